// tt_kernels.h -- launchers of the HIP kernels (enqueue only, no host sync).
#pragma once
#include "tt_internal.h"

namespace tt {

// Measurement hook, implemented by the host library: when per-kernel timing
// is on, records a HIP event on `st` after the named kernel's launch.
void prof_mark(const char* name, hipStream_t st);

// Zero the counters, validate batch offsets (if any), and write the piece
// starts (+ sentinel n) to `starts` and P to w.ctr[CTR_P].  n >= 1.
hipError_t launch_pretokenize(const uint8_t* bytes, int64_t n, const int64_t* offs, int nseq, int pattern,
                              const Work& w, int32_t* starts, hipStream_t st);

// BPE of every piece in w.piece_start, then token offsets and ids into out_ids;
// the total goes to w.ctr[CTR_T].
hipError_t launch_bpe_emit(const uint8_t* bytes, int64_t n, const Tables& tb, const Work& w, int32_t* out_ids,
                           hipStream_t st);

// *out = error code if any data error was flagged, else w.ctr[which].
hipError_t launch_finish_count(const Work& w, int which, int64_t* out, hipStream_t st);

// out_off[s] = token offset of sequence s; out_off[nseq] = T or error code.
hipError_t launch_batch_offsets(const int64_t* offs, int nseq, int64_t n, const Work& w, int64_t* out_off,
                                hipStream_t st);

hipError_t launch_write_zeros(int64_t* out, int cnt, hipStream_t st);
hipError_t launch_write_zero_i32(int32_t* out, hipStream_t st);
hipError_t launch_zero_counters(const Work& w, hipStream_t st);
hipError_t launch_check_offsets(const int64_t* offs, int nseq, int64_t n, const Work& w, hipStream_t st);

}  // namespace tt
