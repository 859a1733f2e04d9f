// tt_kernels.h -- launchers of the HIP kernels (enqueue only, no host sync).
#pragma once
#include "tt_internal.h"

namespace tt {

// Measurement hook, implemented by the host library: when per-kernel timing
// is on, records a HIP event on `st` after the named kernel's launch.
void prof_mark(const char* name, hipStream_t st);

// Pre-tokenize (validating the batch offsets, if any): the per-call counters
// zeroed, piece starts (+ sentinel n) to `starts`, P and the error bits to
// w.ctr; *out_np = P or the error code if out_np is given.  With tables `tb`,
// also the first BPE step of every piece (single bytes, single-token table,
// queues for the merge pass).  n >= 1.
hipError_t launch_pretokenize(const uint8_t* bytes, int64_t n, const int64_t* offs, int nseq, int pattern,
                              const Work& w, int32_t* starts, int64_t* out_np, const Tables* tb, hipStream_t st);

// BPE of the queued pieces, then token offsets and ids into out_ids;
// the total goes to w.ctr[CTR_T] and, if out_n is given, T or the error code
// to *out_n.  If out_starts is given it receives the byte offset of every
// token and, at [T], n.
hipError_t launch_bpe_emit(const uint8_t* bytes, int64_t n, const Tables& tb, const Work& w, int32_t* out_ids,
                           int64_t* out_n, int32_t* out_starts, hipStream_t st);

// *out = error code if any data error was flagged, else w.ctr[which].
hipError_t launch_finish_count(const Work& w, int which, int64_t* out, hipStream_t st);

// out_off[s] = token offset of sequence s; out_off[nseq] = T or error code.
hipError_t launch_batch_offsets(const int64_t* offs, int nseq, int64_t n, const Work& w, int64_t* out_off,
                                hipStream_t st);

// Incremental repair step after the window text[w0, n_new) was encoded into
// win_ids / win_starts (count in info[SI_WIN_CNT]): choose the splice byte
// and, if one qualifies, copy the window's tokens from it over ids / starts
// (t_old tokens of text[0, n_old)).  Results and the next append's window
// starts go to info (device int64[SI_COUNT]), and a copy of info, once final,
// to info_out (the device address of pinned, mapped host memory).
hipError_t launch_splice(const uint8_t* text, int64_t w0, int64_t n_old, int64_t n_new, int pattern, int64_t tail,
                         int32_t* ids, int32_t* starts, int64_t t_old, const int32_t* win_ids,
                         const int32_t* win_starts, const Work& w, int64_t* info, int64_t* info_out, hipStream_t st);
// After a full encode of text[0, n) with its count in info[SI_WIN_CNT].
hipError_t launch_session_full(const uint8_t* text, int64_t n, int64_t tail, const Work& w, int64_t* info,
                               int64_t* info_out, hipStream_t st);

// Device address of the fixed scratch array of the no-alloc encode on the
// current device: looked up with hipGetSymbolAddress on the first call per
// device, then kept.  Allocates nothing.
hipError_t scratch_address(void** out);

hipError_t launch_write_zeros(int64_t* out, int cnt, hipStream_t st);
hipError_t launch_write_zero_i32(int32_t* out, hipStream_t st);
hipError_t launch_zero_counters(const Work& w, hipStream_t st);
hipError_t launch_check_offsets(const int64_t* offs, int nseq, int64_t n, const Work& w, hipStream_t st);

}  // namespace tt
