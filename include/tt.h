/* tt.h -- exact fresh-session byte-level BPE tokenization on one gfx950 GPU.
 *
 * C ABI of libtt.so.  The library reproduces, bit for bit, a sequential
 * ordered-rule regex pre-tokenizer followed by classic byte-level BPE on every
 * pre-token (TokTier, arXiv:2607.29678v1, summary page: the factorisation
 * F = E* o G of Appendix A.1; the run-decomposition pre-tokenizer of §4.1; the
 * per-piece GPU BPE of §4.2; the CPU-sync-free, graph-capturable single
 * request path of §4.3; IDs only, raw array output, §4.3 / §4.4).
 *
 * Conventions
 *  - One tokenizer is loaded per process.  All calls are serialised by the
 *    caller: the device workspace is shared, so two encodes that overlap in
 *    time (on any streams) race.
 *  - Token ids: 0..255 are raw byte values; the merge of rank r makes id
 *    256 + r.  Ids are int32.
 *  - Text is UTF-8 with no BOM handling (U+FEFF is an ordinary char).  A
 *    "char" is a Unicode code point.
 *  - Return values: 0 on success or a negative TT_E* code.  Codes returned
 *    by tt_encode / tt_encode_batch / tt_pretokenize cover only synchronous
 *    argument, state and launch errors; data errors (invalid UTF-8, bad batch
 *    offsets) are written on the device into the count the caller reads.
 */
#ifndef TT_H
#define TT_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TT_OK          0
#define TT_EINVAL     -1  /* bad argument (null pointer, negative size, bad pattern id) */
#define TT_ETABLE     -2  /* merge table invalid (see tt_load_bpe) */
#define TT_ENOMEM     -3  /* host or device allocation failed */
#define TT_EHIP       -4  /* a HIP runtime call or kernel launch failed */
#define TT_EUTF8      -5  /* input is not valid UTF-8 (device-side data error) */
#define TT_ENOTLOADED -6  /* no tokenizer loaded */
#define TT_EOFFSETS   -7  /* batch offsets not monotone / not ending at n (device-side) */
#define TT_ETOOBIG    -8  /* size beyond the library's limits or the tt_reserve size */
#define TT_ESTALE     -9  /* tokenizer replaced since the session was reset (sessions below) */
#define TT_EUNSUPPORTED -10 /* o200k-style rules: a device-side check that every contraction
                              chain's attachment was fixed where it decides a split failed.  The
                              carried chain state covers every chain, so no input is known to
                              reach it; it stays so that such a case could never pass as a
                              wrong split */

#define TT_PATTERN_GPT2   0  /* GPT-2-style rules: lower-case contractions, ' ?letters', ' ?digits',
                                ' ?other', whitespace with the not-followed-by-non-space rule */
#define TT_PATTERN_CL100K 1  /* cl100k-style rules: ASCII case-insensitive contractions, letters
                                with one optional non-letter/digit/newline prefix, 1-3 digit
                                groups, punctuation absorbing following CR/LF, whitespace up to
                                the last CR/LF, then the lookahead rule */
#define TT_PATTERN_O200K  2  /* o200k-style rules: words split by case (upper-type Lu/Lt/Lm/Lo/marks,
                                lower-type Ll/Lm/Lo/marks) with one optional non-letter/mark/digit/
                                newline prefix and an attached ASCII case-insensitive contraction,
                                1-3 digit groups, punctuation absorbing CR, LF and '/', whitespace
                                up to the last CR/LF run, then the lookahead rule.  Sessions
                                (incremental repair) are not offered under these rules. */
#define TT_PATTERN_DEEPSEEK 3 /* DeepSeek-style rules: digit groups of 1-3 and runs of CJK ideographs
                                and kana cut out first; then on each piece by itself: ASCII
                                punctuation followed by ASCII letters, letters/marks with one
                                optional non-CR/LF/letter/punctuation/symbol prefix, ' ?'
                                punctuation/symbol runs absorbing CR/LF, whitespace up to the
                                last CR/LF run, the lookahead rule; other chars stand alone.
                                Sessions are not offered under these rules. */

/* Maximum merges: ids must fit in 20 bits. */
#define TT_MAX_MERGES (1048576 - 256)
/* Maximum bytes of one encode call (offsets are int32 inside the library). */
#define TT_MAX_BYTES  ((int64_t)1 << 30)

/* tt_load_bpe -- load a byte-level BPE merge table and a rule set.
 *
 * Defines the reference tokenizer every encode must equal id for id
 * (TokTier summary page, §1.3: outputs identical to the reference
 * tokenizer, never an approximation): the rule set is the pre-tokenizer G and
 * the merge table the per-piece BPE E of the factorisation F = E* o G
 * (Appendix A.1).
 *
 * merges     host int32[n_merges][2]: (left id, right id) of merge k.
 * ranks      host int32[n_merges]: rank of merge k, a permutation of
 *            0..n_merges-1; merge k makes token id 256 + ranks[k].  May be
 *            NULL, meaning ranks[k] = k.
 * n_merges   0 .. TT_MAX_MERGES.  0 means ids are the UTF-8 bytes.
 * pattern_id TT_PATTERN_GPT2, TT_PATTERN_CL100K, TT_PATTERN_O200K or TT_PATTERN_DEEPSEEK.
 *
 * The table must be consistent: both operands of the merge of rank r are ids
 * below 256 + r (every table learned by BPE training is), and no pair may
 * appear twice.  Otherwise TT_ETABLE and nothing changes.  The arrays are
 * copied; the caller may free them on return.  Builds the device pair-rank
 * tables and the whole-pre-token cache (each token whose own BPE is itself),
 * synchronises the device, and replaces any previously loaded tokenizer.
 * The old tables are freed, so a HIP graph captured before the call must not
 * be replayed after it; the call also ends any tt_reserve (see there).
 * Returns TT_OK, TT_EINVAL, TT_ETABLE, TT_ENOMEM or TT_EHIP.
 */
int tt_load_bpe(const int32_t* merges, const int32_t* ranks, int64_t n_merges, int32_t pattern_id);

/* Option of tt_load_bpe_ex: the whole-word rule of the Llama family
 * (ignore_merges; TokTier summary page, §4.2: the whole pre-token is first
 * matched against the vocabulary, and a match skips the merges).  A piece
 * whose bytes are those of a token becomes that one token (the smallest id
 * if several tokens have the same bytes); any other piece is merged as
 * usual.  Tables learned by BPE training have no token that its own BPE
 * fails to reach, so there the rule changes nothing; it matters for tables
 * that do. */
#define TT_LOAD_IGNORE_MERGES 1u

/* tt_load_bpe_ex -- tt_load_bpe with options.
 *
 * flags      0 (same as tt_load_bpe) or TT_LOAD_IGNORE_MERGES.  With the
 *            rule, every token of 2..16 bytes goes into the whole-pre-token
 *            cache and longer tokens into a hashed whole-word table whose
 *            hits are confirmed byte by byte; tokens longer than 2048 bytes
 *            are not supported (TT_ETABLE).
 * Other arguments, effects and return values as tt_load_bpe; unknown flag
 * bits give TT_EINVAL.
 */
int tt_load_bpe_ex(const int32_t* merges, const int32_t* ranks, int64_t n_merges, int32_t pattern_id,
                   uint32_t flags);

/* tt_reserve -- size the device workspace for inputs of up to max_bytes
 * bytes and up to max_seqs batch sequences, and fix it there.
 *
 * The pages' single-request path sizes its buffers ahead in buckets so that
 * the host never reads a count to size a kernel and the whole chain can run
 * as one captured graph (TokTier summary page, §4.3); this call is that
 * bucket.  Without a reservation an encode that needs more workspace grows it
 * (which synchronises the device and frees the old buffer).  tt_reserve
 * sizes the workspace for exactly max_bytes, rounded up to a multiple of
 * 1 KiB and to at least 64 KiB (freeing a larger one left by earlier calls),
 * and from then on never reallocates it: an encode, batch, pretokenize or
 * session that needs more returns TT_ETOOBIG instead, so a HIP graph
 * captured after the call stays valid.  The
 * reservation (and every graph captured under it) ends at the next
 * tt_reserve, tt_load_bpe / tt_load_bpe_ex or tt_free; a later tt_reserve may
 * resize.  Returns TT_OK, TT_EINVAL, TT_ETOOBIG, TT_ENOMEM, TT_EHIP or
 * TT_ENOTLOADED. */
int tt_reserve(int64_t max_bytes, int32_t max_seqs);

/* tt_encode -- token ids of one text.
 *
 * Exact fresh-session tokenization of one text on the GPU (TokTier summary
 * page, §4): pre-tokenization by run decomposition (§4.1), BPE of every
 * pre-token (§4.2), ids as a raw device array with no host synchronisation
 * inside the call (§4.3) and no byte offsets (§4.4; tt_encode_offsets adds
 * them).
 *
 * dev_bytes  device uint8[n]: the UTF-8 text (caller-owned).
 * n          0 .. TT_MAX_BYTES-1.
 * out_ids    device int32[>= n] (caller-owned).  T <= n always holds, so a
 *            capacity of n never overflows; this is not checked.
 * out_n      device int64[1] (caller-owned): receives T >= 0, or TT_EUTF8
 *            if the text is not valid UTF-8 (out_ids is then unspecified).
 * stream     HIP stream the work is enqueued on (0 = null stream).
 *
 * Enqueues only: no host synchronisation, no allocation once the workspace is
 * large enough (see tt_reserve), graph-capturable.  n == 0 gives *out_n = 0.
 * Returns TT_OK, TT_EINVAL, TT_ETOOBIG (also: n above a tt_reserve),
 * TT_ENOMEM, TT_EHIP or TT_ENOTLOADED.
 */
int tt_encode(const uint8_t* dev_bytes, int64_t n, int32_t* out_ids, int64_t* out_n,
              hipStream_t stream);

/* Largest input of tt_encode_noalloc. */
#define TT_NOALLOC_MAX_BYTES ((int64_t)1 << 21)

/* tt_encode_noalloc -- tt_encode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).
 *
 * Arguments, output and enqueue-only contract as tt_encode, with n at most
 * TT_NOALLOC_MAX_BYTES (2 MiB; larger gives TT_ETOOBIG before any device
 * work).  The call allocates nothing, ever: instead of the library's
 * workspace it uses a fixed 52 MiB device array that every GPU the library
 * is loaded on holds until the process ends, looked up once per device.
 * Every call on one GPU shares that array, which keeps the last call's
 * contents (the kernels reset what they need), so two calls that overlap in
 * time on one GPU race, as do a no-alloc call and any other encode.  The
 * merge tables still come from tt_load_bpe.  Returns TT_OK, TT_EINVAL,
 * TT_ETOOBIG, TT_EHIP or TT_ENOTLOADED.
 */
int tt_encode_noalloc(const uint8_t* dev_bytes, int64_t n, int32_t* out_ids, int64_t* out_n,
                      hipStream_t stream);

/* tt_encode_batch -- token ids of n_seqs independent texts in one call.
 *
 * Each text is a fresh session tokenized on its own (the factorisation of
 * TokTier summary page, Appendix A.1, applied text by text), all of them in
 * one enqueue-only launch chain (§4.3).
 *
 * dev_bytes    device uint8[n]: the texts, concatenated.
 * n            total bytes; must equal dev_offsets[n_seqs].
 * dev_offsets  device int64[n_seqs + 1]: text s is bytes
 *              [dev_offsets[s], dev_offsets[s+1]); dev_offsets[0] == 0,
 *              non-decreasing (empty texts are allowed).  Each text is a
 *              separate fresh session: its end is end-of-text for the
 *              lookahead rules and no pre-token crosses it.
 * n_seqs       >= 1.
 * out_ids      device int32[>= n].
 * out_offsets  device int64[n_seqs + 1]: ids of text s are
 *              out_ids[out_offsets[s] .. out_offsets[s+1]).  On a data error
 *              out_offsets[n_seqs] receives TT_EUTF8 or TT_EOFFSETS.
 * stream       HIP stream.
 * Same enqueue-only contract as tt_encode.
 */
int tt_encode_batch(const uint8_t* dev_bytes, int64_t n, const int64_t* dev_offsets, int32_t n_seqs,
                    int32_t* out_ids, int64_t* out_offsets, hipStream_t stream);

/* tt_pretokenize -- the pre-tokenizer alone (run decomposition, §4.1):
 * byte offsets of every pre-token start.
 *
 * dev_offsets may be NULL (one text of n bytes) or as in tt_encode_batch.
 * out_starts   device int32[>= n + 1]: piece starts in increasing order,
 *              followed by the sentinel n.
 * out_np       device int64[1]: number of pieces P, or TT_EUTF8 / TT_EOFFSETS.
 * Same enqueue-only contract as tt_encode.
 */
int tt_pretokenize(const uint8_t* dev_bytes, int64_t n, const int64_t* dev_offsets, int32_t n_seqs,
                   int32_t* out_starts, int64_t* out_np, hipStream_t stream);

/* tt_encode_offsets -- token ids plus the byte span of every token: the
 * device-side byte-offset export (TokTier summary page, Path C of §8 and of
 * Appendix E; §4.4 and §7 note that the pages' GPU path emits ids only and
 * falls back to the CPU when offsets are needed).
 *
 * dev_bytes, n, dev_offsets, n_seqs: as in tt_pretokenize (dev_offsets NULL
 *              means one text of n bytes).
 * out_ids      device int32[>= n]: the same ids tt_encode / tt_encode_batch
 *              give.
 * out_starts   device int32[>= n + 1]: token i covers bytes
 *              [out_starts[i], out_starts[i+1]) of dev_bytes -- offsets into
 *              the whole buffer, also for a batch -- and out_starts[T] = n.
 *              Token byte spans never split a pre-token boundary but may
 *              split a multi-byte char (byte-level tokens).
 * out_counts   device int64: with dev_offsets NULL, [1] receiving T or
 *              TT_EUTF8; else [n_seqs + 1] as out_offsets of tt_encode_batch.
 *              On a data error out_ids and out_starts are unspecified.
 * Same enqueue-only contract as tt_encode.  Each token's byte length comes
 * from a table built by tt_load_bpe; the extra device work over tt_encode is
 * one gather per token and, for a pre-token of more than 4,096 tokens, one
 * extra read of its ids.
 */
int tt_encode_offsets(const uint8_t* dev_bytes, int64_t n, const int64_t* dev_offsets, int32_t n_seqs,
                      int32_t* out_ids, int32_t* out_starts, int64_t* out_counts, hipStream_t stream);

/* ---------------------------------------------------------------- sessions
 *
 * Incremental repair (TokTier summary page, §3.3, with the splicing theorem
 * of Appendix A.2): a session keeps a growing text, its token ids and the byte
 * start of every token in device memory.  After an append only a tail window
 * (the last tail_bytes of the old text plus the appended bytes) is encoded,
 * and its tokens are spliced in at a pre-token start that the old and the new
 * tokenization provably share: at least 16 bytes into the window and 20 bytes
 * before the old end, and for cl100k-style rules also a change of char class
 * (letter / number / whitespace / other), the pages' synchronisation boundary.
 * Without such a start the window doubles, up to 5 times (§3.3), then the
 * whole text is encoded.  The result always equals a fresh encode of the
 * whole text.  Sessions belong to the loaded tokenizer: after tt_load_bpe or
 * tt_free a session must be reset (TT_ESTALE).  Session calls are
 * host-synchronous (they wait for their stream) and serialised with every
 * other call of the library.
 */
typedef struct tt_session tt_session;

/* tt_session_create -- a session for texts of up to capacity bytes.
 * tail_bytes: first window size behind the old end (0 = 2048; else
 * 64 .. 2^24).  Allocates device memory for the text, ids, token starts and
 * window scratch (17 bytes per byte of capacity) and sizes the shared
 * workspace for capacity bytes.  Needs a loaded tokenizer.  *out receives the
 * session.  Returns TT_OK, TT_EINVAL, TT_ETOOBIG, TT_ENOMEM, TT_EHIP or
 * TT_ENOTLOADED. */
int tt_session_create(int64_t capacity, int64_t tail_bytes, tt_session** out);

/* tt_session_destroy -- synchronise the device and free the session. */
int tt_session_destroy(tt_session* s);

/* tt_session_reset -- start the session over with dev_bytes[0, n) (device,
 * caller-owned, copied): a full encode, ids and byte starts kept in the
 * session.  n <= capacity (else TT_ETOOBIG).  Invalid UTF-8 gives TT_EUTF8
 * and leaves the session empty and unusable until the next reset. */
int tt_session_reset(tt_session* s, const uint8_t* dev_bytes, int64_t n, hipStream_t stream);

/* tt_session_append -- append dev_delta[0, nd) (device, caller-owned,
 * copied) and repair the tokens.  If the text with the append would not be
 * valid UTF-8 (including a char split across appends) the call returns
 * TT_EUTF8 and the session keeps its previous text and tokens.
 * out_info (host int64[4], may be NULL): [0] windows doubled before the splice
 * (0..5), or -1 if the whole text was encoded; [1] bytes encoded by the last
 * window; [2] splice byte; [3] tokens of the whole text.  nd == 0 changes
 * nothing.  Returns TT_OK, TT_EINVAL (not reset), TT_ETOOBIG (capacity),
 * TT_ESTALE, TT_EUTF8 or TT_EHIP. */
int tt_session_append(tt_session* s, const uint8_t* dev_delta, int64_t nd, int64_t* out_info, hipStream_t stream);

/* tt_session_view -- the session's device arrays, valid until the next call
 * on the session: text uint8[n], ids int32[T], starts int32[T + 1] (token i
 * covers bytes [starts[i], starts[i+1]); starts[T] = n).  Any output pointer
 * may be NULL. */
int tt_session_view(const tt_session* s, const uint8_t** text, int64_t* n, const int32_t** ids,
                    const int32_t** starts, int64_t* T);

/* tt_session_read -- enqueue device-to-device copies of the session's text
 * (n bytes), ids (T) and token starts (T + 1) into caller buffers (device;
 * any may be NULL).  Returns TT_OK, TT_EINVAL or TT_EHIP. */
int tt_session_read(const tt_session* s, uint8_t* text_out, int32_t* ids_out, int32_t* starts_out,
                    hipStream_t stream);

/* tt_char_class -- host query of the compiled Unicode class table:
 * 0 other, 1 upper/title-case letter (Lu, Lt), 2 lower-case letter (Ll),
 * 3 modifier/other letter (Lm, Lo), 4 mark (\p{M}), 5 number (\p{N}),
 * 6 White_Space, 7 punctuation (\p{P}), 8 symbol (\p{S}); -1 if cp is not
 * a Unicode scalar value.  No device work. */
int tt_char_class(uint32_t cp);

/* tt_profile -- per-kernel timing of later calls (a measurement aid).
 * enable != 0 creates a small pool of HIP events (this allocates: switch it
 * on outside any graph capture); from then on every encode records an event
 * on its stream after each kernel launch.  enable == 0 synchronises and
 * destroys them.  Returns TT_OK or TT_EHIP. */
int tt_profile(int enable);

/* tt_profile_read -- kernel names and durations (ms, time from the previous
 * event to the event after this kernel) of the last encode / pretokenize
 * call.  Waits for that call to finish.  names[i] are static strings.
 * Returns the number of entries written (<= cap), or TT_EINVAL if profiling
 * is off, or TT_EHIP. */
int tt_profile_read(const char** names, float* ms, int cap);

/* tt_free -- release the tokenizer tables and the workspace (synchronises);
 * ends any tt_reserve and invalidates captured graphs.  Housekeeping: no
 * passage of the pages defines it. */
void tt_free(void);

/* tt_strerror -- static description of a TT_* code.  Housekeeping: no
 * passage of the pages defines it. */
const char* tt_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* TT_H */
