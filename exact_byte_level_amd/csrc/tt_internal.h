// tt_internal.h -- layouts shared by the host table builder and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tt {

// ---------------------------------------------------------------- pre-tokenizer
constexpr int TILE = 1024;              // bytes per pre-tokenizer workgroup
constexpr int PT_THREADS = 256;         // threads per pre-tokenizer workgroup
constexpr int PT_CHUNK = TILE / PT_THREADS;  // 4 contiguous bytes per thread
constexpr int HALO = 16;                // context bytes kept on each side of a tile
constexpr int SPAN = TILE + 2 * HALO;   // decoded positions per tile
constexpr int BMAP_WORDS = (SPAN + 8 + 31) / 32;  // sequence-boundary bitmap
constexpr int RAW_WORDS = (SPAN + 16) / 16;       // raw tile bytes staged in LDS, 16 B words

// Char classes of the run decomposition.  WS = whitespace other than CR/LF,
// WN = CR or LF.  CONT marks a UTF-8 continuation byte, OUT a position
// outside the text.  NONE stands for "no char" (text or sequence edge).
enum : uint32_t { C_NONE = 0, C_L = 1, C_N = 2, C_O = 3, C_WS = 4, C_WN = 5, C_CONT = 6, C_OUT = 7 };

// Per-position code (uint16 in LDS):
//   bits 0-2 class, bit 3 first char of its sequence, bit 4 last char of its
//   sequence, bits 5-8 contraction letter (1..8 = s t r e v m l d, case
//   folded), bit 9 ASCII upper case, bit 10 U+0020, bit 11 apostrophe,
//   bit 12 invalid UTF-8 here, bits 13-14 byte length - 1.
constexpr uint32_t K_SEQ_START = 1u << 3;
constexpr uint32_t K_SEQ_LAST = 1u << 4;
constexpr int K_LETTER_SHIFT = 5;
constexpr uint32_t K_UPPER = 1u << 9;
constexpr uint32_t K_SP = 1u << 10;
constexpr uint32_t K_AP = 1u << 11;
constexpr uint32_t K_BAD = 1u << 12;
constexpr int K_LEN_SHIFT = 13;
constexpr uint32_t K_SLASH = 1u << 15;  // '/'
constexpr int K_FINE_SHIFT = 16;        // 32-bit codes: the Unicode class of a multibyte char (4 bits),
                                        // 7 for ASCII punctuation and symbols
constexpr uint32_t K_CJK = 1u << 20;    // 32-bit codes: a CJK ideograph (U+4E00..U+9FA5) or kana (U+3040..U+30FF)
enum : uint32_t { LT_S = 1, LT_T = 2, LT_R = 3, LT_E = 4, LT_V = 5, LT_M = 6, LT_L = 7, LT_D = 8 };

// ------------------------------------------------------------------------- BPE
constexpr uint32_t RANK_NONE = 0xFFFFFFFFu;
constexpr int ID_BITS = 20;             // token ids < 2^20
constexpr uint32_t ID_MASK = (1u << ID_BITS) - 1;

// 40-bit key of the pair (x, y) (host-side maps).
__host__ __device__ inline uint64_t pair_key(uint32_t x, uint32_t y) {
  return ((uint64_t)x << ID_BITS) | (uint64_t)y;
}
// Pair-rank table for pairs with an operand >= 256 (byte pairs have their own
// direct table): a two-choice (cuckoo) table of 16-byte buckets of two slots
// {key, rank}.  With ids below 2^v (v >= 16 chosen at load time from the
// vocabulary), the 32-bit slot key is (x << (32 - v)) | (y >> p), p = 2 v -
// 32, and the buckets are split into 2^p partitions by (x ^ y) mod 2^p: a
// pair's two buckets lie in its partition, so the partition restores the low
// bits of y that the key drops.  A slot is then 8 bytes and the table holds
// up to 0.8 keys per slot.  Empty slots are {0, RANK_NONE} (no key of the
// table is 0: one of its ids is >= 256).  A lookup is two independent
// 16-byte loads and four compares.
__host__ __device__ inline uint32_t pair_slot_key(uint32_t x, uint32_t y, int kshift, int pbits) {
  return (x << kshift) | (y >> pbits);
}
// Bucket choices of (x, y): m = the xor of two 24-bit products (exact for
// ids < 2^20); choice i = the top bits of the 32-bit product of m's low 24
// bits and PAIR_MUL_i: two independent full-rate 24-bit products of m, which
// a probe computes side by side.
constexpr uint32_t PAIR_MUL_X = 0x9E3779u, PAIR_MUL_Y = 0x7FEB35u;
constexpr uint32_t PAIR_MUL_1 = 0xEBCA6Bu, PAIR_MUL_2 = 0xB2AE35u;
__host__ __device__ inline uint32_t pair_mix(uint32_t x, uint32_t y) {
  return (uint32_t)(x * PAIR_MUL_X) ^ (uint32_t)(y * PAIR_MUL_Y);
}
__host__ __device__ inline uint32_t pair_choice(uint32_t m, uint32_t mul) { return (m & 0xFFFFFFu) * mul; }

// Whole-pre-token table: buckets of CACHE_SLOTS entries in one 128-byte line
// (struct of arrays).  Entry k holds the piece bytes zero-padded into w0[k] /
// w1[k] (little endian) and meta[k] = (id << 5) | len, len in 2..16; a slot
// with len 0 is empty.  Bit 31 of meta[0] is set if some key whose hash lands
// in this bucket (or an earlier one of its probe run) was placed in a later
// bucket: a lookup stops at the first bucket without it.
constexpr int CACHE_MAXLEN = 16;
constexpr int CACHE_SLOTS = 4;
constexpr uint32_t CACHE_MORE = 1u << 31;
struct alignas(128) CacheBucket {
  uint32_t meta[CACHE_SLOTS];
  uint32_t pad0[4];
  uint64_t w0[CACHE_SLOTS];
  uint64_t w1[CACHE_SLOTS];
  uint64_t pad1[4];
};
__host__ __device__ inline uint32_t cache_hash(uint64_t w0, uint64_t w1, uint32_t len, int shift) {
  uint64_t h = (w0 ^ (uint64_t)len * 0xD6E8FEB86659FD93ull) * 0x9E3779B97F4A7C15ull;
  h ^= h >> 29;
  h = (h ^ w1) * 0xBF58476D1CE4E5B9ull;
  h ^= h >> 31;
  return (uint32_t)((h * 0x94D049BB133111EBull) >> shift);
}

// Device-resident tables of the loaded tokenizer (passed by value).
// Whole-word table (the whole-word rule, for pieces longer than
// CACHE_MAXLEN bytes): open addressing over entries
// hash << 32 | length << ID_BITS | id (0 = empty), the hash over the piece's
// bytes read as little-endian 8-byte words (the last one zero-padded); a hit
// is confirmed against the token's bytes.
constexpr int WORD_MAXLEN = 2048;  // longest token the rule serves
__host__ __device__ inline uint64_t word_hash_init(uint32_t len) { return 0x9E3779B97F4A7C15ull * ((uint64_t)len + 1); }
__host__ __device__ inline uint64_t word_hash_step(uint64_t h, uint64_t word) {
  h = (h ^ word) * 0xFF51AFD7ED558CCDull;
  return h ^ (h >> 32);
}

// The classic encoding of RUN_BYTES copies of one byte value: token count,
// ids, and the byte offset of each token (a stitched chunk that is a run of
// one byte takes it from here instead of merging).
constexpr int RUN_BYTES = 32;
struct RunChunk {
  uint32_t cnt;
  uint32_t id[RUN_BYTES];
  uint8_t pos[RUN_BYTES];
};

struct Tables {
  const uint32_t* byte_pair;    // [65536] rank of (x, y), x, y < 256, or RANK_NONE
  const uint4* pair_tab;        // [2^(32 - pair_shift + pair_pbits)] two-choice buckets of two {key, rank} slots
  const CacheBucket* cache;     // [cache_nb]
  const uint32_t* tok_len;      // [2^ID_BITS] byte length of every token (0 past the vocabulary)
  const uint64_t* kids;         // [merges] operands of the merge of rank r: left | right << 32
  const struct RunChunk* runs;  // [256] the encoding of RUN_BYTES copies of each byte
  int pair_shift;               // 32 - (log2(buckets) - pair_pbits): hash bits above the partition
  int pair_kshift;              // 32 - v (slot key: x << pair_kshift | y >> pair_pbits)
  int pair_pbits;               // p = 2 v - 32: partitions 2^p
  uint32_t cache_mask;          // cache_nb - 1
  int cache_shift;              // 64 - log2(cache_nb)
  int cache_probe;              // max buckets visited by any lookup
  int pattern;
  // whole-word rule (word_maxlen > 0): every token of 2..16 bytes is in the
  // cache, longer ones in word_tab
  const uint64_t* word_tab;     // [word_mask + 1]
  const uint32_t* tok_off;      // [vocabulary + 1] offset of each token's bytes in tok_bytes
  const uint8_t* tok_bytes;     // every token's bytes, back to back
  uint32_t word_mask;
  int word_probe;               // longest probe run in word_tab
  int word_maxlen;              // longest token with the rule on, else 0
};

// Device workspace of one encode.
//
// Counters: the last tile of the compaction pass writes P and the error bits
// and zeroes the other per-call counters.
enum : int {
  CTR_P = 0,             // pieces
  CTR_NLONG = 1,         // (unused: long pieces are counted per queue group, qctr[g][4])
  CTR_ERR = 2,           // ERR_* bits
  CTR_T = 4,             // tokens
  CTR_NHUGE = 5,         // pieces with more than HUGE_TOKENS tokens (huge_list)
  CTR_NFALL = 6,         // pieces longer than BIG_BYTES whose stitching failed (fall_list)
  CTR_RESET_END = 12,    // counters [0, CTR_RESET_END) are per call
  CTR_COUNT = 16
};
enum : uint32_t { ERR_UTF8 = 1u, ERR_OFFSETS = 2u, ERR_UNSUP = 4u };
constexpr int TILE_ERR_SHIFT = 29;     // tile_cnt[t] bits 29-31: ERR_* bits of tile t

constexpr int QGROUPS = 8;
constexpr int QCTR_STRIDE = 32;          // words: 128 bytes
constexpr int QCLASS_MINLEN[4] = {2, 9, 17, 33};

struct Work {
  uint32_t* tile_fwd;    // [ntiles] forward run summary of each tile
  uint32_t* tile_bwd;    // [ntiles] backward run summary
  uint32_t* tile_cnt;    // [ntiles] pre-token starts of each tile | error bits << TILE_ERR_SHIFT
  uint8_t* codes;        // [(ntiles + 1) * TILE] cl100k/o200k-style rules: one code byte per text byte
  uint32_t* tile_tail;   // [ntiles] o200k-style rules: CR/LF/'/' tail summary of each tile
  uint32_t* tile_chain;  // [ntiles] o200k-style rules: contraction-chain map of each tile
  uint16_t* flags;       // [ntiles * PT_THREADS] start bits of each thread's PT_CHUNK bytes
  int32_t* piece_start;  // [n + 1]
  int32_t* piece_cnt;    // [n] tokens of each piece
  int32_t* tmp_ids;      // [n] tokens of the piece starting at byte s live at [s, s + cnt)
  uint32_t* tmp_rank;    // [n] pair ranks for the long-piece merge loop; afterwards, for
                         // offset export, the byte length of chunk k of a huge piece
                         // starting at byte s at [s + k]
  int32_t* tok_off;      // [n + 1] token offset of each piece; [P] = T
  uint32_t* tile_tok;    // [ntiles] tokens of the pieces that start in each tile
  uint32_t* tile_pbase;  // [ntiles] index of the first piece that starts in each tile
  // Pieces longer than BIG_BYTES (stitched in k_compact): at the index of the
  // tile holding the piece's last byte (no two such pieces share one), 1 once
  // some tile found a boundary it could not repair; reset by k_pretok.
  int32_t* big_fail;     // [ntiles]
  // Tokens of stitched pieces that start in each tile: [2t] for the piece
  // that covers the tile's first byte, [2t + 1] for the piece that starts in
  // the tile (both included in tile_tok[t]).
  uint32_t* huge_hc;     // [2 * ntiles]
  int32_t* fall_list;    // [n / BIG_BYTES + 1] pieces whose stitching failed
  // Inputs of more than SB_MIN_TILES tiles: sums over each run of SB_TILES
  // tiles of their piece counts (and the OR of their error bits) and of
  // their token counts, so that a tile's prefix reads O(1) cache lines per
  // thread instead of every tile before it (the kernels' SB instantiations).
  uint32_t* sb_cnt;      // [ntiles / SB_TILES + 1]
  uint32_t* sb_err;      // [ntiles / SB_TILES + 1]
  uint32_t* sb_tok;      // [ntiles / SB_TILES + 1]
  int32_t* long_list;    // [QGROUPS][lcap] pieces of LANE_CAP + 1 .. BIG_BYTES bytes, by tile mod QGROUPS
  int32_t* huge_list;    // [n / (HUGE_TOKENS + 1) + 1] pieces with more than HUGE_TOKENS tokens
  // Pieces for group BPE by class c (<= 8, 16, 32, 64 bytes).  Tile t
  // appends to sub-queue g = t % QGROUPS: queue[c] + g * qcap[c], with its
  // count at qctr[g * QCTR_STRIDE + c] (one cache line per sub-queue group,
  // so that appends from different groups do not meet at one atomic unit);
  // pieces of LANE_CAP + 1 .. BIG_BYTES bytes to long_list + g * lcap,
  // counted at qctr[g * QCTR_STRIDE + 4].
  uint32_t* queue[4];
  uint32_t qcap[4];
  uint32_t lcap;
  uint32_t* qctr;        // [QGROUPS * QCTR_STRIDE]
  uint32_t* ctr;         // [CTR_COUNT]
};

constexpr int SB_TILES = 2048;          // tiles per super-block of the two-level tile prefix
constexpr int SB_MIN_TILES = 16384;     // inputs above this many tiles use it

// ------------------------------------------------------------- BPE tiers
constexpr int LANE_CAP = 64;            // pieces up to this many bytes: group BPE in one wavefront
constexpr int BIG_BYTES = 2048;         // longer pieces: merged by the workgroup of the tile they start in
constexpr int EMIT_THREADS = 256;       // emission workgroup (one tile's pieces)
constexpr int HUGE_TOKENS = 64;         // pieces with more tokens are copied by the whole grid

// ------------------------------------------------------------- no-alloc encode
// tt_encode_noalloc carves its workspace out of one fixed device array of
// NOALLOC_SCRATCH_BYTES (the layout of an input of TT_NOALLOC_MAX_BYTES bytes
// needs about 24.5 bytes per input byte, 49 MiB at 2 MiB).
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)52 << 20;
constexpr int NOALLOC_MAX_DEVICES = 64;

// ------------------------------------------------------------- sessions
constexpr int SESSION_LEVELS = 6;       // window sizes tail << 0 .. tail << 5 before a full encode
// info[] of one repair step (device int64; the host reads it after the step)
enum : int {
  SI_STATUS = 0,   // SPLICED, FULL, NONE (no qualifying p in this window), ODD (bookkeeping mismatch)
  SI_ERROR = 1,    // 0 or a negative TT_* data error code of the window encode
  SI_T = 2,        // tokens of the whole text after the step
  SI_P = 3,        // splice byte
  SI_IOLD = 4,     // index of p among A's token starts
  SI_IWIN = 5,     // index of p - w0 among W's token starts
  SI_TWIN = 6,     // tokens of W
  SI_NEXT_W0 = 7,  // [7, 7 + SESSION_LEVELS): window starts for the next append
  SI_WIN_CNT = 14, // the window encode's count (T or error code)
  SI_COUNT = 16
};
enum : int64_t { SS_NONE = 0, SS_SPLICED = 1, SS_FULL = 2, SS_ODD = 3 };

}  // namespace tt
