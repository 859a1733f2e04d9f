// tt_kernels.hip -- HIP kernels (gfx950, wave64) of exact byte-level BPE tokenization.
//
// Method: TokTier (arXiv:2607.29678v1), summary page.
//   §4.1  run decomposition: the ordered-rule regex split is reproduced in
//         parallel from char classes, maximal same-class runs, the offset in a
//         run, a few chars of context and run-level facts (k_tile_summary,
//         k_pretok, k_compact);
//   §4.2  BPE per piece, pieces independent, tiered by length: the
//         whole-piece lookup of single-token pieces (the exact form of the
//         vocabulary short-circuit the page mentions) and queueing by length
//         class in k_compact; group merges of up to 64-byte pieces, one byte
//         position per lane, and exact global-minimum rounds for longer
//         pieces, a wavefront each (k_bpe_merge); past 2 KiB, 32-byte chunks
//         encoded alone and stitched at compatible token pairs by every tile
//         the piece covers (stitch_piece, in k_compact), with the exact
//         rounds by one workgroup as the fallback (big_fallback);
//   §4.3  no host synchronisation between kernels: every size a kernel needs
//         after the first is read on the device (grids are sized for the
//         worst case and exit early), so the chain is graph-capturable.
//
// Passes of one encode: k_tile_summary (every rule set but GPT-2 style),
// k_pretok, k_compact, k_bpe_merge, k_emit.
//
// Hot-path data (all integer; no floating point, no MFMA):
//   bytes   uint8[n]         caller's UTF-8 text
//   codes   uint8[n]         one code byte per text byte (class index, run flags)
//   flags   uint16 per 4 B   pre-token start bits
//   starts  int32[P + 1]     piece byte offsets + sentinel n
//   tmp_ids int32[n]         tokens of the piece starting at byte s at [s, s+cnt)
//   out_ids int32[T]         caller's output
#include "tt_kernels.h"
#include "unicode_table.inc"

namespace tt {

// ------------------------------------------------------------ Unicode classes

constexpr int UNI_L1_PAD = (TT_UNI_L1_SIZE + 15) / 16 * 16;
constexpr int UNI_L2_PAD = TT_UNI_NBLOCKS * 128;
alignas(16) __device__ const uint8_t g_uni_l1[UNI_L1_PAD] = {TT_UNI_L1_DATA};
alignas(16) __device__ const uint8_t g_uni_l2[UNI_L2_PAD] = {TT_UNI_L2_DATA};

// Unicode class (the table's 4-bit value) -> the char class of the rules.
constexpr uint32_t UNI_SINGLE = 9;  // single-class blocks 0..8
__device__ __forceinline__ uint32_t uni_cls(uint32_t u) {
  return u - 1u < 3u ? C_L : u == 5u ? C_N : u == 6u ? C_WS : C_O;
}

struct alignas(16) AsciiTab {
  uint16_t v[128];
};

constexpr uint16_t ascii_code(int c) {
  uint16_t code = C_O;
  bool upper = c >= 'A' && c <= 'Z';
  bool lower = c >= 'a' && c <= 'z';
  if (upper || lower) {
    int lc = c | 0x20;
    uint16_t lt = lc == 's' ? LT_S : lc == 't' ? LT_T : lc == 'r' ? LT_R : lc == 'e' ? LT_E
                : lc == 'v' ? LT_V : lc == 'm' ? LT_M : lc == 'l' ? LT_L : lc == 'd' ? LT_D : 0;
    code = (uint16_t)(C_L | (lt << K_LETTER_SHIFT) | (upper ? K_UPPER : 0));
  } else if (c >= '0' && c <= '9') {
    code = C_N;
  } else if (c == '\n' || c == '\r') {
    code = C_WN;
  } else if (c == '\t' || c == 0x0b || c == 0x0c || c == ' ') {
    code = (uint16_t)(C_WS | (c == ' ' ? K_SP : 0));
  } else if (c == '\'') {
    code = (uint16_t)(C_O | K_AP);
  } else if (c == '/') {
    code = (uint16_t)(C_O | K_SLASH);
  }
  return code;
}

constexpr AsciiTab make_ascii() {
  AsciiTab t{};
  for (int c = 0; c < 128; ++c) t.v[c] = ascii_code(c);
  return t;
}

__device__ const AsciiTab g_ascii = make_ascii();

// Wave-uniform copy of a value every lane already agrees on.  Loops that
// contain wave collectives (shuffles, ballots) take their exit condition from
// such a value, so the compiler keeps the loop uniform and never splits lanes
// of one wavefront onto different paths around a collective.
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ uint32_t cls_of(uint32_t code) { return code & 7u; }
__device__ __forceinline__ bool is_w(uint32_t k) { return k == C_WS || k == C_WN; }
__device__ __forceinline__ bool is_char(uint32_t code) { return cls_of(code) - 1u < 5u; }
__device__ __forceinline__ int clen(uint32_t code) { return (int)((code >> K_LEN_SHIFT) & 3u) + 1; }

// Shared-memory state of one pre-tokenizer tile.
// Codes live in LDS at a padded index (one spare dword per 16 positions), so
// threads that each walk their own run of 16 positions hit distinct banks.
constexpr int CODE_SLOTS = SPAN + 2 * (SPAN / 16) + 4;
__device__ __forceinline__ int cix(int j) { return j + 2 * (j >> 4); }

struct TileSmem {
  uint4 raw[RAW_WORDS];   // bytes of positions [t0 - HALO, t0 - HALO + 16 * RAW_WORDS); 0 outside the text
  uint16_t code[CODE_SLOTS];
  alignas(16) uint16_t ascii[128];
  uint32_t bmap[BMAP_WORDS];
  uint32_t red[8];
  uint64_t bsw[7][17];   // cl100k/o200k-style rules: bit planes of the span's chars (64 per entry)
  uint32_t cbits[34];    // their start bits by char (tiles with non-ASCII bytes)
  int64_t seq_lo, seq_hi;
  uint32_t carry_fwd, carry_bwd, carry_tail, carry_chain;
  int flag;
  // cl100k-style rules: the span's code bytes (by position), its chars in
  // order (code bytes) and their positions, and the tile's start bits
  alignas(16) uint8_t cb[SPAN + 16];
  alignas(16) uint8_t cc[SPAN + 16];
  uint16_t cpos[SPAN];
  uint32_t sbits[TILE / 32];
  // plen[j]: byte length of the char that ends right before position j (0
  // if unknown: no char start there, or the previous char begins outside the
  // span); filled only when the tile has non-ASCII bytes
  alignas(16) uint8_t plen[SPAN + 16];
};

__device__ __forceinline__ bool bmap_bit(const uint32_t* bm, int j) {
  return (bm[j >> 5] >> (j & 31)) & 1u;
}

// First index s in [0, cnt) with a[s] >= v (cnt if none).
__device__ __forceinline__ int64_t lower_bound_i64(const int64_t* a, int64_t cnt, int64_t v) {
  int64_t lo = 0, hi = cnt;
  while (lo < hi) {
    int64_t mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Stage the tile in LDS: raw bytes of [t0 - HALO, t0 + TILE + HALO + 16) with
// one 16-byte load per thread (byte loads only at the text edges or for an
// unaligned text) and the sequence-boundary bitmap.  Returns (the same in
// every thread) whether any staged byte is >= 0x80.
__device__ bool stage_tile(const uint8_t* __restrict__ bytes, int64_t n, const int64_t* __restrict__ offs,
                           int nseq, int64_t t0, TileSmem& sm) {
  const int tid = threadIdx.x;
  const int64_t base = t0 - HALO;
  const bool aligned = (reinterpret_cast<uintptr_t>(bytes) & 15u) == 0;
  for (int i = tid; i < BMAP_WORDS; i += PT_THREADS) sm.bmap[i] = 0;
  for (int i = tid; i < (SPAN + 16) / 16; i += PT_THREADS) reinterpret_cast<uint4*>(sm.plen)[i] = make_uint4(0u, 0u, 0u, 0u);
  if (tid < 16) reinterpret_cast<uint4*>(sm.ascii)[tid] = reinterpret_cast<const uint4*>(g_ascii.v)[tid];
  uint32_t hi_bits = 0;
  for (int i = tid; i < RAW_WORDS; i += PT_THREADS) {
    const int64_t g = base + 16 * (int64_t)i;
    uint4 v;
    if (aligned && g >= 0 && g + 16 <= n) {
      v = *reinterpret_cast<const uint4*>(bytes + g);
    } else {
      uint32_t wv[4] = {0u, 0u, 0u, 0u};
      for (int k = 0; k < 16; ++k) {
        const int64_t q = g + k;
        if (q >= 0 && q < n) wv[k >> 2] |= (uint32_t)bytes[q] << (8 * (k & 3));
      }
      v = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
    sm.raw[i] = v;
    hi_bits |= v.x | v.y | v.z | v.w;
  }
  if (tid == 0) {
    if (offs) {
      sm.seq_lo = lower_bound_i64(offs, (int64_t)nseq + 1, base);
      sm.seq_hi = lower_bound_i64(offs, (int64_t)nseq + 1, base + SPAN + 8);
    } else {
      sm.seq_lo = 0;
      sm.seq_hi = 0;
    }
  }
  const bool na = __syncthreads_or((hi_bits & 0x80808080u) != 0u);
  if (offs) {
    for (int64_t s = sm.seq_lo + tid; s < sm.seq_hi; s += PT_THREADS) {
      int64_t j = offs[s] - base;
      if (j >= 0 && j < (int64_t)BMAP_WORDS * 32) atomicOr(&sm.bmap[j >> 5], 1u << (j & 31));
    }
  } else if (tid == 0 && base <= 0) {
    int64_t j = -base;
    if (j < (int64_t)BMAP_WORDS * 32) sm.bmap[j >> 5] |= 1u << (j & 31);
  }
  __syncthreads();  // the bitmap is complete before any wavefront reads it
  return na;
}


// UTF-8 decode of four contiguous positions p0 .. p0 + 3 held in registers: wb
// the bytes p0 .. p0 + 7 (0 past the text), bm bit i: a sequence starts at
// p0 + i.  The same codes, computed without branches: byte kinds from the
// count of leading one bits, the continuation bytes of a lead checked
// together as one word, the code point assembled from all four payloads and
// shifted to the char's length; then the table blocks and class bits of the
// four are loaded together, so a thread waits for two global loads, not
// eight.  len[k]: byte length of the char at p0 + k (0 if none starts there).
__device__ __forceinline__ void decode4_regs(uint64_t wb, uint32_t bm, int64_t p0, int64_t n, const uint16_t* ascii,
                                             uint32_t code[4], int len_out[4]) {
  uint32_t cp[4];
  bool tab[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t p = p0 + k;
    const uint32_t w4 = (uint32_t)(wb >> (8 * k));  // bytes p .. p + 3
    const uint32_t b0 = w4 & 255u, b1 = (w4 >> 8) & 255u;
    const uint32_t ones = (uint32_t)__clz(~(b0 << 24));  // leading one bits of b0
    const bool start = (bm >> k) & 1u;
    const bool in = p >= 0 && p < n;
    const bool ascii_b = ones == 0u, cont = ones == 1u;
    const bool lead = ones - 2u <= 2u && b0 >= 0xC2u && b0 <= 0xF4u;
    const uint32_t len = lead ? ones : 1u;
    const uint32_t need = (0xFFFFFFFFu >> (32u - 8u * len)) & ~0xFFu;  // the continuation bytes
    const bool conts = (((w4 & 0xC0C0C000u) ^ 0x80808000u) & need) == 0u;
    const bool seq_ok = ((bm >> (k + 1)) & ((1u << (len - 1u)) - 1u)) == 0u;
    const bool second = !((b0 == 0xE0u && b1 < 0xA0u) || (b0 == 0xEDu && b1 > 0x9Fu) || (b0 == 0xF0u && b1 < 0x90u) ||
                          (b0 == 0xF4u && b1 > 0x8Fu));
    const bool good_mb = lead && conts && seq_ok && p + (int64_t)len <= n && second;
    const bool bad_lead = !ascii_b && !cont && !good_mb;
    const uint32_t clen = bad_lead ? 1u : len;
    const uint32_t full = ((b0 & (0x7Fu >> ones)) << 18) | (((w4 >> 8) & 0x3Fu) << 12) | (((w4 >> 16) & 0x3Fu) << 6) |
                          ((w4 >> 24) & 0x3Fu);
    cp[k] = full >> (6u * (4u - len));
    tab[k] = in && good_mb && (cp[k] >> 8) < (uint32_t)TT_UNI_L1_SIZE;  // else class 0 (other)
    // a continuation byte right after a complete char is stray
    const bool last = p + (int64_t)clen >= n || ((bm >> (k + clen)) & 1u);
    const bool stray = !last && !bad_lead && (((uint32_t)(wb >> (8 * (k + clen))) & 0xC0u) == 0x80u);
    uint32_t c = ascii_b ? (uint32_t)ascii[b0 & 127u] : bad_lead ? (C_O | K_BAD) : 0u;
    // printable ASCII that is not a letter, digit or space: punctuation or a symbol
    if (ascii_b && b0 - 0x21u < 0x5Eu && cls_of(c) == C_O) c |= 7u << K_FINE_SHIFT;
    c |= ((clen - 1u) << K_LEN_SHIFT) | (start ? K_SEQ_START : 0u) | (last ? K_SEQ_LAST : 0u) | (stray ? K_BAD : 0u);
    code[k] = !in ? (uint32_t)C_OUT : cont ? (C_CONT | (start ? K_BAD : 0u)) : c;
    len_out[k] = in && !cont ? (int)clen : 0;
  }
  // class of the multibyte chars: block numbers below UNI_SINGLE are
  // single-class blocks (the number is the class)
  uint32_t blk[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) blk[k] = tab[k] ? (uint32_t)g_uni_l1[cp[k] >> 8] : 0u;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (cls_of(code[k]) == 0u) {
      // a valid multibyte char (class bits still 0)
      const uint32_t u = !tab[k] ? 0u : blk[k] < UNI_SINGLE ? blk[k]
                       : (g_uni_l2[blk[k] * 128u + ((cp[k] & 255u) >> 1)] >> ((cp[k] & 1u) * 4u)) & 15u;
      code[k] |= uni_cls(u) | (u << K_FINE_SHIFT);
      if (cp[k] - 0x4E00u <= 0x9FA5u - 0x4E00u || cp[k] - 0x3040u <= 0x30FFu - 0x3040u) code[k] |= K_CJK;
    }
  }
}

// decode4_regs for the four contiguous span positions j .. j + 3 (j a multiple
// of 4) of a staged tile: writes the codes and the predecessor lengths;
// returns whether a char starting at one of the tile's own positions is
// invalid.
__device__ __forceinline__ bool decode4(int64_t n, int64_t base, int j, TileSmem& sm) {
  const uint32_t* raw32 = reinterpret_cast<const uint32_t*>(sm.raw);
  const uint64_t wb = (uint64_t)raw32[j >> 2] | ((uint64_t)raw32[(j >> 2) + 1] << 32);
  const int sh = j & 31;
  const uint32_t b0w = sm.bmap[j >> 5], b1w = sm.bmap[(j >> 5) + 1];
  const uint32_t bm = sh ? (b0w >> sh) | (b1w << (32 - sh)) : b0w;  // bit i: a sequence starts at j + i
  uint32_t code[4];
  int len[4];
  decode4_regs(wb, bm, base + j, n, sm.ascii, code, len);
  bool bad_own = false;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    sm.code[cix(j + k)] = (uint16_t)code[k];
    if (len[k]) sm.plen[j + k + len[k]] = (uint8_t)len[k];
    if ((code[k] & K_BAD) && j + k >= HALO && j + k < HALO + TILE) bad_own = true;
  }
  return bad_own;
}

// Codes of all SPAN positions (non-ASCII chars classed from the two-level
// Unicode table in global memory, where it stays cached), and for non-ASCII
// tiles the predecessor lengths.
// Returns true if some char starting inside the tile is invalid UTF-8.
__device__ bool decode_span(int64_t n, int64_t t0, bool na, TileSmem& sm) {
  const int tid = threadIdx.x;
  bool bad = false;
  if (!na) {
    // every byte is a one-byte char: class from the ASCII table, sequence
    // edges from the bitmap (no invalid UTF-8 is possible)
    const uint8_t* raw = reinterpret_cast<const uint8_t*>(sm.raw);
    const int64_t base = t0 - HALO;
    for (int j = tid; j < SPAN; j += PT_THREADS) {
      const int64_t p = base + j;
      uint32_t c = C_OUT;
      if (p >= 0 && p < n) {
        c = sm.ascii[raw[j]];
        if (bmap_bit(sm.bmap, j)) c |= K_SEQ_START;
        if (p + 1 >= n || bmap_bit(sm.bmap, j + 1)) c |= K_SEQ_LAST;
      }
      sm.code[cix(j)] = (uint16_t)c;
    }
    __syncthreads();
    return false;
  }
  // four contiguous positions per thread: positions 0 .. 1023, and threads
  // 0 .. 7 the last 32 of the span as well
  bad = decode4(n, t0 - HALO, PT_CHUNK * tid, sm);
  if (tid < (SPAN - PT_CHUNK * PT_THREADS) / PT_CHUNK) bad |= decode4(n, t0 - HALO, PT_CHUNK * (PT_THREADS + tid), sm);
  __syncthreads();
  return bad;
}

// The whole tile: stage, then decode every position.  *non_ascii (same in
// every thread) tells whether any staged byte is >= 0x80.
__device__ bool load_tile(const uint8_t* __restrict__ bytes, int64_t n, const int64_t* __restrict__ offs,
                          int nseq, int64_t t0, TileSmem& sm, bool* non_ascii = nullptr) {
  const bool na = stage_tile(bytes, n, offs, nseq, t0, sm);
  if (non_ascii) *non_ascii = na;
  return decode_span(n, t0, na, sm);
}

// ---------------------------------------------------- run-state scan operators
// Forward state of a range of chars, for the trailing run:
//   bit 0 has chars, bit 1 open (the run reaches the range start and no
//   sequence starts there), bits 2-4 class, bits 5-7 class of the char before
//   the run (C_NONE at a sequence start), bits 8-9 run length mod 3.
struct FwdOp {
  static constexpr uint32_t IDENT = 0;
  __device__ static __forceinline__ uint32_t elem(uint32_t code) {
    uint32_t open = (code & K_SEQ_START) ? 0u : 2u;
    return 1u | open | (cls_of(code) << 2) | (1u << 8);
  }
  __device__ static __forceinline__ uint32_t combine(uint32_t a, uint32_t b) {
    if (!(b & 1u)) return a;
    if (!(a & 1u)) return b;
    if (b & 2u) {
      uint32_t ca = (a >> 2) & 7u, cb = (b >> 2) & 7u;
      if (ca == cb) {
        uint32_t len = ((a >> 8) & 3u) + ((b >> 8) & 3u);  // each < 3: the sum mod 3 by one subtraction
        len -= len >= 3u ? 3u : 0u;
        return (a & 0xFFu) | (len << 8);
      }
      return 1u | (cb << 2) | (ca << 5) | (b & 0x300u);
    }
    return b;
  }
  __device__ static __forceinline__ bool closed(uint32_t a) { return (a & 1u) && !(a & 2u); }
};

// Forward state for the o200k-style CR/LF/'/' tails, of the trailing run of
// tail chars (CR, LF, '/'; none starts a sequence inside the run): bit 0 has
// chars, bit 1 open (the whole range is that run), bit 2 active (a tail
// starts in the run: a CR/LF right after an "other" char), bit 3 the range's
// first char is CR/LF and starts no sequence, bit 4 its last char is
// "other", bit 5 its last char is a tail char, bits 6-11 distance from the
// range end back to the first tail start of the run (saturating at 63),
// bits 12-17 the number of chars (saturating at 63).
struct TailOp {
  static constexpr uint32_t IDENT = 0;
  static constexpr uint32_t SAT = 63;
  __device__ static __forceinline__ uint32_t elem(uint32_t code) {
    const uint32_t k = cls_of(code);
    const bool r = k == C_WN || (code & K_SLASH), ss = (code & K_SEQ_START) != 0u;
    return 1u | (r && !ss ? 2u : 0u) | (k == C_WN && !ss ? 8u : 0u) | (k == C_O ? 16u : 0u) | (r ? 32u : 0u) |
           (1u << 12);
  }
  __device__ static __forceinline__ uint32_t combine(uint32_t a, uint32_t b) {
    if (!(b & 1u)) return a;
    if (!(a & 1u)) return b;
    const uint32_t len = min(SAT, ((a >> 12) & SAT) + ((b >> 12) & SAT));
    uint32_t r = 1u | (a & 8u) | (b & 48u) | (len << 12);
    if (b & 2u) {
      const bool a_act = (a & 32u) && (a & 4u), seed = (b & 8u) && (a & 16u);
      const uint32_t blen = (b >> 12) & SAT;
      const uint32_t d = a_act ? min(SAT, ((a >> 6) & SAT) + blen) : seed ? blen : ((b >> 6) & SAT);
      r |= (a & b & 2u) | ((a_act || seed || (b & 4u)) ? 4u : 0u) | (d << 6);
    } else {
      r |= (b & 4u) | (b & (SAT << 6));
    }
    return r;
  }
  __device__ static __forceinline__ bool closed(uint32_t a) { return (a & 1u) && !(a & 2u); }
};

// Contraction-chain state (o200k-style rules) of a range of chars, as a map
// from the state before the range to the state after it.  Phases: 0 no
// chain and the last char is no letter, 1 no chain after a letter, 2 an
// apostrophe that may start a contraction shape, 3 / 4 that apostrophe and
// r or v / l, 5 a whole shape, 6 inside a run of Lm/Lo/marks that began
// right after a whole shape; phases 2-6 also hold whether that shape
// attaches (a chain's first shape attaches after a letter; each later one
// attaches exactly when the one before did not).  Entry p (5 bits at 5 p,
// phases 0-5): bits 0-2 the phase after, bit 4 the attachment after, taken
// as is or, with bit 3, xor the attachment before; phases 0 and 1 keep bits
// 3-4 clear.  Phase 6 needs no entry: it stays 6 over a range of such marks
// and letters only (bit 30) and otherwise goes where phase 1 goes.  Bit 31:
// the range has chars.
struct ChainOp {
  static constexpr uint32_t IDENT = 0, HAS = 1u << 31, ALLB = 1u << 30, REP = 0x2108421u;
  __device__ static __forceinline__ uint32_t entry(uint32_t f, uint32_t p) { return (f >> (5u * p)) & 31u; }
  __device__ static __forceinline__ bool constant(uint32_t f) {
    return (f & 0x3FFFFFFFu) == (f & 31u) * REP && !(f & 8u);
  }
  // the map of one char: idx its o200k-style class index, ss it starts a sequence
  __device__ static __forceinline__ uint32_t elem(uint32_t idx, bool ss) {
    const uint32_t att = ss ? 0u : 16u, t = idx & 7u;
    if (idx == 3u) {  // an apostrophe: after a whole shape it links, unless a sequence starts
      const uint32_t e5 = ss ? 2u : (2u | 8u | 16u);
      return HAS | 2u | ((2u | att) << 5) | (2u << 10) | ((2u | att) << 15) | ((2u | att) << 20) | (e5 << 25);
    }
    if (idx == 23u && !ss)  // Lm/Lo/mark: after a whole shape, phase 6 keeps its attachment
      return HAS | ALLB | (1u * (REP & 0x1FFFFFu)) | (14u << 25);
    if (idx & 16u) {  // a letter: shape letters go on; any other resets to phase 1
      const uint32_t ea = ss ? 1u : t == 1u ? 13u : t == 2u ? 11u : t == 3u ? 12u : 1u;
      const uint32_t er = !ss && t == 4u ? 13u : 1u, el = !ss && t == 3u ? 13u : 1u;
      return HAS | 1u | (1u << 5) | (ea << 10) | (er << 15) | (el << 20) | (1u << 25);
    }
    return HAS;  // any other char: phase 0 from every state
  }
  // entry ea followed by the map b
  __device__ static __forceinline__ uint32_t then(uint32_t ea, uint32_t b) {
    const uint32_t pa = ea & 7u;
    const uint32_t eb = pa == 6u ? ((b & ALLB) ? 14u : entry(b, 1u)) : entry(b, pa);
    return (eb ^ ((eb << 1) & ea & 16u)) & (ea | 0x17u);
  }
  __device__ static __forceinline__ uint32_t combine(uint32_t a, uint32_t b) {
    if (!(b & HAS)) return a;
    if (!(a & HAS)) return b;
    if (constant(b)) return b;
    if (constant(a)) return then(a & 31u, b) * REP | HAS;
    uint32_t r = 0u;
#pragma unroll
    for (uint32_t p = 0; p < 6u; ++p) r |= then(entry(a, p), b) << (5u * p);
    return r | HAS | (a & b & ALLB);
  }
  __device__ static __forceinline__ bool closed(uint32_t a) { return (a & HAS) && constant(a); }
};

// Backward state, for the leading run: bit 0 has chars, bit 1 open (the run
// reaches the range end and the last char does not end its sequence),
// bits 2-4 class, bits 5-7 class of the char after the run (C_NONE at an end).
struct BwdOp {
  static constexpr uint32_t IDENT = 0;
  __device__ static __forceinline__ uint32_t elem(uint32_t code) {
    uint32_t open = (code & K_SEQ_LAST) ? 0u : 2u;
    return 1u | open | (cls_of(code) << 2);
  }
  __device__ static __forceinline__ uint32_t combine(uint32_t a, uint32_t b) {
    if (!(a & 1u)) return b;
    if (!(b & 1u)) return a;
    if (a & 2u) {
      uint32_t ca = (a >> 2) & 7u, cb = (b >> 2) & 7u;
      if (ca == cb) return 1u | (b & 2u) | (ca << 2) | (b & 0xE0u);
      return 1u | (ca << 2) | (cb << 5);
    }
    return a;
  }
};

// Sum as a scan operator.
struct SumOp {
  static constexpr uint32_t IDENT = 0;
  __device__ static __forceinline__ uint32_t combine(uint32_t a, uint32_t b) { return a + b; }
};

// Ordered scans over a wavefront by DPP (operand modifiers of the combining
// VALU instruction: no LDS round trip and no per-lane address registers).
// dpp_id reads another lane's x by dpp_ctrl CTRL in the rows of ROWS; lanes
// without a source, or outside ROWS, read id.  Controls: 0x111.. row shift
// right by 1.., 0x101.. row shift left, 0x142 / 0x143 row broadcast of lane
// 15 / 31, 0x138 / 0x130 wavefront shift right / left by one lane.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_id(uint32_t id, uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, CTRL, ROWS, 0xF, false);
}

// Op with its operands swapped (a scan over lanes whose text order runs from
// the last lane to the first).
template <class Op>
struct RevOp {
  static constexpr uint32_t IDENT = Op::IDENT;
  __device__ static __forceinline__ uint32_t combine(uint32_t a, uint32_t b) { return Op::combine(b, a); }
};

// Inclusive left-to-right scan: Kogge-Stone inside each 16-lane row, then
// the rows before by broadcasts (lane 15 of a row into rows 1 and 3, then
// lane 31 into rows 2 and 3).
template <class Op>
__device__ __forceinline__ uint32_t wave_incl_fwd(uint32_t x, int) {
  x = Op::combine(dpp_id<0x111>(Op::IDENT, x), x);
  x = Op::combine(dpp_id<0x112>(Op::IDENT, x), x);
  x = Op::combine(dpp_id<0x114>(Op::IDENT, x), x);
  x = Op::combine(dpp_id<0x118>(Op::IDENT, x), x);
  x = Op::combine(dpp_id<0x142, 0xA>(Op::IDENT, x), x);
  x = Op::combine(dpp_id<0x143, 0xC>(Op::IDENT, x), x);
  return x;
}

// Inclusive right-to-left scan: Kogge-Stone inside each row, then the totals
// of the rows after (their first lanes, read into scalars).
template <class Op>
__device__ __forceinline__ uint32_t wave_incl_bwd(uint32_t x, int lane) {
  x = Op::combine(x, dpp_id<0x101>(Op::IDENT, x));
  x = Op::combine(x, dpp_id<0x102>(Op::IDENT, x));
  x = Op::combine(x, dpp_id<0x104>(Op::IDENT, x));
  x = Op::combine(x, dpp_id<0x108>(Op::IDENT, x));
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  const uint32_t p2 = Op::combine((uint32_t)__builtin_amdgcn_readlane((int)x, 32), r3);
  const uint32_t p1 = Op::combine((uint32_t)__builtin_amdgcn_readlane((int)x, 16), p2);
  const int row = lane >> 4;
  return Op::combine(x, row == 0 ? p1 : row == 1 ? p2 : row == 2 ? r3 : Op::IDENT);
}

// Exclusive ordered scan over the PT_THREADS threads of a block (left to
// right).  *total receives the whole block's combination.
template <class Op>
__device__ uint32_t block_excl_fwd(uint32_t x, uint32_t* red, uint32_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t inc = wave_incl_fwd<Op>(x, lane);
  uint32_t exc = dpp_id<0x138>(Op::IDENT, inc);
  if (lane == 63) red[wid] = inc;
  __syncthreads();
  uint32_t pre = Op::IDENT, tot = Op::IDENT;
  for (int w = 0; w < PT_THREADS / 64; ++w) {
    if (w < wid) pre = Op::combine(pre, red[w]);
    tot = Op::combine(tot, red[w]);
  }
  *total = tot;
  __syncthreads();
  return Op::combine(pre, exc);
}

// Exclusive ordered scan right to left.
template <class Op>
__device__ uint32_t block_excl_bwd(uint32_t x, uint32_t* red, uint32_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t inc = wave_incl_bwd<Op>(x, lane);
  uint32_t exc = dpp_id<0x130>(Op::IDENT, inc);
  if (lane == 0) red[wid] = inc;
  __syncthreads();
  uint32_t post = Op::IDENT, tot = Op::IDENT;
  for (int w = PT_THREADS / 64 - 1; w >= 0; --w) {
    if (w > wid) post = Op::combine(red[w], post);
    tot = Op::combine(red[w], tot);
  }
  *total = tot;
  __syncthreads();
  return Op::combine(exc, post);
}

// The two run-state scans of a tile in one pass: the exclusive forward scan
// of fx (left to right) and the exclusive backward scan of bx (right to
// left) over the block, with one barrier.  red needs 8 words.
__device__ __forceinline__ void block_excl_fwd_bwd(uint32_t fx, uint32_t bx, uint32_t* red, uint32_t* ef,
                                                   uint32_t* eb) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t incf = wave_incl_fwd<FwdOp>(fx, lane);
  const uint32_t incb = wave_incl_bwd<BwdOp>(bx, lane);
  const uint32_t excf = dpp_id<0x138>(FwdOp::IDENT, incf);
  const uint32_t excb = dpp_id<0x130>(BwdOp::IDENT, incb);
  if (lane == 63) red[wid] = incf;
  if (lane == 0) red[4 + wid] = incb;
  __syncthreads();
  uint32_t pre = FwdOp::IDENT, post = BwdOp::IDENT;
  for (int v = 0; v < PT_THREADS / 64; ++v) {
    if (v < wid) pre = FwdOp::combine(pre, red[v]);
  }
  for (int v = PT_THREADS / 64 - 1; v > wid; --v) post = BwdOp::combine(red[4 + v], post);
  *ef = FwdOp::combine(pre, excf);
  *eb = BwdOp::combine(excb, post);
}

// Butterfly step inside each half of the wavefront: lane l reads lane l ^ d
// (d < 32).  ds_swizzle takes the pattern as an immediate, so a kernel with
// many reductions keeps no per-lane address registers alive for them.
template <int D>
__device__ __forceinline__ uint32_t swz_xor(uint32_t x) {
  static_assert(D > 0 && D < 32, "within a half");
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x1F | (D << 10));
}

// Sum over the wavefront, the same in every lane.
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  x += swz_xor<16>(x);
  x += swz_xor<8>(x);
  x += swz_xor<4>(x);
  x += swz_xor<2>(x);
  x += swz_xor<1>(x);
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 0) + (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
}

__device__ __forceinline__ uint32_t block_sum(uint32_t x, uint32_t* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  x = wave_sum(x);
  if (lane == 0) red[wid] = x;
  __syncthreads();
  uint32_t t = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
  __syncthreads();
  return t;
}

// Exclusive prefix sum over the block; *total receives the block sum.
__device__ __forceinline__ uint32_t block_excl_sum(uint32_t x, uint32_t* red, uint32_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_fwd<SumOp>(x, lane);
  if (lane == 63) red[wid] = inc;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    if (w < wid) pre += red[w];
    tot += red[w];
  }
  *total = tot;
  __syncthreads();
  return pre + inc - x;
}

// ---------------------------------------------------------- chunk summaries

// Thread-chunk positions: tile indices [HALO + PT_CHUNK * tid, + PT_CHUNK).
__device__ __forceinline__ uint32_t chunk_fwd(const TileSmem& sm) {
  uint32_t s = FwdOp::IDENT;
  const int j0 = HALO + PT_CHUNK * threadIdx.x;
#pragma unroll
  for (int k = 0; k < PT_CHUNK; ++k) {
    uint32_t c = sm.code[cix(j0 + k)];
    if (is_char(c)) s = FwdOp::combine(s, FwdOp::elem(c));
  }
  return s;
}

__device__ __forceinline__ uint32_t chunk_bwd(const TileSmem& sm) {
  uint32_t s = BwdOp::IDENT;
  const int j0 = HALO + PT_CHUNK * threadIdx.x;
#pragma unroll
  for (int k = PT_CHUNK - 1; k >= 0; --k) {
    uint32_t c = sm.code[cix(j0 + k)];
    if (is_char(c)) s = BwdOp::combine(BwdOp::elem(c), s);
  }
  return s;
}

// Class index of a char code: 0 no char; letters 1 plain, 2 s/t/m/d, 3 r/v,
// 4 l, 5 e (either case: the contraction letters); 8 digit; 9 other,
// 10 apostrophe; 12 whitespace, 13 space; 14 CR/LF.
__device__ __forceinline__ uint32_t cl_index(uint32_t code) {
  constexpr uint64_t LTAB = 1ull | 2ull << 4 | 2ull << 8 | 3ull << 12 | 5ull << 16 | 3ull << 20 | 2ull << 24 |
                            4ull << 28 | 2ull << 32;  // by letter type 0..8
  constexpr uint32_t CTAB = 8u << (4 * C_N) | 9u << (4 * C_O) | 12u << (4 * C_WS) | 14u << (4 * C_WN);
  const uint32_t k = cls_of(code), lt = (code >> K_LETTER_SHIFT) & 15u;
  if (k == C_L) return (uint32_t)(LTAB >> (4 * lt)) & 15u;
  return ((CTAB >> (4 * k)) & 15u) + ((code >> 10) & 1u) + ((code >> 11) & 1u);  // + K_SP, + K_AP
}

// Code byte of a text byte for the cl100k-style rules (written by
// k_tile_summary, read by k_pretok): bits 0-3 the class index of the char
// starting there (0: no char starts there), bit 4 a sequence starts with that
// char, bit 5 its sequence ends with it, bit 7 invalid UTF-8 starts there.
constexpr uint32_t CB_IDX = 31u, CB_SS = 1u << 5, CB_SL = 1u << 6, CB_BAD = 1u << 7;

// Class index of a char code under the o200k-style rules (5 bits): 0 no
// char; 1 digit, 2 other, 3 apostrophe, 4 '/', 5 whitespace, 6 space, 7
// CR/LF; letter-type chars 16 | (lower case ? 8 : 0) | t, where t is the
// contraction letter type of an ASCII letter (0 none, 1 s/t/m/d, 2 r/v, 3 l,
// 4 e), and 23 for Lm and Lo letters and marks (either case).
__device__ __forceinline__ uint32_t o2_index(uint32_t code) {
  constexpr uint64_t TTAB = 0ull | 1ull << 4 | 1ull << 8 | 2ull << 12 | 4ull << 16 | 2ull << 20 | 1ull << 24 |
                            3ull << 28 | 1ull << 32;  // by letter type 0..8
  // selects from the weakest case to the strongest (flat: no branches)
  const uint32_t k = cls_of(code), fine = (code >> K_FINE_SHIFT) & 15u;
  const bool mb = ((code >> K_LEN_SHIFT) & 3u) != 0u;  // a multibyte char
  const uint32_t lt = (code >> K_LETTER_SHIFT) & 15u;
  const uint32_t ascii_l = 16u | ((code & K_UPPER) ? 0u : 8u) | ((uint32_t)(TTAB >> (4 * lt)) & 15u);
  const uint32_t mb_l = fine == 1u ? 16u : fine == 2u ? 24u : 23u;
  uint32_t c = 0u;
  c = k == C_WN ? 7u : c;
  c = k == C_WS ? ((code & K_SP) ? 6u : 5u) : c;
  c = k == C_O ? ((code & K_AP) ? 3u : (code & K_SLASH) ? 4u : 2u) : c;
  c = k == C_N ? 1u : c;
  c = (k == C_L) | (mb & (k == C_O) & (fine == 4u)) ? (mb ? mb_l : ascii_l) : c;
  return c;
}

// The code with its class as the o200k-style run summaries see it: marks
// are letters, and letters split into three classes (upper case C_L2U, lower
// case C_L, Lm/Lo/marks C_L2B) so that a run of one case is one run.
constexpr uint32_t C_L2U = 6u, C_L2B = 7u;
__device__ __forceinline__ uint32_t o2_sum_code(uint32_t code, uint32_t idx) {  // idx: o2_index(code)
  if (!(idx & 16u)) return code;
  const uint32_t c = (idx & 8u) ? C_L : (idx & 7u) == 7u ? C_L2B : C_L2U;
  return (code & ~7u) | c;
}

// Class index of a char code under the DeepSeek-style rules (5 bits): bits
// 0-3 1 digit, 2 other, 3 whitespace, 4 space, 5 CR/LF, 6 ASCII
// punctuation or symbol, 7 other punctuation or symbol, 8 ASCII letter, 9
// other letter or mark; bit 4 a CJK ideograph or kana; 0 no char.
__device__ __forceinline__ uint32_t ds_index(uint32_t code) {
  // selects from the weakest case to the strongest (flat: no branches)
  const uint32_t k = cls_of(code), fine = (code >> K_FINE_SHIFT) & 15u;
  const bool mb = ((code >> K_LEN_SHIFT) & 3u) != 0u;  // a multibyte char
  uint32_t c = 0u;
  c = k == C_O ? 2u : c;
  c = (k == C_O) & ((fine == 7u) | (fine == 8u)) ? (mb ? 7u : 6u) : c;
  c = (k == C_L) | (mb & (fine == 4u)) ? (mb ? 9u : 8u) : c;
  c = k == C_WN ? 5u : c;
  c = k == C_WS ? ((code & K_SP) ? 4u : 3u) : c;
  c = k == C_N ? 1u : c;
  return c ? c | ((code & K_CJK) ? 16u : 0u) : 0u;
}

// The code with its class as the DeepSeek-style run summaries see it:
// ASCII letters C_L2U; ASCII punctuation/symbols that can start a D1 piece
// (d1: no punctuation, symbol or space of its segment before it) C_L2B; other
// punctuation/symbols C_O; other letters, marks, "other" chars and every
// CJK char C_L.  idx: ds_index(code).
__device__ __forceinline__ uint32_t ds_sum_code(uint32_t code, bool d1, uint32_t idx) {
  const uint32_t c4 = idx & 15u;
  const bool keep = (idx == 0u) | (c4 == 1u) | (c4 - 3u <= 2u);  // no char, digits, whitespace
  uint32_t c = C_L;
  c = c4 == 7u ? C_O : c;
  c = c4 == 6u ? (d1 ? C_L2B : C_O) : c;
  c = c4 == 8u ? C_L2U : c;
  c = (idx & 16u) ? C_L : c;
  return keep ? code : (code & ~7u) | c;
}

template <int PAT>
__device__ __forceinline__ uint32_t code_byte(uint32_t code) {
  return (PAT == 3 ? ds_index(code) : PAT == 2 ? o2_index(code) : cl_index(code)) |
         ((code & K_SEQ_START) ? CB_SS : 0u) | ((code & K_SEQ_LAST) ? CB_SL : 0u) | ((code & K_BAD) ? CB_BAD : 0u);
}

// First index s in [0, cnt) with a[s] >= v (cnt if none), by one wavefront:
// 64 probes per step, so a step narrows the range 64-fold.
template <typename T>
__device__ int64_t wave_lower_bound(const T* __restrict__ a, int64_t cnt, int64_t v, int lane) {
  int64_t lo = 0, hi = cnt;  // the answer lies in [lo, hi]
  while (hi > lo) {
    const int64_t step = (hi - lo + 63) / 64;
    const int64_t q = lo + step * lane;
    const uint64_t m = __ballot(q < hi && (int64_t)a[q] < v);  // lanes 0 .. c - 1 (a is sorted)
    const int64_t c = __popcll(m);
    if (c == 0) return lo;
    const int64_t lo2 = lo + step * (c - 1) + 1;
    hi = min(hi, lo + step * c);
    lo = lo2;
  }
  return lo;
}

// Pass 1 (cl100k-style rules only): decode the tile (4 bytes per thread),
// write one code byte per text byte, and the tile's forward and backward run
// summaries, so that pass 2 can resolve runs that cross tiles (digit-group
// phase, the last newline of a whitespace run, newlines absorbed after
// punctuation) without a second look at distant bytes, and classify its span
// without decoding it again.
template <int PAT>
__global__ __launch_bounds__(PT_THREADS) void k_tile_summary(const uint8_t* __restrict__ bytes, int64_t n,
                                                             const int64_t* __restrict__ offs, int nseq,
                                                             Work w) {
  __shared__ uint16_t ascii[128];
  __shared__ uint32_t sbm[TILE / 32 + 3];  // sequence starts in [t0 - 32, t0 + TILE + 64)
  __shared__ uint32_t red[18];
  __shared__ uint32_t cbl[(4 + TILE) / 4];  // DeepSeek-style: code bytes of [t0 - 4, t0 + TILE)
  const int tid = (int)threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int t = blockIdx.x;
  const int64_t t0 = (int64_t)t * TILE;
  if (tid < 64) reinterpret_cast<uint32_t*>(ascii)[tid] = reinterpret_cast<const uint32_t*>(g_ascii.v)[tid];
  if (tid < TILE / 32 + 3) sbm[tid] = 0u;
  // DeepSeek-style: thread 0 also loads the 4 bytes before the tile (the
  // chars its punctuation test looks back at), in flight with the tile
  uint32_t pre4 = 0u;
  if (PAT == 3 && tid == 0 && t0 >= 4) {
    if ((reinterpret_cast<uintptr_t>(bytes) & 3u) == 0)
      pre4 = *reinterpret_cast<const uint32_t*>(bytes + t0 - 4);
    else
      for (int k = 0; k < 4; ++k) pre4 |= (uint32_t)bytes[t0 - 4 + k] << (8 * k);
  }
  // this thread's 4 bytes and the 4 after them
  const int64_t q = t0 + PT_CHUNK * tid;
  uint32_t d0 = 0u, d1 = 0u;
  if ((reinterpret_cast<uintptr_t>(bytes) & 3u) == 0 && q + 8 <= n) {
    d0 = *reinterpret_cast<const uint32_t*>(bytes + q);
    d1 = *reinterpret_cast<const uint32_t*>(bytes + q + 4);
  } else {
    for (int k = 0; k < 8; ++k)
      if (q + k < n) (k < 4 ? d0 : d1) |= (uint32_t)bytes[q + k] << (8 * (k & 3));
  }
  __syncthreads();
  if (offs) {
    if (wid == 0) {
      const int64_t lo = wave_lower_bound(offs, (int64_t)nseq + 1, t0 - 32, lane);
      const int64_t hi = wave_lower_bound(offs, (int64_t)nseq + 1, t0 + TILE + 64, lane);
      for (int64_t s = lo + lane; s < hi; s += 64) {
        const int j = (int)(offs[s] - (t0 - 32));
        atomicOr(&sbm[j >> 5], 1u << (j & 31));
      }
    }
  } else if (t0 == 0 && tid == 0) {
    sbm[1] = 1u;
  }
  __syncthreads();
  const int sh = (PT_CHUNK * tid) & 31;
  const uint32_t sw0 = sbm[1 + ((PT_CHUNK * tid) >> 5)], sw1 = sbm[2 + ((PT_CHUNK * tid) >> 5)];
  const uint32_t bm = sh ? (sw0 >> sh) | (sw1 << (32 - sh)) : sw0;  // bit i: a sequence starts at q + i
  uint32_t code[4];
  int len[4];
  decode4_regs((uint64_t)d0 | ((uint64_t)d1 << 32), bm, q, n, ascii, code, len);
  uint32_t out = 0u, fv = FwdOp::IDENT, bv = BwdOp::IDENT, tv = TailOp::IDENT;
#pragma unroll
  for (int k = 0; k < 4; ++k) out |= code_byte<PAT>(code[k]) << (8 * k);
  bool cap[4] = {false, false, false, false};
  if (PAT == 3) {
    // whether each ASCII punctuation char may start a D1 piece: look at the
    // char before it.  Thread 0 also decodes the 4 bytes before the tile;
    // each thread then reads the previous thread's 4 code bytes and finds,
    // in the 8-byte window, the nearest char start among the 3 bytes before
    // each of its own (else the 4th byte back: a char is at most 4 bytes).
    uint32_t pcw = 0u;
    if (tid == 0 && t0 >= 4) {
      uint32_t pc[4];
      int pl[4];
      decode4_regs((uint64_t)pre4 | ((uint64_t)d0 << 32), (sbm[0] >> 28) | (sbm[1] << 4), t0 - 4, n, ascii, pc, pl);
      pcw = code_byte<PAT>(pc[0]) | (code_byte<PAT>(pc[1]) << 8) | (code_byte<PAT>(pc[2]) << 16) |
            (code_byte<PAT>(pc[3]) << 24);
    }
    cbl[1 + tid] = out;
    if (tid == 0) cbl[0] = pcw;
    __syncthreads();
    const uint64_t win = (uint64_t)cbl[tid] | ((uint64_t)out << 32);
    // bit 8 i + 7: window byte i starts a char (class index bits nonzero)
    const uint64_t starts = ((win & 0x1F1F1F1F1F1F1F1Full) + 0x7F7F7F7F7F7F7F7Full) & 0x8080808080808080ull;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint64_t m = starts & (0xFFFFFFull << (8 * (k + 1)));  // window bytes k + 1 .. k + 3
      const int pos = m ? (63 - __clzll((long long)m)) >> 3 : k;
      const uint32_t pidx = (uint32_t)(win >> (8 * pos)) & CB_IDX, pc4 = pidx & 15u;
      cap[k] = ((out >> (8 * k)) & CB_IDX) == 6u &&
               ((code[k] & K_SEQ_START) || pidx == 0u || (pidx & 16u) || !(pc4 == 4u || pc4 == 6u || pc4 == 7u));
    }
  }
  bool ch[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    ch[k] = is_char(code[k]);
    // o200k-style summaries see marks as letters and letters by case (class
    // values 6 and 7 included)
    if (PAT == 2) code[k] = o2_sum_code(code[k], (out >> (8 * k)) & CB_IDX);
    if (PAT == 3) code[k] = ds_sum_code(code[k], cap[k], (out >> (8 * k)) & CB_IDX);
    if (ch[k]) {
      fv = FwdOp::combine(fv, FwdOp::elem(code[k]));
      if (PAT == 2) tv = TailOp::combine(tv, TailOp::elem(code[k]));
    }
  }
#pragma unroll
  for (int k = 3; k >= 0; --k)
    if (ch[k]) bv = BwdOp::combine(BwdOp::elem(code[k]), bv);
  *reinterpret_cast<uint32_t*>(w.codes + q) = out;
  const uint32_t wf = wave_incl_fwd<FwdOp>(fv, lane);
  const uint32_t wb = wave_incl_bwd<BwdOp>(bv, lane);
  if (lane == 63) red[wid] = wf;
  if (lane == 0) red[4 + wid] = wb;
  if (PAT == 2) {
    const uint32_t wt = wave_incl_fwd<TailOp>(tv, lane);
    if (lane == 63) red[8 + wid] = wt;
    // the tile's contraction-chain map.  The state at the tile's end can be
    // other than "no chain" only with an apostrophe among its last 3 chars
    // or an Lm/Lo/mark as its last char; else the map is that constant
    // (phase 1 after a letter, else 0).  Otherwise the last wavefront's map
    // of its 256 bytes, when constant (any char that resets the state, as
    // text between chains has), is the tile's; only a tile whose last 256
    // bytes carry a chain state through takes the whole tile's scan below.
    if (wid == PT_THREADS / 64 - 1) {
      uint32_t last = 0u;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (ch[k]) last = (out >> (8 * k)) & CB_IDX;
      const uint32_t x = d0 ^ 0x27272727u;
      const bool open = lane == 63 && ((((x - 0x01010101u) & ~x & 0x80808080u) != 0u) || last == 23u);
      const uint32_t l63 = (uint32_t)__builtin_amdgcn_readlane((int)last, 63);
      uint32_t m = ((l63 & 16u) ? ChainOp::REP : 0u) | ChainOp::HAS;
      bool whole = false;
      if (__ballot(open)) {
        uint32_t cv = ChainOp::IDENT;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (ch[k]) cv = ChainOp::combine(cv, ChainOp::elem((out >> (8 * k)) & CB_IDX, (out >> (8 * k)) & CB_SS));
        const uint32_t m3 = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_fwd<ChainOp>(cv, lane), 63);
        if (ChainOp::closed(m3)) m = m3;
        else whole = true;
      }
      if (lane == 0) {
        red[12] = whole;
        red[13] = m;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    w.tile_fwd[t] = FwdOp::combine(FwdOp::combine(red[0], red[1]), FwdOp::combine(red[2], red[3]));
    w.tile_bwd[t] = BwdOp::combine(BwdOp::combine(red[4], red[5]), BwdOp::combine(red[6], red[7]));
    if (PAT == 2) w.tile_tail[t] = TailOp::combine(TailOp::combine(red[8], red[9]), TailOp::combine(red[10], red[11]));
    if (PAT == 2 && !red[12]) w.tile_chain[t] = red[13];
  }
  if (PAT == 2 && red[12]) {
    // the whole tile's chain map (the same branch in every thread)
    uint32_t cv = ChainOp::IDENT;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (ch[k]) cv = ChainOp::combine(cv, ChainOp::elem((out >> (8 * k)) & CB_IDX, (out >> (8 * k)) & CB_SS));
    const uint32_t wc = wave_incl_fwd<ChainOp>(cv, lane);
    if (lane == 63) red[14 + wid] = wc;
    __syncthreads();
    if (tid == 0)
      w.tile_chain[t] = ChainOp::combine(ChainOp::combine(red[14], red[15]), ChainOp::combine(red[16], red[17]));
  }
}

// Combine the summaries of all tiles left of `t` (Op over src, wavefronts 0
// and 2) / right of `t` (wavefront 1), stopping once the run is closed: first
// the 64 nearest tiles (one per lane; usually a run closes there), then 8 per
// lane, 512 per step.
template <class Op>
__device__ __forceinline__ uint32_t look_back(const uint32_t* __restrict__ src, int t, int lane) {
  constexpr int PER = 8;
  uint32_t acc = Op::IDENT;
  int b = t - 1, per = 1;
  while (b >= 0) {
    // lane 0 holds the tiles next to t: the lanes run right to left in the text
    uint32_t x[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = b - per * lane - i;
      x[i] = i < per && j >= 0 ? src[j] : Op::IDENT;
    }
    uint32_t v = Op::IDENT;
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) v = Op::combine(v, x[i]);
    const uint32_t all = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_bwd<RevOp<Op>>(v, lane), 0);
    acc = uniform(Op::combine(all, acc));
    if (Op::closed(acc)) break;
    b -= 64 * per;
    per = PER;
  }
  return acc;
}

template <int PAT>
__device__ void tile_carries(const Work& w, int t, int ntiles, TileSmem& sm) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  constexpr int PER = 8;
  if (wid == 0) {
    const uint32_t acc = look_back<FwdOp>(w.tile_fwd, t, lane);
    if (lane == 0) sm.carry_fwd = acc;
  } else if (wid == 1) {
    uint32_t acc = BwdOp::IDENT;
    int b = t + 1, per = 1;
    while (b < ntiles) {
      uint32_t x[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int j = b + per * lane + i;
        x[i] = i < per && j < ntiles ? w.tile_bwd[j] : BwdOp::IDENT;
      }
      uint32_t v = BwdOp::IDENT;
#pragma unroll
      for (int i = 0; i < PER; ++i) v = BwdOp::combine(v, x[i]);
      const uint32_t all = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_bwd<BwdOp>(v, lane), 0);
      acc = uniform(BwdOp::combine(acc, all));
      if ((acc & 1u) && !(acc & 2u)) break;
      b += 64 * per;
      per = PER;
    }
    if (lane == 0) sm.carry_bwd = acc;
  } else if (wid == 2 && PAT == 2) {
    const uint32_t acc = look_back<TailOp>(w.tile_tail, t, lane);
    if (lane == 0) sm.carry_tail = acc;
  } else if (wid == 3 && PAT == 2) {
    const uint32_t acc = look_back<ChainOp>(w.tile_chain, t, lane);
    if (lane == 0) sm.carry_chain = acc;
  }
  __syncthreads();
}

// --------------------------------------------------------- boundary predicate

// Code at tile position j of the padded LDS array.
__device__ __forceinline__ uint32_t cat(const uint16_t* c, int j) { return c[cix(j)]; }

// Previous char start before tile position j, or -1 at a sequence start.
// With ASCII (no byte >= 0x80 in the staged span) every byte starts a char.
template <bool ASCII>
__device__ __forceinline__ int prev_char(const uint16_t* c, const uint8_t* pl, int j) {
  if (cat(c, j) & K_SEQ_START) return -1;
  if (ASCII) return j - 1;
  if (pl[j]) return j - pl[j];
  int k = j - 1;
  while (k > 0 && cls_of(cat(c, k)) == C_CONT && k > j - 4) --k;
  return k;
}

// The apostrophe at q starts a piece: it is a one-char "other" run that no
// space in front of it absorbs.
template <bool ASCII>
__device__ __forceinline__ bool ap_starts_piece(const uint16_t* c, const uint8_t* pl, int q) {
  uint32_t cq = cat(c, q);
  if (!(cq & K_AP)) return false;
  if (cq & K_SEQ_START) return true;
  uint32_t cr = cat(c, prev_char<ASCII>(c, pl, q));
  return cls_of(cr) != C_O && !(cr & K_SP);
}

// Length (1 or 2) of a contraction suffix whose first letter is at a, or 0.
template <int PAT, bool ASCII>
__device__ __forceinline__ int contraction_len(const uint16_t* c, const uint8_t* pl, int a) {
  uint32_t ca = cat(c, a);
  if (ca & K_SEQ_START) return 0;
  if (!ap_starts_piece<ASCII>(c, pl, prev_char<ASCII>(c, pl, a))) return 0;
  if (PAT == 0 && (ca & K_UPPER)) return 0;
  uint32_t lt = (ca >> K_LETTER_SHIFT) & 15u;
  if (lt == LT_S || lt == LT_T || lt == LT_M || lt == LT_D) return 1;
  if ((lt == LT_R || lt == LT_V || lt == LT_L) && !(ca & K_SEQ_LAST)) {
    uint32_t c2 = cat(c, a + 1);
    if (PAT == 0 && (c2 & K_UPPER)) return 0;
    uint32_t l2 = (c2 >> K_LETTER_SHIFT) & 15u;
    if ((lt == LT_R && l2 == LT_E) || (lt == LT_V && l2 == LT_E) || (lt == LT_L && l2 == LT_L)) return 2;
  }
  return 0;
}

// Letter at j is the first letter after a contraction suffix.
template <int PAT, bool ASCII>
__device__ __forceinline__ bool after_contraction(const uint16_t* c, const uint8_t* pl, int j) {
  int a = prev_char<ASCII>(c, pl, j);
  if (a < 0) return false;
  if (contraction_len<PAT, ASCII>(c, pl, a) == 1) return true;
  int a2 = prev_char<ASCII>(c, pl, a);
  return a2 >= 0 && contraction_len<PAT, ASCII>(c, pl, a2) == 2;
}

template <bool ASCII>
__device__ __forceinline__ bool pred_gpt2(const uint16_t* c, const uint8_t* pl, int j) {
  uint32_t c0 = cat(c, j);
  if (c0 & K_SEQ_START) return true;
  uint32_t k0 = cls_of(c0);
  int p1 = prev_char<ASCII>(c, pl, j);
  uint32_t c1 = cat(c, p1), k1 = cls_of(c1);
  if (is_w(k0)) {
    if (!is_w(k1)) return true;
    if (c0 & K_SEQ_LAST) return false;
    return !is_w(cls_of(cat(c, j + (ASCII ? 1 : clen(c0)))));
  }
  if (k1 == k0) return k0 == C_L && after_contraction<0, ASCII>(c, pl, j);
  if (c1 & K_SP) return false;
  if (k0 == C_L && contraction_len<0, ASCII>(c, pl, j) > 0) return false;
  return true;
}

// GPT-2-style start bits of a pure-ASCII tile, evaluated on 64-position masks
// instead of position by position, straight from the staged bytes (no decode
// pass: every byte is a char and its class comes from the ASCII table).  A
// wavefront covers its 256 tile positions in windows of 64 lanes: lane i of
// a window reads position P - 4 + i, so each mask holds the 4 positions
// before the window's own 56 (bits 4..59) and 4 after -- the whole reach of
// the rules (a contraction looks at most 4 chars back, the whitespace rule 1
// char ahead).  Class tests become ballots and the rules 64-bit scalar
// operations (X << 1 is "the char before", X >> 1 "the char after").  PLAIN:
// the span holds no text edge and no sequence boundary, so every position is
// a char and none starts or ends a sequence.  Returns the 4 start bits of
// this thread's positions and sets *cnt to the wavefront's start count.
template <bool PLAIN>
__device__ __forceinline__ uint32_t gpt2_ascii_bits(const TileSmem& sm, int64_t n, int64_t t0, uint32_t* cnt) {
  const int lane = (int)(threadIdx.x & 63u);
  const int wbase = HALO + 256 * (int)(threadIdx.x >> 6);  // the wave's first tile position
  const uint8_t* raw = reinterpret_cast<const uint8_t*>(sm.raw);
  uint32_t mine = 0, total = 0;
#pragma unroll
  for (int q = 0; q < 5; ++q) {  // 5 windows of 56 cover 256 positions
    const int P = wbase + 56 * q;
    const int j = P - 4 + lane;  // < 16 * RAW_WORDS
    uint32_t c = sm.ascii[raw[j] & 127u];
    uint64_t CH = ~0ull, SS = 0ull, SL = 0ull;
    if (!PLAIN) {
      const int64_t p = t0 - HALO + j;
      const bool in = p >= 0 && p < n;
      if (!in) c = C_OUT;
      CH = __ballot(in);
      SS = __ballot(in && bmap_bit(sm.bmap, j));
      SL = __ballot(in && (p + 1 >= n || bmap_bit(sm.bmap, j + 1)));
    }
    const uint32_t k = cls_of(c), lt = (c >> K_LETTER_SHIFT) & 15u;
    const uint64_t W = __ballot(k == C_WS || k == C_WN);
    const uint64_t L = __ballot(k == C_L);
    const uint64_t N = __ballot(k == C_N);
    const uint64_t O = __ballot(k == C_O);
    const uint64_t SP = __ballot((c & K_SP) != 0u);
    const uint64_t AP = __ballot((c & K_AP) != 0u);
    uint64_t CLEN = 0ull, AFTER = 0ull;
    if (AP) {
      const bool low = k == C_L && !(c & K_UPPER);
      const uint64_t C1 = __ballot(low && (lt == LT_S || lt == LT_T || lt == LT_M || lt == LT_D));
      const uint64_t CRV = __ballot(low && (lt == LT_R || lt == LT_V));
      const uint64_t CL = __ballot(low && lt == LT_L);
      const uint64_t CE = __ballot(low && lt == LT_E);
      // an apostrophe starts a piece: sequence start, or the char before it
      // is neither "other" nor a space
      const uint64_t APS = AP & (SS | ~((O | SP) << 1));
      // contraction suffix of 1 or 2 lower-case letters starting here
      const uint64_t PRE = ~SS & (APS << 1);
      const uint64_t CLEN1 = PRE & C1;
      const uint64_t CLEN2 = PRE & ~SL & ((CRV & (CE >> 1)) | (CL & (CL >> 1)));
      CLEN = CLEN1 | CLEN2;
      // first letter after a contraction suffix
      AFTER = ~SS & ((CLEN1 << 1) | ((~SS & (CLEN2 << 1)) << 1));
    }
    const uint64_t SAME = (L & (L << 1)) | (N & (N << 1)) | (O & (O << 1)) | (W & (W << 1));
    const uint64_t WB = W & (~(W << 1) | (~SL & ~(W >> 1)));
    const uint64_t NB = ~W & ((SAME & L & AFTER) | (~SAME & ~(SP << 1) & ~(L & CLEN)));
    uint64_t B = CH & (SS | WB | NB);
    // own positions: bits 4..59 that are this wavefront's tile positions
    const int own = min(56, min(wbase + 256, HALO + TILE) - P);
    B = own > 0 ? (B >> 4) & ((1ull << own) - 1ull) : 0ull;
    total += (uint32_t)__popcll(B);
    const int rel = 4 * lane - 56 * q;  // this thread's first position in the window
    if (rel >= 0 && rel < 56) mine = (uint32_t)(B >> rel) & 15u;
  }
  *cnt = total;
  return mine;
}

// fwd_prev: forward run state at the previous char; fwd_here: at this char;
// ends_run: the whitespace run through this char is followed by no CR/LF.
template <bool ASCII>
__device__ __forceinline__ bool pred_cl100k(const uint16_t* c, const uint8_t* pl, int j, uint32_t fwd_prev, uint32_t fwd_here,
                                            bool ends_run) {
  uint32_t c0 = cat(c, j);
  if (c0 & K_SEQ_START) return true;
  uint32_t k0 = cls_of(c0);
  int p1 = prev_char<ASCII>(c, pl, j);
  uint32_t c1 = cat(c, p1), k1 = cls_of(c1);
  switch (k0) {
    case C_N:
      return k1 != C_N || ((fwd_here >> 8) & 3u) == 1u;
    case C_L:
      if (k1 == C_L) return after_contraction<1, ASCII>(c, pl, j);
      if (k1 == C_WS) return false;
      if (k1 == C_O) {
        if (c1 & K_SEQ_START) return false;
        uint32_t c2 = cat(c, prev_char<ASCII>(c, pl, p1));
        return !(cls_of(c2) != C_O && !(c2 & K_SP));
      }
      return true;
    case C_O:
      if (k1 == C_O) return false;
      return !(c1 & K_SP);
    case C_WN:
      if (is_w(k1)) return false;
      return k1 != C_O;
    case C_WS:
      if (!is_w(k1)) return true;
      if (k1 == C_WN) return ends_run || ((fwd_prev >> 5) & 7u) == C_O;
      if (c0 & K_SEQ_LAST) return false;
      return !is_w(cls_of(cat(c, j + (ASCII ? 1 : clen(c0)))));
  }
  return false;
}


// cl100k-style start bits, bit-sliced.  The span's chars in order (char
// index x; own chars [c_lo, e)) are held as bit planes: lane l of a wavefront
// holds bits i = 0..31 of word l, char x = c_lo - 32 + 32 l + i (word 0: the
// chars before the own ones; then the own chars and the right context), so
// one VALU instruction evaluates a rule at up to 1088 positions.  The rules
// read at most four chars back and one ahead, except three facts that a
// whole run decides: a digit starts a group iff its offset in its digit run
// is a multiple of 3; a whitespace char after a CR/LF starts a piece iff its
// run of non-CR/LF whitespace is not followed by a CR/LF, or the CR/LF run
// before it follows an "other" char (which absorbed the CR/LFs).  Runs are
// spread over words with carry chains (a fill by addition, its carries
// between words from two ballots); runs that cross the tile's ends take the
// tile's forward and backward run states.
constexpr int BS_WORDS = 34;            // 1088 chars: 32 before, 1024 own, 32 after
constexpr int BS_CHUNKS = BS_WORDS / 2;  // 64-char ballot chunks

// x from the char S places before / after (bits shifted in across words).
template <int S>
__device__ __forceinline__ uint32_t bs_up(uint32_t x) {
  return __builtin_amdgcn_alignbit(x, dpp_id<0x138>(0u, x), 32 - S);
}
template <int S>
__device__ __forceinline__ uint32_t bs_dn(uint32_t x) {
  return __builtin_amdgcn_alignbit(dpp_id<0x130>(0u, x), x, S);
}

// Bits of R reached from a seed of S going up through contiguous bits of R,
// across words.  S lies in R, at most one seed per block of R.
__device__ __forceinline__ uint32_t bs_fill_up(uint32_t R, uint32_t S, int lane) {
  const uint32_t sum = R + S;
  const uint64_t G = __ballot(sum < R);                  // carry out of the word
  const uint64_t P = G | __ballot(sum == 0xFFFFFFFFu);   // carry out given a carry in
  const uint64_t C = (G + P) ^ G ^ P;                    // carry into each word
  return R & ~(R + S + ((uint32_t)(C >> lane) & 1u));
}

// The same going down (seeds at the blocks' tops): the fill on reversed bits,
// with the carries between words running from the last word to the first.
__device__ __forceinline__ uint32_t bs_fill_down(uint32_t R, uint32_t S, int lane) {
  const uint32_t r = __builtin_bitreverse32(R), s = __builtin_bitreverse32(S);
  const uint32_t sum = r + s;
  const uint64_t G = __builtin_bitreverse64(__ballot(sum < r));
  const uint64_t P = G | __builtin_bitreverse64(__ballot(sum == 0xFFFFFFFFu));
  const uint64_t C = (G + P) ^ G ^ P;
  return __builtin_bitreverse32(r & ~(r + s + ((uint32_t)(C >> (63 - lane)) & 1u)));
}

// Bits of this lane's word with char index in [lo, hi).
__device__ __forceinline__ uint32_t bs_range(int x0, int lo, int hi) {
  const int a = min(max(lo - x0, 0), 32), b = min(max(hi - x0, 0), 32);
  const uint32_t ma = a >= 32 ? 0u : ~0u << a;
  const uint32_t mb = b >= 32 ? ~0u : ~(~0u << b);
  return ma & mb;
}

// Start bits of this lane's word (one wavefront; lanes >= BS_WORDS hold no
// chars).  lf: forward run state of the chars before c_lo; rb: backward run
// state of the chars from e on.
// The three run facts shared by the cl100k- and o200k-style rules, for this
// lane's word: NPH digits at offset 0 mod 3 in their digit run, ENDS
// whitespace chars whose whitespace run is not followed by a CR/LF, ABSO
// CR/LF chars of a CR/LF run that follows an "other" char.
// o_cls: the summary classes that count as "other" for the CR/LF carry.
__device__ __forceinline__ void run_facts(uint32_t N, uint32_t WS, uint32_t WN, uint32_t O, uint32_t SS, uint32_t SL,
                                          int lane, int c_lo, int e, uint32_t lf, uint32_t rb, uint32_t* nph,
                                          uint32_t* ends, uint32_t* abso, uint32_t o_cls = 1u << C_O) {
  const int x0 = c_lo - 32 + 32 * lane;
  // digits at offset 0 mod 3 in their run: fill each run with its start's
  // residue (mod 3) of the char index
  // X0: the span's first char, whose predecessor is not seen (a run start
  // only if a sequence starts there)
  const uint32_t X0 = bs_range(x0, 0, 1);
  const uint32_t Np = bs_up<1>(N);
  const uint32_t RSN = N & (~Np | SS) & ~(X0 & ~SS);
  const uint32_t Q = N & ~RSN;
  const int base = ((x0 % 3) + 3) % 3;
  const uint32_t P0 = 0x49249249u;
  const uint32_t M0 = P0 << ((3 - base) % 3), M1 = P0 << ((4 - base) % 3), M2 = P0 << ((5 - base) % 3);
  uint32_t S0 = RSN & M0, S1 = RSN & M1;
  if ((lf & 1u) && ((lf >> 2) & 7u) == C_N) {
    // the digit run that reaches c_lo, if it began before the span: its
    // start's residue, seeded at the span's first char
    const int r0 = (((c_lo - (int)((lf >> 8) & 3u)) % 3) + 3) % 3;
    if (r0 == 0) S0 |= N & X0;
    if (r0 == 1) S1 |= N & X0;
  }
  const uint32_t F0 = bs_fill_up(Q, bs_up<1>(S0) & Q, lane) | S0;
  const uint32_t F1 = bs_fill_up(Q, bs_up<1>(S1) & Q, lane) | S1;
  const uint32_t F2 = N & ~F0 & ~F1;
  *nph = (F0 & M0) | (F1 & M1) | (F2 & M2);
  // whitespace runs followed by a CR/LF, spread down from the run's top (runs
  // cut at e; one that goes on past e takes the backward state there)
  const uint32_t lim = bs_range(x0, -(1 << 20), e);
  uint32_t FW = WS & bs_dn<1>(WN) & ~SL & lim;
  const bool rb_ws_nl = (rb & 1u) && ((rb >> 2) & 7u) == C_WS && ((rb >> 5) & 7u) == C_WN;
  if (rb_ws_nl) FW |= WS & bs_dn<1>(WS) & ~SL & bs_range(x0, e - 1, e);
  *ends = WS & ~bs_fill_down(WS & ~SL & lim, FW, lane);
  // CR/LF runs right after an "other" char
  const uint32_t RN = WN & ~SS;
  uint32_t SN = RN & ~bs_up<1>(WN) & bs_up<1>(O);
  if ((lf & 1u) && ((lf >> 2) & 7u) == C_WN && ((o_cls >> ((lf >> 5) & 7u)) & 1u)) SN |= RN & X0;
  *abso = bs_fill_up(RN, SN, lane);
}

__device__ uint32_t cl_word_bits(const uint32_t* pl, int lane, int c_lo, int e, uint32_t lf, uint32_t rb) {
  const uint32_t b0 = pl[0], b1 = pl[1], b2 = pl[2], b3 = pl[3], SS = pl[4], SL = pl[5];
  const int x0 = c_lo - 32 + 32 * lane;
  const uint32_t CH = b0 | b1 | b2 | b3;
  const uint32_t L = ~b3 & (b0 | b1 | b2);
  const uint32_t N = b3 & ~b2 & ~b1 & ~b0;
  const uint32_t O = b3 & ~b2 & (b0 ^ b1);
  const uint32_t AP = b3 & ~b2 & b1 & ~b0;
  const uint32_t W = b3 & b2, WS = W & ~b1, SP = WS & b0, WN = W & b1;
  uint32_t NPH, ENDS, ABSO;
  run_facts(N, WS, WN, O, SS, SL, lane, c_lo, e, lf, rb, &NPH, &ENDS, &ABSO);
  // contractions (ASCII letters, either case): the letter after a suffix of
  // one or two letters that follows a piece-starting apostrophe starts a piece
  const uint32_t OSp = bs_up<1>(O | SP);
  uint32_t AFTER = 0u;
  if (__ballot(AP != 0u)) {
    const uint32_t C1 = ~b3 & ~b2 & b1 & ~b0, RV = ~b3 & ~b2 & b1 & b0;
    const uint32_t LL = ~b3 & b2 & ~b1 & ~b0, E = ~b3 & b2 & ~b1 & b0;
    const uint32_t APS = AP & (SS | ~OSp);
    const uint32_t PRE = ~SS & bs_up<1>(APS);
    const uint32_t CLEN1 = PRE & C1;
    const uint32_t CLEN2 = PRE & ~SL & ((RV & bs_dn<1>(E)) | (LL & bs_dn<1>(LL)));
    AFTER = ~SS & (bs_up<1>(CLEN1) | bs_up<1>(~SS & bs_up<1>(CLEN2)));
  }
  const uint32_t Lp = bs_up<1>(L), Op = bs_up<1>(O), WSp = bs_up<1>(WS), Wp = bs_up<1>(W);
  const uint32_t WNp = bs_up<1>(WN), SSp = bs_up<1>(SS), SPp = bs_up<1>(SP);
  const uint32_t BN = N & (~bs_up<1>(N) | NPH);
  const uint32_t BL = L & ((Lp & AFTER) | (~Lp & ~WSp & ~Op) | (Op & ~SSp & bs_up<1>(OSp)));
  const uint32_t BO = O & ~Op & ~SPp;
  const uint32_t BWN = WN & ~Wp & ~Op;
  const uint32_t BWS = WS & (~Wp | (WNp & (ENDS | bs_up<1>(ABSO))) | (WSp & ~SL & ~bs_dn<1>(W)));
  return CH & (SS | BN | BL | BO | BWN | BWS) & bs_range(x0, c_lo, e);
}

// Stage the span's code bytes (k_tile_summary's; none before the text or at
// or past its end).  Returns, the same in every thread, whether some position
// of the span inside the text starts no char (then the chars are compacted
// before the bit planes are taken); *bad: an own position starts invalid
// UTF-8.
__device__ bool stage_codes(int64_t n, int64_t t0, const Work& w, TileSmem& sm, bool* bad) {
  bool gap = false, b = false;
  for (int i = threadIdx.x; i < SPAN / 4; i += PT_THREADS) {
    const int64_t p = t0 - HALO + 4 * (int64_t)i;
    uint32_t v = 0u, in = 0u;
    if (p >= 0 && p < n) {
      v = *reinterpret_cast<const uint32_t*>(w.codes + p);
      in = p + 4 <= n ? ~0u : (1u << (8 * (n - p))) - 1u;  // bytes inside the text
      v &= in;
    }
    // a byte inside the text whose class index is 0 (set the others' low bit)
    const uint32_t nib = (v & 0x1F1F1F1Fu) | (~in & 0x01010101u);
    gap |= ((nib - 0x01010101u) & ~nib & 0x80808080u) != 0u;
    if (i >= HALO / 4 && i < (HALO + TILE) / 4) b |= (v & 0x80808080u) != 0u;
    reinterpret_cast<uint32_t*>(sm.cb)[i] = v;
  }
  *bad = __syncthreads_or(b);
  return __syncthreads_or(gap);
}

// o200k-style start bits of this lane's word (one wavefront; the planes are
// the five class-index bits, sequence start, sequence last).  lf, rb: the
// forward / backward run states (o200k-style classes) before c_lo and from
// e on; tl: the tail state before c_lo; ch: the contraction-chain map of
// the text before the tile.  *unsup (the same in every lane): the word's
// outcome depends on a contraction chain whose head these carries do not
// fix (a check: the chain map covers every such chain).
__device__ uint32_t o2_word_bits(const uint32_t* pl, int lane, int c_lo, int e, uint32_t lf, uint32_t rb, uint32_t tl,
                                 uint32_t ch, bool* unsup) {
  const uint32_t b0 = pl[0], b1 = pl[1], b2 = pl[2], b3 = pl[3], b4 = pl[4], SS = pl[5], SL = pl[6];
  const int x0 = c_lo - 32 + 32 * lane;
  const uint32_t CH = b0 | b1 | b2 | b3 | b4;
  const uint32_t LI = b4, NL = ~b4 & CH;
  const uint32_t LW = b4 & b3;                        // lower case
  const uint32_t BT = b4 & ~b3 & b2 & b1 & b0;        // Lm, Lo, marks
  const uint32_t UC = b4 & ~b3 & ~(b2 & b1 & b0);     // upper case
  const uint32_t C1 = b4 & ~b2 & ~b1 & b0, RV = b4 & ~b2 & b1 & ~b0, LL = b4 & ~b2 & b1 & b0, E = b4 & b2 & ~b1 & ~b0;
  const uint32_t N = NL & ~b2 & ~b1 & b0;
  const uint32_t O = NL & ((~b2 & b1) | (b2 & ~b1 & ~b0));
  const uint32_t AP = NL & ~b2 & b1 & b0;
  const uint32_t SLASH = NL & b2 & ~b1 & ~b0;
  const uint32_t WS = NL & b2 & (b1 ^ b0), SP = NL & b2 & b1 & ~b0, WN = NL & b2 & b1 & b0;
  const uint32_t W = WS | WN;
  const uint32_t X0 = bs_range(x0, 0, 1);
  uint32_t NPH, ENDS, ABSO;
  run_facts(N, WS, WN, O, SS, SL, lane, c_lo, e, lf, rb, &NPH, &ENDS, &ABSO);
  // tails: CR/LF right after an "other" char, then CR, LF and '/' chars
  const uint32_t RT = (WN | SLASH) & ~SS;
  uint32_t ST = WN & bs_up<1>(O) & ~SS;
  if ((tl & 1u) && (tl & 32u) && (tl & 4u)) {
    // the tail through c_lo - 1 started d chars before c_lo (at the span's
    // first char if that lies before the span)
    const int xs = max(c_lo - (int)((tl >> 6) & 63u), 0);
    ST |= RT & bs_range(x0, xs, xs + 1);
  }
  const uint32_t TAIL = bs_fill_up(RT, ST, lane) | ST;
  // contractions: an apostrophe after a letter, with a contraction shape
  // after it, attaches to the word before it
  const uint32_t SSn = bs_dn<1>(SS), SSn2 = bs_dn<2>(SS);
  const uint32_t CS1 = AP & bs_dn<1>(C1) & ~SSn;
  const uint32_t CS2 = AP & ~SSn & ~SSn2 & ((bs_dn<1>(RV) & bs_dn<2>(E)) | (bs_dn<1>(LL) & bs_dn<2>(LL)));
  const uint32_t CAND = (CS1 | CS2) & bs_up<1>(LI) & ~SS;
  const uint32_t LINK = bs_up<2>(CS1) | bs_up<3>(CS2);  // right after a contraction shape: a chain
  // a chain of shapes, each right after the letters of the one before: its
  // first shape (HEAD) attaches when a letter comes before it, and every
  // later one attaches exactly when the one before did not (a word that took
  // a contraction is over; one that did not takes the next).  So a shape's
  // attachment is P (prefix parity of the shapes) xor a base that is the
  // same along the chain: the head's P ^ CAND, filled along the chain's chars.
  const uint32_t CSX = CS1 | CS2;
  const uint32_t LNK = CSX & LINK & ~SS;
  const uint32_t HEAD = CSX & ~LNK;
  const uint32_t RC = CSX | bs_up<1>(CSX) | bs_up<2>(CS2);
  const uint32_t cst = ChainOp::entry(ch, 0u);  // (the text starts in phase 0)
  uint32_t ATT = CAND, UNK = 0u;
  // with no linked shape in the window and no chain carried in, every shape
  // is its chain's head and the rule below gives ATT = CAND
  if (__ballot(LNK != 0u) != 0ull || (cst & 7u) - 2u <= 3u) {
    uint32_t P = CSX;
    P ^= P << 1;
    P ^= P << 2;
    P ^= P << 4;
    P ^= P << 8;
    P ^= P << 16;
    if (__popcll(__ballot(__popc(CSX) & 1) & ((1ull << lane) - 1ull)) & 1) P = ~P;
    // a shape in the window's first three chars may link to one before the
    // window, unless the window starts a sequence: heads there are not known
    const bool seq0 = __ballot((SS & bs_range(x0, 0, 1)) != 0u) != 0ull;
    const uint32_t EDGE = seq0 ? 0u : bs_range(x0, -(1 << 20), 3);
    uint32_t HC = HEAD & ~EDGE;
    uint32_t S1 = HC & (P ^ CAND);
    // a chain that reaches the tile start with its head before the window:
    // the carry (the chain state at the tile start) holds the attachment of
    // its last shape before the tile, which fixes the base for the whole run
    // of chain chars that ends at c_lo - 1 (lane 0, bit 31)
    uint32_t SEED = 0u;
    if ((cst & 7u) - 2u <= 3u) {
      const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)RC, 0);
      const uint32_t h0 = (uint32_t)__builtin_amdgcn_readlane((int)HC, 0);
      const uint32_t g0 = (uint32_t)__builtin_amdgcn_readlane((int)EDGE, 0);
      if (r0 >> 31) {
        const int z = 31 - __clz((int)~r0);  // the char before that run (chars before the text are 0)
        if (!(h0 & (~0u << (z + 1))) && ((g0 >> (z + 1)) & 1u)) {
          const uint32_t p0 = (uint32_t)__builtin_amdgcn_readlane((int)P, 0);
          SEED = lane == 0 ? 1u << (z + 1) : 0u;
          if (((p0 >> 31) ^ (cst >> 4)) & 1u) S1 |= SEED;
        }
      }
    }
    HC |= SEED;
    const uint32_t F = bs_fill_up((RC & ~HC) | S1, S1, lane) | S1;
    // chains whose head is not known: from a run start in the first three chars
    const uint32_t SU0 = RC & EDGE & ~bs_up<1>(RC) & ~SEED;
    UNK = bs_fill_up(RC & ~HC, SU0, lane) | SU0;
    ATT = (CAND | (CSX & EDGE & ~UNK)) & ((~UNK & (P ^ F)) | (UNK & ~LINK));
    UNK &= CSX & (LNK | EDGE);
  }
  const uint32_t IC = bs_up<1>(ATT) | bs_up<2>(ATT & CS2);  // letters of an attached contraction
  const uint32_t AFTER = LI & ~SS & (bs_up<2>(ATT & CS1) | bs_up<3>(ATT & CS2));
  // the run of Lm/Lo/marks (no sequence start in it) that ends at c_lo - 1,
  // if any: the carried chain state says whether it began right after a
  // whole shape that attached, so whether its first char restarts the word,
  // also where that shape or the run's start lies before the window
  uint32_t AFT = AFTER;
  const uint32_t bn0 = (uint32_t)__builtin_amdgcn_readlane((int)(BT & ~SS), 0);
  if (bn0 >> 31) {
    const uint32_t qb = 1u << (32 - __clz((int)~bn0));  // the run's first char (chars before the text are 0)
    if (lane == 0) AFT = (AFTER & ~qb) | (((cst & 7u) == 6u && (cst & 16u)) ? qb : 0u);
  }
  // case rules inside a letter run: PREVW, the last cased char of the word
  // before this char is lower case (Lm/Lo/marks carry it; a restart after a
  // contraction cuts it)
  const uint32_t RB = BT & ~AFT & ~SS;
  uint32_t SB = RB & bs_up<1>(LW);
  if ((lf & 1u) && ((lf >> 2) & 7u) == C_L2B && ((lf >> 5) & 7u) == C_L) {
    // an Lm/Lo/mark run that began before the span, after a lower-case letter
    SB |= RB & X0;
  }
  const uint32_t LWB = bs_fill_up(RB, SB, lane);
  const uint32_t PREVW = bs_up<1>(LW | LWB);
  // ALLU: upper-case chars from which only upper-case chars follow to the
  // letter run's end (runs cut at e; one that goes on past e takes rb)
  const uint32_t lim = bs_range(x0, -(1 << 20), e);
  uint32_t SU = UC & ~SS & (SL | ~bs_dn<1>(LI)) & lim;
  const bool rb_u_end = (rb & 1u) && ((rb >> 2) & 7u) == C_L2U && ((rb >> 5) & 7u) != C_L &&
                        ((rb >> 5) & 7u) != C_L2B;
  if (rb_u_end) SU |= UC & bs_dn<1>(UC) & ~SL & bs_range(x0, e - 1, e);
  const uint32_t ALLU = bs_fill_down(((UC & ~SS & ~SL) | SU) & lim, SU, lane);
  const uint32_t RULEA = UC & PREVW;
  const uint32_t RULEB = UC & bs_up<1>(BT) & ~PREVW & ALLU;
  const uint32_t Lp = bs_up<1>(LI), Op = bs_up<1>(O), TAILp = bs_up<1>(TAIL), SSp = bs_up<1>(SS);
  const uint32_t BL_IN = LI & Lp & ~IC & (AFTER | RULEA | RULEB);
  const uint32_t BL_ST = LI & ~Lp & ~bs_up<1>(WS) & ~IC &
                         (~Op | TAILp | (~SSp & (bs_up<2>(O & ~TAIL) | bs_up<2>(SP))));
  const uint32_t BN = N & (~bs_up<1>(N) | NPH);
  const uint32_t BO = O & ~TAIL & ~bs_up<1>(SP) & (~Op | TAILp) & ~(Lp & ATT);
  const uint32_t Wp = bs_up<1>(W);
  const uint32_t BWN = WN & ~Wp & ~Op;
  const uint32_t BWS = WS & (~Wp | (bs_up<1>(WN) & (ENDS | bs_up<1>(ABSO))) | (bs_up<1>(WS) & ~SL & ~bs_dn<1>(W)));
  const uint32_t own = bs_range(x0, c_lo, e);
  // undecided: a shape of a chain whose head is not known whose own chars
  // or next char lie from c_lo on.  The carried chain state covers every
  // chain that reaches c_lo - 1, so this does not arise; it stays a check.
  const uint32_t reach = UNK & ((CS1 & bs_range(x0, c_lo - 2, e)) | (CS2 & bs_range(x0, c_lo - 3, e)));
  *unsup = __ballot(reach != 0u) != 0ull;
  return CH & (SS | BN | BL_IN | BL_ST | BO | BWN | BWS) & own;
}

// DeepSeek-style start bits of this lane's word (one wavefront; the planes
// are the five class-index bits, sequence start, sequence last).  Digit
// groups and CJK/kana runs cut segments first: SEG marks a segment's first
// char, SEGL its last; inside, the rules see segment ends as text ends.
// lf, rb: the forward / backward run states (DeepSeek-style classes) before
// c_lo and from e on.
__device__ uint32_t ds_word_bits(const uint32_t* pl, int lane, int c_lo, int e, uint32_t lf, uint32_t rb) {
  const uint32_t b0 = pl[0], b1 = pl[1], b2 = pl[2], b3 = pl[3], CJK = pl[4], SS = pl[5], SL = pl[6];
  const int x0 = c_lo - 32 + 32 * lane;
  const uint32_t CH = b0 | b1 | b2 | b3;
  auto eq = [&](uint32_t v) {
    return ((v & 1u) ? b0 : ~b0) & ((v & 2u) ? b1 : ~b1) & ((v & 4u) ? b2 : ~b2) & ((v & 8u) ? b3 : ~b3);
  };
  const uint32_t N = eq(1u), O = eq(2u), WSn = eq(3u), SP = eq(4u), WN = eq(5u), AP1 = eq(6u), PSn = eq(7u);
  const uint32_t AL = eq(8u), LMn = eq(9u);
  const uint32_t WS = WSn | SP, W = WS | WN, PS = AP1 | PSn, LM = AL | LMn;
  // digit groups first: NPH from the shared run facts needs sequence starts
  // only; then segment starts and ends
  uint32_t NPH, ENDS0, ABSO0;
  run_facts(N, WS, WN, PS, SS, SL, lane, c_lo, e, lf, rb, &NPH, &ENDS0, &ABSO0);
  const uint32_t Np = bs_up<1>(N);
  const uint32_t SEG = CH & (SS | (N & (~Np | NPH)) | (~N & Np) | (CJK ^ bs_up<1>(CJK)));
  const uint32_t SEGL = CH & (SL | bs_dn<1>(SEG));
  // whitespace facts again, inside segments
  uint32_t NPH2, ENDS, ABSO;
  run_facts(N, WS, WN, PS, SEG, SEGL, lane, c_lo, e, lf, rb, &NPH2, &ENDS, &ABSO, (1u << C_O) | (1u << C_L2B));
  // D1: an ASCII punctuation char that starts a piece and has ASCII letters
  // after it takes them
  const uint32_t D1S = AP1 & bs_dn<1>(AL) & ~bs_dn<1>(SEG) & (SEG | ~(bs_up<1>(PS) | bs_up<1>(SP)));
  const uint32_t RA = AL & ~SEG;
  uint32_t SA = RA & bs_up<1>(D1S);
  // an ASCII-letter run that began before the span right after a D1 start
  if ((lf & 1u) && ((lf >> 2) & 7u) == C_L2U && ((lf >> 5) & 7u) == C_L2B) SA |= RA & bs_range(x0, 0, 1);
  const uint32_t D1L = bs_fill_up(RA, SA, lane);
  const uint32_t BLM = LM & ((bs_up<1>(LM) & bs_up<1>(D1L) & ~AL) | (bs_up<1>(PS) & ~(bs_up<1>(D1S) & AL)) |
                             bs_up<1>(WN));
  const uint32_t BPS = PS & ~bs_up<1>(PS) & ~bs_up<1>(SP);
  const uint32_t BWN = WN & ~bs_up<1>(W) & ~bs_up<1>(PS);
  const uint32_t BWS = WS & (~bs_up<1>(W) | (bs_up<1>(WN) & (ENDS | bs_up<1>(ABSO))) |
                             (bs_up<1>(WS) & ~SEGL & ~bs_dn<1>(W)));
  const uint32_t BO = O & (~bs_up<1>(O) | (bs_dn<1>(LM) & ~SEGL));
  return CH & (SEG | BLM | BPS | BWN | BWS | BO) & bs_range(x0, c_lo, e);
}

// The tile's cl100k-style start bits: this thread's 4 (its positions
// HALO + 4 tid ...) and, in *cnt, the tile's count (the same in every
// thread).  The code bytes are staged and the tile's carries (sm.carry_fwd /
// carry_bwd) set.  DIRECT: every span position inside the text starts a
// char, so char x is span position x; else the chars are compacted first.
template <int PAT, bool DIRECT>
__device__ uint32_t pat_bits(TileSmem& sm, uint32_t* cnt, bool* unsup) {
  constexpr int NPL = PAT >= 2 ? 7 : 6;  // class-index bits, sequence start, sequence last
  constexpr int NIDX = NPL - 2;
  const int tid = (int)threadIdx.x, lane = tid & 63, wid = (int)uniform((uint32_t)tid >> 6);
  int c_lo = HALO, n_own = TILE, nc = SPAN;
  const uint8_t* chars = sm.cb;
  if (!DIRECT) {
    // the span's chars in order: left halo, own, right halo
    const int j0 = HALO + PT_CHUNK * tid;
    const uint32_t v = reinterpret_cast<const uint32_t*>(sm.cb)[j0 >> 2];
    uint32_t own = 0;
#pragma unroll
    for (int k = 0; k < PT_CHUNK; ++k) own += ((v >> (8 * k)) & CB_IDX) ? 1u : 0u;
    uint32_t n_o;
    const uint32_t own_base = block_excl_sum(own, sm.red, &n_o);
    // the halos, lanes 0..15 the left one and 16..31 the right one (every
    // wavefront counts them, so all agree on the indices; wavefront 0 writes them)
    const int hj = lane < HALO ? lane : TILE + lane;
    const bool hc = lane < 2 * HALO && (sm.cb[hj] & CB_IDX) != 0u;
    const uint64_t hm = __ballot(hc);
    const uint32_t n_left = (uint32_t)__popcll(hm & 0xFFFFull);
    c_lo = (int)uniform(n_left);
    n_own = (int)uniform(n_o);
    nc = c_lo + n_own + (int)__popcll(hm & 0xFFFF0000ull);
    uint32_t at = n_left + own_base;
#pragma unroll
    for (int k = 0; k < PT_CHUNK; ++k) {
      const uint32_t c = (v >> (8 * k)) & 255u;
      if (c & CB_IDX) {
        sm.cc[at] = (uint8_t)c;
        sm.cpos[at] = (uint16_t)(j0 + k);
        ++at;
      }
    }
    if (wid == 0 && hc) {
      const uint32_t below = (uint32_t)__popcll(hm & ((1ull << lane) - 1ull));
      const uint32_t idx = lane < HALO ? below : (uint32_t)(c_lo + n_own) + below - n_left;
      sm.cc[idx] = sm.cb[hj];
      sm.cpos[idx] = (uint16_t)hj;
    }
    if (tid < TILE / 32) sm.sbits[tid] = 0u;
    __syncthreads();
    chars = sm.cc;
  }
  // bit planes, 64 chars per ballot, chunks dealt to the wavefronts
  for (int c = wid; c < BS_CHUNKS; c += PT_THREADS / 64) {
    const int x = c_lo - 32 + 64 * c + lane;
    const uint32_t b = x >= 0 && x < nc ? chars[x] : 0u;
    const uint32_t idx = b & CB_IDX;
    uint64_t m[NPL];
#pragma unroll
    for (int k = 0; k < NIDX; ++k) m[k] = __ballot((idx >> k) & 1u);
    m[NIDX] = __ballot(idx != 0u && (b & CB_SS));
    m[NIDX + 1] = __ballot(idx != 0u && (b & CB_SL));
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < NPL; ++k) sm.bsw[k][c] = m[k];
    }
  }
  __syncthreads();
  if (wid == 0) {
    uint32_t pl[NPL];
#pragma unroll
    for (int k = 0; k < NPL; ++k)
      pl[k] = lane < BS_WORDS ? reinterpret_cast<const uint32_t*>(sm.bsw[k])[lane] : 0u;
    bool uns = false;
    const uint32_t B = PAT == 3 ? ds_word_bits(pl, lane, c_lo, c_lo + n_own, uniform(sm.carry_fwd),
                                               uniform(sm.carry_bwd))
                     : PAT == 2 ? o2_word_bits(pl, lane, c_lo, c_lo + n_own, uniform(sm.carry_fwd),
                                               uniform(sm.carry_bwd), uniform(sm.carry_tail),
                                               uniform(sm.carry_chain), &uns)
                                : cl_word_bits(pl, lane, c_lo, c_lo + n_own, uniform(sm.carry_fwd),
                                               uniform(sm.carry_bwd));
    const uint32_t tot = wave_incl_fwd<SumOp>((uint32_t)__popc(B), lane);
    if (lane == 63) sm.red[0] = tot;
    if (lane == 0) sm.red[1] = uns ? 1u : 0u;
    if (DIRECT) {
      if (lane >= 1 && lane <= TILE / 32) sm.sbits[lane - 1] = B;
    } else if (lane < BS_WORDS) {
      sm.cbits[lane] = B;
    }
  }
  __syncthreads();
  *cnt = sm.red[0];
  *unsup = sm.red[1] != 0u;
  if (!DIRECT) {
    // own char o sits at word 1 + o / 32: its start bit goes to its byte position
#pragma unroll
    for (int k = 0; k < PT_CHUNK; ++k) {
      const int o = PT_CHUNK * tid + k;
      if (o < n_own && ((sm.cbits[1 + (o >> 5)] >> (o & 31)) & 1u)) {
        const int p = (int)sm.cpos[c_lo + o] - HALO;
        atomicOr(&sm.sbits[p >> 5], 1u << (p & 31));
      }
    }
    __syncthreads();
  }
  return (sm.sbits[tid >> 3] >> ((tid & 7) * PT_CHUNK)) & 15u;
}

__device__ __forceinline__ int64_t err_code(uint32_t e) {
  return (e & ERR_OFFSETS) ? -7 : (e & ERR_UTF8) ? -5 : (e & ERR_UNSUP) ? -10 : 0;
}

// Sum over i < cnt of (a[i] & mask) by the whole workgroup of 256 threads:
// coalesced, eight loads in flight per thread.  *hi gets the OR of this
// thread's (a[i] & ~mask).
__device__ uint32_t block_reduce(const uint32_t* __restrict__ a, int cnt, uint32_t mask, uint32_t* red,
                                 uint32_t* hi) {
  uint32_t sum = 0, orv = 0;
  for (int c0 = 0; c0 < cnt; c0 += 256 * 8) {
    uint32_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = c0 + 256 * k + (int)threadIdx.x;
      v[k] = i < cnt ? a[i] : 0u;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sum += v[k] & mask;
      orv |= v[k] & ~mask;
    }
  }
  *hi = orv;
  return block_sum(sum, red);
}

// Sum of (a[i] & mask), i < cnt, for a tile prefix (a = tile_cnt or
// tile_tok), with *hi = this thread's OR of (a[i] & ~mask).  With the
// super-block sums (SB: sb_sum and sb_or, which may be null), the whole runs of
// SB_TILES tiles before cnt come from their sums and only the partial run is
// read tile by tile.
template <bool SB>
__device__ __forceinline__ uint32_t tile_prefix(const uint32_t* __restrict__ a, const uint32_t* __restrict__ sb_sum,
                                                const uint32_t* __restrict__ sb_or, int cnt, uint32_t mask,
                                                uint32_t* red, uint32_t* hi) {
  if (!SB || cnt < SB_TILES) return block_reduce(a, cnt, mask, red, hi);
  const int j = cnt / SB_TILES;
  uint32_t h0, h1, h2 = 0;
  const uint32_t s0 = block_reduce(sb_sum, j, ~0u, red, &h0);
  const uint32_t s1 = block_reduce(a + (int64_t)j * SB_TILES, cnt - j * SB_TILES, mask, red, &h1);
  if (sb_or) block_reduce(sb_or, j, 0u, red, &h2);  // mask 0: the sum is 0, *hi the OR
  *hi = h1 | h2;
  return s0 + s1;
}

// Super-block j: the sum of (a[i] & mask) and the OR of (a[i] & ~mask) over
// tiles [j * SB_TILES, (j + 1) * SB_TILES) (or_out may be null).
__global__ __launch_bounds__(256) void k_sb_sums(const uint32_t* __restrict__ a, int ntiles, uint32_t mask,
                                                 uint32_t* __restrict__ sum_out, uint32_t* __restrict__ or_out) {
  __shared__ uint32_t red[8];
  const int lo = (int)blockIdx.x * SB_TILES;
  uint32_t hi;
  const uint32_t sum = block_reduce(a + lo, min(SB_TILES, ntiles - lo), mask, red, &hi);
  uint32_t orv = 0;
  for (int b = 0; b < 32; ++b)
    if ((~mask >> b) & 1u) orv |= __syncthreads_or((hi >> b) & 1u) ? 1u << b : 0u;
  if (threadIdx.x == 0) {
    sum_out[blockIdx.x] = sum;
    if (or_out) or_out[blockIdx.x] = orv;
  }
}

// Pass 2: pre-token start bits of every byte of a tile and the tile count,
// with the tile's error bits (invalid UTF-8; for a batch, the validity of a
// share of the offsets) above TILE_ERR_SHIFT.
template <int PAT>
__global__ __launch_bounds__(PT_THREADS) void k_pretok(const uint8_t* __restrict__ bytes, int64_t n,
                                                       const int64_t* __restrict__ offs, int nseq, int ntiles,
                                                       Work w) {
  __shared__ TileSmem sm;
  const int t = blockIdx.x;
  const int64_t t0 = (int64_t)t * TILE;
  // no block of this pass uses the counters: reset them for the passes after
  if (t == 0) {
    if (threadIdx.x < CTR_RESET_END) w.ctr[threadIdx.x] = 0u;
    for (int i = threadIdx.x; i < QGROUPS * QCTR_STRIDE; i += PT_THREADS) w.qctr[i] = 0u;
  }
  bool bad_off = false;
  if (offs) {
    for (int64_t q = (int64_t)t * PT_THREADS + threadIdx.x; q <= nseq; q += (int64_t)ntiles * PT_THREADS) {
      const int64_t o = offs[q];
      bad_off |= (q == 0 && o != 0) || (q == nseq && o != n) || o < 0 || o > n || (q < nseq && offs[q + 1] < o);
    }
  }
  uint32_t bits = 0;
  uint32_t cnt;
  bool counted = false, bad, unsup = false;
  int ebits = -1;  // the tile's error flags (bit 0 UTF-8, bit 1 offsets) once gathered
  if (PAT != 0) {
    // cl100k- and o200k-style rules: classes from the code bytes of the
    // summary pass
    const bool gap = stage_codes(n, t0, w, sm, &bad);
    tile_carries<PAT>(w, t, ntiles, sm);
    bits = gap ? pat_bits<PAT, false>(sm, &cnt, &unsup) : pat_bits<PAT, true>(sm, &cnt, &unsup);
    counted = true;
  } else {
    const bool na = stage_tile(bytes, n, offs, nseq, t0, sm);
    // pure-ASCII tiles need no decode pass (their masks come from the bytes)
    bad = na ? decode_span(n, t0, na, sm) : false;
    const int j0 = HALO + PT_CHUNK * threadIdx.x;
    if (!na) {
      uint32_t wc;
      const bool plain = t0 - HALO >= 0 && t0 - HALO + 16 * RAW_WORDS <= n && (!offs || sm.seq_lo == sm.seq_hi);
      bits = plain ? gpt2_ascii_bits<true>(sm, n, t0, &wc) : gpt2_ascii_bits<false>(sm, n, t0, &wc);
      // the wavefronts' counts and offset-check flags (an ASCII tile has no
      // UTF-8 error) through one barrier
      const uint32_t woff = __ballot(bad_off) ? 2u : 0u;
      if ((threadIdx.x & 63u) == 0) {
        sm.red[threadIdx.x >> 6] = wc;
        sm.red[4 + (threadIdx.x >> 6)] = woff;
      }
      __syncthreads();
      cnt = sm.red[0] + sm.red[1] + sm.red[2] + sm.red[3];
      ebits = (int)(sm.red[4] | sm.red[5] | sm.red[6] | sm.red[7]);
      counted = true;
    } else {
#pragma unroll
      for (int k = 0; k < PT_CHUNK; ++k) {
        uint32_t c = sm.code[cix(j0 + k)];
        if (is_char(c) && pred_gpt2<false>(sm.code, sm.plen, j0 + k)) bits |= 1u << k;
      }
    }
  }
  w.flags[(int64_t)t * PT_THREADS + threadIdx.x] = (uint16_t)bits;
  if (!counted) cnt = block_sum(__popc(bits), sm.red);
  if (ebits < 0) ebits = (__syncthreads_or(bad) ? 1 : 0) | (__syncthreads_or(bad_off) ? 2 : 0);
  const uint32_t err = ((ebits & 1) ? ERR_UTF8 : 0u) | ((ebits & 2) ? ERR_OFFSETS : 0u) | (unsup ? ERR_UNSUP : 0u);
  if (threadIdx.x == 0) {
    w.tile_cnt[t] = cnt | (err << TILE_ERR_SHIFT);
    // reset for the long-piece stitching of the next pass
    w.big_fail[t] = 0;
  }
}

// ----------------------------------------------------------------------- BPE

// 24-bit product (x < 2^24) as one full-rate instruction: with __umul24 the
// optimizer saw that only the low 24 bits of these products feed the bucket
// choices and turned them into quarter-rate 32-bit products.
__device__ __forceinline__ uint32_t mul_u24(uint32_t x, uint32_t c) {
  uint32_t r;
  asm("v_mul_u32_u24 %0, %1, %2" : "=v"(r) : "s"(c), "v"(x));
  return r;
}

// Rank of a pair with an operand >= 256 (every pair next to a new token),
// or RANK_NONE: its two buckets loaded together (16 bytes each), four slot
// keys compared; 24-bit products for the hash (exact: ids < 2^20), 32-bit
// byte offsets from the table base.
__device__ __forceinline__ uint32_t pair_rank_new(const Tables& tb, uint32_t x, uint32_t y) {
  const uint32_t mx = mul_u24(x, PAIR_MUL_X) ^ mul_u24(y, PAIR_MUL_Y);
  const uint32_t h1 = __umul24(mx, PAIR_MUL_1), h2 = __umul24(mx, PAIR_MUL_2);  // = pair_choice
  // byte offset of the partition in a row of 2^p buckets
  const uint32_t part = ((x ^ y) & ((1u << tb.pair_pbits) - 1u)) << 4;
  const int rs = tb.pair_pbits + 4;
  const uint32_t o1 = ((h1 >> tb.pair_shift) << rs) | part, o2 = ((h2 >> tb.pair_shift) << rs) | part;
  const char* base = reinterpret_cast<const char*>(tb.pair_tab);
  const uint4 e1 = *reinterpret_cast<const uint4*>(base + o1);
  const uint4 e2 = *reinterpret_cast<const uint4*>(base + o2);
  const uint32_t k = pair_slot_key(x, y, tb.pair_kshift, tb.pair_pbits);
  uint32_t r = e1.x == k ? e1.y : RANK_NONE;
  r = e1.z == k ? e1.w : r;
  r = e2.x == k ? e2.y : r;
  return e2.z == k ? e2.w : r;
}

// pair_rank_new for the lanes with on set, RANK_NONE elsewhere, without a
// branch: the other lanes load the table's first bucket (one cache line for
// all of them) and drop the result.  Inside a merge step some lane of the
// wavefront always probes, so a branch around the probe would skip nothing;
// without it the step's other work can be scheduled into the probe's wait.
__device__ __forceinline__ uint32_t pair_rank_if(const Tables& tb, bool on, uint32_t x, uint32_t y) {
  const uint32_t mx = mul_u24(x, PAIR_MUL_X) ^ mul_u24(y, PAIR_MUL_Y);
  const uint32_t h1 = __umul24(mx, PAIR_MUL_1), h2 = __umul24(mx, PAIR_MUL_2);  // = pair_choice
  const uint32_t part = ((x ^ y) & ((1u << tb.pair_pbits) - 1u)) << 4;
  const int rs = tb.pair_pbits + 4;
  // the offsets masked by an AND the compiler does not see through: as a
  // select it became a branch, or a select of 64-bit addresses
  const uint32_t keep = on ? ~0u : 0u;
  uint32_t o1 = ((h1 >> tb.pair_shift) << rs) | part, o2 = ((h2 >> tb.pair_shift) << rs) | part;
  asm("v_and_b32 %0, %1, %2" : "=v"(o1) : "v"(o1), "v"(keep));
  asm("v_and_b32 %0, %1, %2" : "=v"(o2) : "v"(o2), "v"(keep));
  const char* base = reinterpret_cast<const char*>(tb.pair_tab);
  const uint4 e1 = *reinterpret_cast<const uint4*>(base + o1);
  const uint4 e2 = *reinterpret_cast<const uint4*>(base + o2);
  const uint32_t k = pair_slot_key(x, y, tb.pair_kshift, tb.pair_pbits);
  uint32_t r = e1.x == k ? e1.y : RANK_NONE;
  r = e1.z == k ? e1.w : r;
  r = e2.x == k ? e2.y : r;
  r = e2.z == k ? e2.w : r;
  return on ? r : RANK_NONE;
}

// A merge step's probe: branch-free (LAT, for latency-bound passes: the
// step's other work fills the probe's wait) or behind a branch (fewer
// instructions, for passes bound by instruction issue).
template <bool LAT>
__device__ __forceinline__ uint32_t probe_step(const Tables& tb, bool on, uint32_t x, uint32_t y) {
  if (LAT) return pair_rank_if(tb, on, x, y);
  uint32_t r = RANK_NONE;
  if (on) r = pair_rank_new(tb, x, y);
  return r;
}

// Rank of merging the adjacent pair (x, y), or RANK_NONE: the byte-pair
// table for two bytes, else the two-choice table (both loaded together).
__device__ __forceinline__ uint32_t pair_rank(const Tables& tb, uint32_t x, uint32_t y) {
  const uint32_t bp = tb.byte_pair[((x & 255u) << 8) | (y & 255u)];
  const uint32_t r = pair_rank_new(tb, x, y);
  return (x | y) < 256u ? bp : r;
}

// The whole-word rule for a piece of len bytes at p, CACHE_MAXLEN < len <=
// tb.word_maxlen: the id of the token with exactly these bytes, or
// RANK_NONE.  Linear probing ends at an empty slot; a slot whose hash and
// length match is confirmed against the token's bytes.
__device__ uint32_t word_lookup(const Tables& tb, const uint8_t* __restrict__ p, uint32_t len) {
  uint64_t h = word_hash_init(len);
  for (uint32_t k = 0; k < len; k += 8) {
    uint64_t wd = 0;
    for (uint32_t j = 0; j < 8 && k + j < len; ++j) wd |= (uint64_t)p[k + j] << (8 * j);
    h = word_hash_step(h, wd);
  }
  const uint64_t key = (h >> 32 << 32) | ((uint64_t)len << ID_BITS);
  uint32_t slot = (uint32_t)h & tb.word_mask;
  for (int i = 0; i < tb.word_probe; ++i, slot = (slot + 1) & tb.word_mask) {
    const uint64_t e = tb.word_tab[slot];
    if (e == 0) break;
    if ((e & ~(uint64_t)ID_MASK) != key) continue;
    const uint32_t id = (uint32_t)e & ID_MASK;
    const uint8_t* q = tb.tok_bytes + tb.tok_off[id];
    bool same = true;
    for (uint32_t k = 0; k < len && same; ++k) same = p[k] == q[k];
    if (same) return id;
  }
  return RANK_NONE;
}

// Id of the single-token piece with these bytes (len 2..16), or RANK_NONE.
// One 128-byte bucket per step (the second key word only for len > 8); the
// walk ends at the first bucket that no key's probe run passed.
__device__ __forceinline__ uint32_t cache_lookup(const Tables& tb, uint64_t w0, uint64_t w1, uint32_t len) {
  uint32_t h = cache_hash(w0, w1, len, tb.cache_shift);
  for (int i = 0; i < tb.cache_probe; ++i) {
    const CacheBucket* b = tb.cache + h;
    const uint4 mt = *reinterpret_cast<const uint4*>(b->meta);
    const ulonglong2 a01 = *reinterpret_cast<const ulonglong2*>(&b->w0[0]);
    const ulonglong2 a23 = *reinterpret_cast<const ulonglong2*>(&b->w0[2]);
    ulonglong2 c01 = make_ulonglong2(0ull, 0ull), c23 = make_ulonglong2(0ull, 0ull);
    if (len > 8) {
      c01 = *reinterpret_cast<const ulonglong2*>(&b->w1[0]);
      c23 = *reinterpret_cast<const ulonglong2*>(&b->w1[2]);
    }
    const uint32_t m0 = mt.x & ~CACHE_MORE;
    if ((m0 & 31u) == len && a01.x == w0 && c01.x == w1) return (m0 >> 5) & ID_MASK;
    if ((mt.y & 31u) == len && a01.y == w0 && c01.y == w1) return (mt.y >> 5) & ID_MASK;
    if ((mt.z & 31u) == len && a23.x == w0 && c23.x == w1) return (mt.z >> 5) & ID_MASK;
    if ((mt.w & 31u) == len && a23.y == w0 && c23.y == w1) return (mt.w >> 5) & ID_MASK;
    if (!(mt.x & CACHE_MORE)) return RANK_NONE;
    h = (h + 1) & tb.cache_mask;
  }
  return RANK_NONE;
}

// DPP move: each lane reads another lane's x (dpp_ctrl CTRL); lanes without a
// source keep their own x.  Controls used: 0xB1 / 0x4E quad permutes (lane xor
// 1 / xor 2), 0x141 half-row mirror, 0x140 row mirror, 0x130 wave shift (lane
// i reads lane i + 1).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, 0xF, 0xF, false);
}

// Value of the next lane (wave_shl:1); the last lane reads 0.
__device__ __forceinline__ uint32_t lane_up1(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x130, 0xF, 0xF, true);
}
// Value of the previous lane (wave_shr:1); lane 0 reads 0.
__device__ __forceinline__ uint32_t lane_dn1(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x138, 0xF, 0xF, true);
}

// Minimum over each aligned group of G lanes (G = 2 ... 64): butterflies
// inside a 16-lane row by DPP (folded into the min instructions), then across
// rows by row broadcasts; G = 32 and 64 read the result from the last lane
// of each half / of the wavefront.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_all(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}
// x from another row into the rows of ROWS; the other rows read the identity
// of min, so min(x, dpp_rows(x)) folds into one DPP min.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_rows(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)0xFFFFFFFFu, (int)x, CTRL, ROWS, 0xF, false);
}
template <int G>
__device__ __forceinline__ uint32_t group_min(uint32_t x) {
  x = min(x, dpp_all<0xB1>(x));
  if (G >= 4) x = min(x, dpp_all<0x4E>(x));
  if (G >= 8) x = min(x, dpp_all<0x141>(x));
  if (G >= 16) x = min(x, dpp_all<0x140>(x));
  if (G == 32) {
    x = min(x, dpp_rows<0x142, 0xA>(x));  // rows 1, 3 += rows 0, 2
    x = (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x3E0);  // every lane reads lane 31 of its half
  } else if (G == 64) {
    x = min(x, dpp_rows<0x142, 0xA>(x));
    x = min(x, dpp_rows<0x143, 0xC>(x));  // rows 2, 3 += row 1
    x = (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
  }
  return x;
}

// The classic merge loop on 64 / G sequences at once, one per aligned group
// of G lanes: lane g of a group holds token g of its sequence (id, and with
// TRACK its first byte's offset pos), rk the rank of the pair (token g,
// token g + 1) or RANK_NONE, m the sequence's token count.  Each step takes
// the group minimum of (rank << 6 | position) -- the lowest rank, leftmost
// among equal pairs, exactly the classic choice -- merges that pair, shifts
// the tokens right of it one lane left, and the two lanes next to the new
// token probe the pair-rank table (both probes in flight together).  The
// loop runs while any group of the wavefront still has a merge (ballot: a
// wave-uniform exit around the DPP moves).
template <int G, bool TRACK, bool LAT = true>
__device__ __forceinline__ void group_merge_loop(const Tables& tb, uint32_t& id, uint32_t& rk, uint32_t& pos, int& m) {
  const int g = (int)(threadIdx.x & 63u) & (G - 1);
  for (;;) {
    const uint32_t kmin = group_min<G>((rk << 6) | (uint32_t)g);
    const bool act = kmin < (1u << 26);
    if (__ballot(act) == 0ull) break;
    const int bk = (int)(kmin & 63u);
    const uint32_t nid = 256u + (kmin >> 6);
    const uint32_t id1 = lane_up1(id), id2 = lane_up1(id1), rs = lane_up1(rk);
    const uint32_t pos1 = TRACK ? lane_up1(pos) : 0u;
    const uint32_t rk1 = g == G - 1 ? RANK_NONE : rs;  // nothing enters from the next group
    const bool do_l = LAT ? act & (g == bk - 1) : act && g == bk - 1;  // (bitwise: no branches)
    const bool do_r = LAT ? act & (g == bk) & (bk + 2 < m) : act && g == bk && bk + 2 < m;
    const uint32_t r = probe_step<LAT>(tb, do_l || do_r, do_l ? id : nid, do_l ? nid : id2);
    if (act) {
      const uint32_t nid_here = (g < bk) ? id : ((g == bk) ? nid : id1);
      rk = (g < bk - 1) ? rk : ((g == bk - 1 || g == bk) ? r : rk1);
      id = nid_here;
      if (TRACK && g > bk) pos = pos1;
      --m;
    }
  }
}

// Classic BPE of up to 64 / G queued pieces (queue entries chunk * (64 / G)
// ...), one per aligned group of G lanes, one byte position per lane (piece
// length <= G).  Tokens go to tmp_ids[s, s + cnt).
template <int G, bool LAT>
__device__ void group_bpe(const uint8_t* __restrict__ bytes, const Work& w, const Tables& tb,
                          const uint32_t* queue, int qn, int chunk) {
  const int lane = (int)(threadIdx.x & 63u);
  const int g = lane & (G - 1);
  const int qi = chunk * (64 / G) + lane / G;
  const bool valid = qi < qn;
  uint32_t p = 0;
  int32_t s = 0;
  int m = 0;
  if (valid) {
    p = queue[qi];
    s = w.piece_start[p];
    m = w.piece_start[p + 1] - s;
  }
  uint32_t id = (g < m) ? (uint32_t)bytes[s + g] : 0u;
  const uint32_t nx = lane_up1(id);
  // rk is RANK_NONE wherever no pair starts (g + 1 >= m), so the key of such
  // a lane, (RANK_NONE << 6) | g, lies above every real key (< 2^26)
  uint32_t rk = (g + 1 < m) ? tb.byte_pair[(id << 8) | (nx & 255u)] : RANK_NONE;
  uint32_t pos = 0;
  group_merge_loop<G, false, LAT>(tb, id, rk, pos, m);
  if (valid) {
    if (g < m) w.tmp_ids[s + g] = (int32_t)id;
    if (g == 0) w.piece_cnt[p] = m;
  }
  // token counts into the tiles the pieces start in: the group leaders' tiles
  // and counts are read into scalar registers and runs of equal tiles (the
  // pieces are consecutive queue entries) summed, one atomic per run
  const uint32_t tl = (valid && g == 0) ? (uint32_t)s / TILE : 0xFFFFFFFFu;
  const uint32_t val = (valid && g == 0) ? (uint32_t)m : 0u;
  uint32_t cur_t = 0xFFFFFFFFu, cur_sum = 0;
#pragma unroll
  for (int q = 0; q < 64 / G; ++q) {
    const uint32_t tq = (uint32_t)__builtin_amdgcn_readlane((int)tl, q * G);
    const uint32_t vq = (uint32_t)__builtin_amdgcn_readlane((int)val, q * G);
    if (tq != cur_t) {
      if (cur_t != 0xFFFFFFFFu && lane == 0) atomicAdd(&w.tile_tok[cur_t], cur_sum);
      cur_t = tq;
      cur_sum = 0;
    }
    cur_sum += vq;
  }
  if (cur_t != 0xFFFFFFFFu && lane == 0) atomicAdd(&w.tile_tok[cur_t], cur_sum);
}

// The classic merge loop with four token slots per lane: 64 / G sequences at
// once, one per aligned group of G lanes, token p of a sequence in slot p % 4
// of lane p / 4 of its group (sequences of up to 4 G tokens).  id[k] and
// rk[k] are the token in slot k and the rank of the pair it starts (RANK_NONE
// where no pair starts: at the sequence's last token and after it); m is the
// sequence's token count.  Each step: the group minimum of (rank << 6 |
// position) -- the lowest rank, leftmost among equal pairs, the classic
// choice -- then the tokens after the merged pair move one position left
// (slot k takes slot k + 1, the last slot the next lane's first), the merged
// pair's slot takes the new id, and the pairs on both sides of it get their
// ranks from the pair table: the lane holding the token before the pair
// probes (left, new) and the lane holding the pair probes (new, right), both
// probes of a step in flight together.  Every lane of a wavefront issues the
// step once for all four of its slots, which is what makes more than one
// slot per lane pay: a step costs a wavefront about twice as many
// instructions as with one slot per lane, for four times the positions.
template <int G>
__device__ __forceinline__ uint32_t group_rev(uint32_t x) {  // lane g reads lane G - 1 - g of its group
  return G == 2 ? dpp_all<0xB1>(x) : G == 4 ? dpp_all<0x1B>(x) : G == 8 ? dpp_all<0x141>(x) : dpp_all<0x140>(x);
}

template <int G, bool TRACK = false, bool LAT = true>
__device__ __forceinline__ void group_merge4(const Tables& tb, uint32_t (&id)[4], uint32_t (&rk)[4], int& m,
                                             uint32_t (&pos)[4]) {
  static_assert(G == 2 || G == 4 || G == 8 || G == 16, "groups within one DPP row");
  const int g = (int)(threadIdx.x & 63u) & (G - 1);
  const uint32_t pb = 4u * (uint32_t)g;
  const bool first = g == 0, last = g == G - 1;
  for (;;) {
    const uint32_t k0 = (rk[0] << 6) | pb, k1 = (rk[1] << 6) | (pb + 1u);
    const uint32_t k2 = (rk[2] << 6) | (pb + 2u), k3 = (rk[3] << 6) | (pb + 3u);
    const uint32_t kmin = group_min<G>(min(min(k0, k1), min(k2, k3)));
    const bool act = kmin < (1u << 26);
    if (__ballot(act) == 0ull) break;
    const int bk = (int)(kmin & 63u);
    const uint32_t nid = 256u + (kmin >> 6);
    // slot of the pair's left token if it is in this lane; a group with
    // nothing left to merge keeps every slot (lb past the lane)
    const int lb = act ? bk - (int)pb : 127;
    const uint32_t n0 = lane_up1(id[0]), r0 = lane_up1(rk[0]);
    const uint32_t rn = last ? RANK_NONE : r0;  // nothing enters from the next group
    const uint32_t rv3 = group_rev<G>(id[3]), dn3 = lane_dn1(id[3]);
    const uint32_t p3 = first ? rv3 : dn3;  // the cyclically previous lane's last token
    // One probe per lane: the lane holding the token before the pair probes
    // (that token, new); the lane holding the token three after the pair's
    // left one (lane 0 of the group if that is past the group) probes (new,
    // token after the pair).  No lane has both roles.
    // (LAT: bitwise on the bools, as the short-circuit form compiles into
    // branches; it is the shorter code where instruction issue is the bound)
    const bool do_l = (uint32_t)(lb - 1) < 4u;
    const bool do_r = LAT ? act & (bk + 2 < m) & (((uint32_t)(lb + 3) < 4u) | (first & (bk + 3 >= 4 * G)))
                          : act && bk + 2 < m && ((lb >= -3 && lb <= 0) || (first && bk + 3 >= 4 * G));
    // x = id[lb - 1] (lb in 1..4), y = id[lb + 2] (lb in -2..0) else p3: selects on
    // the bits of the slot number
    const uint32_t a = (uint32_t)(lb - 1), b = (uint32_t)(lb + 2);
    const uint32_t xl = (a & 1u) ? id[1] : id[0], xh = (a & 1u) ? id[3] : id[2];
    const uint32_t x = (a & 2u) ? xh : xl;
    uint32_t y = b == 2u ? id[2] : p3;  // flat selects (nested ones compiled into a branch)
    y = b == 1u ? id[1] : y;
    y = b == 0u ? id[0] : y;
    const uint32_t px = do_l ? x : nid, py = do_l ? nid : y;
    const uint32_t res = probe_step<LAT>(tb, do_l || do_r, px, py);
    // the right probe's result belongs to the lane holding the pair: the
    // prober itself (pair at slot 0) or the cyclically previous lane
    const uint32_t rvr = group_rev<G>(res), upr = lane_up1(res);
    const uint32_t rnx = last ? rvr : upr;
    const uint32_t rl = res, rr = lb == 0 ? res : rnx;
    const bool e0 = lb == 0, e1 = lb == 1, e2 = lb == 2, e3 = lb == 3, e4 = lb == 4;
    const bool t0 = lb > 0, t1 = lb > 1, t2 = lb > 2, t3 = lb > 3, t4 = lb > 4;
    const uint32_t i0 = e0 ? nid : t0 ? id[0] : id[1];
    const uint32_t i1 = e1 ? nid : t1 ? id[1] : id[2];
    const uint32_t i2 = e2 ? nid : t2 ? id[2] : id[3];
    const uint32_t i3 = e3 ? nid : t3 ? id[3] : n0;
    const uint32_t q0 = e0 ? rr : e1 ? rl : t1 ? rk[0] : rk[1];
    const uint32_t q1 = e1 ? rr : e2 ? rl : t2 ? rk[1] : rk[2];
    const uint32_t q2 = e2 ? rr : e3 ? rl : t3 ? rk[2] : rk[3];
    const uint32_t q3 = e3 ? rr : e4 ? rl : t4 ? rk[3] : rn;
    if (TRACK) {  // byte offsets move with the tokens; the new token keeps its left token's
      // slot k keeps its offset while k <= lb, else takes slot k + 1's
      const uint32_t pn = lane_up1(pos[0]);
      pos[0] = lb >= 0 ? pos[0] : pos[1];
      pos[1] = t0 ? pos[1] : pos[2];
      pos[2] = t1 ? pos[2] : pos[3];
      pos[3] = t2 ? pos[3] : pn;
    }
    id[0] = i0; id[1] = i1; id[2] = i2; id[3] = i3;
    rk[0] = q0; rk[1] = q1; rk[2] = q2; rk[3] = q3;
    m -= act ? 1 : 0;
  }
}

// Classic BPE of up to 64 / G queued pieces of at most 4 G bytes (queue
// entries chunk * (64 / G) ...), one per aligned group of G lanes, four byte
// positions per lane.  Tokens go to tmp_ids[s, s + cnt); the pieces' token
// counts are added to the tiles they start in, one atomic per run of pieces
// in one tile.
template <int G, bool LAT>
__device__ void group_bpe4(const uint8_t* __restrict__ bytes, const Work& w, const Tables& tb,
                           const uint32_t* queue, int qn, int chunk) {
  const int lane = (int)(threadIdx.x & 63u);
  const int g = lane & (G - 1);
  const int qi = chunk * (64 / G) + lane / G;
  const bool valid = qi < qn;
  uint32_t p = 0;
  int32_t s = 0;
  int m = 0;
  if (valid) {
    p = queue[qi];
    s = w.piece_start[p];
    m = w.piece_start[p + 1] - s;
  }
  const int pb = 4 * g;
  uint32_t id[4], rk[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) id[k] = pb + k < m ? (uint32_t)bytes[s + pb + k] : 0u;
  const uint32_t n0 = lane_up1(id[0]);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t nx = k < 3 ? id[k + 1] : n0;
    rk[k] = pb + k + 1 < m ? tb.byte_pair[(id[k] << 8) | nx] : RANK_NONE;
  }
  uint32_t pos[4];
  group_merge4<G, false, LAT>(tb, id, rk, m, pos);
  if (valid) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (pb + k < m) w.tmp_ids[s + pb + k] = (int32_t)id[k];
    if (g == 0) w.piece_cnt[p] = m;
  }
  const uint32_t tl = (valid && g == 0) ? (uint32_t)s / TILE : 0xFFFFFFFFu;
  const uint32_t val = (valid && g == 0) ? (uint32_t)m : 0u;
  uint32_t cur_t = 0xFFFFFFFFu, cur_sum = 0;
#pragma unroll
  for (int q = 0; q < 64 / G; ++q) {
    const uint32_t tq = (uint32_t)__builtin_amdgcn_readlane((int)tl, q * G);
    const uint32_t vq = (uint32_t)__builtin_amdgcn_readlane((int)val, q * G);
    if (tq != cur_t) {
      if (cur_t != 0xFFFFFFFFu && lane == 0) atomicAdd(&w.tile_tok[cur_t], cur_sum);
      cur_t = tq;
      cur_sum = 0;
    }
    cur_sum += vq;
  }
  if (cur_t != 0xFFFFFFFFu && lane == 0) atomicAdd(&w.tile_tok[cur_t], cur_sum);
}

__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
  x = min(x, swz_xor<16>(x));
  x = min(x, swz_xor<8>(x));
  x = min(x, swz_xor<4>(x));
  x = min(x, swz_xor<2>(x));
  x = min(x, swz_xor<1>(x));
  return min((uint32_t)__builtin_amdgcn_readlane((int)x, 0), (uint32_t)__builtin_amdgcn_readlane((int)x, 32));
}

// Merge starts of one 64-position chunk: ms[k] = eq[k] && !ms[k-1], ms[-1] =
// cin.  Inside a run of equal pairs this keeps every other position, which is
// what leftmost-first merging does (x x x x -> xx xx).  Runs of ones are
// filled from their start with a carry trick and masked by start parity.
__device__ __forceinline__ uint64_t alt_mask(uint64_t eq, uint64_t cin) {
  const uint64_t E = 0x5555555555555555ull;
  uint64_t starts = eq & ~(eq << 1);
  uint64_t se = starts & E, so = starts & ~E;
  if (cin && (eq & 1ull)) { se &= ~1ull; so |= 1ull; }
  uint64_t fe = eq & ~(eq + se);
  uint64_t fo = eq & ~(eq + so);
  return (fe & E) | (fo & ~E);
}

// A piece longer than LANE_CAP bytes, by one wavefront: exact global-minimum
// rounds.  Each round takes the lowest rank r present, merges every
// occurrence of that pair (alternating inside runs of equal pairs), compacts
// the ids in place and, in the same sweep, carries the rank of every pair that
// did not change and looks up the ranks of the pairs next to a new token.  In
// a consistent table a pair that contains the new token 256 + r ranks above
// r, so this equals the classic loop.  Ids and ranks live in the piece's own
// slice of tmp_ids / tmp_rank.
__device__ void long_bpe(const uint8_t* __restrict__ bytes, const Work& w, const Tables& tb, uint32_t p) {
  const int lane = (int)(threadIdx.x & 63u);
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  const int32_t s = (int32_t)uniform((uint32_t)w.piece_start[p]);
  int m = (int)uniform((uint32_t)(w.piece_start[p + 1] - s));
  uint32_t* I = reinterpret_cast<uint32_t*>(w.tmp_ids) + s;
  uint32_t* R = w.tmp_rank + s;
  uint32_t rmin = RANK_NONE;
  for (int base = 0; base < m; base += 64) {
    const int k = base + lane;
    if (k < m) {
      const uint32_t b = bytes[s + k];
      I[k] = b;
      const uint32_t r = k + 1 < m ? tb.byte_pair[(b << 8) | bytes[s + k + 1]] : RANK_NONE;
      R[k] = r;
      rmin = min(rmin, r);
    }
  }
  rmin = uniform(wave_min(rmin));
  __threadfence_block();
  while (rmin != RANK_NONE) {
    const uint32_t T = 256u + rmin;
    uint64_t cin = 0;
    uint32_t nmin = RANK_NONE;
    int out = 0;
    for (int base = 0; base < m; base += 64) {
      const int k = base + lane;
      const uint32_t id0 = k < m ? I[k] : 0u, id1 = k + 1 < m ? I[k + 1] : 0u, id2 = k + 2 < m ? I[k + 2] : 0u;
      const uint32_t r0 = k + 1 < m ? R[k] : RANK_NONE;
      const uint32_t r1 = k + 2 < m ? R[k + 1] : RANK_NONE;
      const uint32_t r2 = k + 3 < m ? R[k + 2] : RANK_NONE;
      const uint64_t ms = alt_mask(__ballot(r0 == rmin), cin);
      const bool m0 = (ms >> lane) & 1ull;
      const bool prev = lane ? ((ms >> (lane - 1)) & 1ull) : (cin != 0);
      const bool m1 = r1 == rmin && !m0;   // merge starts at k + 1
      const bool m2 = r2 == rmin && !m1;   // merge starts at k + 2
      const bool keep = k < m && !prev;    // the right half of a merge drops out
      const uint32_t nid = m0 ? T : id0;
      // the next surviving token: k + 2 after a merge at k, else k + 1
      const bool has_next = m0 ? (k + 2 < m) : (k + 1 < m);
      const uint32_t nxt = m0 ? (m2 ? T : id2) : (m1 ? T : id1);
      uint32_t nr = RANK_NONE;
      if (keep && has_next) nr = (m0 || m1) ? pair_rank_new(tb, nid, nxt) : r0;
      const uint64_t km = __ballot(keep);
      if (keep) {
        const int o = out + __popcll(km & lt_mask);
        I[o] = nid;
        R[o] = nr;
      }
      nmin = min(nmin, nr);
      out += __popcll(km);
      cin = ms >> 63;
    }
    m = (int)uniform((uint32_t)out);
    rmin = uniform(wave_min(nmin));
    __threadfence_block();
  }
  if (lane == 0) {
    w.piece_cnt[p] = m;
    atomicAdd(&w.tile_tok[s / TILE], (uint32_t)m);
    if (m > HUGE_TOKENS) w.huge_list[atomicAdd(&w.ctr[CTR_NHUGE], 1u)] = (int32_t)p;
  }
}

// Carry functions of the merge-start scan: bit 0 = carry out for carry in 0,
// bit 1 = carry out for carry in 1.  compose(f, g) applies f, then g.
constexpr uint32_t FN_ID = 2u;
__device__ __forceinline__ uint32_t fn_compose(uint32_t f, uint32_t g) {
  const uint32_t h0 = (f & 1u) ? (g >> 1) & 1u : g & 1u;
  const uint32_t h1 = (f & 2u) ? (g >> 1) & 1u : g & 1u;
  return h0 | (h1 << 1);
}
struct FnOp {
  static constexpr uint32_t IDENT = FN_ID;
  __device__ static __forceinline__ uint32_t combine(uint32_t f, uint32_t g) { return fn_compose(f, g); }
};

__device__ __forceinline__ uint32_t block_min(uint32_t x, uint32_t* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  x = wave_min(x);
  if (lane == 0) red[wid] = x;
  __syncthreads();
  uint32_t r = RANK_NONE;
  for (int v = 0; v < (int)(blockDim.x >> 6); ++v) r = min(r, red[v]);
  __syncthreads();
  return r;
}

constexpr int BIG_E = 8;                           // positions per thread and sweep step
constexpr int BIG_STEP = 256 * BIG_E;              // positions per sweep step of the workgroup
constexpr int BIG_LDS = BIG_STEP + 2 + (BIG_STEP + 2) / 32 + 1;  // skewed slots per staged array
__device__ __forceinline__ int big_slot(int i) { return i + (i >> 5); }  // spreads BIG_E-strided reads over the banks

// LDS of big_rounds: the staged ids and ranks of one sweep step plus scan space.
struct BigSmem {
  uint32_t id[BIG_LDS];
  uint32_t rk[BIG_LDS];
  uint32_t sh[16];
};

// Word k of a uint32 array at base (uniform): 32-bit byte offsets let the
// loads take the base from scalar registers.
__device__ __forceinline__ uint32_t big_word(const uint32_t* base, uint32_t k) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(base) + k * 4u);
}

// Rounds 1, 2, ... of piece p = bytes [s, s + m) by one workgroup of 256
// threads (s, m and rmin, the least pair rank left by the first round, are
// the same in every thread): exact global-minimum rounds, as long_bpe, for a
// piece whose stitching failed.  A sweep step's BIG_STEP positions (and two
// more on the right) are staged in LDS with coalesced loads; thread t then
// takes the BIG_E contiguous positions t * BIG_E ... .  Inside a run of equal
// pairs the merge starts alternate, so whether position k starts a merge
// depends on the carry from k - 1: each thread evaluates its positions for
// both carries and a block scan of the resulting carry functions picks the
// right one.  A block prefix sum of the surviving positions places the
// compacted ids; a step writes only left of the next step's positions, and
// all its LDS reads finish (barrier) before the next step is staged.  The
// staged ids and ranks are read from LDS where they are used, which keeps the
// code small enough in registers to live in the merge kernel.
__device__ int big_rounds(const Work& w, const Tables& tb, uint32_t p, int32_t s, int m, uint32_t rmin,
                          BigSmem& sm) {
  const int tid = (int)threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t* I = reinterpret_cast<uint32_t*>(w.tmp_ids) + s;
  uint32_t* R = w.tmp_rank + s;
  uint32_t lx = RANK_NONE, ly = RANK_NONE, lr = RANK_NONE;  // the last pair looked up and its rank
  int first = 0;  // a position at or before the first pair of rank rmin
  while (rmin != RANK_NONE) {
    const uint32_t T = 256u + rmin;
    uint32_t cin = 0, nmin = RANK_NONE;
    int nfirst = 0x7FFFFFFF;  // where this thread's least new rank first occurs
    // the steps before the one holding the pair just before the first pair
    // of rank rmin merge nothing, move nothing and keep their ranks: the
    // sweep starts there, with carry 0
    const int base0 = max(first - 1, 0) / BIG_STEP * BIG_STEP;
    int out = base0;
    for (int base = base0; base < m; base += BIG_STEP) {
      for (int j = 0; j <= BIG_E; ++j) {
        if (j < BIG_E || tid < 2) {
          const uint32_t k = (uint32_t)(base + tid + 256 * j);
          sm.id[big_slot(tid + 256 * j)] = (int)k < m ? big_word(I, k) : 0u;
          sm.rk[big_slot(tid + 256 * j)] = (int)k + 1 < m ? big_word(R, k) : RANK_NONE;
        }
      }
      __syncthreads();
      const int j0 = tid * BIG_E, k0 = base + j0;
      uint32_t eq = 0;
      for (int j = 0; j < BIG_E + 2; ++j) eq |= (sm.rk[big_slot(j0 + j)] == rmin ? 1u : 0u) << j;
      // merge starts of this thread's positions for carry in 0 (msA) and 1 (msB)
      uint32_t msA = 0, msB = 0, a = 0, b = 1;
      for (int j = 0; j < BIG_E; ++j) {
        const uint32_t e = (eq >> j) & 1u;
        a = e & (a ^ 1u);
        b = e & (b ^ 1u);
        msA |= a << j;
        msB |= b << j;
      }
      // carry into this thread: the step's carry through the functions of the threads before it
      const uint32_t inc = wave_incl_fwd<FnOp>(a | (b << 1), lane);
      if (lane == 63) sm.sh[wid] = inc;
      __syncthreads();
      uint32_t before = FN_ID;
      for (int v = 0; v < wid; ++v) before = fn_compose(before, sm.sh[v]);
      before = fn_compose(before, dpp_id<0x138>(FN_ID, inc));
      const uint32_t tc = (cin ? (before >> 1) : before) & 1u;
      const uint32_t ms = tc ? msB : msA;
      const uint32_t lastms = (ms >> (BIG_E - 1)) & 1u;
      const uint32_t msE = ((eq >> BIG_E) & 1u) & (lastms ^ 1u);
      const uint32_t msE1 = ((eq >> (BIG_E + 1)) & 1u) & (msE ^ 1u);
      const uint32_t msx = ms | (msE << BIG_E) | (msE1 << (BIG_E + 1));
      const uint32_t prev = (ms << 1) | tc;  // bit j: a merge starts at position j - 1
      uint32_t keep = 0;
      for (int j = 0; j < BIG_E; ++j)
        if (k0 + j < m && !((prev >> j) & 1u)) keep |= 1u << j;
      if (tid == 255) sm.sh[4] = lastms;
      uint32_t tot;
      int o = out + (int)block_excl_sum(__popc(keep), sm.sh + 8, &tot);
      for (int j = 0; j < BIG_E; ++j) {
        if (!((keep >> j) & 1u)) continue;
        const int k = k0 + j;
        const bool m0 = (msx >> j) & 1u, m1 = (msx >> (j + 1)) & 1u, m2 = (msx >> (j + 2)) & 1u;
        const uint32_t nid = m0 ? T : sm.id[big_slot(j0 + j)];
        const bool has_next = m0 ? (k + 2 < m) : (k + 1 < m);
        const uint32_t nxt = m0 ? (m2 ? T : sm.id[big_slot(j0 + j + 2)]) : (m1 ? T : sm.id[big_slot(j0 + j + 1)]);
        uint32_t nr = RANK_NONE;
        if (has_next && (m0 || m1)) {
          // (merged ids are never bytes; inside runs the same pair recurs)
          if (nid != lx || nxt != ly) {
            lx = nid;
            ly = nxt;
            lr = pair_rank_new(tb, nid, nxt);
          }
          nr = lr;
        } else if (has_next) {
          nr = sm.rk[big_slot(j0 + j)];
        }
        I[o] = nid;
        R[o] = nr;
        if (nr < nmin) {
          nmin = nr;
          nfirst = o;
        }
        ++o;
      }
      out += (int)tot;
      cin = uniform(sm.sh[4]);
      __syncthreads();  // the staged step is read; the next one may overwrite it
    }
    m = (int)uniform((uint32_t)out);
    // the ranks of the skipped steps count for the next minimum (and come
    // before every rewritten position)
    for (int k = tid; k < base0; k += 256) {
      const uint32_t r = big_word(R, (uint32_t)k);
      if (r < nmin || (r == nmin && k < nfirst)) {
        nmin = r;
        nfirst = k;
      }
    }
    rmin = uniform(block_min(nmin, sm.sh + 8));
    first = (int)uniform(block_min(nmin == rmin ? (uint32_t)nfirst : 0x7FFFFFFFu, sm.sh + 8));
  }
  if (tid == 0) {
    w.piece_cnt[p] = m;
    if (m > HUGE_TOKENS) w.huge_list[atomicAdd(&w.ctr[CTR_NHUGE], 1u)] = (int32_t)p;
  }
  return m;
}

// The first round of a piece longer than BIG_BYTES on one share [a, b) of
// it (the piece ends at e): every position holds its byte as id and the rank
// of the byte pair it starts (none at the piece's last byte).  A thread takes
// BIG_E contiguous positions per pass, its loads and lookups issued before
// any is used.  Returns the least rank of the share, the same in every thread.
__device__ uint32_t big_first_round(const uint8_t* __restrict__ bytes, const Work& w, const Tables& tb, int32_t a,
                                    int32_t b, int32_t e, BigSmem& sm) {
  uint32_t rmin = RANK_NONE;
  for (int32_t k0 = a + BIG_E * (int32_t)threadIdx.x; k0 < b; k0 += BIG_E * PT_THREADS) {
    uint32_t by[BIG_E + 1], r[BIG_E];
#pragma unroll
    for (int j = 0; j <= BIG_E; ++j) by[j] = k0 + j < e ? bytes[k0 + j] : 0u;
#pragma unroll
    for (int j = 0; j < BIG_E; ++j) r[j] = k0 + j + 1 < e ? tb.byte_pair[(by[j] << 8) | by[j + 1]] : RANK_NONE;
#pragma unroll
    for (int j = 0; j < BIG_E; ++j) {
      if (k0 + j < b) {
        w.tmp_ids[k0 + j] = (int32_t)by[j];
        w.tmp_rank[k0 + j] = r[j];
        rmin = min(rmin, r[j]);
      }
    }
  }
  return uniform(block_min(rmin, sm.sh + 8));
}


// ------------------------------------------------------------- stitched BPE
//
// A piece longer than BIG_BYTES is cut into chunks of SCH bytes counted from
// its first byte.  Every chunk is encoded on its own; two adjacent chunks
// join as they are when their edge tokens are compatible (tokens_compatible:
// the classic loop on the two tokens' bytes gives back the two tokens).  A
// token sequence whose every adjacent pair is compatible, built from tokens
// that are each their own encoding, is the classic encoding of its bytes, so
// joined chunks are exact.  Where two chunks do not join, a window -- the
// last k tokens of the left chunk and the first k of the right one -- is
// encoded again, and it replaces them if its own edge tokens are compatible
// with the chunk tokens next to it; k doubles up to SK_MAX.  A window takes at
// most (cnt - 1) / 2 tokens of a chunk with a boundary on its other side too,
// so the two windows of one chunk never meet and every adjacent pair of the
// result has been checked.  A boundary that no window within these limits
// repairs makes the piece fall back to exact global-minimum rounds
// (big_fallback, in k_bpe_merge).
//
// Each tile the piece covers encodes the chunks that overlap it and their
// two neighbours, and decides the boundaries between them; a boundary shared
// by two tiles is decided by both, from the same two chunks, the same way.
// The result stays sparse: the id of each token at its first byte in
// tmp_ids, -1 at every other byte of the piece; k_emit compacts it.
constexpr int SCH = RUN_BYTES;           // bytes per chunk
constexpr int SCH_MAX = TILE / SCH + 3;  // chunks a tile's region and its two neighbours can touch
constexpr int SWIN = 64;                 // longest window, bytes
constexpr int SWIN_TOK = 32;             // most tokens a window's encoding may have
constexpr int SK_MAX = 8;                // largest window half, tokens per side

struct StitchSmem {
  uint32_t tok[SCH_MAX][SCH];    // tokens of each chunk
  uint32_t win[SCH_MAX][SWIN_TOK];  // window tokens of boundary b (between chunks b and b + 1)
  int32_t wstart[SCH_MAX];       // first byte of each window
  uint32_t list[SCH_MAX];        // boundaries whose windows are encoded in this pass
  uint32_t red[8];
  uint32_t nlist, nopen, nfail;
  uint8_t pos[SCH_MAX][SCH];     // byte offset of each chunk token in its chunk
  uint8_t wpos[SCH_MAX][SWIN_TOK];  // byte offset of each window token in its window
  uint8_t cnt[SCH_MAX];          // tokens per chunk
  uint8_t wcnt[SCH_MAX];         // window tokens
  uint8_t wlen[SCH_MAX];         // window bytes
  uint8_t kb[SCH_MAX];           // window half of each boundary (0: the chunks join as they are)
  uint8_t state[SCH_MAX];        // 0 joined, 1 open, 2 beyond the limits
};

// Can token b follow token a in a BPE result: does the classic loop on
// bytes(a) + bytes(b) give exactly [a, b]?  The loop builds a and b from
// their operands.  At any moment the pair across the junction is (x, y), x on
// a's right spine (a, right(a), right(right(a)), ...) and y on b's left spine.
// It gets merged if it has a merge whose rank is below the rank that consumes
// x (an equal rank is this same pair further left, which goes first) and not
// above the rank that consumes y (an equal rank is this same pair further
// right, which goes after).  The walk visits the junction pairs from the last
// one, (a, b), back to the two edge bytes: of the two current tokens the one
// made later (the higher rank) steps down to its operand at the junction.
//
// The path of the walk does not depend on the ranks it finds, only its
// verdict does, so the loop runs to the end of the path without an early
// exit: each step's pair probe is then in flight with the child-id load of
// the next step instead of before it.
__device__ bool tokens_compatible(const Tables& tb, uint32_t a, uint32_t b) {
  uint32_t x = a, y = b, cx = RANK_NONE, cy = RANK_NONE;
  bool bad = false;
  for (int it = 0; it < 4 * SCH; ++it) {  // at most depth(a) + depth(b) <= 2 (SWIN - 1) steps
    const uint32_t r = pair_rank(tb, x, y);
    bad |= r != RANK_NONE && r < cx && r <= cy;
    if (x >= 256u && (y < 256u || x > y)) {
      cx = x - 256u;
      x = (uint32_t)(tb.kids[cx] >> 32);
    } else if (y >= 256u) {
      cy = y - 256u;
      y = (uint32_t)tb.kids[cy] & ID_MASK;
    } else {
      return !bad;
    }
  }
  return false;  // not reached for tokens of at most SWIN bytes; refusing only costs the fallback
}

// The stitched encoding of piece [s, e) on the region [a, b) of the tile at
// t0 (all the same in every thread): the region's ids at their token starts
// (-1 elsewhere) into ids_out[a, b).  Returns the number of tokens that start
// in the region, or -1 if some boundary needs a window beyond the limits
// (then nothing is written).
__device__ int stitch_region(const uint8_t* __restrict__ bytes, const Tables& tb, int32_t* __restrict__ ids_out,
                             int32_t s, int32_t e, int32_t a, int32_t b, int64_t t0, StitchSmem& sm) {
  const int tid = (int)threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nc = (e - s + SCH - 1) / SCH;
  const int klo = (a - s) / SCH, khi = (b - 1 - s) / SCH;
  const int c0 = max(klo - 1, 0), c1 = min(khi + 1, nc - 1);
  const int nch = c1 - c0 + 1, nb = nch - 1;
  // 1. each chunk on its own, eight per wavefront and pass: groups of 8
  // lanes, four byte positions per lane
  for (int q = 0; q < nch; q += 32) {
    const int i = q + 8 * wid + (lane >> 3), g = lane & 7, pb = 4 * g;
    const int32_t cs = s + (c0 + i) * SCH;
    const int len = i < nch ? min(SCH, e - cs) : 0;
    uint32_t id[4], rk[4], pos[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      id[k] = pb + k < len ? (uint32_t)bytes[cs + pb + k] : 0u;
      pos[k] = (uint32_t)(pb + k);
    }
    const uint32_t n0 = lane_up1(id[0]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t nx = k < 3 ? id[k + 1] : n0;
      rk[k] = pb + k + 1 < len ? tb.byte_pair[(id[k] << 8) | (nx & 255u)] : RANK_NONE;
    }
    int m = len;
    // a whole chunk of one byte value: its encoding from the run table (the
    // group's least and greatest byte agree)
    const uint32_t lo = group_min<8>(min(min(id[0], id[1]), min(id[2], id[3])));
    const uint32_t hi = ~group_min<8>(~max(max(id[0], id[1]), max(id[2], id[3])));
    if (len == SCH && lo == hi) {
      const RunChunk& rc = tb.runs[lo];
      m = (int)rc.cnt;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        id[k] = pb + k < m ? rc.id[pb + k] : 0u;
        pos[k] = pb + k < m ? rc.pos[pb + k] : 0u;
        rk[k] = RANK_NONE;
      }
    }
    group_merge4<8, true>(tb, id, rk, m, pos);
    if (i < nch) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (pb + k < m) {
          sm.tok[i][pb + k] = id[k];
          sm.pos[i][pb + k] = (uint8_t)pos[k];
        }
      if (g == 0) sm.cnt[i] = (uint8_t)m;
    }
  }
  if (tid == 0) {
    sm.nopen = 0u;
    sm.nfail = 0u;
  }
  __syncthreads();
  // 2. the boundaries: join where the edge tokens are compatible
  if (tid < nb) {
    const bool ok = tokens_compatible(tb, sm.tok[tid][sm.cnt[tid] - 1], sm.tok[tid + 1][0]);
    sm.kb[tid] = 0;
    sm.wcnt[tid] = 0;
    sm.state[tid] = ok ? 0 : 1;
    if (!ok) atomicAdd(&sm.nopen, 1u);
  }
  __syncthreads();
  for (int k = 1; k <= SK_MAX && uniform(sm.nopen) != 0u; k *= 2) {
    if (tid == 0) sm.nlist = 0u;
    __syncthreads();
    if (tid < nb && sm.state[tid] == 1) {
      const int p = sm.cnt[tid], q = sm.cnt[tid + 1];
      // a chunk with a boundary on its other side as well gives a window at
      // most (cnt - 1) / 2 tokens; the piece's first and last chunks all of theirs
      const int kl = c0 + tid > 0 ? (p - 1) / 2 : p;
      const int kr = c0 + tid + 1 < nc - 1 ? (q - 1) / 2 : q;
      const int32_t cs0 = s + (c0 + tid) * SCH, cs1 = cs0 + SCH;
      int32_t ws = 0, we = 0;
      bool fit = k <= kl && k <= kr;
      if (fit) {
        ws = cs0 + sm.pos[tid][p - k];
        we = k < q ? cs1 + sm.pos[tid + 1][k] : min(cs1 + SCH, e);
        fit = we - ws <= SWIN;
      }
      if (!fit) {
        sm.state[tid] = 2;
        atomicAdd(&sm.nfail, 1u);
      } else {
        sm.kb[tid] = (uint8_t)k;
        sm.wstart[tid] = ws;
        sm.wlen[tid] = (uint8_t)(we - ws);
        sm.list[atomicAdd(&sm.nlist, 1u)] = (uint32_t)tid;
      }
    }
    __syncthreads();
    if (uniform(sm.nfail) != 0u) break;
    // the windows, four per wavefront and pass: groups of 16 lanes, four
    // byte positions per lane
    const int nl = (int)uniform(sm.nlist);
    for (int q = 0; q < nl; q += 16) {
      const int wi = q + 4 * wid + (lane >> 4), g = lane & 15, pb = 4 * g;
      const bool valid = wi < nl;
      const int bb = valid ? (int)sm.list[wi] : 0;
      const int32_t ws = valid ? sm.wstart[bb] : 0;
      const int wl = valid ? (int)sm.wlen[bb] : 0;
      uint32_t id[4], rk[4], pos[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        id[k] = pb + k < wl ? (uint32_t)bytes[ws + pb + k] : 0u;
        pos[k] = (uint32_t)(pb + k);
      }
      const uint32_t n0 = lane_up1(id[0]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t nx = k < 3 ? id[k + 1] : n0;
        rk[k] = pb + k + 1 < wl ? tb.byte_pair[(id[k] << 8) | (nx & 255u)] : RANK_NONE;
      }
      int m = wl;
      group_merge4<16, true>(tb, id, rk, m, pos);
      if (valid) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (pb + k < m && pb + k < SWIN_TOK) {
            sm.win[bb][pb + k] = id[k];
            sm.wpos[bb][pb + k] = (uint8_t)pos[k];
          }
        if (g == 0) sm.wcnt[bb] = (uint8_t)m;
      }
    }
    __syncthreads();
    // the window's edge tokens against the chunk tokens next to it
    if (tid < nb && sm.state[tid] == 1 && sm.wcnt[tid] > SWIN_TOK) {
      sm.state[tid] = 2;  // more window tokens than kept: beyond the limits
      atomicAdd(&sm.nfail, 1u);
    }
    if (tid < nb && sm.state[tid] == 1) {
      const int kk = sm.kb[tid], p = sm.cnt[tid], q = sm.cnt[tid + 1], wc = sm.wcnt[tid];
      const bool okl = p - kk < 1 || tokens_compatible(tb, sm.tok[tid][p - kk - 1], sm.win[tid][0]);
      const bool okr = kk >= q || tokens_compatible(tb, sm.win[tid][wc - 1], sm.tok[tid + 1][kk]);
      if (okl && okr) {
        sm.state[tid] = 0;
        atomicSub(&sm.nopen, 1u);
      }
    }
    __syncthreads();
  }
  if (uniform(sm.nopen) != 0u) return -1;
  // 3. the region's image: each final token's id at its first byte, -1 at
  // the others (the barrier orders the two stores of a byte)
  for (int32_t j = a + tid; j < b; j += PT_THREADS) ids_out[j] = -1;
  __syncthreads();
  uint32_t mine = 0;
  for (int k = tid; k < nch * SCH; k += PT_THREADS) {
    const int i = k / SCH, j = k % SCH;
    const int head = i > 0 ? sm.kb[i - 1] : 0, tail = i < nb ? sm.kb[i] : 0;
    if (j >= head && j < (int)sm.cnt[i] - tail) {
      const int32_t at = s + (c0 + i) * SCH + sm.pos[i][j];
      if (at >= a && at < b) {
        ids_out[at] = (int32_t)sm.tok[i][j];
        ++mine;
      }
    }
  }
  for (int k = tid; k < nb * SWIN_TOK; k += PT_THREADS) {
    const int bb = k / SWIN_TOK, j = k % SWIN_TOK;
    if (sm.kb[bb] && j < sm.wcnt[bb]) {
      const int32_t at = sm.wstart[bb] + sm.wpos[bb][j];
      if (at >= a && at < b) {
        ids_out[at] = (int32_t)sm.win[bb][j];
        ++mine;
      }
    }
  }
  return (int)block_sum(mine, sm.red);
}

// stitch_region for piece p, with the failure hand-off: the first tile to
// find a boundary it cannot repair lists the piece for the fallback rounds
// (its other tiles' sparse output is then overwritten there).  Returns the
// tokens that start in the region, 0 on failure.
__device__ uint32_t stitch_piece(const uint8_t* __restrict__ bytes, const Work& w, const Tables& tb, uint32_t p,
                                 int32_t s, int32_t e, int32_t a, int32_t b, int64_t t0, StitchSmem& sm) {
  const int c = stitch_region(bytes, tb, w.tmp_ids, s, e, a, b, t0, sm);
  if (c >= 0) return (uint32_t)c;
  if (threadIdx.x == 0 && atomicCAS(&w.big_fail[(e - 1) / TILE], 0, 1) == 0)
    w.fall_list[atomicAdd(&w.ctr[CTR_NFALL], 1u)] = (int32_t)p;
  return 0u;
}

// Fallback for a piece whose stitching failed: the exact global-minimum
// rounds by the whole workgroup (first round from the bytes, then
// big_rounds), ids contiguous in tmp_ids[s, s + m).  The piece's tokens then
// count in the tile it starts in, and the stitched counts its tiles posted to
// tile_tok are taken back.
__device__ void big_fallback(const uint8_t* __restrict__ bytes, const Work& w, const Tables& tb, uint32_t p,
                             BigSmem& sm) {
  const int32_t s = (int32_t)uniform((uint32_t)w.piece_start[p]);
  const int32_t e = (int32_t)uniform((uint32_t)w.piece_start[p + 1]);
  const uint32_t rmin = big_first_round(bytes, w, tb, s, e, e, sm);
  const int m = big_rounds(w, tb, p, s, e - s, rmin, sm);
  const int ts = s / TILE, te = (e - 1) / TILE;
  for (int t = ts + (int)threadIdx.x; t <= te; t += (int)blockDim.x) {
    uint32_t* hc = &w.huge_hc[t == ts ? 2 * t + 1 : 2 * t];
    const uint32_t add = (t == ts ? (uint32_t)m : 0u) - *hc;  // modulo 2^32: a subtraction
    *hc = 0u;  // no stitched tokens of this piece remain in the tile
    if (add) atomicAdd(&w.tile_tok[t], add);
  }
}

// The last tile before t with a pre-token start, scanning tiles [lo, t)
// down 512 at a time (8 loads in flight per lane), or -1; the same in every
// lane.
__device__ __forceinline__ int last_tile_in(const Work& w, int lo, int t, uint32_t cmask) {
  const int lane = (int)(threadIdx.x & 63u);
  for (int b = t - 1; b >= lo; b -= 512) {
    uint32_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int bb = b - 64 * k - lane;
      v[k] = bb >= lo ? w.tile_cnt[bb] & cmask : 0u;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint64_t nz = __ballot(v[k] != 0u);
      if (nz) return b - 64 * k - (__ffsll((unsigned long long)nz) - 1);
    }
  }
  return -1;
}

// The first tile in (t, hi) with a pre-token start, or hi.
__device__ __forceinline__ int first_tile_in(const Work& w, int t, int hi, uint32_t cmask) {
  const int lane = (int)(threadIdx.x & 63u);
  for (int b = t + 1; b < hi; b += 512) {
    uint32_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int bb = b + 64 * k + lane;
      v[k] = bb < hi ? w.tile_cnt[bb] & cmask : 0u;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint64_t nz = __ballot(v[k] != 0u);
      if (nz) return b + 64 * k + __ffsll((unsigned long long)nz) - 1;
    }
  }
  return hi;
}

// The last pre-token start before tile t (t >= 1; byte 0 always starts one),
// from the tile counts and start bits; the same in every lane.  With SB the
// search skips whole runs of SB_TILES tiles without a start (their sums are
// zero), so its length does not grow with the input.
template <bool SB>
__device__ int32_t last_start_before(const Work& w, int t, uint32_t cmask) {
  const int lane = (int)(threadIdx.x & 63u);
  int f;
  if (SB) {
    const int r0 = t / SB_TILES * SB_TILES;
    f = last_tile_in(w, r0, t, cmask);
    if (f < 0) {
      int j = -1;
      for (int b = t / SB_TILES - 1; b >= 0 && j < 0; b -= 64) {
        const uint64_t nz = __ballot(b - lane >= 0 && w.sb_cnt[b - lane] != 0u);
        if (nz) j = b - (__ffsll((unsigned long long)nz) - 1);
      }
      f = j < 0 ? -1 : last_tile_in(w, j * SB_TILES, (j + 1) * SB_TILES, cmask);
    }
  } else {
    f = last_tile_in(w, 0, t, cmask);
  }
  if (f < 0) return 0;
  for (int q = PT_THREADS - 64; q >= 0; q -= 64) {
    const uint32_t fl = w.flags[(int64_t)f * PT_THREADS + q + lane];
    const uint64_t fm = __ballot(fl != 0u);
    if (fm) {
      const int l = 63 - __clzll((long long)fm);
      const uint32_t flw = (uint32_t)__builtin_amdgcn_readlane((int)fl, l);
      return (int32_t)((int64_t)f * TILE + PT_CHUNK * (q + l) + 31 - __clz(flw));
    }
  }
  return 0;
}

// The first pre-token start after tile t, else n; nc1 = the count of tile
// t + 1 + lane and fl1 = the start bits of tile t + 1's thread lane, loaded
// ahead.  Every wavefront runs the same search; the ballots keep it uniform.
// With SB it skips whole runs of SB_TILES tiles without a start.
template <bool SB>
__device__ int32_t first_start_after(const Work& w, int t, int ntiles, int64_t n, uint32_t cmask, uint32_t nc1,
                                     uint32_t fl1) {
  const int lane = (int)(threadIdx.x & 63u);
  // usually the next tile has a start in its first 256 bytes
  const uint64_t nz1 = __ballot((nc1 & cmask) != 0u);
  const uint64_t fm1 = __ballot(fl1 != 0u);
  if ((nz1 & 1ull) && fm1) {
    const int l = __ffsll((unsigned long long)fm1) - 1;
    const uint32_t flw = (uint32_t)__builtin_amdgcn_readlane((int)fl1, l);
    return (int32_t)((int64_t)(t + 1) * TILE + PT_CHUNK * l + __ffs(flw) - 1);
  }
  int f;
  if (SB) {
    const int r1 = min(ntiles, (t / SB_TILES + 1) * SB_TILES);
    f = first_tile_in(w, t, r1, cmask);
    if (f >= r1) {
      const int nsb = (ntiles + SB_TILES - 1) / SB_TILES;
      int j = nsb;
      for (int b = t / SB_TILES + 1; b < nsb && j >= nsb; b += 64) {
        const uint64_t nz = __ballot(b + lane < nsb && w.sb_cnt[b + lane] != 0u);
        if (nz) j = b + __ffsll((unsigned long long)nz) - 1;
      }
      f = j >= nsb ? ntiles : first_tile_in(w, j * SB_TILES - 1, min(ntiles, (j + 1) * SB_TILES), cmask);
    }
  } else {
    f = first_tile_in(w, t, ntiles, cmask);
  }
  if (f >= ntiles) return (int32_t)n;
  for (int q = 0; q < PT_THREADS; q += 64) {
    const uint32_t fl = w.flags[(int64_t)f * PT_THREADS + q + lane];
    const uint64_t fm = __ballot(fl != 0u);
    if (fm) {
      const int l = __ffsll((unsigned long long)fm) - 1;
      const uint32_t flw = (uint32_t)__builtin_amdgcn_readlane((int)fl, l);
      return (int32_t)((int64_t)f * TILE + PT_CHUNK * (q + l) + __ffs(flw) - 1);
    }
  }
  return (int32_t)n;
}

// Pass 3: piece starts in order, from the counts of the tiles before and a
// block scan of the start bits.  The last tile adds the sentinel n and sets P
// and the error bits; for a bare pre-tokenization it writes P (or the error
// code) to *out_np.  With CLASSIFY, the tile then takes the first BPE step of
// every piece that starts in it: single bytes and pieces found in the
// single-token table finish here; pieces of up to LANE_CAP bytes go to the
// global queue of their length class (<= 8, 16, 32, 64 bytes) for
// k_bpe_merge, longer ones up to BIG_BYTES to the long list (one atomic per
// class and round of 256 pieces reserves the slots).  The end of the tile's
// last piece is the first start in a later tile, found from the tile counts
// and start bits.  A piece longer than BIG_BYTES (only the tile's last one
// and the one its first bytes end can be) is stitched here, each tile doing
// the stretch of it that lies in the tile (stitch_piece).
template <bool CLASSIFY, bool SB>
__global__ __launch_bounds__(PT_THREADS) __attribute__((amdgpu_waves_per_eu(6))) void k_compact(const uint8_t* __restrict__ bytes, Work w, Tables tb,
                                                        int ntiles, int64_t n, int32_t* __restrict__ starts,
                                                        int64_t* __restrict__ out_np) {
  // the piece starts and the staged bytes of the classification, and after
  // it the LDS of big_rounds, in one place
  constexpr size_t SST_BYTES = sizeof(int32_t) * (TILE + 4);
  constexpr size_t CLS_BYTES = SST_BYTES + 16 * ((TILE + CACHE_MAXLEN) / 16);
  constexpr size_t LDS_BYTES = CLS_BYTES > sizeof(StitchSmem) ? CLS_BYTES : sizeof(StitchSmem);
  static_assert(SST_BYTES % 16 == 0, "staged bytes stay 16-byte aligned");
  __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
  __shared__ uint32_t red[8];
  __shared__ uint32_t qn[5], qbase[5];
  int32_t* sst = reinterpret_cast<int32_t*>(lds);                  // [TILE + 1]
  uint4* stage = reinterpret_cast<uint4*>(lds + SST_BYTES);        // [(TILE + CACHE_MAXLEN) / 16]
  StitchSmem& st = *reinterpret_cast<StitchSmem*>(lds);
  const int t = blockIdx.x;
  const int lane = (int)(threadIdx.x & 63u);
  const uint32_t cmask = (1u << TILE_ERR_SHIFT) - 1u;
  const bool last = t == ntiles - 1;
  const int64_t t0 = (int64_t)t * TILE;
  // independent loads first, so that their latencies overlap: this tile's
  // start bits, its bytes (+ CACHE_MAXLEN), the next tile's count and first
  // start bits (where the last piece usually ends), and the first step of the
  // prefix over the tile counts before it
  uint32_t bits = w.flags[(int64_t)t * PT_THREADS + threadIdx.x];
  const bool aligned = (reinterpret_cast<uintptr_t>(bytes) & 15u) == 0;
  uint4 sv = make_uint4(0u, 0u, 0u, 0u);
  const int64_t sg = t0 + 16 * (int64_t)threadIdx.x;
  const bool stage_fast = CLASSIFY && aligned && threadIdx.x < (TILE + CACHE_MAXLEN) / 16 && sg + 16 <= n;
  if (stage_fast) sv = *reinterpret_cast<const uint4*>(bytes + sg);
  const uint32_t nc1 = (CLASSIFY && t + 1 + lane < ntiles) ? w.tile_cnt[t + 1 + lane] : 0u;
  const uint32_t fl1 = (CLASSIFY && t + 1 < ntiles) ? w.flags[(int64_t)(t + 1) * PT_THREADS + lane] : 0u;
  // the previous tile's count, for the end of a long piece that began before this tile
  const uint32_t prev_cnt = (CLASSIFY && t > 0) ? w.tile_cnt[t - 1] : 0u;
  uint32_t hi;
  // the last tile also folds its own count and error bits into the totals
  const uint32_t base = tile_prefix<SB>(w.tile_cnt, w.sb_cnt, w.sb_err, last ? t + 1 : t, cmask, red, &hi) -
                        (last ? (w.tile_cnt[t] & cmask) : 0u);
  uint32_t tot;
  uint32_t lpos = block_excl_sum(__popc(bits), red, &tot);
  uint32_t pos = base + lpos;
  const int64_t p0 = t0 + (int64_t)PT_CHUNK * threadIdx.x;
  while (bits) {
    const int k = __ffs(bits) - 1;
    bits &= bits - 1;
    starts[pos++] = (int32_t)(p0 + k);
    if (CLASSIFY) sst[lpos++] = (int32_t)(p0 + k);
  }
  if (last) {
    const uint32_t e = (__syncthreads_or(hi & (ERR_UTF8 << TILE_ERR_SHIFT)) ? ERR_UTF8 : 0u) |
                       (__syncthreads_or(hi & (ERR_OFFSETS << TILE_ERR_SHIFT)) ? ERR_OFFSETS : 0u) |
                       (__syncthreads_or(hi & (ERR_UNSUP << TILE_ERR_SHIFT)) ? ERR_UNSUP : 0u);
    const uint32_t P = base + tot;
    if (threadIdx.x == 0) {
      w.ctr[CTR_P] = P;
      w.ctr[CTR_ERR] = e;
      starts[P] = (int32_t)n;
      if (out_np) *out_np = e ? err_code(e) : (int64_t)P;
    }
  }
  if (threadIdx.x == 0) w.tile_pbase[t] = base;
  if (!CLASSIFY) return;
  if (tot == 0) {
    // the whole tile lies inside one piece; if it is longer than BIG_BYTES,
    // this tile's part of its stitched encoding
    const int32_t sp = last_start_before<SB>(w, t, cmask);
    const int32_t ep = first_start_after<SB>(w, t, ntiles, n, cmask, nc1, fl1);
    uint32_t hh = 0;
    if (ep - sp > BIG_BYTES)
      hh = stitch_piece(bytes, w, tb, base - 1, sp, ep, (int32_t)t0, (int32_t)min<int64_t>(ep, t0 + TILE), t0, st);
    if (threadIdx.x == 0) {
      w.tile_tok[t] = hh;
      w.huge_hc[2 * t] = hh;
      w.huge_hc[2 * t + 1] = 0u;
    }
    return;
  }
  // end of the last piece: the first start after this tile, else n
  const int32_t e_next = first_start_after<SB>(w, t, ntiles, n, cmask, nc1, fl1);
  if (threadIdx.x == 0) sst[tot] = e_next;
  // the tile's bytes plus CACHE_MAXLEN, for single bytes and table keys
  if (threadIdx.x < (TILE + CACHE_MAXLEN) / 16) {
    if (!stage_fast) {
      uint32_t wv[4] = {0u, 0u, 0u, 0u};
      for (int k = 0; k < 16; ++k)
        if (sg + k < n) wv[k >> 2] |= (uint32_t)bytes[sg + k] << (8 * (k & 3));
      sv = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
    stage[threadIdx.x] = sv;
  }
  if (threadIdx.x < 5) qn[threadIdx.x] = 0;
  __syncthreads();
  const uint8_t* sb = reinterpret_cast<const uint8_t*>(stage);
  uint32_t fin = 0;  // pieces of one token finished here
  for (uint32_t k0 = 0; k0 < tot; k0 += PT_THREADS) {
    const uint32_t k = k0 + threadIdx.x;
    const uint32_t p = base + k;
    int cls = -1;
    uint32_t slot = 0;
    if (k < tot) {
      const int32_t s = sst[k];
      const int32_t len = sst[k + 1] - s;
      const int off = (int)(s - t0);
      // the whole-word rule, for pieces longer than the cache's keys
      const uint32_t word = len > CACHE_MAXLEN && len <= tb.word_maxlen
                                ? word_lookup(tb, bytes + s, (uint32_t)len)
                                : RANK_NONE;
      if (word != RANK_NONE) {
        w.tmp_ids[s] = (int32_t)word;
        w.piece_cnt[p] = 1;
        ++fin;
      } else if (len > BIG_BYTES) {
        // only a tile's last piece can be this long: the tile stitches it below
      } else if (len > LANE_CAP) {
        cls = 4;
      } else if (len == 1) {
        w.tmp_ids[s] = sb[off];
        w.piece_cnt[p] = 1;
        ++fin;
      } else {
        uint32_t hit = RANK_NONE;
        if (len <= CACHE_MAXLEN) {
          // the key's bytes from three aligned 8-byte LDS reads, shifted and
          // masked to the piece (a byte-by-byte loop under len compiled into
          // sixteen branches, each waiting for its read): the staging ends
          // at byte TILE + CACHE_MAXLEN, so the reads up to (off & ~7) + 24
          // stay inside it for every off in the tile
          static_assert(CACHE_MAXLEN == 16 && (TILE + CACHE_MAXLEN) % 8 == 0, "three 8-byte words cover a key");
          const uint64_t* sq = reinterpret_cast<const uint64_t*>(stage);
          const int q = off >> 3, sh = (off & 7) * 8;
          const uint64_t q0 = sq[q], q1 = sq[q + 1], q2 = sq[q + 2];
          uint64_t w0 = sh ? (q0 >> sh) | (q1 << (64 - sh)) : q0;
          uint64_t w1 = sh ? (q1 >> sh) | (q2 << (64 - sh)) : q1;
          w0 = len >= 8 ? w0 : w0 & ((1ull << (8 * len)) - 1ull);
          w1 = len >= 16 ? w1 : len > 8 ? w1 & ((1ull << (8 * (len - 8))) - 1ull) : 0ull;
          hit = cache_lookup(tb, w0, w1, (uint32_t)len);
        }
        if (hit != RANK_NONE) {
          w.tmp_ids[s] = (int32_t)hit;
          w.piece_cnt[p] = 1;
          ++fin;
        } else {
          cls = len <= 8 ? 0 : len <= 16 ? 1 : len <= 32 ? 2 : 3;
        }
      }
      if (cls >= 0) slot = atomicAdd(&qn[cls], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 5) {
      const uint32_t c = qn[threadIdx.x];
      uint32_t* ctr = &w.qctr[(t % QGROUPS) * QCTR_STRIDE + threadIdx.x];
      qbase[threadIdx.x] = c ? atomicAdd(ctr, c) : 0u;
    }
    __syncthreads();
    if (cls >= 0) {
      uint32_t* q = cls < 4 ? w.queue[cls] + (t % QGROUPS) * w.qcap[cls]
                            : reinterpret_cast<uint32_t*>(w.long_list) + (t % QGROUPS) * w.lcap;
      q[qbase[cls] + slot] = p;
    }
    // another round reuses the class counts and reads qbase again: a barrier
    // between (after the last round the block sum below orders what follows)
    if (k0 + PT_THREADS < tot) {
      if (threadIdx.x < 5) qn[threadIdx.x] = 0;
      __syncthreads();
    }
  }
  // tokens of the tile's finished pieces; merged pieces add theirs later
  const uint32_t tok = block_sum(fin, red);
  // pieces longer than BIG_BYTES, stitched (this tile's part of each): the
  // bytes before the tile's first start end a piece that began before the
  // tile (that long only if the tile before has no start), and the tile's
  // last piece (its end comes from this tile's search)
  const int32_t fs = (int32_t)uniform((uint32_t)sst[0]);
  const int32_t ls = (int32_t)uniform((uint32_t)sst[tot - 1]);
  const int32_t le = (int32_t)uniform((uint32_t)sst[tot]);
  __syncthreads();  // the classification's LDS is read; the stitching reuses it
  uint32_t hh = 0, ht = 0;
  if (t > 0 && fs > t0 && (prev_cnt & cmask) == 0u) {
    const int32_t sp = last_start_before<SB>(w, t, cmask);
    if (fs - sp > BIG_BYTES) hh = stitch_piece(bytes, w, tb, base - 1, sp, fs, (int32_t)t0, fs, t0, st);
  }
  if (le - ls > BIG_BYTES) {
    // count 0 marks the sparse layout (a fallback writes its real count)
    if (threadIdx.x == 0) w.piece_cnt[base + tot - 1] = 0;
    ht = stitch_piece(bytes, w, tb, base + tot - 1, ls, le, ls, (int32_t)min<int64_t>(le, t0 + TILE), t0, st);
  }
  if (threadIdx.x == 0) {
    w.tile_tok[t] = tok + hh + ht;
    w.huge_hc[2 * t] = hh;
    w.huge_hc[2 * t + 1] = ht;
  }
}

// Pass 5: BPE of the queued pieces.  Work items are wavefront loads: one long
// piece, one piece of 33-64 bytes, eight of <= 32, sixteen of <= 16 or
// thirty-two of <= 8, numbered longest class first and dealt round-robin to
// the wavefronts (of the XCD that compacted their tiles, for queued pieces),
// so the longest merge chains start first.  The item index is the same in
// every lane, so the loop and the class branches are scalar.
constexpr int MERGE_THREADS = 256;
constexpr int64_t MERGE_SMALL = (int64_t)1 << 21;  // inputs up to 2 MiB: the 4-wave merge pass
// WAVES: wavefronts per SIMD the register budget is made for.  An input of
// up to MERGE_SMALL bytes has fewer work items than a 4-wave grid has
// wavefronts, and its time is its longest merge chains: 4 waves per SIMD
// give those chains registers (no spills) and the SIMDs to themselves.
// Larger inputs keep 8 waves per SIMD to hide the probes' latency.
template <int WAVES>
__global__ __launch_bounds__(MERGE_THREADS) __attribute__((amdgpu_waves_per_eu(WAVES, WAVES))) void k_bpe_merge(const uint8_t* __restrict__ bytes, Work w, Tables tb) {
  __shared__ uint32_t pre[6], qlen[5];
  __shared__ BigSmem big;  // LDS of the fallback rounds
  const uint32_t x = blockIdx.x % QGROUPS;
  // this group's queue counts, loaded with the fallback count (their loads
  // overlap); class c's count goes to qlen[c], so that an item's first
  // load is its queue entries
  const uint32_t qk = threadIdx.x < 5 ? w.qctr[x * QCTR_STRIDE + 4 - threadIdx.x] : 0u;
  // pieces whose stitching failed: exact rounds, a whole workgroup each, first
  const uint32_t nfall = w.ctr[CTR_NFALL];
  for (uint32_t f = blockIdx.x; f < nfall; f += gridDim.x)
    big_fallback(bytes, w, tb, uniform((uint32_t)w.fall_list[f]), big);
  const uint32_t wid = threadIdx.x >> 6;
  // the workgroups of group x = blockIdx mod QGROUPS take sub-queue x, the
  // pieces of the tiles t = x mod QGROUPS.  Workgroups are dealt to the 8
  // XCDs in turn, so these are the XCD that compacted those tiles and will
  // emit them: the pieces' starts, bytes and output ids stay in one L2.
  // (The grid has at least QGROUPS workgroups.)
  const uint32_t nwx = (gridDim.x - x + QGROUPS - 1) / QGROUPS * (MERGE_THREADS / 64);
  const uint32_t wx = uniform((blockIdx.x / QGROUPS) * (MERGE_THREADS / 64) + wid);
  // work items per class, longest first: a long piece (65 bytes .. BIG_BYTES,
  // exact rounds by the wavefront) or a 33-64 byte piece alone (their merge
  // chains are the kernel's critical path: one token slot per lane keeps the
  // steps short); 32 / 16 / 8 shorter pieces together, four token slots per
  // lane.  pre[i]: items before class 4 - i.
  if (threadIdx.x < 5) {
    const uint32_t c = 4u - threadIdx.x;
    qlen[c] = qk;
    pre[threadIdx.x + 1] = c >= 3u ? qk : (qk + (32u >> c) - 1) >> (5 - c);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    pre[0] = 0u;
    for (int i = 1; i <= 5; ++i) pre[i] += pre[i - 1];
  }
  __syncthreads();
  const uint32_t total = uniform(pre[5]);
  // rounds of nwx items, every other round dealt in reverse: the waves that
  // drew the longest items in one round draw the shortest in the next.  A
  // wavefront's issue priority follows its item's length class, so that the
  // SIMDs favour the longest merge chains over the short items that fill in
  // around them.
  for (uint32_t rnd = 0, u = wx; u < total; ++rnd, u = rnd * nwx + ((rnd & 1u) ? nwx - 1u - wx : wx)) {
    const uint32_t i = u < uniform(pre[1]) ? 0u : u < uniform(pre[2]) ? 1u : u < uniform(pre[3]) ? 2u
                     : u < uniform(pre[4]) ? 3u : 4u;
    const uint32_t c = 4u - i;
    const uint32_t item = u - uniform(pre[i]);
    if (c == 4) {
      __builtin_amdgcn_s_setprio(3);
      long_bpe(bytes, w, tb, uniform((uint32_t)w.long_list[x * w.lcap + item]));
      continue;
    }
    const uint32_t qn = uniform(qlen[c]);
    const uint32_t* q = w.queue[c] + x * w.qcap[c];
    if (c == 3) {
      __builtin_amdgcn_s_setprio(3);
      group_bpe<64, WAVES == 4>(bytes, w, tb, q, (int)qn, (int)item);
    } else if (c == 2) {
      __builtin_amdgcn_s_setprio(2);
      group_bpe4<8, WAVES == 4>(bytes, w, tb, q, (int)qn, (int)item);
    } else if (c == 1) {
      __builtin_amdgcn_s_setprio(1);
      group_bpe4<4, WAVES == 4>(bytes, w, tb, q, (int)qn, (int)item);
    } else {
      __builtin_amdgcn_s_setprio(0);
      group_bpe4<2, WAVES == 4>(bytes, w, tb, q, (int)qn, (int)item);
    }
  }
}

// ------------------------------------------------------------------ emission

constexpr uint32_t HUGE_CHUNK = 4096;  // tokens per grid work item of a huge piece
static_assert(HUGE_CHUNK % (EMIT_THREADS * 8) == 0, "a chunk is whole passes of 8 tokens per thread");

// Byte-offset export only: chunk k of a huge piece (tokens [k * HUGE_CHUNK,
// (k + 1) * HUGE_CHUNK)) gets its byte length written to tmp_rank[s + k] (s =
// the piece's first byte; the piece's ranks are dead by now and its byte
// range is at least as long as its chunk count), for every chunk but the
// last.  Items (piece, chunk) are dealt round-robin to the workgroups.
__global__ __launch_bounds__(EMIT_THREADS) void k_chunk_sums(Work w, const uint32_t* __restrict__ tok_len) {
  __shared__ uint32_t red[8];
  const uint32_t nhuge = w.ctr[CTR_NHUGE];
  uint32_t item = 0;
  for (uint32_t h = 0; h < nhuge; ++h) {
    const uint32_t p = (uint32_t)w.huge_list[h];
    const uint32_t cc = (uint32_t)w.piece_cnt[p];
    const uint32_t nit = (cc + HUGE_CHUNK - 1) / HUGE_CHUNK - 1;  // chunks before the last
    const uint32_t first = (blockIdx.x + gridDim.x - item % gridDim.x) % gridDim.x;
    item += nit;
    if (first >= nit) continue;
    const uint32_t src = (uint32_t)w.piece_start[p];
    for (uint32_t ch = first; ch < nit; ch += gridDim.x) {
      const int32_t* ids = w.tmp_ids + src + ch * HUGE_CHUNK;
      uint32_t sum = 0;
      for (uint32_t k0 = 0; k0 < HUGE_CHUNK; k0 += EMIT_THREADS * 8) {
        uint32_t id[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) id[j] = (uint32_t)ids[k0 + EMIT_THREADS * j + threadIdx.x];
#pragma unroll
        for (int j = 0; j < 8; ++j) sum += tok_len[id[j] & ID_MASK];
      }
      sum = block_sum(sum, red);
      if (threadIdx.x == 0) w.tmp_rank[src + ch] = sum;
    }
  }
}

// The tokens of a stitched piece that start in [a, b) (inside one tile; their
// ids sit at their first byte in tmp_ids, -1 at the other bytes), in byte
// order to out_ids[off ...) (and with OFFS their first bytes to out_starts),
// never past cap.  Returns their number, the same in every thread.
template <bool OFFS>
__device__ uint32_t emit_sparse(const Work& w, int32_t a, int32_t b, uint32_t off, uint32_t cap,
                                int32_t* __restrict__ out_ids, int32_t* __restrict__ out_starts, uint32_t* red) {
  const int32_t j0 = a + 4 * (int32_t)threadIdx.x;  // 4 bytes per thread: b - a <= TILE
  int32_t v[4];
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[k] = j0 + k < b ? w.tmp_ids[j0 + k] : -1;
    c += v[k] >= 0 ? 1u : 0u;
  }
  uint32_t tot;
  uint32_t o = off + block_excl_sum(c, red, &tot);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (v[k] < 0) continue;
    if (o < cap) {
      out_ids[o] = v[k];
      if (OFFS) out_starts[o] = j0 + k;
    }
    ++o;
  }
  return tot;
}

// Pass 6, one workgroup per tile: the output offset of the tile's pieces (the
// tokens of the tiles before it plus a block scan of their counts) and the
// copy of their tokens: up to 8 by the piece's own thread, up to HUGE_TOKENS
// by a wavefront.  Pieces with more tokens are cut into HUGE_CHUNK-token items
// dealt round-robin to the workgroups, each of which works out the piece's
// offset itself.  The last tile writes T (and tok_off[P]); *out_n, if given,
// gets T or the error code.  No copy goes past cap (= n).
//
// OFFS: also the byte offset of every token (device-side offset export, the
// summary page's Path C, §8 / Appendix E): a token's start is its piece's
// first byte plus the byte lengths of the tokens before it in the piece -- a
// running sum in the piece's thread, a wavefront scan, or for a huge piece a
// workgroup scan that starts from the byte lengths of the earlier chunks
// (k_chunk_sums).  out_starts[T] = cap.
template <bool OFFS, bool SB>
__global__ __launch_bounds__(EMIT_THREADS) void k_emit(Work w, int ntiles, int32_t* __restrict__ out_ids,
                                                       int64_t* __restrict__ out_n, uint32_t cap,
                                                       int32_t* __restrict__ out_starts,
                                                       const uint32_t* __restrict__ tok_len) {
  __shared__ uint32_t red[8];
  const int t = blockIdx.x;
  const int lane = (int)(threadIdx.x & 63u);
  const uint32_t cmask = (1u << TILE_ERR_SHIFT) - 1u;
  uint32_t hi;
  const uint32_t pbase = w.tile_pbase[t];
  const uint32_t np = w.tile_cnt[t] & cmask;
  const uint32_t hh = uniform(w.huge_hc[2 * t]), ht = uniform(w.huge_hc[2 * t + 1]);
  const uint32_t nhuge = uniform(w.ctr[CTR_NHUGE]);  // read now: the loads below overlap it
  uint32_t off0 = tile_prefix<SB>(w.tile_tok, w.sb_tok, nullptr, t, ~0u, red, &hi);
  const int32_t t0 = t * TILE;
  const int32_t tend = (int32_t)min(cap, (uint32_t)(t0 + TILE));
  // a stitched piece that began before the tile: its tokens that start here
  // come first (a nonzero stitched count marks it; a fallback zeroes it)
  if (hh) {
    const int32_t pe = np ? (int32_t)uniform((uint32_t)w.piece_start[pbase]) : tend;
    off0 += emit_sparse<OFFS>(w, t0, pe, off0, cap, out_ids, out_starts, red);
  }
  for (uint32_t k0 = 0; k0 < np; k0 += EMIT_THREADS) {
    const uint32_t k = k0 + threadIdx.x;
    const bool live = k < np;
    const uint32_t p = pbase + k;
    const uint32_t c = live ? (uint32_t)w.piece_cnt[p] : 0u;
    const uint32_t src = live ? (uint32_t)w.piece_start[p] : 0u;
    uint32_t tot;
    const uint32_t off = off0 + block_excl_sum(c, red, &tot);
    if (live) {
      w.tok_off[p] = (int32_t)off;
      if (c <= 8) {
        uint32_t at = src;
#pragma unroll
        for (uint32_t j = 0; j < 8; ++j)
          if (j < c) {
            const int32_t id = w.tmp_ids[src + j];
            out_ids[off + j] = id;
            if (OFFS) {
              out_starts[off + j] = (int32_t)at;
              at += tok_len[(uint32_t)id & ID_MASK];
            }
          }
      }
    }
    uint64_t big = __ballot(live && c > 8 && c <= (uint32_t)HUGE_TOKENS);
    while (big) {
      const int l = __ffsll((unsigned long long)big) - 1;
      big &= big - 1;
      const uint32_t cs = (uint32_t)__builtin_amdgcn_readlane((int)src, l);
      const uint32_t co = (uint32_t)__builtin_amdgcn_readlane((int)off, l);
      const uint32_t cc = (uint32_t)__builtin_amdgcn_readlane((int)c, l);
      const bool in = (uint32_t)lane < cc;
      const int32_t id = in ? w.tmp_ids[cs + lane] : 0;
      if (in) out_ids[co + lane] = id;
      if (OFFS) {
        const uint32_t len = in ? tok_len[(uint32_t)id & ID_MASK] : 0u;
        const uint32_t inc = wave_incl_fwd<SumOp>(len, lane);
        if (in) out_starts[co + lane] = (int32_t)(cs + inc - len);
      }
    }
    off0 += tot;
  }
  // the tile's last piece, if stitched: its tokens that start in the tile
  if (ht) {
    const int32_t ls = (int32_t)uniform((uint32_t)w.piece_start[pbase + np - 1]);
    off0 += emit_sparse<OFFS>(w, ls, tend, off0, cap, out_ids, out_starts, red);
  }
  if (t == ntiles - 1 && threadIdx.x == 0) {
    w.ctr[CTR_T] = off0;
    w.tok_off[pbase + np] = (int32_t)off0;
    if (OFFS && off0 <= cap) out_starts[off0] = (int32_t)cap;
    if (out_n) {
      const uint32_t e = w.ctr[CTR_ERR];
      *out_n = e ? err_code(e) : (int64_t)off0;
    }
  }
  // huge pieces: work item i = (piece, chunk) goes to workgroup i mod grid
  uint32_t item = 0;
  for (uint32_t h = 0; h < nhuge; ++h) {
    const uint32_t p = (uint32_t)w.huge_list[h];
    const uint32_t cc = (uint32_t)w.piece_cnt[p];
    const uint32_t nch = (cc + HUGE_CHUNK - 1) / HUGE_CHUNK;
    uint32_t first = (blockIdx.x + gridDim.x - item % gridDim.x) % gridDim.x;  // my first chunk of this piece
    item += nch;
    if (first >= nch) continue;
    // offset: tokens of the tiles before the piece's tile and of the pieces before it in its tile
    const uint32_t src = (uint32_t)w.piece_start[p];
    const int tp = (int)(src / TILE);
    const uint32_t pb = w.tile_pbase[tp];
    // (plus the tokens of a stitched piece that began before that tile and
    // start in it: they come before the tile's own pieces)
    const uint32_t dst = tile_prefix<SB>(w.tile_tok, w.sb_tok, nullptr, tp, ~0u, red, &hi) + w.huge_hc[2 * tp] +
                         block_reduce(reinterpret_cast<const uint32_t*>(w.piece_cnt) + pb, (int)(p - pb), ~0u, red, &hi);
    for (uint32_t ch = first; ch < nch; ch += gridDim.x) {
      const uint32_t k1 = min(min(cc, (ch + 1) * HUGE_CHUNK), cap - min(cap, dst));  // never past the output
      if (!OFFS) {
        // eight loads in flight per thread, then their stores
        for (uint32_t k0 = ch * HUGE_CHUNK; k0 < k1; k0 += EMIT_THREADS * 8) {
          int32_t v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t k = k0 + EMIT_THREADS * j + threadIdx.x;
            v[j] = k < k1 ? w.tmp_ids[src + k] : 0;
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t k = k0 + EMIT_THREADS * j + threadIdx.x;
            if (k < k1) out_ids[dst + k] = v[j];
          }
        }
        continue;
      }
      // byte offset of the chunk's first token: the earlier chunks' lengths
      uint32_t at = src + block_reduce(w.tmp_rank + src, (int)ch, ~0u, red, &hi);
      for (uint32_t b0 = ch * HUGE_CHUNK; b0 < k1; b0 += EMIT_THREADS * 8) {
        const uint32_t kb = b0 + 8u * threadIdx.x;  // 8 consecutive tokens per thread
        int32_t id[8];
        uint32_t len[8], sum = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) id[j] = kb + j < k1 ? w.tmp_ids[src + kb + j] : 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          len[j] = kb + j < k1 ? tok_len[(uint32_t)id[j] & ID_MASK] : 0u;
          sum += len[j];
        }
        uint32_t tot;
        uint32_t a = at + block_excl_sum(sum, red, &tot);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (kb + j < k1) {
            out_ids[dst + kb + j] = id[j];
            out_starts[dst + kb + j] = (int32_t)a;
            a += len[j];
          }
        at += tot;
      }
    }
  }
}

// ------------------------------------------------------- incremental repair
//
// A session holds a text A (n_old bytes), its token ids and the byte start of
// every token.  After Δ is appended, the window W = X[w0, n_new) of X = A + Δ
// is encoded on its own, and X's tokens are A's tokens before a splice byte p
// followed by W's tokens from p (TokTier summary page, §3.3 and the splicing
// theorem of Appendix A.2).  p qualifies when
//   (1) p is a pre-token start of W, with w0 + 16 <= p and p + 20 <= n_old;
//   (2) cl100k-style rules only: the chars at p - 1 and p differ in class
//       (letter / number / whitespace / other): a class-run start.
// Why this is exact: every start decision of both rule sets reads at most 4
// chars to the left (an apostrophe 3 chars back and the char before it) and
// 4 to the right (16 bytes hold at least 4 chars; 20 bytes at least 5).  The
// GPT-2-style rules read nothing else, so W's starts at or after p are X's,
// and A's starts before p are X's.  The cl100k-style rules also read the
// whole run they sit in (digit groups count from the run start, whitespace
// runs look at their newlines and their end): from a run start p on, every
// run lies inside W with its left neighbour inside W too, and every run
// before p ends at or before p, inside A and at least 5 chars before A's end.
// Pre-tokens are encoded independently (Appendix A.1), so equal pre-tokens
// give equal tokens.  This is the pages' char-class synchronisation boundary,
// with the two rule sets' exact reach in place of the generic matched-token
// certificate.


// class of the char starting at byte q (the text is valid UTF-8): 1 letter,
// 2 number, 3 other, 4 whitespace
__device__ uint32_t class4_at(const uint8_t* __restrict__ text, int64_t q) {
  const uint32_t b0 = text[q];
  if (b0 < 0x80u) {
    const uint32_t c = cls_of(g_ascii.v[b0]);
    return c == C_L ? 1u : c == C_N ? 2u : is_w(c) ? 4u : 3u;
  }
  uint32_t cp, len;
  if (b0 < 0xE0u) { cp = b0 & 0x1Fu; len = 2; }
  else if (b0 < 0xF0u) { cp = b0 & 0x0Fu; len = 3; }
  else { cp = b0 & 0x07u; len = 4; }
  for (uint32_t k = 1; k < len; ++k) cp = (cp << 6) | (text[q + k] & 0x3Fu);
  const uint32_t hi = cp >> 8;
  uint32_t u = 0;
  if (hi < (uint32_t)TT_UNI_L1_SIZE) {
    const uint32_t blk = g_uni_l1[hi];
    u = blk < UNI_SINGLE ? blk : (g_uni_l2[blk * 128u + ((cp & 255u) >> 1)] >> ((cp & 1u) * 4u)) & 15u;
  }
  const uint32_t c = uni_cls(u);
  return c == C_L ? 1u : c == C_N ? 2u : c == C_WS ? 4u : 3u;
}

// start of the char that ends right before byte q (q > 0)
__device__ __forceinline__ int64_t prev_char_start(const uint8_t* __restrict__ text, int64_t q) {
  int64_t s = q - 1;
  for (int k = 0; k < 3 && s > 0 && (text[s] & 0xC0u) == 0x80u; ++k) --s;
  return s;
}

// window starts of the next append for a text of n bytes: char starts at or
// before n - (tail << k), or 0
// The session's info words to the host's copy (pinned, mapped host memory
// that kernels only write): by the thread that wrote the last of them.
__device__ __forceinline__ void publish_info(const int64_t* info, int64_t* __restrict__ out) {
#pragma unroll
  for (int i = 0; i < SI_COUNT; ++i) out[i] = info[i];
}

__device__ void session_next_windows(const uint8_t* __restrict__ text, int64_t n, int64_t tail, int64_t* info) {
  for (int k = 0; k < SESSION_LEVELS; ++k) {
    int64_t s = n - (tail << k);
    if (s <= 0) {
      s = 0;
    } else {
      for (int j = 0; j < 3 && s > 0 && (text[s] & 0xC0u) == 0x80u; ++j) --s;
    }
    info[SI_NEXT_W0 + k] = s;
  }
}

// One workgroup: pick the splice byte (the first qualifying pre-token start
// of the window) and the token indices on both sides.
__global__ __launch_bounds__(256) void k_splice_find(const uint8_t* __restrict__ text, int64_t w0, int64_t n_old,
                                                     int pattern, int32_t* __restrict__ starts, int64_t t_old,
                                                     const int32_t* __restrict__ win_starts, Work w,
                                                     int64_t* __restrict__ info, int64_t n_new, int64_t tail,
                                                     int32_t* __restrict__ ids, const int32_t* __restrict__ win_ids,
                                                     bool do_copy, int64_t* __restrict__ info_out) {
  __shared__ uint32_t red[8];
  __shared__ int64_t sh_io, sh_iw;
  __shared__ int sh_status;
  const int64_t wc = info[SI_WIN_CNT];
  const uint32_t err = w.ctr[CTR_ERR];
  if (wc < 0 || err) {
    if (threadIdx.x == 0) {
      info[SI_STATUS] = SS_NONE;
      info[SI_ERROR] = wc < 0 ? wc : err_code(err);
      publish_info(info, info_out);
    }
    return;
  }
  const uint32_t P = w.ctr[CTR_P];
  int64_t p = -1;
  if (w0 == 0) {
    p = 0;  // the window is the whole text
  } else {
    const int64_t lo = 16, hi = n_old - 20 - w0;  // window-relative range of p
    // first piece starting at or after lo (each wavefront searches 64-way)
    const uint32_t a = (uint32_t)wave_lower_bound(w.piece_start, (int64_t)P, lo, (int)(threadIdx.x & 63u));
    for (uint32_t k0 = a; k0 < P; k0 += 256) {
      const uint32_t k = k0 + threadIdx.x;
      uint32_t best = 0xFFFFFFFFu;
      const int64_t q = k < P ? (int64_t)w.piece_start[k] : hi + 1;
      if (q <= hi) {
        bool ok = true;
        if (pattern == 1) {
          const int64_t g = w0 + q;
          ok = class4_at(text, g) != class4_at(text, prev_char_start(text, g));
        }
        if (ok) best = k;
      }
      best = block_min(best, red);
      if (best != 0xFFFFFFFFu) {
        p = w0 + (int64_t)w.piece_start[best];
        break;
      }
      // no piece of this batch qualified; stop once the batch ran past hi
      const int64_t last = (int64_t)w.piece_start[min(k0 + 255u, P - 1u)];
      if (last > hi) break;
    }
  }
  if (threadIdx.x < 64) {
    const int lane = (int)threadIdx.x;
    if (lane == 0) {
      info[SI_ERROR] = 0;
      info[SI_TWIN] = wc;
    }
    int status = SS_NONE;
    int64_t iw = 0, io = 0;
    if (p >= 0) {
      // token index of p on both sides, by 64-way searches of one wavefront.
      // In the old text every token index below t_old - (n_old - w0) - 1
      // starts before w0 < p (tokens are at least a byte long and end at
      // n_old), so that search starts there
      iw = wave_lower_bound(win_starts, wc, p - w0, lane);
      const int64_t ob = max<int64_t>(0, t_old - (n_old - w0) - 1);
      io = ob + wave_lower_bound(starts + ob, t_old - ob, p, lane);
      // p must start a token on both sides (it does whenever the reach
      // argument holds; a mismatch falls back to a full encode)
      const bool odd = iw > wc || win_starts[iw] != (int32_t)(p - w0) || io > t_old || starts[io] != (int32_t)p;
      status = odd ? SS_ODD : SS_SPLICED;
      if (lane == 0) {
        info[SI_P] = p;
        info[SI_IOLD] = io;
        info[SI_IWIN] = iw;
        info[SI_T] = io + (wc - iw);
      }
    }
    if (lane == 0) {
      info[SI_STATUS] = status;
      publish_info(info, info_out);  // final unless the splice below adds the next windows
      sh_status = status;
      sh_io = io;
      sh_iw = iw;
    }
  }
  // the splice itself, for a window small enough for one workgroup (else
  // k_splice_copy does it): W's tokens from p over the session's arrays
  // from A's token index of p (the check above read starts[io] first)
  if (!do_copy) return;
  __syncthreads();
  if (sh_status != SS_SPLICED) return;
  const int64_t io = sh_io, iw = sh_iw;
  for (int64_t i = iw + (int64_t)threadIdx.x; i < wc; i += 256) {
    ids[io + (i - iw)] = win_ids[i];
    starts[io + (i - iw)] = (int32_t)(win_starts[i] + w0);
  }
  if (threadIdx.x == 0) {
    starts[io + (wc - iw)] = (int32_t)n_new;
    session_next_windows(text, n_new, tail, info);
    publish_info(info, info_out);
  }
}

// The splice itself: W's tokens from p (ids, and starts shifted by w0) over
// the session's arrays from A's token index of p; the end sentinel; the next
// append's window starts.
__global__ __launch_bounds__(256) void k_splice_copy(const uint8_t* __restrict__ text, int64_t w0, int64_t n_new,
                                                     int64_t tail, int32_t* __restrict__ ids,
                                                     int32_t* __restrict__ starts,
                                                     const int32_t* __restrict__ win_ids,
                                                     const int32_t* __restrict__ win_starts,
                                                     int64_t* __restrict__ info, int64_t* __restrict__ info_out) {
  if (info[SI_STATUS] != SS_SPLICED) return;
  const int64_t io = info[SI_IOLD], iw = info[SI_IWIN], wc = info[SI_TWIN];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = iw + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < wc; i += stride) {
    ids[io + (i - iw)] = win_ids[i];
    starts[io + (i - iw)] = (int32_t)(win_starts[i] + w0);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    starts[io + (wc - iw)] = (int32_t)n_new;
    session_next_windows(text, n_new, tail, info);
    publish_info(info, info_out);
  }
}

// After a full encode of the session text into its own arrays (count in
// info[SI_WIN_CNT]): status, T and the next append's window starts.
__global__ void k_session_full(const uint8_t* __restrict__ text, int64_t n, int64_t tail, Work w,
                               int64_t* __restrict__ info, int64_t* __restrict__ info_out) {
  const int64_t c = info[SI_WIN_CNT];
  const uint32_t err = w.ctr[CTR_ERR];
  info[SI_STATUS] = SS_FULL;
  info[SI_ERROR] = c < 0 ? c : (err ? err_code(err) : 0);
  info[SI_T] = c < 0 ? 0 : c;
  info[SI_P] = 0;
  session_next_windows(text, n, tail, info);
  publish_info(info, info_out);
}

// ------------------------------------------------------------- small kernels

__global__ void k_zero(uint32_t* ctr, int cnt) {
  if ((int)threadIdx.x < cnt) ctr[threadIdx.x] = 0;
}

__global__ void k_check_offsets(const int64_t* __restrict__ offs, int nseq, int64_t n, uint32_t* ctr) {
  int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s > nseq) return;
  int64_t o = offs[s];
  bool bad = (s == 0 && o != 0) || (s == nseq && o != n) || o < 0 || o > n || (s < nseq && offs[s + 1] < o);
  if (bad) atomicOr(&ctr[CTR_ERR], ERR_OFFSETS);
}

__global__ void k_finish_count(const uint32_t* ctr, int which, int64_t* out) {
  uint32_t e = ctr[CTR_ERR];
  *out = e ? err_code(e) : (int64_t)ctr[which];
}

// One wavefront per sequence (and one for the total): the first piece that
// starts at or after the sequence's first byte, by a 64-way search.
constexpr int BATCH_OFF_WAVES = 4;
__global__ __launch_bounds__(64 * BATCH_OFF_WAVES) void k_batch_offsets(const int64_t* __restrict__ offs, int nseq,
                                                                      int64_t n, Work w,
                                                                      int64_t* __restrict__ out_off) {
  const int s = blockIdx.x * BATCH_OFF_WAVES + (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63u);
  if (s > nseq) return;
  if (s == nseq) {
    const uint32_t e = w.ctr[CTR_ERR];
    if (lane == 0) out_off[s] = e ? err_code(e) : (int64_t)w.ctr[CTR_T];
    return;
  }
  int64_t o = offs[s];
  o = o < 0 ? 0 : (o > n ? n : o);
  const int64_t lo = wave_lower_bound(w.piece_start, (int64_t)w.ctr[CTR_P], o, lane);
  if (lane == 0) out_off[s] = (int64_t)w.tok_off[lo];
}

__global__ void k_write_zero_i64(int64_t* out, int cnt) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < cnt) out[i] = 0;
}

__global__ void k_write_zero_i32(int32_t* out) { *out = 0; }

// ------------------------------------------------------- fixed scratch array
// The workspace of tt_encode_noalloc, for callers that cannot allocate: one
// array per device, held from module load until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is a stand-in,
// not a device address); it looks up the device address once per device and
// passes that.
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];
static void* scratch_dev[NOALLOC_MAX_DEVICES];  // looked-up address per device, null until then

hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return hipErrorInvalidDevice;
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return hipSuccess;
}

// ---------------------------------------------------------------- launchers

static inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
static inline int capped_grid(int64_t items, int per, int cap) {
  const int g = ceil_div(items, per);
  return g < 1 ? 1 : (g > cap ? cap : g);
}

hipError_t launch_pretokenize(const uint8_t* bytes, int64_t n, const int64_t* offs, int nseq, int pattern,
                              const Work& w, int32_t* starts, int64_t* out_np, const Tables* tb, hipStream_t st) {
  const int ntiles = ceil_div(n, TILE);
  if (pattern == 1) {
    hipLaunchKernelGGL(k_tile_summary<1>, dim3(ntiles), dim3(PT_THREADS), 0, st, bytes, n, offs, nseq, w);
    prof_mark("k_tile_summary", st);
    hipLaunchKernelGGL(k_pretok<1>, dim3(ntiles), dim3(PT_THREADS), 0, st, bytes, n, offs, nseq, ntiles, w);
    prof_mark("k_pretok<1>", st);
  } else if (pattern == 2) {
    hipLaunchKernelGGL(k_tile_summary<2>, dim3(ntiles), dim3(PT_THREADS), 0, st, bytes, n, offs, nseq, w);
    prof_mark("k_tile_summary", st);
    hipLaunchKernelGGL(k_pretok<2>, dim3(ntiles), dim3(PT_THREADS), 0, st, bytes, n, offs, nseq, ntiles, w);
    prof_mark("k_pretok<2>", st);
  } else if (pattern == 3) {
    hipLaunchKernelGGL(k_tile_summary<3>, dim3(ntiles), dim3(PT_THREADS), 0, st, bytes, n, offs, nseq, w);
    prof_mark("k_tile_summary", st);
    hipLaunchKernelGGL(k_pretok<3>, dim3(ntiles), dim3(PT_THREADS), 0, st, bytes, n, offs, nseq, ntiles, w);
    prof_mark("k_pretok<3>", st);
  } else {
    hipLaunchKernelGGL(k_pretok<0>, dim3(ntiles), dim3(PT_THREADS), 0, st, bytes, n, offs, nseq, ntiles, w);
    prof_mark("k_pretok<0>", st);
  }
  // large inputs: the two-level tile prefix (sums of the tile counts per
  // super-block first); smaller ones sum the tile counts directly
  const bool sb = ntiles > SB_MIN_TILES;
  if (sb) {
    hipLaunchKernelGGL(k_sb_sums, dim3(ceil_div(ntiles, SB_TILES)), dim3(256), 0, st, w.tile_cnt, ntiles,
                       (1u << TILE_ERR_SHIFT) - 1u, w.sb_cnt, w.sb_err);
    prof_mark("k_sb_sums", st);
  }
  const dim3 g(ntiles), b(PT_THREADS);
  if (tb && sb) hipLaunchKernelGGL((k_compact<true, true>), g, b, 0, st, bytes, w, *tb, ntiles, n, starts, out_np);
  if (tb && !sb) hipLaunchKernelGGL((k_compact<true, false>), g, b, 0, st, bytes, w, *tb, ntiles, n, starts, out_np);
  if (!tb && sb)
    hipLaunchKernelGGL((k_compact<false, true>), g, b, 0, st, bytes, w, Tables{}, ntiles, n, starts, out_np);
  if (!tb && !sb)
    hipLaunchKernelGGL((k_compact<false, false>), g, b, 0, st, bytes, w, Tables{}, ntiles, n, starts, out_np);
  prof_mark("k_compact", st);
  return hipGetLastError();
}

hipError_t launch_bpe_emit(const uint8_t* bytes, int64_t n, const Tables& tb, const Work& w, int32_t* out_ids,
                           int64_t* out_n, int32_t* out_starts, hipStream_t st) {
  // enough wavefronts to fill the chip; each one loops over work items
  if (n <= MERGE_SMALL)
    hipLaunchKernelGGL(k_bpe_merge<4>, dim3(max(QGROUPS, capped_grid(n, 256, 1024))), dim3(MERGE_THREADS), 0, st,
                       bytes, w, tb);
  else  // every queue group has workgroups either way
    hipLaunchKernelGGL(k_bpe_merge<8>, dim3(max(QGROUPS, capped_grid(n, 256, 2048))), dim3(MERGE_THREADS), 0, st,
                       bytes, w, tb);
  prof_mark("k_bpe_merge", st);
  const int ntiles = ceil_div(n, TILE);
  const bool sb = ntiles > SB_MIN_TILES;  // the two-level tile prefix, as in pre-tokenization
  if (sb) {
    hipLaunchKernelGGL(k_sb_sums, dim3(ceil_div(ntiles, SB_TILES)), dim3(256), 0, st, w.tile_tok, ntiles, ~0u,
                       w.sb_tok, nullptr);
    prof_mark("k_sb_sums", st);
  }
  const dim3 g(ntiles), b(EMIT_THREADS);
  if (out_starts) {
    // a piece of more than HUGE_CHUNK tokens has more than HUGE_CHUNK bytes
    if (n > (int64_t)HUGE_CHUNK) {
      hipLaunchKernelGGL(k_chunk_sums, dim3(capped_grid(n, HUGE_CHUNK, 1024)), dim3(EMIT_THREADS), 0, st, w,
                         tb.tok_len);
      prof_mark("k_chunk_sums", st);
    }
    if (sb)
      hipLaunchKernelGGL((k_emit<true, true>), g, b, 0, st, w, ntiles, out_ids, out_n, (uint32_t)n, out_starts,
                         tb.tok_len);
    else
      hipLaunchKernelGGL((k_emit<true, false>), g, b, 0, st, w, ntiles, out_ids, out_n, (uint32_t)n, out_starts,
                         tb.tok_len);
  } else {
    if (sb)
      hipLaunchKernelGGL((k_emit<false, true>), g, b, 0, st, w, ntiles, out_ids, out_n, (uint32_t)n, nullptr, nullptr);
    else
      hipLaunchKernelGGL((k_emit<false, false>), g, b, 0, st, w, ntiles, out_ids, out_n, (uint32_t)n, nullptr,
                         nullptr);
  }
  prof_mark("k_emit", st);
  return hipGetLastError();
}

hipError_t launch_finish_count(const Work& w, int which, int64_t* out, hipStream_t st) {
  hipLaunchKernelGGL(k_finish_count, dim3(1), dim3(1), 0, st, w.ctr, which, out); prof_mark("k_finish_count", st);
  return hipGetLastError();
}

hipError_t launch_batch_offsets(const int64_t* offs, int nseq, int64_t n, const Work& w, int64_t* out_off,
                                hipStream_t st) {
  hipLaunchKernelGGL(k_batch_offsets, dim3(ceil_div((int64_t)nseq + 1, BATCH_OFF_WAVES)), dim3(64 * BATCH_OFF_WAVES), 0, st,
                     offs, nseq, n, w,
                     out_off); prof_mark("k_batch_offsets", st);
  return hipGetLastError();
}

hipError_t launch_write_zeros(int64_t* out, int cnt, hipStream_t st) {
  if (cnt > 0) {
    hipLaunchKernelGGL(k_write_zero_i64, dim3(ceil_div(cnt, 256)), dim3(256), 0, st, out, cnt);
    prof_mark("k_write_zero_i64", st);
  }
  return hipGetLastError();
}

hipError_t launch_write_zero_i32(int32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(k_write_zero_i32, dim3(1), dim3(1), 0, st, out); prof_mark("k_write_zero_i32", st);
  return hipGetLastError();
}

hipError_t launch_zero_counters(const Work& w, hipStream_t st) {
  hipLaunchKernelGGL(k_zero, dim3(1), dim3(64), 0, st, w.ctr, (int)CTR_RESET_END); prof_mark("k_zero", st);
  return hipGetLastError();
}

hipError_t launch_splice(const uint8_t* text, int64_t w0, int64_t n_old, int64_t n_new, int pattern, int64_t tail,
                         int32_t* ids, int32_t* starts, int64_t t_old, const int32_t* win_ids,
                         const int32_t* win_starts, const Work& w, int64_t* info, int64_t* info_out, hipStream_t st) {
  // a window of up to 64 KiB (at most that many tokens) is spliced by the
  // search's own workgroup; a larger one by the grid-wide copy after it
  const bool fused = n_new - w0 <= ((int64_t)1 << 16);
  hipLaunchKernelGGL(k_splice_find, dim3(1), dim3(256), 0, st, text, w0, n_old, pattern, starts, t_old, win_starts, w,
                     info, n_new, tail, ids, win_ids, fused, info_out);
  prof_mark("k_splice_find", st);
  if (!fused) {
    hipLaunchKernelGGL(k_splice_copy, dim3(capped_grid(n_new - w0, 4096, 1024)), dim3(256), 0, st, text, w0, n_new,
                       tail, ids, starts, win_ids, win_starts, info, info_out);
    prof_mark("k_splice_copy", st);
  }
  return hipGetLastError();
}

hipError_t launch_session_full(const uint8_t* text, int64_t n, int64_t tail, const Work& w, int64_t* info,
                               int64_t* info_out, hipStream_t st) {
  hipLaunchKernelGGL(k_session_full, dim3(1), dim3(1), 0, st, text, n, tail, w, info, info_out);
  prof_mark("k_session_full", st);
  return hipGetLastError();
}

hipError_t launch_check_offsets(const int64_t* offs, int nseq, int64_t n, const Work& w, hipStream_t st) {
  hipLaunchKernelGGL(k_check_offsets, dim3(ceil_div((int64_t)nseq + 1, 256)), dim3(256), 0, st, offs, nseq, n, w.ctr); prof_mark("k_check_offsets", st);
  return hipGetLastError();
}

}  // namespace tt
