// tt_api.cpp -- C ABI of libtt: tokenizer loading, device tables, workspace,
// and the enqueue-only encode entry points declared in include/tt.h.
#include <algorithm>
#include <new>
#include <string>
#include <cstring>
#include <mutex>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "tt.h"
#include "tt_kernels.h"
#include "unicode_table.inc"

namespace {

using namespace tt;

const uint8_t h_uni_l1[TT_UNI_L1_SIZE] = {TT_UNI_L1_DATA};
const uint8_t h_uni_l2[TT_UNI_NBLOCKS * 128] = {TT_UNI_L2_DATA};

struct State {
  bool loaded = false;
  int pattern = 0;
  int64_t n_merges = 0;
  uint64_t generation = 0;  // bumped by every load and free: sessions keep the one they began with
  int device = -1;
  uint32_t* d_byte_pair = nullptr;
  uint32_t* d_pair = nullptr;
  CacheBucket* d_cache = nullptr;
  uint32_t* d_tok_len = nullptr;
  uint64_t* d_kids = nullptr;
  RunChunk* d_runs = nullptr;
  uint64_t* d_word = nullptr;
  uint32_t* d_tok_off = nullptr;
  uint8_t* d_tok_bytes = nullptr;
  bool ignore_merges = false;
  Tables tb{};
  void* d_ws = nullptr;
  int64_t ws_n = 0;     // bytes of input the workspace is sized for
  bool ws_fixed = false;  // set by tt_reserve: the workspace is never reallocated
  Work w{};
};

State g;
std::mutex g_mu;

constexpr int64_t SESSION_DEFAULT_TAIL = 2048;
constexpr int64_t SESSION_MIN_TAIL = 64;
constexpr int64_t SESSION_MAX_TAIL = (int64_t)1 << 24;

// Per-kernel timing (measurement aid): events recorded after each launch.
constexpr int PROF_CAP = 64;
struct Prof {
  bool on = false;
  hipEvent_t start = nullptr;
  hipEvent_t ev[PROF_CAP] = {};
  const char* name[PROF_CAP] = {};
  int n = 0;
} g_prof;

void prof_begin(hipStream_t st) {
  if (!g_prof.on) return;
  g_prof.n = 0;
  (void)hipEventRecord(g_prof.start, st);
}

template <class T>
void free_dev(T*& p) {
  if (p) (void)hipFree((void*)p);
  p = nullptr;
}

uint64_t next_pow2(uint64_t v) {
  uint64_t p = 1;
  while (p < v) p <<= 1;
  return p;
}

int log2_u64(uint64_t p) {
  int k = 0;
  while ((1ull << k) < p) ++k;
  return k;
}

// Classic lowest-rank-first BPE on the host, used once per token when the
// whole-piece table is built (which token byte strings encode to themselves).
std::vector<uint32_t> host_bpe(const std::vector<uint32_t>& in,
                               const std::unordered_map<uint64_t, uint32_t>& rank) {
  std::vector<uint32_t> ids = in;
  for (;;) {
    uint32_t best = RANK_NONE;
    size_t bi = 0;
    for (size_t i = 0; i + 1 < ids.size(); ++i) {
      auto it = rank.find(pair_key(ids[i], ids[i + 1]));
      if (it != rank.end() && it->second < best) {
        best = it->second;
        bi = i;
      }
    }
    if (best == RANK_NONE) return ids;
    ids[bi] = 256u + best;
    ids.erase(ids.begin() + (ptrdiff_t)bi + 1);
  }
}

void release_tables() {
  ++g.generation;
  free_dev(g.d_byte_pair);
  free_dev(g.d_pair);
  free_dev(g.d_cache);
  free_dev(g.d_tok_len);
  free_dev(g.d_kids);
  free_dev(g.d_runs);
  free_dev(g.d_word);
  free_dev(g.d_tok_off);
  free_dev(g.d_tok_bytes);
  g.loaded = false;
  g.ws_fixed = false;  // graphs captured under a reservation hold the old tables
}

void release_workspace() {
  if (g.d_ws) (void)hipFree(g.d_ws);
  g.d_ws = nullptr;
  g.ws_n = 0;
  g.w = Work{};
  g.ws_fixed = false;
}

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

// Carve the workspace for inputs of up to n bytes.
size_t layout(int64_t n, char* base, Work* w) {
  const size_t ntiles = (size_t)((n + TILE - 1) / TILE) + 1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  const size_t nn = (size_t)n + 1;
  Work t{};
  t.tile_fwd = (uint32_t*)take(ntiles * 4);
  t.tile_bwd = (uint32_t*)take(ntiles * 4);
  t.tile_cnt = (uint32_t*)take(ntiles * 4);
  t.codes = (uint8_t*)take(ntiles * TILE + 64);
  t.tile_tail = (uint32_t*)take(ntiles * 4);
  t.tile_chain = (uint32_t*)take(ntiles * 4);
  t.flags = (uint16_t*)take(ntiles * PT_THREADS * 2);
  t.piece_start = (int32_t*)take((nn + 1) * 4);
  t.piece_cnt = (int32_t*)take(nn * 4);
  t.tmp_ids = (int32_t*)take(nn * 4);
  t.tmp_rank = (uint32_t*)take(nn * 4);
  t.tok_off = (int32_t*)take((nn + 1) * 4);
  t.tile_tok = (uint32_t*)take(ntiles * 4);
  t.tile_pbase = (uint32_t*)take(ntiles * 4);
  t.big_fail = (int32_t*)take(ntiles * 4);
  t.huge_hc = (uint32_t*)take(ntiles * 2 * 4);
  t.fall_list = (int32_t*)take((nn / BIG_BYTES + 2) * 4);
  t.sb_cnt = (uint32_t*)take((ntiles / SB_TILES + 2) * 4);
  t.sb_err = (uint32_t*)take((ntiles / SB_TILES + 2) * 4);
  t.sb_tok = (uint32_t*)take((ntiles / SB_TILES + 2) * 4);
  // a class-c sub-queue takes the pieces of at least QCLASS_MINLEN[c] bytes
  // that start in every QGROUPS-th tile (long pieces: LANE_CAP + 1 bytes)
  const size_t tiles_per_group = (ntiles + QGROUPS - 1) / QGROUPS;
  t.lcap = (uint32_t)(tiles_per_group * (TILE / (LANE_CAP + 1) + 1));
  t.long_list = (int32_t*)take((size_t)t.lcap * QGROUPS * 4);
  t.huge_list = (int32_t*)take((nn / (HUGE_TOKENS + 1) + 2) * 4);
  for (int c = 0; c < 4; ++c) {
    t.qcap[c] = (uint32_t)(tiles_per_group * (TILE / QCLASS_MINLEN[c] + 1));
    t.queue[c] = (uint32_t*)take((size_t)t.qcap[c] * QGROUPS * 4);
  }
  t.qctr = (uint32_t*)take(QGROUPS * QCTR_STRIDE * 4);
  t.ctr = (uint32_t*)take(CTR_COUNT * 4);
  if (w) *w = t;
  return off;
}

// Input bytes a workspace for n bytes is sized for: n rounded up to whole
// tiles, at least 64 KiB.
int64_t workspace_size(int64_t n) {
  const int64_t want = std::max<int64_t>(n, (int64_t)1 << 16);
  return (want + TILE - 1) / TILE * TILE;
}

// Make the workspace large enough for n input bytes (synchronises if it
// grows).  A reserved workspace is never reallocated: graphs captured after
// tt_reserve hold its address.
int ensure_workspace(int64_t n) {
  if (n <= g.ws_n && g.d_ws) return TT_OK;
  if (g.ws_fixed) return TT_ETOOBIG;
  const int64_t want = workspace_size(n);
  if (hipDeviceSynchronize() != hipSuccess) return TT_EHIP;
  release_workspace();
  size_t bytes = layout(want, nullptr, nullptr);
  void* p = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return TT_ENOMEM;
  }
  g.d_ws = p;
  g.ws_n = want;
  layout(want, (char*)p, &g.w);
  return TT_OK;
}

template <class T>
int upload(T** dst, const std::vector<T>& src) {
  void* p = nullptr;
  if (hipMalloc(&p, src.size() * sizeof(T)) != hipSuccess) {
    (void)hipGetLastError();
    return TT_ENOMEM;
  }
  if (hipMemcpy(p, src.data(), src.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(p);
    return TT_EHIP;
  }
  *dst = (T*)p;
  return TT_OK;
}

int check_stream_state() {
  if (!g.loaded) return TT_ENOTLOADED;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != g.device) return TT_EINVAL;
  return TT_OK;
}

}  // namespace

// A session's device-resident state: the text so far, its token ids and the
// byte start of every token (plus the end), window scratch, and the repair
// step's info block (device and pinned host copies).
struct tt_session {
  int64_t cap = 0;
  int64_t tail = SESSION_DEFAULT_TAIL;
  int64_t n = 0, T = 0;
  uint64_t gen = 0;
  bool valid = false;
  uint8_t* text = nullptr;
  int32_t* ids = nullptr;
  int32_t* starts = nullptr;
  int32_t* win_ids = nullptr;
  int32_t* win_starts = nullptr;
  int64_t* info_dev = nullptr;
  int64_t* info_host = nullptr;  // pinned, mapped: the kernels that finish a step write it
  int64_t* info_map = nullptr;   // its device address
  int64_t next_w0[SESSION_LEVELS] = {};
};

namespace {

void session_release(tt_session* s) {
  free_dev(s->text);
  free_dev(s->ids);
  free_dev(s->starts);
  free_dev(s->win_ids);
  free_dev(s->win_starts);
  free_dev(s->info_dev);
  if (s->info_host) (void)hipHostFree(s->info_host);
  s->info_host = nullptr;
}

// Read the info block of the last step (one stream synchronisation).
int session_read_info(tt_session* s, hipStream_t st) {
  // the step's last kernel wrote info_host through its mapped address
  if (hipStreamSynchronize(st) != hipSuccess) return TT_EHIP;
  return TT_OK;
}

void session_take_windows(tt_session* s) {
  for (int k = 0; k < SESSION_LEVELS; ++k) s->next_w0[k] = s->info_host[SI_NEXT_W0 + k];
}

// Full encode of the session text [0, n) into the session arrays.
int session_full(tt_session* s, int64_t n, hipStream_t st) {
  if (launch_pretokenize(s->text, n, nullptr, 1, g.pattern, g.w, g.w.piece_start, nullptr, &g.tb, st) != hipSuccess ||
      launch_bpe_emit(s->text, n, g.tb, g.w, s->ids, s->info_dev + SI_WIN_CNT, s->starts, st) != hipSuccess ||
      launch_session_full(s->text, n, s->tail, g.w, s->info_dev, s->info_map, st) != hipSuccess)
    return TT_EHIP;
  return session_read_info(s, st);
}

}  // namespace

void tt::prof_mark(const char* name, hipStream_t st) {
  if (!g_prof.on || g_prof.n >= PROF_CAP) return;
  (void)hipEventRecord(g_prof.ev[g_prof.n], st);
  g_prof.name[g_prof.n++] = name;
}

extern "C" {

int tt_load_bpe(const int32_t* merges, const int32_t* ranks, int64_t n_merges, int32_t pattern_id) {
  return tt_load_bpe_ex(merges, ranks, n_merges, pattern_id, 0u);
}

int tt_load_bpe_ex(const int32_t* merges, const int32_t* ranks, int64_t n_merges, int32_t pattern_id,
                   uint32_t flags) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (pattern_id < TT_PATTERN_GPT2 || pattern_id > TT_PATTERN_DEEPSEEK) return TT_EINVAL;
  if (flags & ~(uint32_t)TT_LOAD_IGNORE_MERGES) return TT_EINVAL;
  const bool whole = (flags & TT_LOAD_IGNORE_MERGES) != 0;
  if (n_merges < 0 || n_merges > TT_MAX_MERGES) return TT_EINVAL;
  if (n_merges > 0 && !merges) return TT_EINVAL;
  const size_t M = (size_t)n_merges;

  // merge of rank r: (x, y) -> 256 + r
  std::vector<uint32_t> mx(M), my(M);
  std::vector<char> seen(M, 0);
  for (size_t k = 0; k < M; ++k) {
    int64_t r = ranks ? ranks[k] : (int64_t)k;
    if (r < 0 || r >= n_merges || seen[r]) return TT_ETABLE;
    seen[r] = 1;
    mx[r] = (uint32_t)merges[2 * k];
    my[r] = (uint32_t)merges[2 * k + 1];
  }
  std::unordered_map<uint64_t, uint32_t> rank;
  rank.reserve(M * 2 + 1);
  for (size_t r = 0; r < M; ++r) {
    if ((int64_t)(int32_t)mx[r] < 0 || (int64_t)(int32_t)my[r] < 0 || mx[r] >= 256 + r || my[r] >= 256 + r)
      return TT_ETABLE;
    if (!rank.emplace(pair_key(mx[r], my[r]), (uint32_t)r).second) return TT_ETABLE;
  }

  // byte-pair table
  std::vector<uint32_t> byte_pair(65536, RANK_NONE);
  for (size_t r = 0; r < M; ++r)
    if (mx[r] < 256 && my[r] < 256) byte_pair[(mx[r] << 8) | my[r]] = (uint32_t)r;

  // pair-rank table for pairs with an operand >= 256: two-choice buckets of
  // two slots in 256 partitions, load factor <= 0.8; a failed insertion
  // doubles the table
  size_t n_pairs = 0;
  for (size_t r = 0; r < M; ++r) n_pairs += (mx[r] >= 256 || my[r] >= 256);
  // ids below 2^v: slot keys x << (32 - v) | y >> p with 2^p partitions
  int v_bits = 16;
  while (v_bits < ID_BITS && ((uint64_t)1 << v_bits) < 256 + (uint64_t)M) ++v_bits;
  const int kshift = 32 - v_bits, pbits = 2 * v_bits - 32;
  const uint32_t pmask = (1u << pbits) - 1u;
  uint64_t pair_nb = std::max<uint64_t>(next_pow2((uint64_t)(n_pairs / 1.6) + 1), 1024);  // buckets
  std::vector<uint32_t> pair_tab;  // 4 words per bucket: key 0, rank 0, key 1, rank 1
  int pair_shift = 0;
  for (;;) {
    pair_shift = 32 - (log2_u64(pair_nb) - pbits);
    pair_tab.assign(pair_nb * 4, 0u);
    for (uint64_t i = 0; i < pair_nb * 2; ++i) pair_tab[2 * i + 1] = RANK_NONE;
    // the two buckets of a pair
    auto buckets = [&](uint32_t x, uint32_t y, uint64_t* b1, uint64_t* b2) {
      const uint32_t m = pair_mix(x, y), part = (x ^ y) & pmask;
      *b1 = ((uint64_t)(pair_choice(m, PAIR_MUL_1) >> pair_shift) << pbits) | part;
      *b2 = ((uint64_t)(pair_choice(m, PAIR_MUL_2) >> pair_shift) << pbits) | part;
    };
    bool ok = true;
    uint64_t lcg = 0x9E3779B97F4A7C15ull;  // eviction choices (fixed seed: the table is reproducible)
    for (size_t r = 0; r < M && ok; ++r) {
      if (mx[r] < 256 && my[r] < 256) continue;
      uint32_t cx = mx[r], cy = my[r], crank = (uint32_t)r;
      ok = false;
      uint64_t b1, b2;
      buckets(cx, cy, &b1, &b2);
      uint64_t b = b1;
      for (int kick = 0; kick < 2000; ++kick) {
        // a free slot in either bucket
        int free_slot = -1;
        uint64_t fb = 0;
        for (uint64_t cand : {b1, b2}) {
          for (int sl = 0; sl < 2 && free_slot < 0; ++sl)
            if (pair_tab[cand * 4 + 2 * sl] == 0u) {
              free_slot = sl;
              fb = cand;
            }
          if (free_slot >= 0) break;
        }
        if (free_slot >= 0) {
          pair_tab[fb * 4 + 2 * free_slot] = pair_slot_key(cx, cy, kshift, pbits);
          pair_tab[fb * 4 + 2 * free_slot + 1] = crank;
          ok = true;
          break;
        }
        // evict a slot of bucket b (alternating buckets along the walk) and
        // move its key to that key's other bucket
        lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
        const int sl = (int)(lcg >> 63);
        const uint32_t ek = pair_tab[b * 4 + 2 * sl], er = pair_tab[b * 4 + 2 * sl + 1];
        pair_tab[b * 4 + 2 * sl] = pair_slot_key(cx, cy, kshift, pbits);
        pair_tab[b * 4 + 2 * sl + 1] = crank;
        cx = ek >> kshift;
        cy = ((ek & ((1u << kshift) - 1u)) << pbits) | (((uint32_t)b ^ cx) & pmask);
        crank = er;
        uint64_t e1, e2;
        buckets(cx, cy, &e1, &e2);
        b1 = e1;
        b2 = e2;
        b = (b == e1) ? e2 : e1;  // the evicted key goes to its other bucket
      }
    }
    if (ok) break;
    pair_nb *= 2;
  }

  // whole-pre-token table: token t of 2..16 bytes whose own BPE is [t]
  std::vector<std::vector<uint8_t>> tok(256 + M);
  for (int b = 0; b < 256; ++b) tok[b] = {(uint8_t)b};
  for (size_t r = 0; r < M; ++r) {
    tok[256 + r] = tok[mx[r]];
    tok[256 + r].insert(tok[256 + r].end(), tok[my[r]].begin(), tok[my[r]].end());
  }
  // byte length of every token, for offset export: 2^ID_BITS entries so that
  // any id masked to ID_BITS indexes inside the table
  std::vector<uint32_t> tok_len((size_t)1 << ID_BITS, 0u);
  for (size_t t = 0; t < tok.size(); ++t) tok_len[t] = (uint32_t)std::min<size_t>(tok[t].size(), 0xFFFFFFFFu);
  // operands of every merge, for the token-pair compatibility walk of the
  // long-piece stitching (one entry even for an empty table)
  std::vector<uint64_t> kids(std::max<size_t>(M, 1), 0ull);
  for (size_t r = 0; r < M; ++r) kids[r] = (uint64_t)mx[r] | ((uint64_t)my[r] << 32);
  // the encoding of RUN_BYTES copies of each byte value (host classic loop)
  std::vector<RunChunk> runs(256);
  for (uint32_t b = 0; b < 256; ++b) {
    std::vector<uint32_t> out = host_bpe(std::vector<uint32_t>(RUN_BYTES, b), rank);
    RunChunk& rc = runs[b];
    std::memset(&rc, 0, sizeof(rc));
    rc.cnt = (uint32_t)out.size();
    uint32_t at = 0;
    for (size_t k = 0; k < out.size(); ++k) {
      rc.id[k] = out[k];
      rc.pos[k] = (uint8_t)at;
      at += (uint32_t)tok[out[k]].size();
    }
  }
  // whole-pre-token table: tokens of 2..16 bytes whose own BPE is
  // themselves; with the whole-word rule, every token (the smallest id of
  // each byte string), and the longer ones go to the whole-word table
  std::vector<uint32_t> single, words;
  size_t word_maxlen = 0;
  if (whole) {
    std::unordered_map<std::string, uint32_t> first;
    first.reserve(tok.size() * 2);
    for (size_t t = 256; t < tok.size(); ++t) {
      const std::string key(tok[t].begin(), tok[t].end());
      if (!first.emplace(key, (uint32_t)t).second) continue;  // a later id with the same bytes
      if (tok[t].size() > (size_t)WORD_MAXLEN) return TT_ETABLE;
      if (tok[t].size() <= (size_t)CACHE_MAXLEN) {
        single.push_back((uint32_t)t);
      } else {
        words.push_back((uint32_t)t);
        word_maxlen = std::max(word_maxlen, tok[t].size());
      }
    }
  } else {
    for (size_t r = 0; r < M; ++r) {
      const auto& bs = tok[256 + r];
      if (bs.size() < 2 || bs.size() > (size_t)CACHE_MAXLEN) continue;
      std::vector<uint32_t> ids(bs.begin(), bs.end());
      std::vector<uint32_t> out = host_bpe(ids, rank);
      if (out.size() == 1 && out[0] == 256u + r) single.push_back((uint32_t)(256 + r));
    }
  }
  // buckets of CACHE_SLOTS entries, load factor <= 1/2
  const uint64_t cache_nb = std::max<uint64_t>(next_pow2((single.size() * 2 + CACHE_SLOTS - 1) / CACHE_SLOTS), 256);
  const int cache_shift = 64 - log2_u64(cache_nb);
  std::vector<CacheBucket> cache(cache_nb);
  std::memset(cache.data(), 0, cache.size() * sizeof(CacheBucket));
  int cache_probe = 1;
  for (uint32_t t : single) {
    const auto& bs = tok[t];
    uint64_t w0 = 0, w1 = 0;
    for (size_t k = 0; k < bs.size(); ++k) {
      if (k < 8) w0 |= (uint64_t)bs[k] << (8 * k);
      else w1 |= (uint64_t)bs[k] << (8 * (k - 8));
    }
    uint32_t h = cache_hash(w0, w1, (uint32_t)bs.size(), cache_shift);
    for (int visited = 1;; ++visited, h = (uint32_t)((h + 1) & (cache_nb - 1))) {
      CacheBucket& b = cache[h];
      int slot = -1;
      for (int s = 0; s < CACHE_SLOTS; ++s)
        if ((b.meta[s] & ~CACHE_MORE) == 0) { slot = s; break; }
      if (slot >= 0) {
        b.w0[slot] = w0;
        b.w1[slot] = w1;
        b.meta[slot] |= (t << 5) | (uint32_t)bs.size();
        cache_probe = std::max(cache_probe, visited);
        break;
      }
      b.meta[0] |= CACHE_MORE;  // the probe run goes on past this full bucket
    }
  }

  // whole-word table: open addressing, load factor <= 1/2; a token's bytes
  // at tok_off[t] in tok_bytes
  std::vector<uint64_t> word_tab;
  std::vector<uint32_t> tok_off;
  std::vector<uint8_t> tok_blob;
  int word_probe = 0;
  if (whole) {
    const uint64_t ns = std::max<uint64_t>(next_pow2(words.size() * 2 + 1), 64);
    word_tab.assign(ns, 0ull);
    for (uint32_t t : words) {
      const auto& bs = tok[t];
      uint64_t h = word_hash_init((uint32_t)bs.size());
      for (size_t k = 0; k < bs.size(); k += 8) {
        uint64_t wd = 0;
        for (size_t j = 0; j < 8 && k + j < bs.size(); ++j) wd |= (uint64_t)bs[k + j] << (8 * j);
        h = word_hash_step(h, wd);
      }
      const uint64_t e = (h >> 32 << 32) | ((uint64_t)bs.size() << ID_BITS) | t;
      uint64_t pos = h & (ns - 1);
      int run = 1;
      while (word_tab[pos] != 0) {
        pos = (pos + 1) & (ns - 1);
        ++run;
      }
      word_tab[pos] = e;
      word_probe = std::max(word_probe, run);
    }
    tok_off.resize(tok.size() + 1);
    for (size_t t = 0; t < tok.size(); ++t) {
      tok_off[t] = (uint32_t)tok_blob.size();
      tok_blob.insert(tok_blob.end(), tok[t].begin(), tok[t].end());
    }
    tok_off[tok.size()] = (uint32_t)tok_blob.size();
  }

  if (hipDeviceSynchronize() != hipSuccess) return TT_EHIP;
  release_tables();
  int rc;
  if ((rc = upload(&g.d_byte_pair, byte_pair)) != TT_OK || (rc = upload(&g.d_pair, pair_tab)) != TT_OK ||
      (rc = upload(&g.d_cache, cache)) != TT_OK || (rc = upload(&g.d_tok_len, tok_len)) != TT_OK ||
      (rc = upload(&g.d_kids, kids)) != TT_OK || (rc = upload(&g.d_runs, runs)) != TT_OK ||
      (whole && ((rc = upload(&g.d_word, word_tab)) != TT_OK || (rc = upload(&g.d_tok_off, tok_off)) != TT_OK ||
                 (rc = upload(&g.d_tok_bytes, tok_blob)) != TT_OK))) {
    release_tables();
    return rc;
  }
  // the device address of the no-alloc scratch array, looked up once here
  void* scratch_ptr = nullptr;
  if (hipGetDevice(&g.device) != hipSuccess || scratch_address(&scratch_ptr) != hipSuccess) {
    (void)hipGetLastError();
    release_tables();
    return TT_EHIP;
  }
  g.pattern = pattern_id;
  g.n_merges = n_merges;
  g.tb.byte_pair = g.d_byte_pair;
  g.tb.pair_tab = reinterpret_cast<const uint4*>(g.d_pair);
  g.tb.cache = g.d_cache;
  g.tb.tok_len = g.d_tok_len;
  g.tb.kids = g.d_kids;
  g.tb.runs = g.d_runs;
  g.tb.pair_shift = pair_shift;
  g.tb.pair_kshift = kshift;
  g.tb.pair_pbits = pbits;
  g.tb.cache_mask = (uint32_t)(cache_nb - 1);
  g.tb.cache_shift = cache_shift;
  g.tb.cache_probe = cache_probe;
  g.tb.pattern = pattern_id;
  g.tb.word_tab = g.d_word;
  g.tb.tok_off = g.d_tok_off;
  g.tb.tok_bytes = g.d_tok_bytes;
  g.tb.word_mask = whole ? (uint32_t)(word_tab.size() - 1) : 0u;
  g.tb.word_probe = word_probe;
  g.tb.word_maxlen = whole ? (int)std::max<size_t>(word_maxlen, (size_t)CACHE_MAXLEN) : 0;
  g.ignore_merges = whole;
  g.loaded = true;
  return TT_OK;
}

int tt_reserve(int64_t max_bytes, int32_t max_seqs) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (max_bytes < 0 || max_seqs < 0) return TT_EINVAL;
  if (max_bytes >= TT_MAX_BYTES) return TT_ETOOBIG;
  int rc = check_stream_state();
  if (rc != TT_OK) return rc;
  // the workspace takes exactly the reserved size (a larger one left by
  // earlier calls is given back), so that the limit is the one asked for
  g.ws_fixed = false;
  if (g.d_ws && g.ws_n != workspace_size(max_bytes)) {
    if (hipDeviceSynchronize() != hipSuccess) return TT_EHIP;
    release_workspace();
  }
  if ((rc = ensure_workspace(max_bytes)) != TT_OK) return rc;
  g.ws_fixed = true;
  return TT_OK;
}

int tt_encode(const uint8_t* dev_bytes, int64_t n, int32_t* out_ids, int64_t* out_n, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (n < 0 || !out_n || (n > 0 && (!dev_bytes || !out_ids))) return TT_EINVAL;
  if (n >= TT_MAX_BYTES) return TT_ETOOBIG;
  int rc = check_stream_state();
  if (rc != TT_OK) return rc;
  if (n == 0) return launch_write_zeros(out_n, 1, stream) == hipSuccess ? TT_OK : TT_EHIP;
  if ((rc = ensure_workspace(n)) != TT_OK) return rc;
  prof_begin(stream);
  if (launch_pretokenize(dev_bytes, n, nullptr, 1, g.pattern, g.w, g.w.piece_start, nullptr, &g.tb, stream) != hipSuccess ||
      launch_bpe_emit(dev_bytes, n, g.tb, g.w, out_ids, out_n, nullptr, stream) != hipSuccess)
    return TT_EHIP;
  return TT_OK;
}

int tt_encode_noalloc(const uint8_t* dev_bytes, int64_t n, int32_t* out_ids, int64_t* out_n, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (n < 0 || !out_n || (n > 0 && (!dev_bytes || !out_ids))) return TT_EINVAL;
  if (n > TT_NOALLOC_MAX_BYTES) return TT_ETOOBIG;
  int rc = check_stream_state();
  if (rc != TT_OK) return rc;
  void* base = nullptr;  // the scratch array's device address (never its host-side name)
  if (scratch_address(&base) != hipSuccess) return TT_EHIP;
  if (n == 0) return launch_write_zeros(out_n, 1, stream) == hipSuccess ? TT_OK : TT_EHIP;
  const int64_t want = (n + TILE - 1) / TILE * TILE;
  if (layout(want, nullptr, nullptr) > NOALLOC_SCRATCH_BYTES) return TT_ETOOBIG;
  Work w{};
  layout(want, static_cast<char*>(base), &w);
  prof_begin(stream);
  if (launch_pretokenize(dev_bytes, n, nullptr, 1, g.pattern, w, w.piece_start, nullptr, &g.tb, stream) != hipSuccess ||
      launch_bpe_emit(dev_bytes, n, g.tb, w, out_ids, out_n, nullptr, stream) != hipSuccess)
    return TT_EHIP;
  return TT_OK;
}

int tt_encode_batch(const uint8_t* dev_bytes, int64_t n, const int64_t* dev_offsets, int32_t n_seqs,
                    int32_t* out_ids, int64_t* out_offsets, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (n < 0 || n_seqs < 1 || !dev_offsets || !out_offsets || (n > 0 && (!dev_bytes || !out_ids)))
    return TT_EINVAL;
  if (n >= TT_MAX_BYTES || n_seqs >= (int64_t)1 << 30) return TT_ETOOBIG;
  int rc = check_stream_state();
  if (rc != TT_OK) return rc;
  if ((rc = ensure_workspace(n)) != TT_OK) return rc;
  if (n == 0) {
    if (launch_zero_counters(g.w, stream) != hipSuccess ||
        launch_check_offsets(dev_offsets, n_seqs, n, g.w, stream) != hipSuccess ||
        launch_write_zeros(out_offsets, n_seqs, stream) != hipSuccess ||
        launch_finish_count(g.w, CTR_T, out_offsets + n_seqs, stream) != hipSuccess)
      return TT_EHIP;
    return TT_OK;
  }
  prof_begin(stream);
  if (launch_pretokenize(dev_bytes, n, dev_offsets, n_seqs, g.pattern, g.w, g.w.piece_start, nullptr, &g.tb,
                         stream) !=
          hipSuccess ||
      launch_bpe_emit(dev_bytes, n, g.tb, g.w, out_ids, nullptr, nullptr, stream) != hipSuccess ||
      launch_batch_offsets(dev_offsets, n_seqs, n, g.w, out_offsets, stream) != hipSuccess)
    return TT_EHIP;
  return TT_OK;
}

int tt_pretokenize(const uint8_t* dev_bytes, int64_t n, const int64_t* dev_offsets, int32_t n_seqs,
                   int32_t* out_starts, int64_t* out_np, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (n < 0 || !out_starts || !out_np || (n > 0 && !dev_bytes) || (dev_offsets && n_seqs < 1)) return TT_EINVAL;
  if (n >= TT_MAX_BYTES || n_seqs >= (int64_t)1 << 30) return TT_ETOOBIG;
  int rc = check_stream_state();
  if (rc != TT_OK) return rc;
  if ((rc = ensure_workspace(n)) != TT_OK) return rc;
  const int nseq = dev_offsets ? n_seqs : 1;
  if (n == 0) {
    if (launch_zero_counters(g.w, stream) != hipSuccess ||
        (dev_offsets && launch_check_offsets(dev_offsets, nseq, n, g.w, stream) != hipSuccess) ||
        launch_write_zero_i32(out_starts, stream) != hipSuccess ||
        launch_finish_count(g.w, CTR_P, out_np, stream) != hipSuccess)
      return TT_EHIP;
    return TT_OK;
  }
  prof_begin(stream);
  if (launch_pretokenize(dev_bytes, n, dev_offsets, nseq, g.pattern, g.w, out_starts, out_np, nullptr, stream) != hipSuccess)
    return TT_EHIP;
  return TT_OK;
}

int tt_encode_offsets(const uint8_t* dev_bytes, int64_t n, const int64_t* dev_offsets, int32_t n_seqs,
                      int32_t* out_ids, int32_t* out_starts, int64_t* out_counts, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (n < 0 || !out_starts || !out_counts || (n > 0 && (!dev_bytes || !out_ids)) || (dev_offsets && n_seqs < 1))
    return TT_EINVAL;
  if (n >= TT_MAX_BYTES || n_seqs >= (int64_t)1 << 30) return TT_ETOOBIG;
  int rc = check_stream_state();
  if (rc != TT_OK) return rc;
  if ((rc = ensure_workspace(n)) != TT_OK) return rc;
  const int nseq = dev_offsets ? n_seqs : 1;
  if (n == 0) {
    if (launch_zero_counters(g.w, stream) != hipSuccess ||
        (dev_offsets && launch_check_offsets(dev_offsets, nseq, n, g.w, stream) != hipSuccess) ||
        launch_write_zero_i32(out_starts, stream) != hipSuccess ||
        (dev_offsets && launch_write_zeros(out_counts, nseq, stream) != hipSuccess) ||
        launch_finish_count(g.w, CTR_T, dev_offsets ? out_counts + nseq : out_counts, stream) != hipSuccess)
      return TT_EHIP;
    return TT_OK;
  }
  prof_begin(stream);
  if (launch_pretokenize(dev_bytes, n, dev_offsets, nseq, g.pattern, g.w, g.w.piece_start, nullptr, &g.tb, stream) !=
          hipSuccess ||
      launch_bpe_emit(dev_bytes, n, g.tb, g.w, out_ids, dev_offsets ? nullptr : out_counts, out_starts, stream) !=
          hipSuccess ||
      (dev_offsets && launch_batch_offsets(dev_offsets, nseq, n, g.w, out_counts, stream) != hipSuccess))
    return TT_EHIP;
  return TT_OK;
}

int tt_session_create(int64_t capacity, int64_t tail_bytes, tt_session** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!out || capacity < 0 || tail_bytes < 0 || (tail_bytes && tail_bytes < SESSION_MIN_TAIL)) return TT_EINVAL;
  if (capacity >= TT_MAX_BYTES || tail_bytes > SESSION_MAX_TAIL) return TT_ETOOBIG;
  *out = nullptr;
  int rc = check_stream_state();
  if (rc != TT_OK) return rc;
  if ((rc = ensure_workspace(capacity)) != TT_OK) return rc;
  tt_session* s = new (std::nothrow) tt_session();
  if (!s) return TT_ENOMEM;
  s->cap = capacity;
  s->tail = tail_bytes ? tail_bytes : SESSION_DEFAULT_TAIL;
  const size_t c1 = (size_t)capacity + 1;
  bool ok = hipMalloc((void**)&s->text, c1 + 16) == hipSuccess && hipMalloc((void**)&s->ids, c1 * 4) == hipSuccess &&
            hipMalloc((void**)&s->starts, c1 * 4) == hipSuccess && hipMalloc((void**)&s->win_ids, c1 * 4) == hipSuccess &&
            hipMalloc((void**)&s->win_starts, c1 * 4) == hipSuccess &&
            hipMalloc((void**)&s->info_dev, SI_COUNT * sizeof(int64_t)) == hipSuccess &&
            hipHostMalloc((void**)&s->info_host, SI_COUNT * sizeof(int64_t),
                          hipHostMallocMapped | hipHostMallocCoherent) == hipSuccess &&
            hipHostGetDevicePointer((void**)&s->info_map, s->info_host, 0) == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    session_release(s);
    delete s;
    return TT_ENOMEM;
  }
  *out = s;
  return TT_OK;
}

int tt_session_destroy(tt_session* s) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!s) return TT_EINVAL;
  (void)hipDeviceSynchronize();
  session_release(s);
  delete s;
  return TT_OK;
}

int tt_session_reset(tt_session* s, const uint8_t* dev_bytes, int64_t n, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!s || n < 0 || (n > 0 && !dev_bytes)) return TT_EINVAL;
  if (n > s->cap) return TT_ETOOBIG;
  if (g.loaded && g.pattern >= TT_PATTERN_O200K) return TT_EINVAL;  // no splice rule for these rules
  int rc = check_stream_state();
  if (rc != TT_OK) return rc;
  s->valid = false;
  s->n = s->T = 0;
  if ((rc = ensure_workspace(std::max<int64_t>(n, 1))) != TT_OK) return rc;
  prof_begin(stream);
  if (n == 0) {
    if (launch_write_zero_i32(s->starts, stream) != hipSuccess || hipStreamSynchronize(stream) != hipSuccess)
      return TT_EHIP;
    for (int k = 0; k < SESSION_LEVELS; ++k) s->next_w0[k] = 0;
  } else {
    if (hipMemcpyAsync(s->text, dev_bytes, (size_t)n, hipMemcpyDeviceToDevice, stream) != hipSuccess) return TT_EHIP;
    if ((rc = session_full(s, n, stream)) != TT_OK) return rc;
    if (s->info_host[SI_ERROR] != 0) return (int)s->info_host[SI_ERROR];
    s->n = n;
    s->T = s->info_host[SI_T];
    session_take_windows(s);
  }
  s->gen = g.generation;
  s->valid = true;
  return TT_OK;
}

int tt_session_append(tt_session* s, const uint8_t* dev_delta, int64_t nd, int64_t* out_info, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!s || nd < 0 || (nd > 0 && !dev_delta)) return TT_EINVAL;
  int rc = check_stream_state();
  if (rc != TT_OK) return rc;
  if (!s->valid) return TT_EINVAL;
  if (s->gen != g.generation) return TT_ESTALE;
  if (g.pattern >= TT_PATTERN_O200K) return TT_EINVAL;
  if (nd > s->cap - s->n) return TT_ETOOBIG;
  int64_t info[4] = {0, 0, -1, s->T};
  if (nd == 0) {
    if (out_info) std::memcpy(out_info, info, sizeof(info));
    return TT_OK;
  }
  const int64_t n_old = s->n, n_new = s->n + nd;
  if ((rc = ensure_workspace(n_new)) != TT_OK) return rc;
  prof_begin(stream);
  if (hipMemcpyAsync(s->text + n_old, dev_delta, (size_t)nd, hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return TT_EHIP;
  int64_t prev = -1;
  bool odd = false;
  for (int k = 0; k < SESSION_LEVELS && !odd; ++k) {
    const int64_t w0 = s->next_w0[k];
    if (w0 == prev) continue;
    prev = w0;
    const int64_t nw = n_new - w0;
    if (launch_pretokenize(s->text + w0, nw, nullptr, 1, g.pattern, g.w, g.w.piece_start, nullptr, &g.tb, stream) !=
            hipSuccess ||
        launch_bpe_emit(s->text + w0, nw, g.tb, g.w, s->win_ids, s->info_dev + SI_WIN_CNT, s->win_starts, stream) !=
            hipSuccess ||
        launch_splice(s->text, w0, n_old, n_new, g.pattern, s->tail, s->ids, s->starts, s->T, s->win_ids,
                      s->win_starts, g.w, s->info_dev, s->info_map, stream) != hipSuccess)
      return TT_EHIP;
    if ((rc = session_read_info(s, stream)) != TT_OK) return rc;
    const int64_t* h = s->info_host;
    if (h[SI_ERROR] != 0) return (int)h[SI_ERROR];  // Δ rejected; the session is unchanged
    if (h[SI_STATUS] == SS_SPLICED) {
      s->n = n_new;
      s->T = h[SI_T];
      session_take_windows(s);
      info[0] = k;
      info[1] = nw;
      info[2] = h[SI_P];
      info[3] = s->T;
      if (out_info) std::memcpy(out_info, info, sizeof(info));
      return TT_OK;
    }
    odd = h[SI_STATUS] == SS_ODD;
  }
  // no window qualified: encode the whole text
  if ((rc = session_full(s, n_new, stream)) != TT_OK) return rc;
  if (s->info_host[SI_ERROR] != 0) {
    s->valid = false;
    return (int)s->info_host[SI_ERROR];
  }
  s->n = n_new;
  s->T = s->info_host[SI_T];
  session_take_windows(s);
  info[0] = -1;
  info[1] = n_new;
  info[2] = 0;
  info[3] = s->T;
  if (out_info) std::memcpy(out_info, info, sizeof(info));
  return TT_OK;
}

int tt_session_view(const tt_session* s, const uint8_t** text, int64_t* n, const int32_t** ids,
                    const int32_t** starts, int64_t* T) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!s) return TT_EINVAL;
  if (text) *text = s->text;
  if (n) *n = s->n;
  if (ids) *ids = s->ids;
  if (starts) *starts = s->starts;
  if (T) *T = s->T;
  return TT_OK;
}

int tt_session_read(const tt_session* s, uint8_t* text_out, int32_t* ids_out, int32_t* starts_out,
                    hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!s || !s->valid) return TT_EINVAL;
  if ((text_out && s->n &&
       hipMemcpyAsync(text_out, s->text, (size_t)s->n, hipMemcpyDeviceToDevice, stream) != hipSuccess) ||
      (ids_out && s->T &&
       hipMemcpyAsync(ids_out, s->ids, (size_t)s->T * 4, hipMemcpyDeviceToDevice, stream) != hipSuccess) ||
      (starts_out &&
       hipMemcpyAsync(starts_out, s->starts, (size_t)(s->T + 1) * 4, hipMemcpyDeviceToDevice, stream) != hipSuccess))
    return TT_EHIP;
  return TT_OK;
}

int tt_char_class(uint32_t cp) {
  if (cp > 0x10FFFF || (cp >= 0xD800 && cp <= 0xDFFF)) return -1;
  uint32_t hi = cp >> 8;
  if (hi >= (uint32_t)TT_UNI_L1_SIZE) return 0;
  uint32_t byte = h_uni_l2[h_uni_l1[hi] * 128u + ((cp & 255u) >> 1)];
  return (int)((byte >> ((cp & 1u) * 4u)) & 15u);
}

int tt_profile(int enable) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (enable && !g_prof.on) {
    if (hipEventCreate(&g_prof.start) != hipSuccess) return TT_EHIP;
    for (int i = 0; i < PROF_CAP; ++i)
      if (hipEventCreate(&g_prof.ev[i]) != hipSuccess) return TT_EHIP;
    g_prof.on = true;
    g_prof.n = 0;
  } else if (!enable && g_prof.on) {
    (void)hipDeviceSynchronize();
    (void)hipEventDestroy(g_prof.start);
    for (int i = 0; i < PROF_CAP; ++i) (void)hipEventDestroy(g_prof.ev[i]);
    g_prof = Prof{};
  }
  return TT_OK;
}

int tt_profile_read(const char** names, float* ms, int cap) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_prof.on || (cap > 0 && (!names || !ms))) return TT_EINVAL;
  if (g_prof.n == 0) return 0;
  if (hipEventSynchronize(g_prof.ev[g_prof.n - 1]) != hipSuccess) return TT_EHIP;
  int k = std::min(cap, g_prof.n);
  for (int i = 0; i < k; ++i) {
    names[i] = g_prof.name[i];
    if (hipEventElapsedTime(&ms[i], i ? g_prof.ev[i - 1] : g_prof.start, g_prof.ev[i]) != hipSuccess) return TT_EHIP;
  }
  return k;
}

void tt_free(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  (void)hipDeviceSynchronize();
  release_workspace();
  release_tables();
}

const char* tt_strerror(int code) {
  switch (code) {
    case TT_OK: return "ok";
    case TT_EINVAL: return "invalid argument";
    case TT_ETABLE: return "invalid merge table";
    case TT_ENOMEM: return "out of memory";
    case TT_EHIP: return "HIP runtime error";
    case TT_EUTF8: return "input is not valid UTF-8";
    case TT_ENOTLOADED: return "no tokenizer loaded";
    case TT_EOFFSETS: return "invalid batch offsets";
    case TT_ETOOBIG: return "size beyond library limits";
    case TT_ESTALE: return "tokenizer replaced since the session began";
    case TT_EUNSUPPORTED: return "input case not decided by the o200k-style GPU rules";
    default: return "unknown error";
  }
}

}  // extern "C"
