// Fixed-budget sparse attention for gfx950 (kvpop_budget_mask_fwd).
//
// KVpop paper, Section 3: every KV head keeps s sink tokens (the first
// positions), a protected window of the w most recent tokens, and the top-k
// of the eligible tokens E_d = [s, d-w] (Section 3.1, Eq. 4) ranked by static
// priorities.  Section 3.2 ("Running top-k sparse attention"): sort once by
// priority, and the retained long-range keys of query d are exactly the
// eligible tokens whose rank is at most c_d, the rank of the k-th best
// eligible token.  The pages compute c_d with a sequential Fenwick-tree sweep;
// here every c_d is an independent query on a wavelet matrix over the ranks
// (k-th smallest value in the prefix [s, d-w]), which gives the same integers
// for all d in parallel.
//
// Pipeline (all on the caller's stream):
//   1. sort:    2048-key chunks sorted in LDS (bitonic), on 64-bit sort keys
//               (descending score, ascending index) formed from the scores;
//   2. rank:    rank(t) = sum over chunks of the number of smaller keys, and
//               its inverse order[rank(t)] = t;
//   3. wavelet: one workgroup per (batch, KV head) builds the log2(S) levels
//               (bitvectors + per-word prefix counts) by stable partitions,
//               inside LDS when the eligible range fits (32768 tokens);
//   4. cutoff:  c_d for every d (KVPOP_CUTOFF_ALL when |E_d| < k, _NONE when
//               k = 0);
//   5. lists:   per query block [d0, d1] the union of the keys any of its
//               queries may keep: [0, s) below the window, the eligible
//               tokens of [s, d0-w] with rank <= c_{d0}, and (d0-w, d1], with
//               the keys that every query of the block keeps listed first;
//   6. forward: attention over the listed keys; tiles of the shared part
//               need no mask, the rest use the per-element membership
//               t <= d and (t < s or t > d-w or rank(t) <= c_d).
#include "attn_fwd.h"
#include "launch.h"

namespace kvpop {

constexpr int RANK_CH = 2048;
constexpr int CUT_ALL = 2147483647;
constexpr int CUT_NONE = -1;

struct BudgetLayout {
  size_t sorted, rank, order, cutoff, arr0, arr1, bits, prefix, zeros, lists, spans, lens, lens_full, lstatus,
      qorder, total;
  int S_pad, nchunks, L, nw1, nqb, QB, cap;
};

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

static BudgetLayout budget_layout(const ShapeInfo &s, int sinks, int window, int topk) {
  BudgetLayout lo{};
  const size_t BH = (size_t)s.B * s.Hkv;
  lo.nchunks = (s.S + RANK_CH - 1) / RANK_CH;
  lo.S_pad = lo.nchunks * RANK_CH;
  lo.L = 1;
  while ((1ll << lo.L) < (long long)s.S) ++lo.L;
  lo.nw1 = (s.S + 31) / 32 + 1;
  const int HG = fwd_heads_per_block(s.Hq / s.Hkv);
  lo.QB = 32 * (4 / HG);
  lo.nqb = (s.S + lo.QB - 1) / lo.QB;
  // room for the longest list, padded to whole tiles of the attention kernel
  long long cap = (long long)sinks + topk + window + lo.QB;
  if (cap > s.S) cap = s.S;
  lo.cap = (int)((cap + KVPOP_FWD_KT - 1) / KVPOP_FWD_KT * KVPOP_FWD_KT);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = al256(off + bytes);
    return o;
  };
  lo.sorted = take(BH * lo.S_pad * 8);
  lo.rank = take(BH * s.S * 4);
  lo.order = take(BH * s.S * 4);
  lo.cutoff = take(BH * s.S * 4);
  lo.arr0 = take(BH * s.S * 4);
  lo.arr1 = take(BH * s.S * 4);
  lo.bits = take(BH * lo.L * lo.nw1 * 4);
  lo.prefix = take(BH * lo.L * lo.nw1 * 4);
  lo.zeros = take(BH * lo.L * 4);
  lo.lists = take(BH * lo.nqb * (size_t)lo.cap * 4);
  lo.spans = take(BH * lo.nqb * (size_t)lo.cap * 8);
  lo.lens = take(BH * lo.nqb * 4);
  lo.lens_full = take(BH * lo.nqb * 4);
  lo.lstatus = take(BH * lo.nqb * 4);
  lo.qorder = take(BH * lo.nqb * 4);
  lo.total = off;
  return lo;
}

size_t budget_workspace_bytes(const ShapeInfo &s, int sinks, int window, int topk) {
  return budget_layout(s, sinks, window, topk).total;
}

BudgetListsInfo budget_lists_info(const ShapeInfo &s, int sinks, int window, int topk) {
  const BudgetLayout lo = budget_layout(s, sinks, window, topk);
  BudgetListsInfo li{};
  li.lists = lo.lists;
  li.spans = lo.spans;
  li.lens = lo.lens;
  li.lens_full = lo.lens_full;
  li.status = lo.lstatus;
  li.nqb = lo.nqb;
  li.QB = lo.QB;
  li.cap = lo.cap;
  li.tile = KVPOP_FWD_KT;
  return li;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Sort key: ascending order = descending score, then ascending index.  -0.0
// is folded into +0.0 and NaN into -inf before the order-preserving map.
__device__ __forceinline__ uint64_t score_key(float sc, int t) {
  if (sc != sc) sc = -INFINITY;
  if (sc == 0.f) sc = 0.f;
  const uint32_t u = __float_as_uint(sc);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)(~ord) << 32) | (uint32_t)t;
}

// The sort key of position t of sequence bh (t < S_pad): formed from the
// scores (the budget mask), or read from a key array (the teacher, whose keys
// come from its own priorities).  Positions past S sort last.
template <bool FROM_SCORES>
__device__ __forceinline__ uint64_t key_at(const void *src, size_t bh, int t, int S, int S_pad) {
  if constexpr (FROM_SCORES) {
    return (t < S) ? score_key(reinterpret_cast<const float *>(src)[bh * S + t], t) : ~0ull;
  } else {
    return reinterpret_cast<const uint64_t *>(src)[bh * S_pad + t];
  }
}

// Bitonic sort of one 2048-key chunk in LDS; 1024 threads, so every stage
// is one compare-exchange per thread.
template <bool FROM_SCORES>
__global__ void __launch_bounds__(1024) budget_sort_chunks(const void *src, uint64_t *sorted, int S, int S_pad) {
  static_assert(RANK_CH == 2048, "one compare-exchange per thread and stage");
  __shared__ uint64_t sh[RANK_CH];
  const size_t bh = blockIdx.y;
  const int t0 = (int)blockIdx.x * RANK_CH;
  const size_t base = bh * S_pad + t0;
  const int tid = threadIdx.x;
  sh[tid] = key_at<FROM_SCORES>(src, bh, t0 + tid, S, S_pad);
  sh[tid + 1024] = key_at<FROM_SCORES>(src, bh, t0 + tid + 1024, S, S_pad);
  __syncthreads();
  for (int k = 2; k <= RANK_CH; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int i = 2 * tid - (tid & (j - 1));  // the lower index of this thread's pair
      const int ixj = i + j;
      const bool up = (i & k) == 0;
      const uint64_t a = sh[i], b = sh[ixj];
      if ((a > b) == up) {
        sh[i] = b;
        sh[ixj] = a;
      }
      __syncthreads();
    }
  }
  sorted[base + tid] = sh[tid];
  sorted[base + tid + 1024] = sh[tid + 1024];
}

// rank(t) = the number of keys below key(t), summed over the sorted chunks,
// and its inverse, order[rank(t)] = t.  A workgroup ranks 256 tokens: it
// stages one sorted chunk at a time in LDS (coalesced, double-buffered, the
// next chunk's loads in flight during the current search) and each thread
// runs a branch-free lower-bound search of fixed depth there, instead of
// scattered probes through L2.
template <bool FROM_SCORES>
__global__ void __launch_bounds__(256) budget_rank(const void *src, const uint64_t *sorted, int *rank, int *order,
                                                   int S, int S_pad, int nchunks) {
  __shared__ uint64_t ch[2][RANK_CH];
  constexpr int PER = RANK_CH / 256;
  const int tid = threadIdx.x;
  const int t = blockIdx.x * 256 + tid;
  const size_t bh = blockIdx.y;
  const uint64_t key = key_at<FROM_SCORES>(src, bh, min(t, S_pad - 1), S, S_pad);
  const uint64_t *srt = sorted + bh * S_pad;
  uint64_t stage[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) stage[e] = srt[tid + 256 * e];
  int cnt = 0;
  for (int c = 0; c < nchunks; ++c) {
    uint64_t *buf = ch[c & 1];
#pragma unroll
    for (int e = 0; e < PER; ++e) buf[tid + 256 * e] = stage[e];
    __syncthreads();
    if (c + 1 < nchunks) {
#pragma unroll
      for (int e = 0; e < PER; ++e) stage[e] = srt[(size_t)(c + 1) * RANK_CH + tid + 256 * e];
    }
    int lo = 0;
#pragma unroll
    for (int step = RANK_CH / 2; step > 0; step >>= 1)
      if (buf[lo + step - 1] < key) lo += step;
    cnt += lo + (buf[lo] < key ? 1 : 0);
    // the buffer written next iteration is the other one; a barrier there
    // (after its writes) orders them against this iteration's reads of it
  }
  if (t < S) {
    rank[bh * S + t] = cnt;
    if (cnt < S) order[bh * S + cnt] = t;  // keys are distinct: a permutation of [0, S)
  }
}

// Block-wide exclusive scan of one int per thread (1024 threads).
__device__ __forceinline__ int block_excl_scan_1024(int x, int *sh_waves, int &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sh_waves[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    const int v = sh_waves[w];
    if (w < wave) before += v;
    tot += v;
  }
  __syncthreads();
  total = tot;
  return before + incl - x;
}

// The wavelet matrix of one (batch, KV head) holds the ranks of positions
// [base, S): base = sinks for an unpacked sequence (no eligible set starts
// earlier), 0 for packed documents (each document's eligible set starts at
// its own offset).
struct WaveletParams {
  const int *rank;
  int *arr0, *arr1;
  uint32_t *bits;
  int *prefix, *zeros;
  int S, base, L, nw1;
};

// One workgroup (1024 threads) per (batch, KV head): levels from the top bit
// down; each level stores the bit of every element of the current
// arrangement and then partitions it stably (zeros first).
__global__ void __launch_bounds__(1024) budget_wavelet_build(const WaveletParams p) {
  __shared__ int sh_waves[16];
  const size_t bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_e = p.S - p.base;
  if (n_e <= 0) return;
  int *cur = p.arr0 + bh * p.S;
  int *nxt = p.arr1 + bh * p.S;
  for (int i = tid; i < n_e; i += 1024) cur[i] = p.rank[bh * p.S + p.base + i];
  __threadfence();
  __syncthreads();
  const int wpt = (p.nw1 + 1023) / 1024;  // words per thread in the scan
  for (int lvl = p.L - 1; lvl >= 0; --lvl) {
    uint32_t *bl = p.bits + (bh * p.L + lvl) * p.nw1;
    int *pl = p.prefix + (bh * p.L + lvl) * p.nw1;
    for (int base = 0; base < 32 * p.nw1; base += 1024) {
      const int i = base + tid;
      const int bit = (i < n_e) ? ((cur[i] >> lvl) & 1) : 0;
      const uint64_t m = __ballot(bit);
      const int w0 = (base + 64 * wave) / 32;
      if (lane == 0 && w0 < p.nw1) bl[w0] = (uint32_t)m;
      if (lane == 0 && w0 + 1 < p.nw1) bl[w0 + 1] = (uint32_t)(m >> 32);
    }
    __threadfence();
    __syncthreads();
    int local = 0;
    for (int q = 0; q < wpt; ++q) {
      const int w = tid * wpt + q;
      if (w < p.nw1) local += __popc(bl[w]);
    }
    int ones;
    int run = block_excl_scan_1024(local, sh_waves, ones);
    for (int q = 0; q < wpt; ++q) {
      const int w = tid * wpt + q;
      if (w < p.nw1) {
        pl[w] = run;
        run += __popc(bl[w]);
      }
    }
    const int Z = n_e - ones;
    if (tid == 0) p.zeros[bh * p.L + lvl] = Z;
    __threadfence();
    __syncthreads();
    for (int i = tid; i < n_e; i += 1024) {
      const int v = cur[i];
      const int w = i >> 5;
      const int before = pl[w] + __popc(bl[w] & ((1u << (i & 31)) - 1u));
      const int pos = ((v >> lvl) & 1) ? Z + before : i - before;
      if (pos >= 0 && pos < n_e) nxt[pos] = v;
    }
    __threadfence();
    __syncthreads();
    int *tmp = cur;
    cur = nxt;
    nxt = tmp;
  }
}

// The same levels built inside LDS when the eligible range fits, every level
// by a workgroup of its own.  The arrangement a level partitions is the
// eligible ranks stably sorted by the bits above the level, the bit just above
// it most significant: each partition by a bit makes that bit the leading key
// and keeps the previous order among equals.  So a level's workgroup builds
// its arrangement directly by an LSD radix sort on 4-bit digits of that key
// (at most ceil((L-1)/4) passes, against L partitions in sequence), then
// stores the level's bit words, prefix counts and zero count like the
// sequential build.  Both arrangements (16-bit ranks) and the digit counts
// stay in LDS.
constexpr int WV_LDS_MAX = 32768;  // eligible tokens per (batch, KV head)
constexpr int WV_LDS_WORDS = WV_LDS_MAX / 32 + 32;

template <int WV_PER_THREAD>
__global__ void __launch_bounds__(1024) budget_wavelet_levels(const WaveletParams p) {
  // Thread tid holds elements tid + 1024*j (j < WV_PER_THREAD): the 64
  // elements of one wave and j form a group of consecutive indices, and the
  // groups run in index order j-major, then wave.  A radix pass ranks each
  // element within its group by matching its digit across the group's
  // ballots (kept, with the digit, two elements per register), counts each
  // digit per group, scans the counts digit-major and scatters.  Slots past
  // n_e take the largest digit, so (the sort being stable and they being
  // last) they stay past n_e.
  constexpr int N_MAX = WV_PER_THREAD * 1024;  // eligible tokens this instance holds
  constexpr int NG = WV_PER_THREAD * 16;       // groups of 64
  constexpr int CS = NG + 2;                   // digit row stride: one group's 16 digits hit 16 banks
  constexpr int NCNT = 16 * CS;
  static_assert(N_MAX <= WV_LDS_MAX, "fits the LDS arrays' budget");
  __shared__ uint16_t arr[2][N_MAX + 64];
  __shared__ __align__(16) uint16_t cnt[NCNT + 8];
  __shared__ uint32_t wl[WV_LDS_WORDS];
  __shared__ int sh_waves[16];
  const int lvl = (int)blockIdx.x % p.L;
  const size_t bh = blockIdx.x / p.L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_e = p.S - p.base;
  if (n_e <= 0 || n_e > N_MAX || p.nw1 > WV_LDS_WORDS) return;  // host picks this kernel only when it fits
  uint32_t *bl = p.bits + (bh * p.L + lvl) * p.nw1;
  int *pl = p.prefix + (bh * p.L + lvl) * p.nw1;
  const int nb = p.L - 1 - lvl;  // key bits: bit L-1-kp of a rank is key bit kp
  if (lvl <= 1 && nb > 12 && (1 << p.L) <= N_MAX) {
    // Levels 0 and 1 of a long range, which would take four radix passes.
    // A key's bucket holds only the 2 or 4 rank values that differ in the
    // bits at and below the level, so the level is built in one step: each
    // rank value's position is tabulated, the buckets' counts are scanned in
    // key order (the key being the bits above the level, reversed), and an
    // element's slot is its key's first slot plus the members of its bucket
    // that precede it in position.  Only the level's bit words are formed.
    uint16_t *pos_of = arr[0];  // position of each rank value, 0xffff where absent
    uint16_t *kbase = arr[1];   // first slot of each key
    const int nv = 1 << p.L, nk = 1 << nb, bsz = 2 << lvl;
    for (int x = tid; x < nv / 2; x += 1024) reinterpret_cast<uint32_t *>(pos_of)[x] = 0xffffffffu;
    for (int w = tid; w < p.nw1; w += 1024) wl[w] = 0u;
    __syncthreads();
    const int *src = p.rank + bh * p.S + p.base;
    int v[WV_PER_THREAD];
#pragma unroll
    for (int j = 0; j < WV_PER_THREAD; ++j) {
      const int i = tid + 1024 * j;
      v[j] = i < n_e ? src[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < WV_PER_THREAD; ++j) {
      const int i = tid + 1024 * j;
      if (i < n_e) pos_of[v[j]] = (uint16_t)i;  // ranks are distinct and below S <= nv
    }
    __syncthreads();
    auto bucket_count = [&](int k) {
      const int m = (int)(__brev((unsigned)k) >> (32 - nb));
      int c = 0;
      for (int u = 0; u < bsz; ++u) c += pos_of[m * bsz + u] != 0xffff ? 1 : 0;
      return c;
    };
    const int kpt = (nk + 1023) / 1024;  // keys per thread, contiguous
    int local = 0;
    for (int q = 0; q < kpt; ++q) {
      const int k = tid * kpt + q;
      if (k < nk) local += bucket_count(k);
    }
    int total;
    int run = block_excl_scan_1024(local, sh_waves, total);
    for (int q = 0; q < kpt; ++q) {
      const int k = tid * kpt + q;
      if (k < nk) {
        kbase[k] = (uint16_t)run;
        run += bucket_count(k);
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < WV_PER_THREAD; ++j) {
      const int i = tid + 1024 * j;
      if (i < n_e && ((v[j] >> lvl) & 1)) {
        const int m = v[j] >> (lvl + 1);
        int slot = kbase[__brev((unsigned)m) >> (32 - nb)];
        for (int u = 0; u < bsz; ++u) slot += pos_of[m * bsz + u] < i ? 1 : 0;  // absent values read 0xffff
        atomicOr(&wl[slot >> 5], 1u << (slot & 31));
      }
    }
  } else {
    {
      const int *src = p.rank + bh * p.S + p.base;
      int r[WV_PER_THREAD];
#pragma unroll
      for (int j = 0; j < WV_PER_THREAD; ++j) r[j] = src[min(tid + 1024 * j, n_e - 1)];
#pragma unroll
      for (int j = 0; j < WV_PER_THREAD; ++j) arr[0][tid + 1024 * j] = (uint16_t)r[j];
    }
    for (int w = 32 * WV_PER_THREAD + tid; w < p.nw1; w += 1024) wl[w] = 0u;  // words past the ballots' reach
    __syncthreads();
    const uint64_t below = (1ull << lane) - 1ull;
    int cur = 0;
    for (int pass = 0; 4 * pass < nb; ++pass) {
      const uint16_t *a = arr[cur];
      uint16_t *b = arr[cur ^ 1];
      for (int e = tid; e < (NCNT + 8) / 2; e += 1024) reinterpret_cast<uint32_t *>(cnt)[e] = 0u;
      __syncthreads();
      // per element: digit (4 bits) and rank among the group's equal digits
      // (6 bits), two elements per register
      uint32_t dr[WV_PER_THREAD / 2];
#pragma unroll
      for (int j = 0; j < WV_PER_THREAD; ++j) {
        // groups of eight reads: the compiler barrier keeps it from hoisting
        // all of them (with the packed ranks they would exceed 128 registers)
        if (j % 8 == 0) asm volatile("" ::: "memory");
        const uint32_t v = a[tid + 1024 * j];
        int d = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kp = 4 * pass + q;
          if (kp < nb) d |= (int)((v >> (p.L - 1 - kp)) & 1u) << q;
        }
        d = (tid + 1024 * j < n_e) ? d : 15;
        uint64_t m = ~0ull;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint64_t bq = __ballot((d >> q) & 1);
          m &= ((d >> q) & 1) ? bq : ~bq;
        }
        const int rk = __popcll(m & below);
        if (rk == 0) cnt[d * CS + 16 * j + wave] = (uint16_t)__popcll(m);  // the digit's lowest lane
        const uint32_t e = (uint32_t)(d | (rk << 4));
        dr[j / 2] = (j & 1) ? (dr[j / 2] | (e << 16)) : e;
      }
      __syncthreads();
      // exclusive scan of the counts, digit-major (a row's two pad entries are 0)
      constexpr int PER = (NCNT + 1023) / 1024;
      int local = 0;
      for (int e = 0; e < PER; ++e) {
        const int idx = tid * PER + e;
        local += idx < NCNT ? cnt[idx] : 0;
      }
      int total;
      int run = block_excl_scan_1024(local, sh_waves, total);
      for (int e = 0; e < PER; ++e) {  // each thread rewrites only its own entries
        const int idx = tid * PER + e;
        if (idx < NCNT) {
          const int c = cnt[idx];
          cnt[idx] = (uint16_t)run;
          run += c;
        }
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < WV_PER_THREAD; ++j) {
        if (j % 8 == 0) asm volatile("" ::: "memory");
        const uint32_t e = (dr[j / 2] >> (16 * (j & 1))) & 0xffffu;
        const int d = (int)(e & 15u), rk = (int)(e >> 4);
        const int pos = (int)cnt[d * CS + 16 * j + wave] + rk;
        b[pos < N_MAX ? pos : N_MAX + lane] = a[tid + 1024 * j];
      }
      __syncthreads();
      cur ^= 1;
    }
    // this level's bits of the arrangement
    const uint16_t *a = arr[cur];
#pragma unroll
    for (int j = 0; j < WV_PER_THREAD; ++j) {
      const int i = tid + 1024 * j;
      const int bit = (i < n_e) ? (int)(a[i] >> lvl) & 1 : 0;
      const uint64_t m = __ballot(bit);
      wl[32 * j + 2 * wave + (lane & 1)] = (lane & 1) ? (uint32_t)(m >> 32) : (uint32_t)m;
    }
  }
  __syncthreads();
  const int wpt = (p.nw1 + 1023) / 1024;  // words per thread in the scan
  int local = 0;
  for (int q = 0; q < wpt; ++q) {
    const int w = tid * wpt + q;
    if (w < p.nw1) local += __popc(wl[w]);
  }
  int ones;
  int run = block_excl_scan_1024(local, sh_waves, ones);
  for (int q = 0; q < wpt; ++q) {
    const int w = tid * wpt + q;
    if (w < p.nw1) {
      pl[w] = run;
      bl[w] = wl[w];
      run += __popc(wl[w]);
    }
  }
  if (tid == 0) p.zeros[bh * p.L + lvl] = n_e - ones;
}

// The per-level LDS build when the eligible range fits (16 or 32 elements per
// thread, whichever holds it), else the sequential global-memory build.
static void launch_wavelet_build(const WaveletParams &wp, int BH, hipStream_t st) {
  const int n_e = wp.S - wp.base;
  const bool lds_ok = wp.S <= 65536 && wp.nw1 <= WV_LDS_WORDS;
  if (lds_ok && n_e <= 16 * 1024)
    hipLaunchKernelGGL(budget_wavelet_levels<16>, dim3(BH * wp.L), dim3(1024), 0, st, wp);
  else if (lds_ok && n_e <= WV_LDS_MAX)
    hipLaunchKernelGGL(budget_wavelet_levels<32>, dim3(BH * wp.L), dim3(1024), 0, st, wp);
  else
    hipLaunchKernelGGL(budget_wavelet_build, dim3(BH), dim3(1024), 0, st, wp);
}

// k-th smallest (0-based kk) of the ranks of positions base+l .. base+r-1
// on the wavelet matrix of (batch, KV head) bh.
__device__ int wavelet_kth(const WaveletParams &p, size_t bh, int l, int r, int kk) {
  const int n_e = p.S - p.base;
  int val = 0;
  for (int lvl = p.L - 1; lvl >= 0; --lvl) {
    const uint32_t *bl = p.bits + (bh * p.L + lvl) * p.nw1;
    const int *pl = p.prefix + (bh * p.L + lvl) * p.nw1;
    const int ol = pl[l >> 5] + __popc(bl[l >> 5] & ((1u << (l & 31)) - 1u));
    const int orr = pl[r >> 5] + __popc(bl[r >> 5] & ((1u << (r & 31)) - 1u));
    const int zin = (r - l) - (orr - ol);
    if (kk < zin) {
      l -= ol;
      r -= orr;
    } else {
      kk -= zin;
      const int Z = p.zeros[bh * p.L + lvl];
      l = Z + ol;
      r = Z + orr;
      val |= 1 << lvl;
    }
    l = min(max(l, 0), n_e);  // stays in range for a well-formed matrix; guards the reads otherwise
    r = min(max(r, l), n_e);
  }
  return val;
}

// c_d: the topk-th smallest rank of E_d = [start(d) + sinks, d - window],
// start(d) the first position of d's document.
__global__ void __launch_bounds__(256) budget_cutoffs(const WaveletParams p, const int *cu, int n_docs, int sinks,
                                                      int window, int topk, int *cutoff) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  const size_t bh = blockIdx.y;
  if (d >= p.S) return;
  const int e_lo = find_doc(cu, n_docs, p.S, d).start + sinks;
  const long long m_e = (long long)d - window - e_lo + 1;  // |E_d|
  int res;
  if (topk <= 0) res = CUT_NONE;
  else if (m_e < topk) res = CUT_ALL;
  else res = wavelet_kth(p, bh, e_lo - p.base, e_lo - p.base + (int)m_e, topk - 1);
  cutoff[bh * p.S + d] = res;
}

struct ListParams {
  const int *rank, *order, *cutoff;
  const int *cu;  // document offsets, or nullptr for one document per batch row
  int *lists, *lens, *lens_full, *status;
  int2 *spans;
  int S, n_docs, sinks, window, topk, QB, nqb, cap;
};

// Key list of query block [d0, d1].  Within a document [a, e), query d keeps
// the sinks [a, a+s), its window (d-w, d] and the eligible tokens of
// E_d = [a+s, d-w] with rank <= c_d.
//
// Every listed key t comes with the span [lo, hi) of query positions that
// keep it, so that the attention kernel's element mask is lo <= d < hi.  The
// queries keeping t form one interval: t itself onwards (causal); while t is
// in their window (d < t + w) or a sink; then, once eligible, while
// rank(t) <= c_d, which holds on a prefix since c_d does not rise; and never
// past the document's end e.  So lo = t and hi is e for a sink, else the
// first d >= t + w with c_d < rank(t), or e if no query of the block has
// one (found by a binary search over the block's cutoffs).
//
// A block inside one document gets two segments:
//   full:    the sinks below the window, the eligible tokens of [a+s, d0-w]
//            with rank <= c_{d1}, then the positions (d1-w, d0].  Every query
//            of the block keeps all of them (c_d is non-increasing, so
//            c_{d1} <= c_d; and (d1-w, d0] is inside every query's window
//            and at or before every query), so their tiles need no
//            per-element mask (their spans are the whole sequence);
//   partial: the eligible tokens with c_{d1} < rank <= c_{d0}, then the
//            rest of the window region (d0-w, d1]; these are masked per
//            element with their spans.
// The size of the full segment is known before the sweep: E_{d1} holds
// exactly topk tokens of rank <= c_{d1}, so E_{d0} holds topk minus those in
// (d0-w, d1-w] (at most QB-1 reads).
// A block that spans documents lists, for each document's part [p0, p1],
// the sinks below p0's window, the eligible tokens of E_{p0} with
// rank <= c_{p0} and the positions (p0-w, p1] of the document, all in the
// partial segment (the spans end at the document's end).  Only the first
// part can reach back before d0, so the list still holds at most
// s + k + w + QB - 1 keys.
// The eligible tokens are found by whichever sweep is shorter: over the
// positions, or over the ranks [0, c] through the inverse permutation
// (late blocks: c is about topk while the eligible range grows with d0).
// The attention kernel needs no order inside a segment.
constexpr int LIST_QB_MAX = 128;
__global__ void __launch_bounds__(256) budget_lists(const ListParams p) {
  __shared__ int sh_w[2][4];
  __shared__ int sh_sub;
  __shared__ int sh_c[LIST_QB_MAX];  // c_d of the block's queries
  const int qb = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d0 = qb * p.QB, d1 = min(p.S - 1, d0 + p.QB - 1);
  const int *rk = p.rank + bh * p.S;
  const int *ord = p.order + bh * p.S;
  const int *cut = p.cutoff + bh * p.S;
  int *list = p.lists + (bh * p.nqb + qb) * (size_t)p.cap;
  int2 *span = p.spans + (bh * p.nqb + qb) * (size_t)p.cap;
  if (tid < d1 - d0 + 1) sh_c[tid] = cut[d0 + tid];
  __syncthreads();
  int off_f = 0, off_p = 0;
  constexpr int EVERY = 0x7fffffff;  // span end of keys kept to the end of the sequence
  // Spans are read only for the masked tiles: every tile of the partial
  // segment, and the last tile of the full segment when the full segment
  // ends inside it.  Full entries before span_from get none (the bulk of
  // the list: writing them all would triple the list's bytes).
  int span_from = 0;

  // first query in [from, to] with c_d < r, else `none` (c_d does not rise
  // inside one document, so the predicate holds on a suffix)
  auto first_below = [&](int r, int from, int to, int none) {
    if (from > to || sh_c[to - d0] >= r) return none;
    int lo = from, hi = to;  // the answer lies in [lo, hi]
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sh_c[mid - d0] < r) hi = mid; else lo = mid + 1;
    }
    return lo;
  };
  // span of a non-sink key t of rank r whose document's queries in the block
  // are [q0, q1] and whose document ends at e
  auto span_of = [&](int t, int r, int q0, int q1, int e) {
    return make_int2(t, first_below(r, max(q0, t + p.window), q1, e));
  };

  // Appends the eligible tokens t in [lo, hi] with rank <= c_any: those with
  // rank <= c_all at off_f (full segment), the others at off_p (partial, with
  // their spans among the queries [q0, q1] of a document ending at e).  The
  // loads of up to LIST_PF chunks of 256 go out before the first chunk is
  // used (one memory round trip per LIST_PF chunks, not per chunk).
  auto sweep = [&](int lo, int hi, int c_all, int c_any, int q0, int q1, int e) {
    const int n_pos = max(0, hi - lo + 1);
    if (n_pos == 0 || c_any == CUT_NONE) return;
    const bool by_rank = c_any != CUT_ALL && c_any + 1 < n_pos;
    const int n_sweep = by_rank ? c_any + 1 : n_pos;
    constexpr int LIST_PF = 8;
    for (int base0 = 0; base0 < n_sweep; base0 += 256 * LIST_PF) {
      int tv[LIST_PF], rv[LIST_PF];
#pragma unroll
      for (int u = 0; u < LIST_PF; ++u) {
        const int x = base0 + 256 * u + tid;
        tv[u] = -1;
        rv[u] = INT32_MAX;
        if (x < n_sweep) {
          if (by_rank) {
            rv[u] = x;
            tv[u] = ord[x];
          } else {
            tv[u] = lo + x;
            rv[u] = rk[tv[u]];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < LIST_PF; ++u) {
        if (base0 + 256 * u >= n_sweep) break;  // uniform over the workgroup
        const int t = tv[u], r = rv[u];
        const bool elig = t >= lo && t <= hi;
        const bool ff = elig && r <= c_all;
        const bool fp = elig && r > c_all && r <= c_any;
        const uint64_t mf = __ballot(ff), mp = __ballot(fp);
        if (lane == 0) {
          sh_w[0][wave] = __popcll(mf);
          sh_w[1][wave] = __popcll(mp);
        }
        __syncthreads();
        int bf = 0, bp = 0, tf = 0, tp = 0;
        for (int w = 0; w < 4; ++w) {
          if (w < wave) {
            bf += sh_w[0][w];
            bp += sh_w[1][w];
          }
          tf += sh_w[0][w];
          tp += sh_w[1][w];
        }
        if (ff) {
          const int slot = off_f + bf + __popcll(mf & lanemask_lt(lane));
          if (slot < p.cap) {
            list[slot] = t;
            if (slot >= span_from) span[slot] = make_int2(0, EVERY);
          }
        }
        if (fp) {
          const int slot = off_p + bp + __popcll(mp & lanemask_lt(lane));
          if (slot < p.cap) {
            list[slot] = t;
            span[slot] = span_of(t, r, q0, q1, e);
          }
        }
        off_f += tf;
        off_p += tp;
        __syncthreads();
      }
    }
  };
  // positions [lo, lo + n) at off_p, skipping [skip_lo, skip_lo + n_skip),
  // with their spans (sinks: kept to the document's end e)
  auto append_range = [&](int lo, int n, int skip_lo, int n_skip, int e_lo, int q0, int q1, int e) {
    for (int i = tid; i < n && off_p + i < p.cap; i += 256) {
      const int t = (n_skip == 0 || lo + i < skip_lo) ? lo + i : lo + i + n_skip;
      list[off_p + i] = t;
      span[off_p + i] = t < e_lo ? make_int2(t, e) : span_of(t, rk[t], q0, q1, e);
    }
    off_p += n;
  };

  const Doc doc0 = find_doc(p.cu, p.n_docs, p.S, d0);
  int status = 0;
  if (d1 < doc0.end) {
    // the block lies inside one document
    const int a = doc0.start, e = doc0.end, e_lo = a + p.sinks;
    const int c0 = sh_c[0], c1 = sh_c[d1 - d0];
    const int a_end = max(a, min(min(e_lo, d0 - p.window + 1), d1 + 1));  // sinks below the window: [a, a_end)
    const int n_a = a_end - a;
    const int b_hi = d0 - p.window;  // E_{d0} = [e_lo, b_hi]
    const int n_e0 = max(0, b_hi - e_lo + 1);
    int n_bfull;
    if (c1 == CUT_NONE) {
      n_bfull = 0;
    } else if (c1 == CUT_ALL) {
      n_bfull = n_e0;
    } else {
      if (tid == 0) sh_sub = 0;
      __syncthreads();
      const int lo = max(e_lo, b_hi + 1), hi = d1 - p.window;  // E_{d1} \ E_{d0}
      const int t = lo + tid;
      if (t <= hi && rk[t] <= c1) atomicAdd(&sh_sub, 1);  // LDS counter, at most QB-1 increments
      __syncthreads();
      n_bfull = p.topk - sh_sub;
    }
    // the window region R = (d0-w, d1] of the document: its part (d1-w, d0]
    // lies inside every query's window and at or before every query of the
    // block, so it joins the unmasked segment; the rest of R is masked per
    // element
    const int c_lo = max(a, d0 - p.window + 1);                 // first position of R
    const int wc_lo = max(c_lo, d1 - p.window + 1), wc_hi = d0;  // (d1-w, d0], possibly empty
    const int n_wc = max(0, wc_hi - wc_lo + 1);
    const int n_full = n_a + n_bfull + n_wc;
    span_from = n_full / KVPOP_FWD_KT * KVPOP_FWD_KT;
    for (int i = tid; i < n_a && i < p.cap; i += 256) {
      list[i] = a + i;
      if (i >= span_from) span[i] = make_int2(0, EVERY);
    }
    for (int i = tid; i < n_wc && n_a + n_bfull + i < p.cap; i += 256) {
      list[n_a + n_bfull + i] = wc_lo + i;
      if (n_a + n_bfull + i >= span_from) span[n_a + n_bfull + i] = make_int2(0, EVERY);
    }
    off_f = n_a;
    off_p = n_full;
    sweep(e_lo, b_hi, c1, c0, d0, d1, e);
    if (off_f != n_a + n_bfull) status |= 2;
    // the masked part of R: all of R when (d1-w, d0] is empty, else
    // (d0-w, d1-w] then (d0, d1]
    append_range(c_lo, d1 - c_lo + 1 - n_wc, wc_lo, n_wc, e_lo, d0, d1, e);
    off_f += n_wc;
  } else {
    // the block spans documents: every part's keys are masked per element
    for (int m_lo = doc0.start; m_lo <= d1;) {
      const Doc dm = find_doc(p.cu, p.n_docs, p.S, m_lo);
      const int a = dm.start, e = dm.end, e_lo = a + p.sinks;
      const int p0 = max(d0, a), p1 = min(d1, e - 1);
      const int a_end = max(a, min(min(e_lo, p0 - p.window + 1), p1 + 1));
      append_range(a, a_end - a, 0, 0, e_lo, p0, p1, e);
      sweep(e_lo, p0 - p.window, CUT_NONE, sh_c[p0 - d0], p0, p1, e);
      const int c_lo = max(a, p0 - p.window + 1);
      append_range(c_lo, max(0, p1 - c_lo + 1), 0, 0, e_lo, p0, p1, e);
      m_lo = e;
    }
  }
  // pad the list to whole tiles: position S (a row past the end of K and V,
  // which the attention kernel's loads return as zeros) kept by no query
  const int n_pad = (min(off_p, p.cap) + KVPOP_FWD_KT - 1) / KVPOP_FWD_KT * KVPOP_FWD_KT;
  for (int i = min(off_p, p.cap) + tid; i < n_pad; i += 256) {
    list[i] = p.S;
    span[i] = make_int2(EVERY, EVERY);
  }
  if (tid == 0) {
    p.lens[bh * p.nqb + qb] = min(off_p, p.cap);
    p.lens_full[bh * p.nqb + qb] = min(off_f, p.cap);
    // 0 when the list is whole: bit 0 = entries past the capacity were
    // dropped, bit 1 = the sweep found a different number of shared keys
    // than the count the segment was laid out for
    p.status[bh * p.nqb + qb] = status | (off_p > p.cap ? 1 : 0);
  }
}

// The order of the sparse forward's query blocks over packed documents.  A
// block's work is its list, whose length follows the block's position inside
// its document rather than in the sequence, so latest-first is no longer
// largest-first: blocks are ranked by tile count (descending), later blocks
// first among equals (the order without documents), and run in that order,
// which puts the short lists of early and short documents in the last
// round.  A block's rank is the number of the head's blocks ahead of it.
// Each workgroup ranks 64 of one head's blocks (one per lane); its four
// waves each count the blocks ahead within a quarter of the head's tile
// counts, held in LDS, and the quarters' counts are summed.
constexpr int BLOCK_ORDER_MAX = 1024;  // query blocks per head the ranking takes
constexpr int ORDER_ROWS = 64;         // blocks ranked per workgroup
constexpr int ORDER_SLICES = 4;        // waves per workgroup, one slice of the counts each
__global__ void __launch_bounds__(ORDER_ROWS *ORDER_SLICES) budget_block_order(const int *lens, int *qorder, int nqb,
                                                                               int KT) {
  __shared__ __align__(16) unsigned short tl[BLOCK_ORDER_MAX];
  __shared__ int part[ORDER_SLICES][ORDER_ROWS];
  if (nqb <= 0 || nqb > BLOCK_ORDER_MAX) return;  // the host launches this only when the head's blocks fit
  const int per_head = (nqb + ORDER_ROWS - 1) / ORDER_ROWS;
  const size_t bh = blockIdx.x / per_head;
  const int i0 = (int)(blockIdx.x % per_head) * ORDER_ROWS;
  // the table is padded to whole 8-count reads in every slice; padding holds 0
  // and a real block 1 + its tile count (saturated at 16 bits), so padding is
  // never ahead of a block and the ranks stay a permutation
  constexpr int STEP = 8 * ORDER_SLICES;
  const int npad = (nqb + STEP - 1) / STEP * STEP;  // <= BLOCK_ORDER_MAX, a multiple of STEP
  for (int j = threadIdx.x; j < npad; j += ORDER_ROWS * ORDER_SLICES)
    tl[j] = j < nqb ? (unsigned short)min((lens[bh * nqb + j] + KT - 1) / KT + 1, 0xffff) : 0;
  __syncthreads();
  const int lane = threadIdx.x % ORDER_ROWS, slice = threadIdx.x / ORDER_ROWS;
  const int i = i0 + lane;
  const int ti = i < nqb ? (int)tl[i] : 0;
  const int span = npad / ORDER_SLICES;
  int r = 0;
  // all lanes of a wave read the same eight counts at a time (a broadcast LDS read)
  for (int j0 = slice * span; j0 < (slice + 1) * span; j0 += 8) {
    const uint4 w = *reinterpret_cast<const uint4 *>(&tl[j0]);
    const unsigned wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tj = (int)((wv[e >> 1] >> (16 * (e & 1))) & 0xffffu);
      r += (int)(tj > ti) | ((int)(tj == ti) & (int)(j0 + e > i));
    }
  }
  part[slice][lane] = r;
  __syncthreads();
  if (slice == 0 && i < nqb) {
    int rank = 0;
#pragma unroll
    for (int q = 0; q < ORDER_SLICES; ++q) rank += part[q][lane];
    qorder[bh * nqb + rank] = i;
  }
}

template <typename T, int D>
static hipError_t run_sparse(const FwdParams &fp, int grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, true, true>), dim3(grid), dim3(256), 0, st, fp);
  return hipGetLastError();
}

hipError_t launch_budget(const ShapeInfo &s, const void *q, const void *k, const void *v,
                         const float *scores, int sinks, int window, int topk, void *o, float *lse,
                         int *rank_out, int *cutoff_out, void *ws, hipStream_t st) {
  const BudgetLayout lo = budget_layout(s, sinks, window, topk);
  char *w = reinterpret_cast<char *>(ws);
  const int BH = s.B * s.Hkv;
  uint64_t *sorted = reinterpret_cast<uint64_t *>(w + lo.sorted);
  int *rank = rank_out ? rank_out : reinterpret_cast<int *>(w + lo.rank);
  int *cutoff = cutoff_out ? cutoff_out : reinterpret_cast<int *>(w + lo.cutoff);

  int *order = reinterpret_cast<int *>(w + lo.order);
  hipLaunchKernelGGL(budget_sort_chunks<true>, dim3(lo.nchunks, BH), dim3(1024), 0, st, scores, sorted, s.S, lo.S_pad);
  hipLaunchKernelGGL(budget_rank<true>, dim3((s.S + 255) / 256, BH), dim3(256), 0, st, scores, sorted, rank, order, s.S,
                     lo.S_pad, lo.nchunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  WaveletParams wp{};
  wp.rank = rank;
  wp.arr0 = reinterpret_cast<int *>(w + lo.arr0);
  wp.arr1 = reinterpret_cast<int *>(w + lo.arr1);
  wp.bits = reinterpret_cast<uint32_t *>(w + lo.bits);
  wp.prefix = reinterpret_cast<int *>(w + lo.prefix);
  wp.zeros = reinterpret_cast<int *>(w + lo.zeros);
  wp.S = s.S;
  wp.base = s.cu != nullptr ? 0 : sinks;
  wp.L = lo.L;
  wp.nw1 = lo.nw1;
  if (topk > 0 && s.S - wp.base > 0) launch_wavelet_build(wp, BH, st);
  hipLaunchKernelGGL(budget_cutoffs, dim3((s.S + 255) / 256, BH), dim3(256), 0, st, wp, s.cu, s.n_docs, sinks, window,
                     topk, cutoff);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  ListParams lp{};
  lp.rank = rank;
  lp.order = order;
  lp.cutoff = cutoff;
  lp.lists = reinterpret_cast<int *>(w + lo.lists);
  lp.spans = reinterpret_cast<int2 *>(w + lo.spans);
  lp.lens = reinterpret_cast<int *>(w + lo.lens);
  lp.lens_full = reinterpret_cast<int *>(w + lo.lens_full);
  lp.status = reinterpret_cast<int *>(w + lo.lstatus);
  lp.cu = s.cu;
  lp.n_docs = s.n_docs;
  lp.topk = topk;
  lp.S = s.S;
  lp.sinks = sinks;
  lp.window = window;
  lp.QB = lo.QB;
  lp.nqb = lo.nqb;
  lp.cap = lo.cap;
  hipLaunchKernelGGL(budget_lists, dim3(lo.nqb, BH), dim3(256), 0, st, lp);
  e = hipGetLastError();
  if (e != hipSuccess || o == nullptr) return e;  // no outputs: the mask alone

  FwdParams fp{};
  fp.q = q;
  fp.k = k;
  fp.v = v;
  fp.o = o;
  fp.lse = lse;
  fp.B = s.B;
  fp.S = s.S;
  fp.Hq = s.Hq;
  fp.Hkv = s.Hkv;
  fp.G = s.Hq / s.Hkv;
  fp.HG = fwd_heads_per_block(fp.G);
  fp.scale_log2 = s.scale * kLog2e;
  fp.cu = s.cu;
  fp.n_docs = s.n_docs;
  fp.lists = lp.lists;
  fp.spans = lp.spans;
  fp.list_len = lp.lens;
  fp.list_len_full = lp.lens_full;
  fp.list_cap = lo.cap;
  if (s.cu != nullptr && lo.nqb <= BLOCK_ORDER_MAX) {
    int *qorder = reinterpret_cast<int *>(w + lo.qorder);
    fp.qorder = qorder;
    const int per_head = (lo.nqb + ORDER_ROWS - 1) / ORDER_ROWS;
    hipLaunchKernelGGL(budget_block_order, dim3(BH * per_head), dim3(ORDER_ROWS * ORDER_SLICES), 0, st, lp.lens,
                       qorder, lo.nqb, KVPOP_FWD_KT);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int grid = lo.nqb * s.B * s.Hkv * (fp.G / fp.HG);
  if (s.dtype == 0 && s.D == 128) return run_sparse<bf16, 128>(fp, grid, st);
  if (s.dtype == 0 && s.D == 64) return run_sparse<bf16, 64>(fp, grid, st);
  if (s.dtype == 1 && s.D == 64) return run_sparse<float, 64>(fp, grid, st);
  return hipErrorInvalidValue;
}

// ===========================================================================
// Teacher labels at the eviction boundary (KVpop paper, Section 3.1, Eqs.
// 4-6) and the boundary-aware retention loss (Eq. 7).
//
// The teacher ranks the eligible tokens E_d = [s, d-w] by effective scores
// (the target minus a per-head decay of lambda per Delta positions of age)
// and keeps the top-k.  Section 3.2's running threshold over static
// priorities applies: pi(t) = y(t) + (lambda/Delta)*t (the age term's
// query-dependent part is shared by all eligible tokens; exact when
// lambda = 0 or Delta = 1).  The rank/wavelet engine of the budget mask then
// gives, for every d, the boundary rank b_d = the min(k, |E_d|)-th smallest
// rank of E_d (the last kept token), the boundary token of that rank, and the
// label of the newly eligible token d-w: rank(d-w) <= b_d.

__global__ void __launch_bounds__(256) teacher_keys(const float *y, const float *lam, int delta, uint64_t *keys,
                                                    int S, int S_pad, int Hkv) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const size_t bh = blockIdx.y;
  if (t >= S_pad) return;
  uint64_t key = ~0ull;
  if (t < S) {
    const float c = (lam != nullptr) ? __fdiv_rn(lam[bh % Hkv], (float)delta) : 0.f;
    const float pri = __fadd_rn(y[bh * S + t], __fmul_rn(c, (float)t));  // no contraction: same rounding as the reference
    key = score_key(pri, t);
  }
  keys[bh * S_pad + t] = key;
}

struct TeacherParams {
  WaveletParams wp;
  const int *rank, *order;
  int *label, *boundary, *brank;
  int window, topk;
};

__global__ void __launch_bounds__(256) teacher_bounds(const TeacherParams p) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  const size_t bh = blockIdx.y;
  const int S = p.wp.S;
  if (d >= S) return;
  const long long m_e = (long long)d - p.window - p.wp.base + 1;  // |E_d| (the matrix starts at the sinks)
  int lab = -1, bnd = -1, br = -1;
  if (p.topk > 0 && m_e > 0) {
    const int m = (int)m_e;
    br = wavelet_kth(p.wp, bh, 0, m, min(p.topk, m) - 1);
    if (br >= 0 && br < S) bnd = p.order[bh * S + br];
    lab = (p.rank[bh * S + d - p.window] <= br) ? 1 : 0;
  }
  p.label[bh * S + d] = lab;
  p.boundary[bh * S + d] = bnd;
  if (p.brank != nullptr) p.brank[bh * S + d] = br;
}

struct TeacherLayout {
  size_t keys, sorted, rank, order, arr0, arr1, bits, prefix, zeros, total;
  int S_pad, nchunks, L, nw1;
};

static TeacherLayout teacher_layout(int B, int Hkv, int S) {
  TeacherLayout lo{};
  const size_t BH = (size_t)B * Hkv;
  lo.nchunks = (S + RANK_CH - 1) / RANK_CH;
  lo.S_pad = lo.nchunks * RANK_CH;
  lo.L = 1;
  while ((1ll << lo.L) < (long long)S) ++lo.L;
  lo.nw1 = (S + 31) / 32 + 1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = al256(off + bytes);
    return o;
  };
  lo.keys = take(BH * lo.S_pad * 8);
  lo.sorted = take(BH * lo.S_pad * 8);
  lo.rank = take(BH * S * 4);
  lo.order = take(BH * S * 4);
  lo.arr0 = take(BH * S * 4);
  lo.arr1 = take(BH * S * 4);
  lo.bits = take(BH * lo.L * lo.nw1 * 4);
  lo.prefix = take(BH * lo.L * lo.nw1 * 4);
  lo.zeros = take(BH * lo.L * 4);
  lo.total = off;
  return lo;
}

size_t teacher_workspace_bytes(int B, int Hkv, int S) { return teacher_layout(B, Hkv, S).total; }

hipError_t launch_teacher(int B, int Hkv, int S, const float *y, const float *lam, int delta, int sinks, int window,
                          int topk, int *label, int *boundary, int *rank_out, int *brank_out, void *ws,
                          hipStream_t st) {
  const TeacherLayout lo = teacher_layout(B, Hkv, S);
  char *w = reinterpret_cast<char *>(ws);
  const int BH = B * Hkv;
  uint64_t *keys = reinterpret_cast<uint64_t *>(w + lo.keys);
  uint64_t *sorted = reinterpret_cast<uint64_t *>(w + lo.sorted);
  int *rank = rank_out ? rank_out : reinterpret_cast<int *>(w + lo.rank);
  int *order = reinterpret_cast<int *>(w + lo.order);
  hipLaunchKernelGGL(teacher_keys, dim3(lo.S_pad / 256, BH), dim3(256), 0, st, y, lam, delta, keys, S, lo.S_pad, Hkv);
  hipLaunchKernelGGL(budget_sort_chunks<false>, dim3(lo.nchunks, BH), dim3(1024), 0, st, keys, sorted, S, lo.S_pad);
  hipLaunchKernelGGL(budget_rank<false>, dim3((S + 255) / 256, BH), dim3(256), 0, st, keys, sorted, rank, order, S,
                     lo.S_pad, lo.nchunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  TeacherParams tp{};
  WaveletParams &wp = tp.wp;
  wp.rank = rank;
  wp.arr0 = reinterpret_cast<int *>(w + lo.arr0);
  wp.arr1 = reinterpret_cast<int *>(w + lo.arr1);
  wp.bits = reinterpret_cast<uint32_t *>(w + lo.bits);
  wp.prefix = reinterpret_cast<int *>(w + lo.prefix);
  wp.zeros = reinterpret_cast<int *>(w + lo.zeros);
  wp.S = S;
  wp.base = sinks;
  wp.L = lo.L;
  wp.nw1 = lo.nw1;
  if (topk > 0 && S - sinks > 0) launch_wavelet_build(wp, BH, st);
  tp.rank = rank;
  tp.order = order;
  tp.label = label;
  tp.boundary = boundary;
  tp.brank = brank_out;
  tp.window = window;
  tp.topk = topk;
  hipLaunchKernelGGL(teacher_bounds, dim3((S + 255) / 256, BH), dim3(256), 0, st, tp);
  return hipGetLastError();
}

// ---- Eq. 7: loss per query position and the gradient of the sum ----
// loss_d = omega_d * softplus(-sign_d * x_d), x_d = (r(d-w) - r(t_bnd(d)))/tau.
// Token d-w receives +g_d and the boundary token -g_d, g_d = dloss_d/dx_d /
// tau.  Many d share one boundary token; since the boundary rank rises while
// |E_d| < k and then falls (c_d is non-increasing), the d's of one boundary
// token form at most one run before d* = s+w+k-1 and one from d* on.  Each
// run is summed in d order by the thread of its first d and stored in that
// phase's slot of the token, so the reduction is deterministic and needs no
// atomics.

struct LossParams {
  const float *pred, *weight;
  const int *label, *boundary;
  float *loss, *grad, *gterm, *slot0, *slot1;
  float *segsum;  // [BH][S]: in-wave sum of the segment a head lane starts
  int *wf_b;      // [BH][nwv]: boundary of each 64-position wave's first element
  int *wf_whole;  // [BH][nwv]: whether that wave is one segment
  float *wf_sum;  // [BH][nwv]: sum of the wave's first segment
  int S, window, dstar, nwv;
  float inv_tau;
};

__global__ void __launch_bounds__(256) boundary_loss_terms(const LossParams p) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  const size_t bh = blockIdx.y;
  if (d >= p.S) return;
  const size_t i = bh * p.S + d;
  const int lab = p.label[i], b = p.boundary[i], a = d - p.window;
  float loss = 0.f, g = 0.f;
  if (lab >= 0 && b >= 0 && b < p.S && a >= 0) {
    const float sgn = lab == 1 ? 1.f : -1.f;
    const float om = p.weight ? p.weight[i] : 1.f;
    const float x = (p.pred[bh * p.S + a] - p.pred[bh * p.S + b]) * p.inv_tau;
    const float z = -sgn * x;
    loss = om * (fmaxf(z, 0.f) + log1pf(expf(-fabsf(z))));
    const float sig = expf(fminf(z, 0.f)) / (1.f + expf(-fabsf(z)));
    g = -sgn * om * sig * p.inv_tau;
  }
  p.loss[i] = loss;
  p.gterm[i] = g;
  p.slot0[i] = 0.f;
  p.slot1[i] = 0.f;
}

// The gradient of a boundary token b collects the terms of the consecutive
// positions d whose boundary is b (a run).  Sums in a fixed order (so the
// result is reproducible), in two levels: each wave of 64 positions forms
// the sum of every segment of equal boundary inside it by a segmented
// suffix scan, and records its first segment; the head of a run then adds
// the first segments of the following waves while the run continues.
__device__ __forceinline__ int loss_boundary_at(const LossParams &p, size_t bh, int d) {
  if (d >= p.S) return -2;
  const int b = p.boundary[bh * p.S + d];
  return (b >= 0 && b < p.S) ? b : -1;
}

__global__ void __launch_bounds__(256) boundary_loss_segments(const LossParams p) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  const size_t bh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int b = loss_boundary_at(p, bh, d);
  float x = (d < p.S) ? p.gterm[bh * p.S + d] : 0.f;
  const int b_up = __shfl_up(b, 1);
  const bool head = lane == 0 || b != b_up;
  const uint64_t H = __ballot(head);
  const uint64_t above = lane == 63 ? 0ull : (H & (~0ull << (lane + 1)));
  const int end = above ? __ffsll((long long)above) - 1 : 64;  // first lane of the next segment
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_down(x, o);
    if (lane + o < end) x += y;
  }
  if (d < p.S && head) p.segsum[bh * p.S + d] = x;
  if (lane == 0 && d < p.S) {
    const size_t w = bh * p.nwv + d / 64;
    p.wf_b[w] = b;
    p.wf_whole[w] = H == 1ull;
    p.wf_sum[w] = x;
  }
}

__global__ void __launch_bounds__(256) boundary_loss_runs(const LossParams p) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  const size_t bh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int b = loss_boundary_at(p, bh, d);
  const int b_up = __shfl_up(b, 1);
  const bool head = lane == 0 || b != b_up;
  const uint64_t H = __ballot(head);
  if (d >= p.S || b < 0 || !head) return;
  if (lane == 0 && d > 0 && loss_boundary_at(p, bh, d - 1) == b) return;  // continues the previous wave's run
  float sum = p.segsum[bh * p.S + d];
  const uint64_t above = lane == 63 ? 0ull : (H & (~0ull << (lane + 1)));
  if (above == 0ull) {  // the segment reaches the end of its wave: follow the run
    bool go = true;
    for (int w0 = d / 64 + 1; go && w0 < p.nwv; w0 += 8) {
      int fb[8], fw[8];
      float fs[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int w = w0 + j;
        const size_t i = bh * p.nwv + min(w, p.nwv - 1);
        fb[j] = w < p.nwv ? p.wf_b[i] : -3;
        fw[j] = p.wf_whole[i];
        fs[j] = p.wf_sum[i];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (go) {
          if (fb[j] != b) {
            go = false;
          } else {
            sum += fs[j];
            if (!fw[j]) go = false;
          }
        }
      }
    }
  }
  float *slot = (d < p.dstar) ? p.slot0 : p.slot1;
  slot[bh * p.S + b] = sum;
}

__global__ void __launch_bounds__(256) boundary_loss_grad(const LossParams p) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const size_t bh = blockIdx.y;
  if (t >= p.S) return;
  const size_t i = bh * p.S + t;
  const float g_new = (t + p.window < p.S) ? p.gterm[i + p.window] : 0.f;
  p.grad[i] = g_new - p.slot0[i] - p.slot1[i];
}

static int loss_waves(int S) { return (S + 63) / 64; }

size_t boundary_loss_workspace_bytes(int B, int Hkv, int S) {
  const size_t BH = (size_t)B * Hkv;
  return 4 * al256(BH * S * 4) + 3 * al256(BH * loss_waves(S) * 4);
}

hipError_t launch_boundary_loss(int B, int Hkv, int S, const float *pred, const int *label, const int *boundary,
                                int sinks, int window, int topk, float tau, const float *weight, float *loss,
                                float *grad, void *ws, hipStream_t st) {
  LossParams lp{};
  const size_t n = al256((size_t)B * Hkv * S * 4);
  char *w = reinterpret_cast<char *>(ws);
  lp.pred = pred;
  lp.weight = weight;
  lp.label = label;
  lp.boundary = boundary;
  lp.loss = loss;
  lp.grad = grad;
  const size_t nw = al256((size_t)B * Hkv * loss_waves(S) * 4);
  lp.gterm = reinterpret_cast<float *>(w);
  lp.slot0 = reinterpret_cast<float *>(w + n);
  lp.slot1 = reinterpret_cast<float *>(w + 2 * n);
  lp.segsum = reinterpret_cast<float *>(w + 3 * n);
  lp.wf_b = reinterpret_cast<int *>(w + 4 * n);
  lp.wf_whole = reinterpret_cast<int *>(w + 4 * n + nw);
  lp.wf_sum = reinterpret_cast<float *>(w + 4 * n + 2 * nw);
  lp.nwv = loss_waves(S);
  lp.S = S;
  lp.window = window;
  const long long ds = (long long)sinks + window + topk - 1;
  lp.dstar = (int)min(max(ds, 0ll), (long long)S);
  lp.inv_tau = 1.f / tau;
  const dim3 grid((S + 255) / 256, B * Hkv);
  hipLaunchKernelGGL(boundary_loss_terms, grid, dim3(256), 0, st, lp);
  hipLaunchKernelGGL(boundary_loss_segments, grid, dim3(256), 0, st, lp);
  hipLaunchKernelGGL(boundary_loss_runs, grid, dim3(256), 0, st, lp);
  hipLaunchKernelGGL(boundary_loss_grad, grid, dim3(256), 0, st, lp);
  return hipGetLastError();
}

}  // namespace kvpop
