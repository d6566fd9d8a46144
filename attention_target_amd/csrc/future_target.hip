// Transposed-attention future target for gfx950.
//
// KVpop paper, Section 3.2 ("Transposed-attention target computation",
// Eq. 8): the future mass of key t is a reduction over the column t of the
// attention matrix, ln sum_{d >= t+w} exp(s_{d,t} - L_d), evaluated with keys
// in the role of queries.  Section 3.1 (Eqs. 2-3) turns the per-query-head
// masses into the target (mean over the N_t future queries, epsilon, max or
// sum over the query heads of a KV head).
//
// Work decomposition
//  * A block is (batch row, KV head, document, key tile of 256 keys, query
//    chunk of DT queries).  Its four waves each keep 64 keys of K resident in
//    registers (the MFMA A operand) for the whole block; when that grid would
//    be small (short sequences), blocks of 128 keys, 32 per wave, instead.
//  * Query tiles of 64 positions stream through double-buffered, swizzled
//    LDS together with -L_d/scale (precomputed once per call by a small
//    elementwise kernel).  The tiles are fetched by buffer loads that write
//    straight into LDS, with the swizzle folded into each lane's source
//    offset, so no registers or LDS stores are spent on staging.  For every
//    query head of the group each wave computes S = Q K^T (32 queries x 64
//    keys per half tile) with MFMA.  The MFMA addend is -L_d/scale, so the
//    accumulator is q_d.k_t - L_d/scale and the exp2 argument is that times
//    scale*log2(e): per element a multiply, exp2 and one add into the
//    per-lane sum of the lane's key remain on the VALU.  (Folding the scale
//    into K instead would save the multiply, but rounding scale*K to bf16
//    perturbs each logit by up to 2^-9 of sum_i |q_i k_i| * scale, e.g.
//    0.04 nats at logits near 30.)  No running max is needed: with the dense
//    normaliser s_{d,t} <= L_d.
//  * The masks d >= t + w and "inside the document" are applied only on the
//    sub-tiles that cross them.
//  * At the end the two halves of each wave add their sums (one shuffle)
//    and write one partial per key and query chunk into the workspace; a
//    second small kernel adds the chunks in a fixed order, applies the mean,
//    epsilon and the aggregation over query heads, and takes the log.  There
//    are no atomics, so results are bitwise reproducible.
//  * Blocks are ordered (batch, KV head, document, chunk descending, key tile)
//    and dealt out so that each XCD (one L2) receives a contiguous range:
//    concurrently running blocks of an XCD share the same query chunk.
//    When B*Hkv is a multiple of 8, every XCD receives whole sequences, and
//    a table written before the launch orders its blocks by size, largest
//    first (longest-processing-time order): the last round then holds the
//    small blocks on the diagonal, not a full-size block started late.
#include <mutex>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace kvpop {

// Keys per wave come in 32-key column blocks (NCB of them): two (256 keys per
// block) when the grid is large, one (128 keys, twice the blocks) when it
// would otherwise leave the GPU partly idle.
constexpr int TGT_SMALL_GRID = 2048;  // blocks below which NCB = 1 is used
template <int NCB>
constexpr int tgt_kt() { return 4 * 32 * NCB; }  // keys per block: 4 waves

struct TgtParams {
  const void *q, *k;
  const float *nl;  // -L/scale per query, [B, Hq, S]
  float *part;
  int B, S, Hq, Hkv, G, window;
  float scale_log2;
  const int *cu;
  int n_docs;
  int DT, nch_max, blocks_per_seq, total_blocks, Hp, kt;
  const unsigned long long *order;  // per-XCD block order (see TgtOrder), or nullptr
  int sx;                           // sequences per XCD when `order` is set
};

// Number of key tiles of a document of length n that meet query chunk j.
__host__ __device__ __forceinline__ int tgt_tiles_in_chunk(int n, int j, int DT, int w, int KT) {
  const int qend = min(n, (j + 1) * DT) - 1;
  if (qend - w < 0) return 0;
  return min((n + KT - 1) / KT, (qend - w) / KT + 1);
}
__host__ __device__ __forceinline__ int tgt_blocks_in_doc(int n, int DT, int w, int KT) {
  const int nch = (n + DT - 1) / DT;
  int c = 0;
  for (int j = 0; j < nch; ++j) c += tgt_tiles_in_chunk(n, j, DT, w, KT);
  return c;
}
// Size of a block in 32-query halves: the rows of its chunk [cq0, cq1) from
// the 32-aligned row where its first key's future begins (the rows its first
// wave computes).
__host__ __device__ __forceinline__ int tgt_block_halves(int cq0, int cq1, int first_future) {
  const int qs = max(cq0, first_future);
  return (cq1 - (cq0 + ((qs - cq0) & ~31)) + 31) / 32;
}

// Block order within an XCD.  Each XCD runs sx = B*Hkv/8 whole sequences,
// sx * blocks_per_seq blocks, taken largest first: by size in halves
// (descending), then by sequence, then in enumeration order (document,
// chunk descending, key tile).  Sizes within one (document, chunk) group
// never rise with the key tile, so blocks of one size are contiguous there.
// Sorting every block by size has a cost in memory traffic: each size class
// spans all chunks, so the diagonal blocks re-read their queries from
// memory instead of sharing them in L2 with the full blocks of their chunk
// (the target's HBM bytes at S=16384 rise 1.6x, to about 0.65 TB/s, far from
// the HBM roof).  Moving only the blocks of at most a quarter chunk to the
// end kept the traffic but not the shorter last round.
// Entry = tile | chunk << 16 | sequence << 32 | document << 48.  The table is
// the same for every XCD and is written by the first workgroup of
// future_target_neg_lse, which runs before the target kernel on the stream.
constexpr int TGT_ORDER_MAX_GROUPS = 64;           // (document, chunk) groups per sequence: one per lane
struct TgtOrder {
  unsigned long long *order;  // [cap = sx * blocks_per_seq], or nullptr: no table
  int cap;                    // entries; the builder writes none past it
  const int *cu;
  int n_docs, S, DT, window, KT, sx, n_groups;
};

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  return v;
}

// Written by the four waves of one workgroup without LDS (which the host
// kernel's other workgroups would then reserve too): lane g of every wave
// owns group g (at most 64 groups, checked on the host); per-class prefixes
// over the groups and the class bases are wave scans.  Each wave computes
// the same positions and writes a quarter of the entries.
constexpr int TGT_ORDER_MAX_DIAG = 1024 / 128 + 1;  // tiles past the full ones in a group: <= DT/KT + 1
__device__ void tgt_build_order(const TgtOrder &o) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // documents (lane d): length and first group; groups run document by
  // document, chunks descending
  int dl = 0, dc = 0;
  if (lane < o.n_docs) {
    dl = o.cu != nullptr ? o.cu[lane + 1] - o.cu[lane] : o.S;
    dc = dl > 0 ? (dl + o.DT - 1) / o.DT : 0;
  }
  const int dg = wave_incl_scan(dc) - dc;
  // this lane's group: the last non-empty document whose first group is <= lane
  int m = -1, mlen = 0, mdg = 0;
  for (int d = 0; d < o.n_docs; ++d) {
    const int gd = __shfl(dg, d), ld = __shfl(dl, d);
    if (gd <= lane && ld > 0) {
      m = d;
      mlen = ld;
      mdg = gd;
    }
  }
  int j = m >= 0 ? (mlen + o.DT - 1) / o.DT - 1 - (lane - mdg) : -1;
  const bool valid = lane < o.n_groups && m >= 0 && j >= 0;  // else: offsets disagree with the host's
  int cq0 = 0, cq1 = 0, nt = 0, nfull = 0, cf = -1;
  if (valid) {
    cq0 = j * o.DT;
    cq1 = min(mlen, cq0 + o.DT);
    nt = tgt_tiles_in_chunk(mlen, j, o.DT, o.window, o.KT);
    // a tile is full (its block starts at the chunk's first row) when its
    // first future row t0 + w is at most cq0 + 31: the first nfull tiles, all
    // of one size; the others each have a size of their own
    const int lim = cq0 + 31 - o.window;
    nfull = lim < 0 ? 0 : min(nt, lim / o.KT + 1);
    cf = nfull > 0 ? tgt_block_halves(cq0, cq1, cq0) : -1;
  }
  const int nd = min(nt - nfull, TGT_ORDER_MAX_DIAG);
  int dcls[TGT_ORDER_MAX_DIAG];
#pragma unroll
  for (int k = 0; k < TGT_ORDER_MAX_DIAG; ++k)
    dcls[k] = k < nd ? tgt_block_halves(cq0, cq1, (nfull + k) * o.KT + o.window) : -1;
  // classes from the largest down: the running base is the number of
  // entries of all larger classes.  Only the classes some group holds are
  // scanned (a few of the DT/32 sizes): each scan is a chain of cross-lane
  // steps.
  int basec = 0, pos_f = 0, tot_f = 0;  // the host keeps the table below 2^31 entries
  int pos_d[TGT_ORDER_MAX_DIAG], tot_d[TGT_ORDER_MAX_DIAG];
#pragma unroll
  for (int k = 0; k < TGT_ORDER_MAX_DIAG; ++k) pos_d[k] = tot_d[k] = 0;
  unsigned long long held = cf > 0 ? 1ull << cf : 0ull;  // classes are 1 .. DT/32 <= 32
#pragma unroll
  for (int k = 0; k < TGT_ORDER_MAX_DIAG; ++k) held |= dcls[k] > 0 ? 1ull << dcls[k] : 0ull;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) held |= __shfl_xor(held, d);
  unsigned long long todo = ((unsigned long long)__builtin_amdgcn_readfirstlane((unsigned)(held >> 32)) << 32) |
                            (unsigned)__builtin_amdgcn_readfirstlane((unsigned)held);
  while (todo != 0ull) {
    const int c = 63 - __builtin_clzll(todo);
    todo &= ~(1ull << c);
    int v = c == cf ? nfull : 0;
#pragma unroll
    for (int k = 0; k < TGT_ORDER_MAX_DIAG; ++k) v += dcls[k] == c ? 1 : 0;
    const int incl = wave_incl_scan(v);
    const int tot = __shfl(incl, 63);
    const int at = basec + (incl - v);
    if (c == cf) {
      pos_f = at;
      tot_f = tot;
    }
#pragma unroll
    for (int k = 0; k < TGT_ORDER_MAX_DIAG; ++k)
      if (dcls[k] == c) {
        pos_d[k] = at;
        tot_d[k] = tot;
      }
    basec += o.sx * tot;
  }
  if (!valid) return;
  // (positions past cap arise only when the device offsets describe more
  // blocks than the host's copy; those entries are dropped)
  const unsigned long long gbits = ((unsigned long long)j << 16) | ((unsigned long long)m << 48);
  for (int sq = 0; sq < o.sx; ++sq) {
    for (int r = wave; r < nfull; r += 4) {
      const int at = pos_f + sq * tot_f + r;
      if (at < o.cap) o.order[at] = gbits | (unsigned)r | ((unsigned long long)sq << 32);
    }
#pragma unroll
    for (int k = 0; k < TGT_ORDER_MAX_DIAG; ++k)
      if (k < nd && (k & 3) == wave) {
        const int at = pos_d[k] + sq * tot_d[k];
        if (at < o.cap) o.order[at] = gbits | (unsigned)(nfull + k) | ((unsigned long long)sq << 32);
      }
  }
}

// -L/scale for every query (mul = -1/scale): the MFMA addend of the target
// kernel, in the units of the raw logits q.k.  With a block-order table to
// write, the first workgroup writes it and the others shift by one.
__global__ void __launch_bounds__(256) future_target_neg_lse(const float *lse, float *nl, float mul, size_t count,
                                                             const TgtOrder o) {
  if (o.order != nullptr && blockIdx.x == 0) {
    tgt_build_order(o);
    return;
  }
  const size_t i = (size_t)(blockIdx.x - (o.order != nullptr ? 1 : 0)) * 256 + threadIdx.x;
  if (i < count) nl[i] = lse[i] * mul;
}

// Waves per SIMD the register budget is cut to: three for bf16; the fp32
// correctness path at D=128 needs more registers and runs two.
template <typename T, int D>
constexpr int tgt_waves() { return (sizeof(T) == 2 || D == 64) ? 3 : 2; }

template <typename T, int D, bool SUM_HEADS, int NCB>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(tgt_waves<T, D>()))) future_target_kernel(const TgtParams p) {
  constexpr int KT = tgt_kt<NCB>();
  using QTile = SwizzledTile<T, D>;
  constexpr int NJ = D / 16;
  constexpr int QT = 64;                                // queries per LDS stage
  constexpr int ROWB = D * (int)sizeof(T);              // bytes per query row
  constexpr int QBYTES = QT * ROWB;
  constexpr int LOADS = QBYTES / 1024 / 4;              // 1 KB direct loads per wave and stage
  static_assert(QBYTES % 4096 == 0 && LOADS >= 1, "stage must split into 1 KB loads per wave");

  __shared__ __align__(16) char q_lds[2][QBYTES];
  __shared__ __align__(16) float nl_lds[2][QT];

  // ---- which block ----
  const int per_xcd = (p.total_blocks + 7) / 8;
  const int v = ((int)blockIdx.x % 8) * per_xcd + (int)blockIdx.x / 8;
  if (v >= p.total_blocks) return;
  int bh, r, j, dstart = 0, n = p.S;
  if (p.order != nullptr) {
    // the grid is exactly 8 * sx * blocks_per_seq: entry blockIdx/8 of the table
    const unsigned long long e = p.order[blockIdx.x / 8];
    r = (int)(e & 0xffff);
    j = (int)((e >> 16) & 0xffff);
    const int sq = (int)((e >> 32) & 0xffff), m = (int)(e >> 48);
    if (sq >= p.sx || m >= p.n_docs) return;
    bh = ((int)blockIdx.x % 8) * p.sx + sq;
    if (p.cu != nullptr) {
      dstart = p.cu[m];
      n = p.cu[m + 1] - dstart;
    }
    if (n <= 0 || dstart < 0 || dstart + n > p.S) return;  // host and device offsets disagree
    const int nch = (n + p.DT - 1) / p.DT;
    if (nch > p.nch_max || j >= nch || r >= tgt_tiles_in_chunk(n, j, p.DT, p.window, KT)) return;
  } else {
    bh = v / p.blocks_per_seq;
    r = v % p.blocks_per_seq;
    bool found = false;
    for (int m = 0; m < p.n_docs; ++m) {
      if (p.cu != nullptr) {
        dstart = p.cu[m];
        n = p.cu[m + 1] - dstart;
      }
      const int cnt = tgt_blocks_in_doc(n, p.DT, p.window, KT);
      if (r < cnt) {
        found = true;
        break;
      }
      r -= cnt;
    }
    if (!found || n <= 0 || dstart < 0 || dstart + n > p.S) return;  // host and device offsets disagree
    const int nch = (n + p.DT - 1) / p.DT;
    if (nch > p.nch_max) return;
    j = nch - 1;
    for (; j >= 0; --j) {
      const int nt = tgt_tiles_in_chunk(n, j, p.DT, p.window, KT);
      if (r < nt) break;
      r -= nt;
    }
    if (j < 0) return;
  }
  const int b = bh / p.Hkv, h = bh % p.Hkv;
  const int t0 = r * KT;  // doc-local first key of the block

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hf = lane >> 5;
  const int tw = t0 + 32 * NCB * wave;  // doc-local first key of this wave
  const int w = p.window;

  // ---- resident K fragments (B operand) ----
  // S = Q K^T puts queries on the rows (registers) and keys on the columns
  // (lanes), so every lane accumulates the column sum of one key.  With the
  // MFMA addend holding -L_d/scale, the accumulator times scale*log2(e) is
  // the exp2 argument s_{d,t}*log2(e) - L_d*log2(e).
  const T *kbase = reinterpret_cast<const T *>(p.k) + ((size_t)b * p.Hkv + h) * (size_t)p.S * D;
  Frag<T> kf[NCB][NJ];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int key = min(tw + 32 * cb + col, n - 1);
    const T *kr = kbase + (size_t)(dstart + key) * D + 8 * hf;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      load_frag(kf[cb][jj], kr + 16 * jj);
    }
  }

  // ---- query stages of this chunk: 64 rows each, from qs_al (32-aligned) ----
  const int cq0 = j * p.DT, cq1 = min(n, (j + 1) * p.DT);
  const int qs = max(cq0, t0 + w);
  const int qs_al = cq0 + ((qs - cq0) & ~31);
  const int n_st = (cq1 - qs_al + QT - 1) / QT;
  const int n_it = p.G * n_st;

  float acc[NCB][2];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb][0] = acc[cb][1] = 0.f;

  // Direct-to-LDS loads: load k of this wave fills LDS chunks
  // [(wave*LOADS + k)*64, +64) of a stage, lane by lane.  Each lane fetches
  // the global chunk that the swizzle places at its LDS chunk.
  auto src_off = [&](int k) {
    const int pch = (wave * LOADS + k) * 64 + lane;  // LDS chunk index in the stage
    const int row = pch / QTile::kChunks, slot = pch % QTile::kChunks;
    return row * ROWB + ((slot ^ QTile::swz(row)) << 4);
  };
  int a_off[NJ];  // bf16: this lane's A-operand chunks (query row `col`)
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) a_off[jj] = QTile::off(col, 2 * jj + hf);
  auto read_a = [&](Frag<T> &a, const char *base, int jj) {
    if constexpr (sizeof(T) == 2) QTile::read_at(a, base, a_off[jj]);
    else QTile::read(a, base, col, 16 * jj + 8 * hf);
  };

  auto q_of = [&](int it, int &gg, int &q0) {
    gg = it / n_st;
    q0 = qs_al + QT * (it % n_st);
  };
  // Starts the loads of stage `it` (64 rows of one head and their -L/scale)
  // into LDS buffer `buf`.  The buffers end at the document end, so rows past
  // it arrive as zeros; they are masked out below.
  auto fetch = [&](auto bufc, int it) {
    constexpr int buf = decltype(bufc)::value;
    int gg, q0;
    q_of(it, gg, q0);
    const int g = h * p.G + gg;
    const int rows = min(QT, n - q0);
    const size_t row0 = ((size_t)b * p.Hq + g) * p.S + dstart + q0;
    const auto qr = make_rsrc(reinterpret_cast<const T *>(p.q) + row0 * D, rows * ROWB);
#pragma unroll
    for (int k = 0; k < LOADS; ++k) lds_load16(qr, q_lds[buf] + (wave * LOADS + k) * 1024, src_off(k));
    if (wave == 0) lds_load4(make_rsrc(p.nl + row0, rows * 4), nl_lds[buf], lane * 4);
  };
  auto write_partial = [&](int hp) {
    // the two lane halves hold complementary query rows of the same key
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      float tot = acc[cb][0] + acc[cb][1];
      tot += __shfl_xor(tot, 32);
      const int key = tw + 32 * cb + col;
      if (hf == 0 && key < n) p.part[(((size_t)b * p.Hp + hp) * p.nch_max + j) * p.S + dstart + key] = tot;
      acc[cb][0] = acc[cb][1] = 0.f;
    }
  };
  // One half stage: 32 query rows starting at row `h32` of the stage.
  const float cs = p.scale_log2;
  // LDS addresses for the asm reads: this lane's Q chunks and its addend
  // quarter, relative to buffer 0 / half 0 (the rest is an immediate)
  unsigned a_abs[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) a_abs[jj] = (unsigned)(size_t)&q_lds[0][0] + a_off[jj];
  const unsigned nl_abs = (unsigned)(size_t)&nl_lds[0][0] + 16 * hf;
  auto half = [&](auto bufc, auto hhc, int q0) {
    constexpr int buf = decltype(bufc)::value, hh = decltype(hhc)::value;
    const char *ql = q_lds[buf] + 32 * hh * ROWB;
    const float *nl = nl_lds[buf] + 32 * hh;
    f32x16 s[NCB];
    if constexpr (sizeof(T) == 2 && NJ % 4 == 0) {
      // The reads are asm: through ordinary loads the compiler cannot tell
      // them from the next stage's direct-to-LDS loads in flight and waits
      // for all of those first.  Each asm block waits for its own reads
      // before it ends (its outputs are never in flight outside it): the
      // first brings the addends and the Q chunks of k-steps 0..3, the second
      // those of k-steps 4..7 while the first group's MFMAs run.  Outputs are
      // early-clobber: a block issues several reads, so no result register
      // may share a register with an address not yet consumed.
      constexpr int QO = buf * QBYTES + 32 * hh * ROWB;
      constexpr int NO = (buf * QT + 32 * hh) * 4;
      f32x4 nv[4];
      Frag<T> a[4];
      asm volatile(
          "ds_read_b128 %0, %8 offset:%13\n\t"
          "ds_read_b128 %1, %8 offset:%14\n\t"
          "ds_read_b128 %2, %8 offset:%15\n\t"
          "ds_read_b128 %3, %8 offset:%16\n\t"
          "ds_read_b128 %4, %9 offset:%17\n\t"
          "ds_read_b128 %5, %10 offset:%17\n\t"
          "ds_read_b128 %6, %11 offset:%17\n\t"
          "ds_read_b128 %7, %12 offset:%17\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(nv[0]), "=&v"(nv[1]), "=&v"(nv[2]), "=&v"(nv[3]), "=&v"(a[0].v), "=&v"(a[1].v), "=&v"(a[2].v),
            "=&v"(a[3].v)
          : "v"(nl_abs), "v"(a_abs[0]), "v"(a_abs[1]), "v"(a_abs[2]), "v"(a_abs[3]), "i"(NO), "i"(NO + 32),
            "i"(NO + 64), "i"(NO + 96), "i"(QO)
          : "memory");
      // accumulators start at -L/scale of the query row held by each register
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
#pragma unroll
          for (int e = 0; e < 4; ++e) s[cb][4 * i4 + e] = nv[i4][e];
#pragma unroll
      for (int j4 = 0; j4 < NJ; j4 += 4) {
        if (j4 > 0) {
          asm volatile(
              "ds_read_b128 %0, %4 offset:%8\n\t"
              "ds_read_b128 %1, %5 offset:%8\n\t"
              "ds_read_b128 %2, %6 offset:%8\n\t"
              "ds_read_b128 %3, %7 offset:%8\n\t"
              "s_waitcnt lgkmcnt(0)"
              : "=&v"(a[0].v), "=&v"(a[1].v), "=&v"(a[2].v), "=&v"(a[3].v)
              : "v"(a_abs[j4]), "v"(a_abs[j4 + 1]), "v"(a_abs[j4 + 2]), "v"(a_abs[j4 + 3]), "i"(QO)
              : "memory");
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) mma(s[cb], a[jj], kf[cb][j4 + jj]);
      }
    } else {
      // accumulators start at -L/scale of the query row held by each
      // register (read twice from LDS rather than kept in a third tile)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 v4 = *reinterpret_cast<const f32x4 *>(&nl[8 * i4 + 4 * hf]);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[cb][4 * i4 + e] = v4[e];
        }
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        Frag<T> a;
        read_a(a, ql, jj);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) mma(s[cb], a, kf[cb][jj]);
      }
    }
    const int tlast = tw + 32 * NCB - 1;
    const bool interior = (q0 >= tlast + w) && (q0 + 31 < n) && (tlast < n);
    if (interior) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[cb][i & 1] += fast_exp2(s[cb][i] * cs);
    } else {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int t = tw + 32 * cb + col;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int d = q0 + c_row(i, hf);
          const float pv = fast_exp2(s[cb][i] * cs);
          acc[cb][i & 1] += (d >= t + w && d < n && t < n) ? pv : 0.f;
        }
      }
    }
  };
  // One stage: wait for this wave's loads of stage `it`, publish them with a
  // barrier (which also retires every read of the other buffer), start the
  // loads of stage it+1 into the other buffer, then compute on this one.
  auto step = [&](auto bufc, int it) {
    constexpr int buf = decltype(bufc)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (it + 1 < n_it) fetch(std::integral_constant<int, 1 - buf>{}, it + 1);

    int gg, q0;
    q_of(it, gg, q0);
    static_for<2>([&](auto hhc) {
      const int qh = q0 + 32 * decltype(hhc)::value;
      // the half must meet a key of this wave and lie inside the chunk
      if (qh < cq1 && qh + 31 >= tw + w && tw < n) half(bufc, hhc, qh);
    });
    if constexpr (!SUM_HEADS) {
      if ((it + 1) % n_st == 0) write_partial(h * p.G + gg);
    }
  };

  fetch(std::integral_constant<int, 0>{}, 0);
  for (int it = 0; it < n_it; it += 2) {
    step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < n_it) step(std::integral_constant<int, 1>{}, it + 1);
  }
  if constexpr (SUM_HEADS) write_partial(h);
}

struct FinParams {
  const float *part;
  float *out;
  int B, S, Hq, Hkv, G, window, DT, nch_max, Hp, Hout, agg, mean, kt;
  float eps;
  const int *cu;
  int n_docs;
};

__global__ void __launch_bounds__(256) future_target_finalize(const FinParams p) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= p.S) return;
  const int ho = blockIdx.y, b = blockIdx.z;
  const Doc dd = find_doc(p.cu, p.n_docs, p.S, t);
  const int n = dd.end - dd.start, pos = t - dd.start;
  const int N = max(0, n - pos - p.window);
  const int fq = (pos / p.kt) * p.kt + p.window;
  const int nch = (n + p.DT - 1) / p.DT;
  const int jlo = (fq <= n - 1) ? fq / p.DT : nch;
  const float scale = p.mean ? (N > 0 ? 1.f / (float)N : 0.f) : 1.f;
  // the chunks are added in index order; their loads are issued eight at a
  // time (one after the other, each add would wait for its own load)
  auto mass = [&](int hp) {
    const float *pp = p.part + ((size_t)b * p.Hp + hp) * p.nch_max * (size_t)p.S + t;
    float s = 0.f;
    int jj = jlo;
    for (; jj + 8 <= nch; jj += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = pp[(size_t)(jj + u) * p.S];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; jj < nch; ++jj) s += pp[(size_t)jj * p.S];
    return s * scale;
  };
  float y;
  if (p.agg == 0) {
    y = logf(mass(ho) + p.eps);
  } else if (p.agg == 1) {
    y = -INFINITY;
    for (int gg = 0; gg < p.G; ++gg) y = fmaxf(y, logf(mass(ho * p.G + gg) + p.eps));
  } else {
    y = logf(mass(ho) + p.eps);
  }
  p.out[((size_t)b * p.Hout + ho) * p.S + t] = y;
}

// ---------------------------------------------------------------------------
// host side

int tgt_chunk(int max_doc) {
  if (max_doc <= 4096) return 192;
  if (max_doc <= 8192) return 512;
  return 1024;
}

// Workspace: per-chunk partial sums [B, Hp, n_chunks, S] (Hp = Hkv for the
// SUM aggregation, which adds a group's query heads inside the kernel, else
// Hq), then the normaliser in logit units -L/scale [B, Hq, S], then (at a
// 256-byte boundary) the block-order table when one is used.  Every value
// the kernels read is written by the same call, so the workspace needs no
// clearing.
static size_t tgt_partial_floats(const ShapeInfo &s, int Hp) {
  const int DT = tgt_chunk(s.max_doc);
  const size_t nch_max = (size_t)((s.max_doc + DT - 1) / DT);
  return (size_t)s.B * Hp * nch_max * s.S;
}
static int tgt_partial_heads(const ShapeInfo &s, int agg) { return agg == 0 ? s.Hkv : s.Hq; }
// (document, chunk) groups of one sequence
static long long tgt_groups(const ShapeInfo &s, int DT) {
  if (s.cu_host == nullptr) return (s.S + DT - 1) / DT;
  long long g = 0;
  for (int m = 0; m < s.n_docs; ++m) g += (s.cu_host[m + 1] - s.cu_host[m] + DT - 1) / DT;
  return g;
}
// Blocks of one sequence for any window and key tile (the most: w = 0,
// 128-key tiles).
static long long tgt_blocks_bound(const ShapeInfo &s) {
  const int DT = tgt_chunk(s.max_doc);
  long long per_seq = 0;
  if (s.cu_host != nullptr) {
    for (int m = 0; m < s.n_docs; ++m) per_seq += tgt_blocks_in_doc(s.cu_host[m + 1] - s.cu_host[m], DT, 0, tgt_kt<1>());
  } else {
    per_seq = tgt_blocks_in_doc(s.S, DT, 0, tgt_kt<1>());
  }
  return per_seq;
}
// Whether the blocks run in the size order of a table: every XCD must get
// whole sequences, and the groups, the builder's 16-bit counts and the entry
// fields must fit.
static bool tgt_ordered(const ShapeInfo &s) {
  const int DT = tgt_chunk(s.max_doc);
  const long long nseq = (long long)s.B * s.Hkv;
  return nseq % 8 == 0 && nseq / 8 < 65536 && s.n_docs <= TGT_ORDER_MAX_GROUPS && (s.cu == nullptr) == (s.cu_host == nullptr) &&
         DT <= 1024 && tgt_groups(s, DT) <= TGT_ORDER_MAX_GROUPS && tgt_blocks_bound(s) < 65536 &&
         nseq / 8 * tgt_blocks_bound(s) < 2147483647ll;
}
// Bytes of the table for any window and key tile, plus the alignment.
static size_t tgt_order_bytes(const ShapeInfo &s) {
  if (!tgt_ordered(s)) return 0;
  return 256 + sizeof(unsigned long long) * (size_t)((long long)s.B * s.Hkv / 8) * (size_t)tgt_blocks_bound(s);
}
static size_t tgt_base_bytes(const ShapeInfo &s, int Hp) {
  return (tgt_partial_floats(s, Hp) + (size_t)s.B * s.Hq * s.S) * sizeof(float);
}
size_t tgt_workspace_bytes(const ShapeInfo &s) { return tgt_base_bytes(s, s.Hq) + tgt_order_bytes(s); }
size_t tgt_workspace_bytes_for(const ShapeInfo &s, int agg) {
  return tgt_base_bytes(s, tgt_partial_heads(s, agg)) + tgt_order_bytes(s);
}

// Scratch of the no-allocation entry point (kvpop_future_target_noalloc):
// one array per GPU, held until the process ends.  Host code never passes
// the array's name to a kernel (on the host it only stands for the symbol):
// each device's address comes from hipGetSymbolAddress, looked up once per
// device with that device current, and kernels receive that address.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void **out) {
  static std::mutex mu;
  static void *addr[kMaxScratchDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

template <typename T, int D, bool SUM>
static hipError_t launch_tgt(const TgtParams &tp, int grid, hipStream_t st) {
  if (tp.kt == tgt_kt<1>())
    hipLaunchKernelGGL((future_target_kernel<T, D, SUM, 1>), dim3(grid), dim3(256), 0, st, tp);
  else
    hipLaunchKernelGGL((future_target_kernel<T, D, SUM, 2>), dim3(grid), dim3(256), 0, st, tp);
  return hipGetLastError();
}

long long tgt_grid_blocks(const ShapeInfo &s, int window) {
  const int DT = tgt_chunk(s.max_doc);
  auto count = [&](int KT) {
    long long c = 0;
    if (s.cu_host != nullptr) {
      for (int m = 0; m < s.n_docs; ++m) c += tgt_blocks_in_doc(s.cu_host[m + 1] - s.cu_host[m], DT, window, KT);
    } else {
      c = tgt_blocks_in_doc(s.S, DT, window, KT);
    }
    return c * s.B * s.Hkv;
  };
  const long long big = count(tgt_kt<2>());
  return big < TGT_SMALL_GRID ? count(tgt_kt<1>()) : big;
}

hipError_t launch_future_target(const ShapeInfo &s, const void *q, const void *k, const float *lse,
                                int window, int agg, int mean, float eps, float *target,
                                void *ws, hipStream_t st) {
  TgtParams tp{};
  tp.q = q;
  tp.k = k;
  tp.part = reinterpret_cast<float *>(ws);
  float *nl = tp.part + tgt_partial_floats(s, tgt_partial_heads(s, agg));
  tp.nl = nl;
  tp.B = s.B;
  tp.S = s.S;
  tp.Hq = s.Hq;
  tp.Hkv = s.Hkv;
  tp.G = s.Hq / s.Hkv;
  tp.window = window;
  tp.scale_log2 = s.scale * kLog2e;
  tp.cu = s.cu;
  tp.n_docs = s.n_docs;
  tp.DT = tgt_chunk(s.max_doc);
  tp.nch_max = (s.max_doc + tp.DT - 1) / tp.DT;
  auto blocks_per_seq = [&](int KT) {
    long long c = 0;
    if (s.cu_host != nullptr) {
      for (int m = 0; m < s.n_docs; ++m) c += tgt_blocks_in_doc(s.cu_host[m + 1] - s.cu_host[m], tp.DT, window, KT);
    } else {
      c = tgt_blocks_in_doc(s.S, tp.DT, window, KT);
    }
    return c;
  };
  tp.kt = tgt_kt<2>();
  long long per_seq = blocks_per_seq(tp.kt);
  if (per_seq * s.B * s.Hkv < TGT_SMALL_GRID) {
    tp.kt = tgt_kt<1>();
    per_seq = blocks_per_seq(tp.kt);
  }
  if (per_seq * s.B * s.Hkv > kMaxGridBlocks) return hipErrorInvalidConfiguration;  // rejected by the ABI first
  tp.blocks_per_seq = (int)per_seq;
  tp.total_blocks = (int)(per_seq * s.B * s.Hkv);
  const bool sum = (agg == 0);
  tp.Hp = tgt_partial_heads(s, agg);
  TgtOrder ord{};
  if (tgt_ordered(s)) {
    const size_t off = (tgt_base_bytes(s, tp.Hp) + 255) & ~(size_t)255;
    ord.order = reinterpret_cast<unsigned long long *>(reinterpret_cast<char *>(ws) + off);
    ord.cu = s.cu;
    ord.n_docs = s.n_docs;
    ord.S = s.S;
    ord.DT = tp.DT;
    ord.window = window;
    ord.KT = tp.kt;
    ord.sx = s.B * s.Hkv / 8;
    ord.n_groups = (int)tgt_groups(s, tp.DT);
    ord.cap = ord.sx * tp.blocks_per_seq;
    tp.order = ord.order;
    tp.sx = ord.sx;
  }
  hipError_t e = hipSuccess;
  if (tp.total_blocks > 0) {
    const size_t count = (size_t)s.B * s.Hq * s.S;
    const float mul = (float)(-1.0 / (double)s.scale);
    const unsigned nl_blocks = (unsigned)((count + 255) / 256) + (ord.order != nullptr ? 1u : 0u);
    hipLaunchKernelGGL(future_target_neg_lse, dim3(nl_blocks), dim3(256), 0, st, lse, nl, mul, count, ord);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int grid = 8 * ((tp.total_blocks + 7) / 8);
    if (s.dtype == 0 && s.D == 128) e = sum ? launch_tgt<bf16, 128, true>(tp, grid, st) : launch_tgt<bf16, 128, false>(tp, grid, st);
    else if (s.dtype == 0 && s.D == 64) e = sum ? launch_tgt<bf16, 64, true>(tp, grid, st) : launch_tgt<bf16, 64, false>(tp, grid, st);
    else if (s.dtype == 1 && s.D == 64) e = sum ? launch_tgt<float, 64, true>(tp, grid, st) : launch_tgt<float, 64, false>(tp, grid, st);
    else if (s.dtype == 1 && s.D == 128) e = sum ? launch_tgt<float, 128, true>(tp, grid, st) : launch_tgt<float, 128, false>(tp, grid, st);
    else return hipErrorInvalidValue;
    if (e != hipSuccess) return e;
  }
  FinParams fp{};
  fp.part = tp.part;
  fp.out = target;
  fp.B = s.B;
  fp.S = s.S;
  fp.Hq = s.Hq;
  fp.Hkv = s.Hkv;
  fp.G = tp.G;
  fp.window = window;
  fp.DT = tp.DT;
  fp.kt = tp.kt;
  fp.nch_max = tp.nch_max;
  fp.Hp = tp.Hp;
  fp.Hout = (agg == 2) ? s.Hq : s.Hkv;
  fp.agg = agg;
  fp.mean = mean;
  fp.eps = eps;
  fp.cu = s.cu;
  fp.n_docs = s.n_docs;
  hipLaunchKernelGGL(future_target_finalize, dim3((s.S + 255) / 256, fp.Hout, s.B), dim3(256), 0, st, fp);
  return hipGetLastError();
}

}  // namespace kvpop
