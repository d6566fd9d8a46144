// Attention forward with log-sum-exp for gfx950: dense causal (packed
// documents allowed) and budget-masked sparse variants.
//
// Dense:  L_d = ln sum_{t<=d, same doc} exp(s_{d,t}), O_d = sum_t exp(s-L) v_t
//         (the causal normaliser of the KVpop paper, Section 3.2).
// Sparse: the same over the per-KV-head budget mask of Section 3 / 3.2
//         (sinks, protected window, running top-k by static rank), reading
//         only the keys listed for the query block; each listed key carries
//         the span [lo, hi) of query positions that keep it.
//
// Work decomposition: one workgroup = 4 waves = one block of QB query
// positions x HG query heads of one KV head (HG = min(G, 4), QB = 32*4/HG), so
// each K/V tile brought to LDS serves every query head of the group.  Each
// wave owns 32 queries of one head and computes S^T = K Q^T with MFMA: a lane
// then owns one query column, so the online-softmax max and sum are reductions
// over the lane's registers plus one exchange with the other lane half.  P^T
// (bf16) is directly the B operand of O^T = V^T P^T.  V stays in its natural
// row layout in LDS and the V^T operand is gathered with gfx950's transposed
// LDS reads.  K/V tiles are double-buffered (one barrier per tile), the
// softmax scale is folded into the exp2 argument, and row maxima are formed
// only for tiles whose exponentials against the running maximum could exceed
// a fixed bound (then the running output is rescaled).
#pragma once

#include "common.h"

namespace kvpop {

struct FwdParams {
  const void *q, *k, *v;
  void *o;
  float *lse;
  int B, S, Hq, Hkv, G, HG;
  float scale_log2;  // softmax scale * log2(e)
  const int *cu;
  int n_docs;
  // budget-masked mode
  const int *lists;     // [B*Hkv][nqb][list_cap] key positions (two segments, see budget_lists)
  const int2 *spans;    // [B*Hkv][nqb][list_cap]: per listed key, the queries [lo, hi) that keep it
  const int *list_len;       // [B*Hkv][nqb]
  const int *list_len_full;  // [B*Hkv][nqb]: leading entries kept by every query of the block
  int list_cap;
  const int *qorder;  // [B*Hkv][nqb]: the order in which query blocks run (packed documents), or nullptr
};

#ifndef KVPOP_FWD_KT
#define KVPOP_FWD_KT 32
#endif
#ifndef KVPOP_FWD_WAVES
#define KVPOP_FWD_WAVES 3
#endif

template <typename T, int D>
struct FwdTiles {
  static constexpr int KT = KVPOP_FWD_KT;                 // keys per tile
  static constexpr int EPC = 16 / (int)sizeof(T);         // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;                     // 16-byte chunks per row
  static constexpr int ROWB = D * (int)sizeof(T);         // bytes per row
  static constexpr int K_BYTES = KT * ROWB;
  static constexpr int STAGE = 2 * K_BYTES;               // K tile, then V tile
  static constexpr int LOADS = K_BYTES / 4096;            // 1 KB direct loads per wave and tensor
  static_assert(KT * CPR % 256 == 0 && K_BYTES % 4096 == 0, "tile must split evenly over 4 waves");
  static_assert(KT % 32 == 0, "a masked tile's spans load in 256-byte pieces");
  // V rows keep their natural layout; 16-byte chunk c of row r sits at slot
  // c ^ vswz(r), so that the transposed 8-byte reads of four consecutive
  // rows (or two rows of the other bank half, for 128-byte rows) hit
  // distinct banks.
  __device__ static __forceinline__ int vswz(int r) { return ROWB >= 256 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
  __device__ static __forceinline__ int voff(int r, int c) { return r * ROWB + ((c ^ vswz(r)) << 4); }
};

// Bound on the unnormalised probabilities exp2(s*c - m_run) that the
// running maximum m_run may leave before it is raised (2^8: far from fp32 or
// bf16 overflow, and a tile's sum of them stays exact enough in fp32).
constexpr float kProbBound = 256.f;

// A operand of O^T = V^T P^T for the 16-key step j and the 32 head-dim rows
// of block nb: lane l needs V[keys 16j + 4*hf + {0..3} and 16j + 8 + 4*hf +
// {0..3}][32*nb + l%32] (the key order of the P^T fragment).
//
// ds_read_tr16_b64: within each group of 16 lanes, lane i returns element
// i%4 of the 4-element (8-byte) pieces read by lanes i/4, i/4+4, i/4+8 and
// i/4+12.  Lane jj of a group therefore reads row k0 + jj/4 at columns
// d0 + 4*(jj%4).  With the V swizzle the byte offset of that piece is
//   16*ROWB*j + (4*hf + x)*ROWB + 64*(nb ^ y) + 32*grp + 8*(jj%4)
// (x = jj/4, y = the swizzle bits of x), plus 8*ROWB for keys 8..15 of the
// step: vt_off() gives the per-lane part for each nb once, the rest are
// immediates.
template <int ROWB>
__device__ __forceinline__ int vt_off(int lane, int nb) {
  const int hf = lane >> 5, grp = (lane >> 4) & 1, jj = lane & 15, x = jj >> 2;
  const int y = ROWB >= 256 ? x : ((x >> 1) & 1);
  return (4 * hf + x) * ROWB + 64 * (nb ^ y) + 32 * grp + 8 * (jj & 3);
}
template <int ROWB, int OFF>
__device__ __forceinline__ void load_vt(Frag<bf16> &a, const char *vl, int off_nb) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const char *p0 = vl + off_nb + OFF;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(__attribute__((address_space(3))) char *)(size_t)p0);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)(__attribute__((address_space(3))) char *)(size_t)(p0 + 8 * ROWB));
  const s16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  a.v = __builtin_bit_cast(bf16x8, w);
}
// The same two reads written out in asm, with their own wait for LDS.
// Through the builtin the compiler cannot tell them from the direct-to-LDS
// loads of the next tile that are still in flight and waits for all of those
// first (that buffer is never read here).  The budget-masked kernel gathers
// rows that often miss in L2, so that wait costs it ~9%; the dense kernel's
// loads mostly hit and there the asm form, which the compiler cannot schedule
// around, is 2% slower.  `addr` is the LDS address of the piece for keys
// 0..3 without OFF.  The outputs are early-clobber so that neither result
// register can take the address register the second read still needs.
template <int ROWB, int OFF>
__device__ __forceinline__ void load_vt_asm(Frag<bf16> &a, unsigned addr) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x4 lo, hi;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %2 offset:%3\n\t"
      "ds_read_b64_tr_b16 %1, %2 offset:%4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo), "=&v"(hi)
      : "v"(addr), "i"(OFF), "i"(OFF + 8 * ROWB)
      : "memory");
  const s16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  a.v = __builtin_bit_cast(bf16x8, w);
}
// fp32 V (correctness path): eight scalar reads through the swizzle.
template <int ROWB>
__device__ __forceinline__ void load_vt(Frag<float> &a, const char *vl, int j, int nb, int lane) {
  using Tl = FwdTiles<float, ROWB / 4>;
  const int hf = lane >> 5, d = 32 * nb + (lane & 31);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r0 = 16 * j + 4 * hf + e, r1 = r0 + 8;
    a.lo[e] = *reinterpret_cast<const float *>(vl + Tl::voff(r0, d >> 2) + 4 * (d & 3));
    a.hi[e] = *reinterpret_cast<const float *>(vl + Tl::voff(r1, d >> 2) + 4 * (d & 3));
  }
}

template <typename T, int D, bool WITH_O, bool SPARSE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KVPOP_FWD_WAVES))) attn_fwd_kernel(const FwdParams p) {
  using Tiles = FwdTiles<T, D>;
  using KTile = SwizzledTile<T, D>;
  constexpr int NJ = D / 16;  // k-steps over the head dimension
  constexpr int NB = D / 32;  // 32-dim blocks of O^T
  constexpr int KT = Tiles::KT;
  constexpr int NRB = KT / 32;  // 32-key row blocks of S^T per tile
  constexpr int CPR = Tiles::CPR;
  constexpr int ROWB = Tiles::ROWB;
  constexpr int LOADS = Tiles::LOADS;

  // two stages of (K tile, V tile): one barrier per tile
  __shared__ __align__(16) char smem[2][Tiles::STAGE];
  __shared__ __align__(16) int2 span_lds[2][KT];  // per listed key of a masked tile: its query span [lo, hi)

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hf = lane >> 5;
  const int HG = p.HG, QB = 32 * (4 / HG), NG = p.G / HG;
  const int nqb = (p.S + QB - 1) / QB;
  const int per_qb = p.B * p.Hkv * NG;
  int qb = nqb - 1 - (int)blockIdx.x / per_qb;  // latest (heaviest) query blocks first
  int rr = (int)blockIdx.x % per_qb;
  const int ng = rr % NG;
  rr /= NG;
  const int h = rr % p.Hkv, b = rr / p.Hkv;
  // over packed documents a budget list's length follows the block's
  // position in its document, so those blocks run in the order of a table
  // sorted by list length
  if constexpr (SPARSE) {
    if (p.qorder != nullptr) qb = p.qorder[((size_t)b * p.Hkv + h) * nqb + (int)blockIdx.x / per_qb];
  }
  const int g = h * p.G + ng * HG + wave % HG;
  const int q0 = qb * QB + 32 * (wave / HG);  // first query of this wave
  const int qpos = q0 + col;
  const bool qvalid = qpos < p.S;
  const int qc = qvalid ? qpos : p.S - 1;
  const bool wave_active = q0 < p.S;

  const size_t bh_kv = (size_t)b * p.Hkv + h;
  const T *kbase = reinterpret_cast<const T *>(p.k) + bh_kv * (size_t)p.S * D;
  const T *vbase = reinterpret_cast<const T *>(p.v) + bh_kv * (size_t)p.S * D;
  const T *qrow = reinterpret_cast<const T *>(p.q) + (((size_t)b * p.Hq + g) * p.S + qc) * D;

  // Q^T fragments of this lane's query (B operand), kept in registers.
  Frag<T> qf[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) load_frag(qf[j], qrow + 16 * j + 8 * hf);

  // Key range.
  int kbeg = 0, kend = 0, n_tiles = 0, list_len = 0, full_tiles = 0;
  const int *list = nullptr;
  int wq_last = 0, wds_first = 0, wds_last = 0, qdoc_start = 0;
  const int2 *spans = nullptr;
  if constexpr (!SPARSE) {
    const int blk_first = qb * QB;
    const int blk_last = min(p.S - 1, qb * QB + QB - 1);
    kbeg = find_doc(p.cu, p.n_docs, p.S, blk_first).start;
    kend = blk_last + 1;
    n_tiles = (kend - kbeg + KT - 1) / KT;
    qdoc_start = find_doc(p.cu, p.n_docs, p.S, qc).start;
    wq_last = min(p.S - 1, q0 + 31);
    wds_first = find_doc(p.cu, p.n_docs, p.S, min(q0, p.S - 1)).start;
    wds_last = find_doc(p.cu, p.n_docs, p.S, wq_last).start;
  } else {
    const size_t tile_id = bh_kv * nqb + qb;
    list = p.lists + tile_id * p.list_cap;
    list_len = min(p.list_len[tile_id], p.list_cap);
    n_tiles = (list_len + KT - 1) / KT;
    full_tiles = min(p.list_len_full[tile_id], list_len) / KT;
    spans = p.spans + tile_id * p.list_cap;
  }

  f32x16 o_acc[WITH_O ? NB : 1];
#pragma unroll
  for (int nb = 0; nb < (WITH_O ? NB : 1); ++nb) o_acc[nb] = f32x16{};
  // Running maximum (in log2 units, i.e. already times scale*log2e) and the
  // running sum of this lane half's keys; the halves are added at the end.
  float m_run = -INFINITY, l_run = 0.f;
  bool started = false;  // every row of the wave has a finite m_run
  const float c = p.scale_log2;

  // budget-masked path: the raw list entries of this lane's rows of the next
  // tile's gathers (loaded one tile ahead).  They are checked only when
  // used, a tile later: checking them on arrival would wait on the list
  // loads right away, and with them (loads complete in order) on the
  // gathers issued just before.
  int kraw[SPARSE ? LOADS : 1];
  int vt_base[NB];  // per-lane part of the transposed V reads
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) vt_base[nb] = vt_off<ROWB>(lane, nb);

  // Dense keys are contiguous: each wave issues LOADS buffer loads of 1 KB
  // per tensor that write straight into the LDS stage (lane l at +16*l), the
  // swizzles folded into each lane's source offset.  Rows past kend arrive
  // as zeros (they are masked anyway).
  // Each lane's source offsets within a tile (the swizzles folded in) are
  // the same for every tile: computed once and kept (opaque to the compiler,
  // which would otherwise recompute them on every tile).
  int koff[SPARSE ? 1 : LOADS], voff[SPARSE ? 1 : LOADS];
  if constexpr (!SPARSE) {
#pragma unroll
    for (int k = 0; k < LOADS; ++k) {
      const int pch = (wave * LOADS + k) * 64 + lane;  // chunk position in the tile
      const int r = pch / CPR, slot = pch % CPR;
      koff[k] = r * ROWB + ((slot ^ KTile::swz(r)) << 4);
      voff[k] = r * ROWB + ((slot ^ Tiles::vswz(r)) << 4);
      asm volatile("" : "+v"(koff[k]), "+v"(voff[k]));
    }
  }
  auto fetch_dense = [&](int tile, int buf) {
    if constexpr (!SPARSE) {
      const int tb = kbeg + tile * KT;
      const int rows = min(KT, kend - tb);
      const auto kr = make_rsrc(kbase + (size_t)tb * D, rows * ROWB);
      const auto vr = make_rsrc(vbase + (size_t)tb * D, rows * ROWB);
#pragma unroll
      for (int k = 0; k < LOADS; ++k) {
        lds_load16(kr, smem[buf] + (wave * LOADS + k) * 1024, koff[k]);
        lds_load16(vr, smem[buf] + Tiles::K_BYTES + (wave * LOADS + k) * 1024, voff[k]);
      }
    }
  };

  // Gathered keys: the same direct-to-LDS loads, each lane's source row
  // taken from the list (positions loaded a tile earlier by load_keys).
  // The buffers span the whole (batch, KV head) sequence.  Per-lane
  // constants of the gathers, recomputed where used (a few integer
  // operations; kept, they would hold six registers through the loop): the
  // row of the tile a load serves and the swizzled chunk offsets of K and V
  // in that row.
  auto g_row = [&](int k) { return ((wave * LOADS + k) * 64 + lane) / CPR; };
  auto g_koff = [&](int k) {
    const int pch = (wave * LOADS + k) * 64 + lane;
    return ((pch % CPR) ^ KTile::swz(pch / CPR)) << 4;
  };
  auto g_voff = [&](int k) {
    const int pch = (wave * LOADS + k) * 64 + lane;
    return ((pch % CPR) ^ Tiles::vswz(pch / CPR)) << 4;
  };
  // The list entries and spans of a tile come through buffer resources over
  // the block's list, which the list builder pads to whole tiles with the
  // row S (past the end of K and V: its loads return zeros) and a span that
  // no query meets.  The whole offset is in the per-lane register: the
  // resource's range check does not cover the scalar offset.
  auto load_keys = [&](int tile) {
    if constexpr (SPARSE) {
      const auto lr = make_rsrc(list, p.list_cap * 4);
#pragma unroll
      for (int k = 0; k < LOADS; ++k)
        kraw[k] = (int)__builtin_amdgcn_raw_buffer_load_b32(lr, (tile * KT + g_row(k)) * 4, 0, 0);
    }
  };
  // Entries are positions in [0, S] (S: padding).  Since S * ROWB < 2^31
  // (checked on the host), the byte offset of an entry needs no clamp: any
  // other value would fall outside the resource and read zeros as well.
  auto fetch_sparse = [&](int buf, int tile) {
    if constexpr (SPARSE) {
      const auto kr = make_rsrc(kbase, p.S * ROWB);
      const auto vr = make_rsrc(vbase, p.S * ROWB);
#pragma unroll
      for (int k = 0; k < LOADS; ++k) {
        const int row = kraw[k] * ROWB;
        lds_load16(kr, smem[buf] + (wave * LOADS + k) * 1024, row + g_koff(k));
        lds_load16(vr, smem[buf] + Tiles::K_BYTES + (wave * LOADS + k) * 1024, row + g_voff(k));
      }
      // Spans are read only by masked tiles, and go straight to LDS with the
      // tile's rows: KT x 8 bytes in 4-byte pieces, 64 per load of wave 0.
      // (Held in a register from a tile ahead instead, the span was spilled
      // across the masked tiles' compute, and its reload waited for every
      // gather in flight.)
      if (wave == 0 && tile >= full_tiles) {
        const auto sr = make_rsrc(spans, p.list_cap * 8);
#pragma unroll
        for (int i = 0; i < KT * 8 / 256; ++i)
          lds_load4(sr, &span_lds[buf][32 * i], (tile * KT + 32 * i) * 8 + lane * 4);
      }
    }
  };

  if constexpr (SPARSE) {
    // tile 0's list entries are loaded before the list length arrives (their
    // addresses do not depend on it), so its gathers wait for one round
    // trip less
    load_keys(0);
    if (n_tiles > 0) {
      fetch_sparse(0, 0);
      load_keys(1);
    }
  } else if (n_tiles > 0) {
    fetch_dense(0, 0);
  }
  // One tile: wait for its loads, publish them with a barrier (which also
  // retires every read of the other buffer), start the next tile's loads,
  // then compute.  FULL tiles need no element mask.  Tiles of each kind form
  // contiguous ranges, so each kind runs in a loop of its own with
  // straight-line code (a per-tile choice would merge the two paths' S tiles
  // and cost a register copy of both per tile).
  auto tile_step = [&](int tile, auto full_c) {
    constexpr bool FULL = decltype(full_c)::value;
    const int buf = tile & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tile + 1 < n_tiles) {
      if constexpr (SPARSE) {
        fetch_sparse(buf ^ 1, tile + 1);  // key positions loaded during the previous tile
        if (tile + 2 < n_tiles) load_keys(tile + 2);
      } else {
        fetch_dense(tile + 1, buf ^ 1);
      }
    }

    // Which of this wave's elements can be valid in this tile?
    bool any = wave_active;
    const int tb = kbeg + tile * KT;
    if constexpr (!SPARSE) any = any && tb <= wq_last && tb + KT - 1 >= wds_first;
    if (any) {
      const char *kl = smem[buf];
      const char *vl = smem[buf] + Tiles::K_BYTES;
      f32x16 s[NRB];
      // S^T tile.  z is an opaque zero: it keeps the LDS reads of a second
      // pass inside that pass (read once for both, they would hold 32 more
      // registers through the first).
      auto logits = [&](int z) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          s[rb] = f32x16{};
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            Frag<T> a;
            KTile::read(a, kl + z, 32 * rb + col, 16 * j + 8 * hf);
            mma(s[rb], a, qf[j]);
          }
        }
      };
      // element mask: disallowed logits become -inf
      auto apply_mask = [&](int z) {
        if constexpr (!FULL) {
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              // the 4 rows of registers 4*i4 .. 4*i4+3 are adjacent: their
              // spans arrive in two 16-byte reads
              int4 pr[2];
              if constexpr (SPARSE) {
                // one group of four rows at a time: read all at once, the
                // spans would hold 32 registers through the masking
                asm volatile("" ::: "memory");
                const int r0 = 32 * rb + c_row(4 * i4, hf) + z;
                pr[0] = *reinterpret_cast<const int4 *>(&span_lds[buf][r0]);
                pr[1] = *reinterpret_cast<const int4 *>(&span_lds[buf][r0 + 2]);
              }
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int i = 4 * i4 + e;
                bool ok;
                if constexpr (!SPARSE) {
                  const int t = tb + 32 * rb + c_row(i, hf);
                  ok = qvalid && t <= qpos && t >= qdoc_start;
                } else {
                  // the key's span of keeping queries
                  const int lo = (e & 1) ? pr[e >> 1].z : pr[e >> 1].x;
                  const int hi = (e & 1) ? pr[e >> 1].w : pr[e >> 1].y;
                  ok = qvalid && qpos >= lo && qpos < hi;
                }
                s[rb][i] = ok ? s[rb][i] : -INFINITY;
              }
            }
          }
        }
      };
      // row maximum over both lane halves, in log2 units
      auto row_max = [&]() {
        float mx = -INFINITY;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[rb][i]);
        return fmaxf(mx, __shfl_xor(mx, 32)) * c;
      };
      auto rescale_to = [&](float m_new) {
        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
        if constexpr (WITH_O) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) o_acc[nb] *= alpha;
        }
        m_run = m_new;
      };
      // P^T in place: exponentials against m, summed per lane
      auto exponentials = [&](float m) {
        float lt = 0.f;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float pv = fast_exp2(__builtin_fmaf(s[rb][i], c, -m));
            s[rb][i] = pv;
            lt += pv;
          }
        }
        return lt;
      };

      // Once every row of the wave has a running maximum, a tile first takes
      // its exponentials against it directly.  A sum of non-negative terms
      // bounds each of them, so when every lane's sum stays within the bound
      // no probability exceeds it and the row maxima are not needed.
      // Otherwise (a larger or non-finite sum), and while some row has no
      // maximum yet, the tile is redone against its exact masked maximum,
      // which also brings the running one to where later tiles pass again.
      float lt = 0.f;
      // Masked tiles of the budget-masked forward (a few per block) always
      // take the exact path: one copy of the masking code instead of two.
      constexpr bool FAST = FULL || !SPARSE;
      bool exact = !FAST || !started;
      if (FAST && started) {
        int z = 0;
        asm volatile("" : "+s"(z));
        logits(z);
        apply_mask(z);
        lt = exponentials(m_run);
        exact = __ballot(!(lt <= kProbBound)) != 0;
      }
      if (exact) {
        // z differs from the first block's: its LDS reads must not be
        // merged with those (that would keep 32 more registers live)
        int z = 0;
        asm volatile("" : "+s"(z));
        logits(z);
        apply_mask(z);
        const float mxc = row_max();
        if (__ballot(mxc > m_run) != 0) rescale_to(fmaxf(m_run, mxc));
        lt = exponentials(m_run == -INFINITY ? 0.f : m_run);
        started = __ballot(m_run == -INFINITY) == 0;
      }
      l_run += lt;

      if constexpr (WITH_O) {
        // 16-key steps j as compile-time constants: the V reads take the
        // step's offset as an immediate
        static_for<KT / 16>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          Frag<T> pf;
          if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e = 0; e < 8; ++e) pf.v[e] = (bf16)s[j >> 1][8 * (j & 1) + e];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              pf.lo[e] = s[j >> 1][8 * (j & 1) + e];
              pf.hi[e] = s[j >> 1][8 * (j & 1) + 4 + e];
            }
          }
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            Frag<T> a;
            if constexpr (sizeof(T) == 2 && SPARSE) {
              load_vt_asm<ROWB, Tiles::K_BYTES + 16 * ROWB * j>(a, (unsigned)(size_t)smem[buf] + vt_base[nb]);
            } else if constexpr (sizeof(T) == 2) {
              load_vt<ROWB, 16 * ROWB * j>(a, vl, vt_base[nb]);
            } else {
              load_vt<ROWB>(a, vl, j, nb, lane);
            }
            mma(o_acc[nb], a, pf);
          }
        });
      }
    }

  };
  int f0 = 0, f1 = 0;  // the unmasked tiles are [f0, f1)
  if constexpr (SPARSE) {
    f1 = full_tiles;
  } else {
    // tb >= wds_last, tb + KT - 1 <= q0 and tb + KT - 1 < kend, tb = kbeg + tile * KT
    f0 = max(0, (wds_last - kbeg + KT - 1) / KT);
    const int last = min(q0, kend - 1) - (KT - 1) - kbeg;  // tb - kbeg <= last
    f1 = last >= 0 ? min(n_tiles, last / KT + 1) : 0;
    f1 = max(f1, f0);
  }
  for (int tile = 0; tile < f0; ++tile) tile_step(tile, std::false_type{});
  for (int tile = f0; tile < f1; ++tile) tile_step(tile, std::true_type{});
  for (int tile = f1; tile < n_tiles; ++tile) tile_step(tile, std::false_type{});

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!qvalid) return;
  const size_t row = ((size_t)b * p.Hq + g) * p.S + qpos;
  if (hf == 0) p.lse[row] = (l_tot > 0.f) ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  if constexpr (WITH_O) {
    const float inv_l = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    T *orow = reinterpret_cast<T *>(p.o) + row * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = 32 * nb + 8 * i4 + 4 * hf;
        if constexpr (sizeof(T) == 2) {
          bf16x4 w = {(bf16)(o_acc[nb][4 * i4 + 0] * inv_l), (bf16)(o_acc[nb][4 * i4 + 1] * inv_l),
                      (bf16)(o_acc[nb][4 * i4 + 2] * inv_l), (bf16)(o_acc[nb][4 * i4 + 3] * inv_l)};
          *reinterpret_cast<bf16x4 *>(orow + d0) = w;
        } else {
          f32x4 w = {o_acc[nb][4 * i4 + 0] * inv_l, o_acc[nb][4 * i4 + 1] * inv_l,
                     o_acc[nb][4 * i4 + 2] * inv_l, o_acc[nb][4 * i4 + 3] * inv_l};
          *reinterpret_cast<f32x4 *>(orow + d0) = w;
        }
      }
    }
  }
}

}  // namespace kvpop
