// Attention forward with log-sum-exp for gfx950: dense causal (packed
// documents allowed) and budget-masked sparse variants.
//
// Dense:  L_d = ln sum_{t<=d, same doc} exp(s_{d,t}), O_d = sum_t exp(s-L) v_t
//         (the causal normaliser of the KVpop paper, Section 3.2).
// Sparse: the same over the per-KV-head budget mask of Section 3 / 3.2
//         (sinks, protected window, running top-k by static rank), reading
//         only the keys listed for the query block.
//
// Work decomposition: one workgroup = 4 waves = one block of QB query
// positions x HG query heads of one KV head (HG = min(G, 4), QB = 32*4/HG), so
// each K/V tile brought to LDS serves every query head of the group.  Each
// wave owns 32 queries of one head and computes S^T = K Q^T with MFMA: a lane
// then owns one query column, so the online-softmax max and sum are reductions
// over the lane's registers plus one exchange with the other lane half.  P^T
// (bf16) is directly the B operand of O^T = V^T P^T; V is transposed into LDS.
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
  const int *lists;     // [B*Hkv][nqb][list_cap] key positions, ascending
  const int *list_len;  // [B*Hkv][nqb]
  const int *rank;      // [B*Hkv][S]
  const int *cutoff;    // [B*Hkv][S]
  int list_cap, sinks, window;
};

template <typename T, int D>
struct FwdTiles {
  static constexpr int KT = 64;      // keys per tile
  static constexpr int VT_LD = 68;   // V^T row length (64 keys + pad), elements
  static constexpr int EPC = 16 / (int)sizeof(T);        // elements per 16-byte chunk
  static constexpr int K_CHUNKS = KT * D / EPC;           // 16-byte chunks of a K tile
  static constexpr int K_PER_THREAD = K_CHUNKS / 256;
  static constexpr int V_ITEMS = (KT / 4) * (D / EPC);    // (4-key group, chunk) items
  static constexpr int V_PER_THREAD = (V_ITEMS + 255) / 256;
  static_assert(K_CHUNKS % 256 == 0, "K tile must split evenly over 256 threads");
};

template <typename T, int D, bool WITH_O, bool SPARSE>
__global__ void __launch_bounds__(256) attn_fwd_kernel(const FwdParams p) {
  using Tiles = FwdTiles<T, D>;
  using KTile = SwizzledTile<T, D>;
  constexpr int NJ = D / 16;  // k-steps over the head dimension
  constexpr int NB = D / 32;  // 32-dim blocks of O^T
  constexpr int KT = Tiles::KT;
  constexpr int VT_LD = Tiles::VT_LD;
  constexpr int EPC = Tiles::EPC;
  constexpr int CPR = D / EPC;  // chunks per row

  __shared__ __align__(16) char k_lds[KT * D * sizeof(T)];
  __shared__ __align__(16) T vt_lds[D * VT_LD];
  __shared__ int kpos_lds[KT];
  __shared__ int krank_lds[KT];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hf = lane >> 5;
  const int HG = p.HG, QB = 32 * (4 / HG), NG = p.G / HG;
  const int nqb = (p.S + QB - 1) / QB;
  const int per_qb = p.B * p.Hkv * NG;
  const int qb = nqb - 1 - (int)blockIdx.x / per_qb;  // latest (heaviest) query blocks first
  int rr = (int)blockIdx.x % per_qb;
  const int ng = rr % NG;
  rr /= NG;
  const int h = rr % p.Hkv, b = rr / p.Hkv;
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
  int kbeg = 0, kend = 0, n_tiles = 0, list_len = 0;
  const int *list = nullptr;
  int wq_last = 0, wds_first = 0, wds_last = 0, qdoc_start = 0, cut_q = 0;
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
    cut_q = p.cutoff[bh_kv * p.S + qc];
  }

  f32x16 o_acc[WITH_O ? NB : 1];
#pragma unroll
  for (int nb = 0; nb < (WITH_O ? NB : 1); ++nb) o_acc[nb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // Prefetch registers for one K/V tile.
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 kreg[Tiles::K_PER_THREAD];
  u32x4 vreg[Tiles::V_PER_THREAD][4];
  int my_kpos = INT32_MAX, my_krank = 0;

  auto key_of = [&](int tile, int r, bool &valid) -> int {
    if constexpr (!SPARSE) {
      const int t = kbeg + tile * KT + r;
      valid = t < kend;
      return valid ? t : kbeg;
    } else {
      const int idx = tile * KT + r;
      valid = idx < list_len;
      const int t = valid ? list[idx] : 0;
      valid = valid && t >= 0 && t < p.S;
      return valid ? t : 0;
    }
  };

  auto prefetch = [&](int tile) {
#pragma unroll
    for (int c = 0; c < Tiles::K_PER_THREAD; ++c) {
      const int li = tid + 256 * c;
      const int r = li / CPR, ch = li % CPR;
      bool valid;
      const int t = key_of(tile, r, valid);
      kreg[c] = *reinterpret_cast<const u32x4 *>(kbase + (size_t)t * D + ch * EPC);
    }
#pragma unroll
    for (int it = 0; it < Tiles::V_PER_THREAD; ++it) {
      const int item = tid + 256 * it;
      if (item < Tiles::V_ITEMS) {
        const int kg = item / CPR, ch = item % CPR;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bool valid;
          const int t = key_of(tile, 4 * kg + e, valid);
          vreg[it][e] = *reinterpret_cast<const u32x4 *>(vbase + (size_t)t * D + ch * EPC);
        }
      }
    }
    if (tid < KT) {
      bool valid;
      const int t = key_of(tile, tid, valid);
      my_kpos = valid ? t : INT32_MAX;
      if constexpr (SPARSE) my_krank = valid ? p.rank[bh_kv * p.S + t] : INT32_MAX;
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int c = 0; c < Tiles::K_PER_THREAD; ++c) {
      const int li = tid + 256 * c;
      const int r = li / CPR, ch = li % CPR;
      *reinterpret_cast<u32x4 *>(k_lds + KTile::off(r, ch)) = kreg[c];
    }
#pragma unroll
    for (int it = 0; it < Tiles::V_PER_THREAD; ++it) {
      const int item = tid + 256 * it;
      if (item < Tiles::V_ITEMS) {
        const int kg = item / CPR, ch = item % CPR;
        const T *e0 = reinterpret_cast<const T *>(&vreg[it][0]);
        const T *e1 = reinterpret_cast<const T *>(&vreg[it][1]);
        const T *e2 = reinterpret_cast<const T *>(&vreg[it][2]);
        const T *e3 = reinterpret_cast<const T *>(&vreg[it][3]);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          T *dst = vt_lds + (ch * EPC + e) * VT_LD + 4 * kg;
          if constexpr (sizeof(T) == 2) {
            bf16x4 w = {e0[e], e1[e], e2[e], e3[e]};
            *reinterpret_cast<bf16x4 *>(dst) = w;
          } else {
            f32x4 w = {e0[e], e1[e], e2[e], e3[e]};
            *reinterpret_cast<f32x4 *>(dst) = w;
          }
        }
      }
    }
    if (tid < KT) {
      kpos_lds[tid] = my_kpos;
      krank_lds[tid] = my_krank;
    }
  };

  if (n_tiles > 0) prefetch(0);
  for (int tile = 0; tile < n_tiles; ++tile) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (tile + 1 < n_tiles) prefetch(tile + 1);

    // Which of this wave's elements can be valid in this tile?
    bool any = wave_active, full = false;
    const int tb = kbeg + tile * KT;
    if constexpr (!SPARSE) {
      any = any && tb <= wq_last && tb + KT - 1 >= wds_first;
      full = tb >= wds_last && tb + KT - 1 <= q0 && tb + KT - 1 < kend;
    }
    if (!any) continue;

    f32x16 s[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      s[rb] = f32x16{};
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        Frag<T> a;
        KTile::read(a, k_lds, 32 * rb + col, 16 * j + 8 * hf);
        mma(s[rb], a, qf[j]);
      }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[rb][i] * p.scale_log2;
        if (!full) {
          const int r = 32 * rb + c_row(i, hf);
          bool ok;
          if constexpr (!SPARSE) {
            const int t = tb + r;
            ok = qvalid && t <= qpos && t >= qdoc_start;
          } else {
            const int t = kpos_lds[r];
            const int rk = krank_lds[r];
            ok = qvalid && t <= qpos && (t < p.sinks || t > qpos - p.window || rk <= cut_q);
          }
          x = ok ? x : -INFINITY;
        }
        s[rb][i] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float sum = 0.f;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(s[rb][i] - m_use);
        s[rb][i] = pv;
        sum += pv;
      }
    }
    sum += __shfl_xor(sum, 32);
    l_run = l_run * alpha + sum;
    m_run = m_new;

    if constexpr (WITH_O) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o_acc[nb] *= alpha;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
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
          const T *vr = vt_lds + (32 * nb + col) * VT_LD + 16 * j + 4 * hf;
          Frag<T> a;
          if constexpr (sizeof(T) == 2) {
            const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(vr);
            const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(vr + 8);
            a.v = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          } else {
            a.lo = *reinterpret_cast<const f32x4 *>(vr);
            a.hi = *reinterpret_cast<const f32x4 *>(vr + 8);
          }
          mma(o_acc[nb], a, pf);
        }
      }
    }
  }

  if (!qvalid) return;
  const size_t row = ((size_t)b * p.Hq + g) * p.S + qpos;
  if (hf == 0) p.lse[row] = (l_run > 0.f) ? (m_run + fast_log2(l_run)) * kLn2 : -INFINITY;
  if constexpr (WITH_O) {
    const float inv_l = (l_run > 0.f) ? 1.f / l_run : 0.f;
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
