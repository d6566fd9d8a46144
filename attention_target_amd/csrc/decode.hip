// Fixed-budget decoding for gfx950 (kvpop_decode_init, kvpop_decode_step).
//
// KVpop paper, Section 3: every KV head keeps s sink tokens, a protected
// window of the w most recent tokens, and the k best eligible tokens by
// static priority, so the per-head cache never exceeds B = s + w + k slots
// (Section 4.3 measures the resulting flat memory at decode time).  Each
// step (Section 3.2, "Running top-k sparse attention"): the new token enters
// the window; token d-w leaves it and competes for the top-k; if the top-k is
// full and the newcomer beats the worst retained token, that token is
// evicted for good (with static priorities a dropped token can never return:
// the set of better tokens only grows).  The query then attends over the
// retained slots, which are exactly the budget mask's row d.
//
// State per (batch row, KV head), caller-owned device memory:
//   slot K, V   [C, D] (C = s + w + k): slots [0, s) sinks, [s, s+w) the
//               window ring (token t >= s at s + t mod w), [s+w, C) the
//               top-k set in no particular order;
//   slot pos    [C] int32, -1 when empty;  slot key [C] uint64, the
//               order key (descending priority, then ascending index);
//   topk count  int32.
// Kernels: decode_update (one workgroup per (b, h)), decode_attn (split
// over slot chunks, G query heads per workgroup, fp32 online softmax),
// decode_combine (merges the chunks per query head).
#include "common.h"
#include "launch.h"

namespace kvpop {

constexpr int DEC_CHUNK = 128;  // slots per attention workgroup
constexpr int DEC_WAVES = 16;   // waves per attention workgroup
constexpr int DEC_ROWS = DEC_CHUNK / DEC_WAVES;  // slot rows per wave
constexpr int DEC_MAX_SLOTS = 1 << 20;  // the C-ABI rejects larger caches
constexpr int DEC_MAX_CHUNKS = DEC_MAX_SLOTS / DEC_CHUNK;  // merge weights held in LDS

__device__ __forceinline__ uint64_t decode_key(float sc, int t) {
  if (sc != sc) sc = -INFINITY;
  if (sc == 0.f) sc = 0.f;
  const uint32_t u = __float_as_uint(sc);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)(~ord) << 32) | (uint32_t)t;
}

struct DecodeState {
  void *k, *v;
  int *pos;
  uint64_t *key;
  int *count;
  float *part;  // [B*Hq][nchunk][D + 2]
};

DecodeState decode_state_view(const DecodeShapeInfo &s, void *base) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t BH = (size_t)s.B * s.Hkv, C = (size_t)s.C;
  const size_t es = s.dtype == 0 ? 2 : 4;
  char *p = reinterpret_cast<char *>(base);
  DecodeState st{};
  size_t off = 0;
  st.k = p + off;
  off = al(off + BH * C * s.D * es);
  st.v = p + off;
  off = al(off + BH * C * s.D * es);
  st.pos = reinterpret_cast<int *>(p + off);
  off = al(off + BH * C * 4);
  st.key = reinterpret_cast<uint64_t *>(p + off);
  off = al(off + BH * C * 8);
  st.count = reinterpret_cast<int *>(p + off);
  off = al(off + BH * 4);
  st.part = reinterpret_cast<float *>(p + off);
  return st;
}

size_t decode_state_bytes(const DecodeShapeInfo &s) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t BH = (size_t)s.B * s.Hkv, C = (size_t)s.C;
  const size_t es = s.dtype == 0 ? 2 : 4;
  const size_t nch = (C + DEC_CHUNK - 1) / DEC_CHUNK;
  return 2 * al(BH * C * s.D * es) + al(BH * C * 4) + al(BH * C * 8) + al(BH * 4) +
         al((size_t)s.B * s.Hq * nch * (s.D + 2) * 4);
}

struct DecParams {
  DecodeState st;
  const void *q, *k, *v;
  const float *score;
  void *o;
  float *lse;
  int B, Hq, Hkv, G, D, C, sinks, window, topk, d, nchunk, dtype;
  float scale_log2;
};

__global__ void __launch_bounds__(256) decode_init_kernel(DecParams p) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t n = (size_t)p.B * p.Hkv * p.C;
  if (i < n) {
    p.st.pos[i] = -1;
    p.st.key[i] = ~0ull;
  }
  if (i < (size_t)p.B * p.Hkv) p.st.count[i] = 0;
}

template <typename T>
__device__ __forceinline__ void copy_row(T *dst, const T *src, int D) {
  for (int e = threadIdx.x; e < D; e += 256) dst[e] = src[e];
}

// One workgroup per (batch row, KV head): the newly eligible token competes
// for the top-k, then the new token takes its sink or window slot.
template <typename T>
__global__ void __launch_bounds__(256) decode_update(DecParams p) {
  __shared__ uint64_t red_key[4];
  __shared__ int red_slot[4];
  __shared__ int sh_target;
  const int bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = p.sinks, w = p.window, k = p.topk, d = p.d, D = p.D;
  T *sk = reinterpret_cast<T *>(p.st.k) + (size_t)bh * p.C * D;
  T *sv = reinterpret_cast<T *>(p.st.v) + (size_t)bh * p.C * D;
  int *pos = p.st.pos + (size_t)bh * p.C;
  uint64_t *key = p.st.key + (size_t)bh * p.C;
  const T *knew = reinterpret_cast<const T *>(p.k) + (size_t)bh * D;
  const T *vnew = reinterpret_cast<const T *>(p.v) + (size_t)bh * D;
  const float sc_new = p.score[bh];

  // 1. token e = d - w becomes eligible at this step (with w = 0, the new token)
  const int e = d - w;
  if (e >= s && k > 0) {
    const int src = (w > 0) ? s + e % w : -1;  // its window slot
    const uint64_t ke = (w > 0) ? key[src] : decode_key(sc_new, d);
    const int n = p.st.count[bh];
    if (tid == 0) sh_target = -1;
    __syncthreads();
    if (n < k) {
      if (tid == 0) sh_target = s + w + n;
    } else {
      // worst retained top-k slot: the largest key
      uint64_t best = 0;
      int bslot = -1;
      for (int j = tid; j < k; j += 256) {
        const uint64_t kj = key[s + w + j];
        if (bslot < 0 || kj > best) {
          best = kj;
          bslot = s + w + j;
        }
      }
      for (int o = 32; o > 0; o >>= 1) {
        const uint64_t ob = __shfl_xor(best, o);
        const int os = __shfl_xor(bslot, o);
        if (os >= 0 && (bslot < 0 || ob > best || (ob == best && os < bslot))) {
          best = ob;
          bslot = os;
        }
      }
      if (lane == 0) {
        red_key[wave] = best;
        red_slot[wave] = bslot;
      }
      __syncthreads();
      if (tid == 0) {
        uint64_t wk = 0;
        int ws = -1;
        for (int q = 0; q < 4; ++q)
          if (red_slot[q] >= 0 && (ws < 0 || red_key[q] > wk)) {
            wk = red_key[q];
            ws = red_slot[q];
          }
        sh_target = (ws >= 0 && ke < wk) ? ws : -1;
      }
    }
    __syncthreads();
    const int target = sh_target;
    if (target >= 0) {
      if (w > 0) {
        copy_row(sk + (size_t)target * D, sk + (size_t)src * D, D);
        copy_row(sv + (size_t)target * D, sv + (size_t)src * D, D);
      } else {
        copy_row(sk + (size_t)target * D, knew, D);
        copy_row(sv + (size_t)target * D, vnew, D);
      }
      if (tid == 0) {
        pos[target] = e;
        key[target] = ke;
        if (n < k) p.st.count[bh] = n + 1;
      }
    }
    __syncthreads();  // the window slot is read before the new token overwrites it
  }
  // 2. the new token: a sink, or the window ring
  int slot = -1;
  if (d < s) slot = d;
  else if (w > 0) slot = s + d % w;
  if (slot >= 0) {
    copy_row(sk + (size_t)slot * D, knew, D);
    copy_row(sv + (size_t)slot * D, vnew, D);
    if (tid == 0) {
      pos[slot] = d;
      key[slot] = decode_key(sc_new, d);
    }
  }
}

// Eight consecutive elements of a slot row, fetched with 16-byte loads.
template <typename T>
struct Row8;
template <>
struct Row8<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16 *src) { v = *reinterpret_cast<const bf16x8 *>(src); }
  __device__ __forceinline__ float operator[](int e) const { return (float)v[e]; }
};
template <>
struct Row8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float *src) {
    a = *reinterpret_cast<const f32x4 *>(src);
    b = *reinterpret_cast<const f32x4 *>(src + 4);
  }
  __device__ __forceinline__ float operator[](int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

// Sum over each aligned group of LPR (8 or 16) lanes, the total in every lane
// of the group: two quad permutations, then the half-row and row mirrors,
// each a DPP-modified add (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int LPR>
__device__ __forceinline__ float lane_group_sum(float x) {
  static_assert(LPR == 8 || LPR == 16, "lane groups of 8 or 16");
  x = dpp_add<0xB1>(x);   // quad_perm [1,0,3,2]
  x = dpp_add<0x4E>(x);   // quad_perm [2,3,0,1]
  x = dpp_add<0x141>(x);  // row_half_mirror: lane i <- 7-i within 8
  if constexpr (LPR == 16) x = dpp_add<0x140>(x);  // row_mirror: lane i <- 15-i within 16
  return x;
}

// Workgroup (chunk, b*Hkv + h): the G query heads of KV head h against slots
// [chunk*DEC_CHUNK, +DEC_CHUNK).  The kernel is bound by latency, not by
// bandwidth or arithmetic, so the chunk is spread over DEC_WAVES waves of
// DEC_ROWS rows each (two or more waves per SIMD), and every wave issues all
// of its K, V and slot-position loads before it computes anything.  Lane l
// covers 8 elements at 8*(l % LPR) of a slot row (LPR = D/8 lanes per row,
// RPW = 64/LPR rows per load instruction).  Phases:
//   1. logits: per-lane partial dot products finished by a DPP sum over the
//      LPR lanes of a row, written to LDS (-inf for empty slots);
//   2. one wave per query head reduces that head's maximum and sum of
//      exponentials over the chunk;
//   3. each wave forms its rows' probabilities and partial PV sums, reduced
//      over the rows of the wave, then over the waves through LDS.
// G (query heads per KV head) and D are template parameters so that register
// arrays are indexed statically and every reduction is unrolled.
template <typename T, int G, int D>
__global__ void __launch_bounds__(DEC_WAVES * 64) decode_attn(DecParams p) {
  constexpr int EPL = 8;                // elements per lane and row
  constexpr int LPR = D / EPL;          // lanes per row: 16 (D=128) or 8 (D=64)
  constexpr int RPW = 64 / LPR;         // rows per load instruction: 4 or 8
  constexpr int NRG = DEC_ROWS / RPW;   // row groups per wave: 2 or 1
  static_assert(DEC_ROWS % RPW == 0, "whole row groups per wave");
  static_assert(G <= DEC_WAVES, "one wave per query head in phase 2");
  __shared__ float lg[G][DEC_CHUNK];
  __shared__ float ml[G][2];  // per head: maximum (log2 units) and sum
  __shared__ float osum[DEC_WAVES][G][D];
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.Hkv, h = bh % p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r_in = lane / LPR, c = lane % LPR;
  const T *sk = reinterpret_cast<const T *>(p.st.k) + (size_t)bh * p.C * D;
  const T *sv = reinterpret_cast<const T *>(p.st.v) + (size_t)bh * p.C * D;
  const int *pos = p.st.pos + (size_t)bh * p.C;
  const int j0 = chunk * DEC_CHUNK;
  const int nslots = min(DEC_CHUNK, p.C - j0);

  // every load of this wave, up front; rows past the chunk's end re-read
  // its last row and are masked
  Row8<T> kr[NRG], vr[NRG];
  bool ok[NRG];
#pragma unroll
  for (int i = 0; i < NRG; ++i) {
    const int j = wave * DEC_ROWS + i * RPW + r_in;
    const int jj = min(j, nslots - 1);
    const size_t off = (size_t)(j0 + jj) * D + c * EPL;
    kr[i].load(sk + off);
    vr[i].load(sv + off);
    ok[i] = j < nslots && pos[j0 + jj] >= 0;
  }
  float qv[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    Row8<T> qr;
    qr.load(reinterpret_cast<const T *>(p.q) + ((size_t)b * p.Hq + h * G + g) * D + c * EPL);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[g][e] = qr[e];
  }

  // 1. logits (log2 units)
#pragma unroll
  for (int i = 0; i < NRG; ++i) {
    const int j = wave * DEC_ROWS + i * RPW + r_in;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float x = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) x += qv[g][e] * kr[i][e];
      x = lane_group_sum<LPR>(x);
      if (c == 0) lg[g][j] = ok[i] ? x * p.scale_log2 : -INFINITY;
    }
  }
  __syncthreads();

  // 2. wave g: maximum and sum of exponentials of head g over the chunk
  if (wave < G) {
    const int g = wave;
    const float x0 = lg[g][lane], x1 = lg[g][lane + 64];
    float m = fmaxf(x0, x1);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float mu = m == -INFINITY ? 0.f : m;
    float l = exp2f(x0 - mu) + exp2f(x1 - mu);  // -inf: 0
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
    if (lane == 0) {
      ml[g][0] = m;
      ml[g][1] = l;
    }
  }
  __syncthreads();

  // 3. probabilities and partial outputs; masked rows contribute zero
  // whatever their V holds
  float acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
#pragma unroll
  for (int i = 0; i < NRG; ++i) {
    const int j = wave * DEC_ROWS + i * RPW + r_in;
    float vf[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) vf[e] = ok[i] ? vr[i][e] : 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float m = ml[g][0];
      const float pg = ok[i] ? exp2f(lg[g][j] - m) : 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] += pg * vf[e];
    }
  }
  // reduce over the row groups of the wave (lanes with the same c)
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = acc[g][e];
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) x += __shfl_xor(x, o);
      acc[g][e] = x;
    }
  if (r_in == 0)
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) osum[wave][g][c * EPL + e] = acc[g][e];
  __syncthreads();
  for (int i = tid; i < G * D; i += DEC_WAVES * 64) {
    const int g = i / D, e = i % D;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) sum += osum[w][g][e];
    float *pp = p.st.part + (((size_t)b * p.Hq + h * G + g) * p.nchunk + chunk) * (D + 2);
    pp[e] = sum;
    if (e == 0) {
      pp[D] = ml[g][0];
      pp[D + 1] = ml[g][1];
    }
  }
}

// One workgroup per (b, query head): merge the chunks.  Chunk maxima and
// sums are read by parallel threads into LDS and the merge weights computed
// once; each thread then sums one output dimension over the chunks, eight
// independent loads at a time.
template <typename T>
__global__ void __launch_bounds__(256) decode_combine(DecParams p) {
  __shared__ float wgt[DEC_MAX_CHUNKS];
  __shared__ float red[4];
  const int bg = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int D = p.D, nc = p.nchunk;
  const float *pp = p.st.part + (size_t)bg * nc * (D + 2);
  float m = -INFINITY;
  for (int c = tid; c < nc; c += 256) {
    const float mc = pp[(size_t)c * (D + 2) + D];
    wgt[c] = mc;
    m = fmaxf(m, mc);
  }
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float mu = m == -INFINITY ? 0.f : m;
  __syncthreads();
  float l = 0.f;
  for (int c = tid; c < nc; c += 256) {
    const float mc = wgt[c];
    const float wc = mc == -INFINITY ? 0.f : exp2f(mc - mu);
    wgt[c] = wc;
    l += wc * pp[(size_t)c * (D + 2) + D + 1];
  }
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
  __syncthreads();  // every weight written before any thread reads them
  if (lane == 0) red[wave] = l;
  __syncthreads();
  l = red[0] + red[1] + red[2] + red[3];
  for (int e = tid; e < D; e += 256) {
    float acc = 0.f;
#pragma unroll 8
    for (int c = 0; c < nc; ++c) acc += pp[(size_t)c * (D + 2) + e] * wgt[c];
    reinterpret_cast<T *>(p.o)[(size_t)bg * D + e] = (T)(l > 0.f ? acc / l : 0.f);
  }
  if (tid == 0) p.lse[bg] = l > 0.f ? (mu + log2f(l)) * kLn2 : -INFINITY;
}

static DecParams decode_params(const DecodeShapeInfo &s, void *state) {
  DecParams p{};
  p.st = decode_state_view(s, state);
  p.B = s.B;
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.G = s.Hq / s.Hkv;
  p.D = s.D;
  p.C = s.C;
  p.sinks = s.sinks;
  p.window = s.window;
  p.topk = s.topk;
  p.nchunk = (s.C + DEC_CHUNK - 1) / DEC_CHUNK;
  p.dtype = s.dtype;
  p.scale_log2 = s.scale * kLog2e;
  return p;
}

hipError_t launch_decode_init(const DecodeShapeInfo &s, void *state, hipStream_t st) {
  DecParams p = decode_params(s, state);
  const size_t n = (size_t)s.B * s.Hkv * s.C;
  hipLaunchKernelGGL(decode_init_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <typename T, int D>
static bool launch_attn_g(const DecParams &p, dim3 grid, hipStream_t st) {
  switch (p.G) {
    case 1: hipLaunchKernelGGL((decode_attn<T, 1, D>), grid, dim3(DEC_WAVES * 64), 0, st, p); return true;
    case 2: hipLaunchKernelGGL((decode_attn<T, 2, D>), grid, dim3(DEC_WAVES * 64), 0, st, p); return true;
    case 3: hipLaunchKernelGGL((decode_attn<T, 3, D>), grid, dim3(DEC_WAVES * 64), 0, st, p); return true;
    case 4: hipLaunchKernelGGL((decode_attn<T, 4, D>), grid, dim3(DEC_WAVES * 64), 0, st, p); return true;
    case 5: hipLaunchKernelGGL((decode_attn<T, 5, D>), grid, dim3(DEC_WAVES * 64), 0, st, p); return true;
    case 6: hipLaunchKernelGGL((decode_attn<T, 6, D>), grid, dim3(DEC_WAVES * 64), 0, st, p); return true;
    case 7: hipLaunchKernelGGL((decode_attn<T, 7, D>), grid, dim3(DEC_WAVES * 64), 0, st, p); return true;
    case 8: hipLaunchKernelGGL((decode_attn<T, 8, D>), grid, dim3(DEC_WAVES * 64), 0, st, p); return true;
    default: return false;
  }
}

template <typename T>
static hipError_t run_decode(DecParams &p, hipStream_t st) {
  hipLaunchKernelGGL(decode_update<T>, dim3(p.B * p.Hkv), dim3(256), 0, st, p);
  const dim3 grid(p.nchunk, p.B * p.Hkv);
  if (p.D == 128) {
    if (!launch_attn_g<T, 128>(p, grid, st)) return hipErrorInvalidValue;
  } else if (p.D == 64) {
    if (!launch_attn_g<T, 64>(p, grid, st)) return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(decode_combine<T>, dim3(p.B * p.Hq), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_decode_step(const DecodeShapeInfo &s, void *state, int position, const void *q, const void *k,
                              const void *v, const float *score, void *o, float *lse, hipStream_t st) {
  DecParams p = decode_params(s, state);
  p.q = q;
  p.k = k;
  p.v = v;
  p.score = score;
  p.o = o;
  p.lse = lse;
  p.d = position;
  return s.dtype == 0 ? run_decode<bf16>(p, st) : run_decode<float>(p, st);
}

}  // namespace kvpop
