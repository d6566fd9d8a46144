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

// Workgroup (chunk, b*Hkv + h): the G query heads of KV head h against slots
// [chunk*DEC_CHUNK, +DEC_CHUNK).  Thread j owns slot j of the chunk for the
// logits; the partial output is accumulated per (head, dimension).
template <typename T>
__global__ void __launch_bounds__(256) decode_attn(DecParams p) {
  __shared__ float qs[8][256];           // up to 8 query heads, D <= 256
  __shared__ float pr[8][DEC_CHUNK];     // probabilities of the chunk
  __shared__ int vld[DEC_CHUNK];         // slot holds a retained token
  __shared__ float red[8][4];
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.Hkv, h = bh % p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G, D = p.D;
  const T *sk = reinterpret_cast<const T *>(p.st.k) + (size_t)bh * p.C * D;
  const T *sv = reinterpret_cast<const T *>(p.st.v) + (size_t)bh * p.C * D;
  const int *pos = p.st.pos + (size_t)bh * p.C;
  for (int i = tid; i < G * D; i += 256) {
    const int g = i / D, e = i % D;
    qs[g][e] = (float)reinterpret_cast<const T *>(p.q)[((size_t)b * p.Hq + h * G + g) * D + e];
  }
  __syncthreads();
  const int j0 = chunk * DEC_CHUNK;
  // logits (log2 units) of slot tid for every head; invalid slots are -inf
  float lg[8];
  const int slot = j0 + tid;
  const bool valid = tid < DEC_CHUNK && slot < p.C && pos[slot] >= 0;
  if (tid < DEC_CHUNK) vld[tid] = valid ? 1 : 0;
#pragma unroll
  for (int g = 0; g < 8; ++g) lg[g] = -INFINITY;
  if (valid) {
    const T *kr = sk + (size_t)slot * D;
    for (int g = 0; g < G; ++g) {
      float acc = 0.f;
      for (int e = 0; e < D; ++e) acc += qs[g][e] * (float)kr[e];
      lg[g] = acc * p.scale_log2;
    }
  }
  // per-head max over the chunk
  float mx[8];
  for (int g = 0; g < G; ++g) {
    float m = lg[g];
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) red[g][wave] = m;
  }
  __syncthreads();
  for (int g = 0; g < G; ++g) mx[g] = fmaxf(fmaxf(red[g][0], red[g][1]), fmaxf(red[g][2], red[g][3]));
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    const float m = mx[g] == -INFINITY ? 0.f : mx[g];
    const float pv = valid ? exp2f(lg[g] - m) : 0.f;
    if (tid < DEC_CHUNK) pr[g][tid] = pv;
    float l = pv;
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
    if (lane == 0) red[g][wave] = l;
  }
  __syncthreads();
  // partial output: thread (g, e) sums over the chunk's slots in order
  const int nslots = min(DEC_CHUNK, p.C - j0);
  for (int i = tid; i < G * D; i += 256) {
    const int g = i / D, e = i % D;
    float acc = 0.f;
    for (int j = 0; j < nslots; ++j)  // empty slots hold no data (possibly not even numbers)
      if (vld[j]) acc += pr[g][j] * (float)sv[(size_t)(j0 + j) * D + e];
    float *pp = p.st.part + (((size_t)b * p.Hq + h * G + g) * p.nchunk + chunk) * (D + 2);
    pp[e] = acc;
    if (e == 0) {
      pp[D] = mx[g];
      pp[D + 1] = red[g][0] + red[g][1] + red[g][2] + red[g][3];
    }
  }
}

// One workgroup per (b, query head): merge the chunks.
template <typename T>
__global__ void __launch_bounds__(256) decode_combine(DecParams p) {
  const int bg = blockIdx.x;
  const int D = p.D;
  const float *pp = p.st.part + (size_t)bg * p.nchunk * (D + 2);
  float m = -INFINITY;
  for (int c = 0; c < p.nchunk; ++c) m = fmaxf(m, pp[c * (D + 2) + D]);
  const float mu = m == -INFINITY ? 0.f : m;
  float l = 0.f;
  for (int c = 0; c < p.nchunk; ++c) {
    const float mc = pp[c * (D + 2) + D];
    if (mc != -INFINITY) l += pp[c * (D + 2) + D + 1] * exp2f(mc - mu);
  }
  for (int e = threadIdx.x; e < D; e += 256) {
    float acc = 0.f;
    for (int c = 0; c < p.nchunk; ++c) {
      const float mc = pp[c * (D + 2) + D];
      if (mc != -INFINITY) acc += pp[c * (D + 2) + e] * exp2f(mc - mu);
    }
    reinterpret_cast<T *>(p.o)[(size_t)bg * D + e] = (T)(l > 0.f ? acc / l : 0.f);
  }
  if (threadIdx.x == 0) p.lse[bg] = l > 0.f ? (mu + log2f(l)) * kLn2 : -INFINITY;
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

template <typename T>
static hipError_t run_decode(DecParams &p, hipStream_t st) {
  hipLaunchKernelGGL(decode_update<T>, dim3(p.B * p.Hkv), dim3(256), 0, st, p);
  hipLaunchKernelGGL(decode_attn<T>, dim3(p.nchunk, p.B * p.Hkv), dim3(256), 0, st, p);
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
