// Fixed-budget decoding for gfx950 (kvpop_decode_init, kvpop_decode_step).
//
// KVpop paper, Section 3: every KV head keeps s sink tokens, a protected
// window of the w most recent tokens, and the k best eligible tokens by
// static priority, so the per-head cache never exceeds B = s + w + k tokens
// (the paper text's results section, Inference efficiency and Fig. 4, and
// Section 4.3 of the Korean summary measure the resulting flat memory at
// decode time).  Each
// step (Section 3.2, "Running top-k sparse attention"): the new token enters
// the window; token d-w leaves it and competes for the top-k; if the top-k is
// full and the newcomer beats the worst retained token, that token is
// evicted for good (with static priorities a dropped token can never return:
// the set of better tokens only grows).  The query then attends over the
// retained tokens, which are exactly the budget mask's row d.
//
// State per (batch row, KV head), caller-owned device memory:
//   slot K, V   [C, D], C = s + R + k with R = w + 1 ring slots (0 if w = 0):
//               slots [0, s) sinks, [s, s+R) the window ring (token t >= s
//               at s + t mod R), [s+R, C) the top-k set in fill order;
//   slot pos    [C] int32, -1 when empty;  slot key [C] uint64, the order
//               key (descending priority, then ascending index);
//   count, worst slot and worst key of the top-k, two copies each, selected
//               by the parity of the step (one is read, the other written);
//   chunk partials of the attention.
// The ring has one slot more than the window so that within one step the
// token that leaves the window (d-w) and the token that enters it (d) never
// share a slot: the row of d-w is read (to copy it into the top-k) while the
// row of d is written, by different workgroups with no ordering between
// them.
//
// One step is two launches:
//   decode_step_kernel  one workgroup per (64-slot chunk, b, KV head).
//                       Every workgroup of (b, h) takes the same insert /
//                       evict decision from the state, attends over its
//                       chunk with this step's changes substituted (the
//                       leaving token masked, the entering token and the new
//                       token read from their sources), then writes the
//                       slots of its chunk that change; the chunk-0
//                       workgroup writes the next step's count and worst key;
//   decode_combine      merges the chunk partials per query head.  (A merge
//                       by the last workgroup to finish needs device-scope
//                       release fences, which write back the whole L2 on
//                       this chip and cost far more than a second launch.)
#include "common.h"
#include "launch.h"

namespace kvpop {

constexpr int DEC_CHUNK = 64;                    // slots per workgroup
// Waves per workgroup: 8, of 8 slot rows each.  64-slot chunks give 264
// workgroups at one batch row, 8 KV heads and a 2048-token budget, enough to
// reach every CU; 128-slot chunks left half of them idle (16.0 against
// 14.3 us per step).
__host__ __device__ constexpr int dec_waves(int) { return 8; }
constexpr int DEC_MAX_SLOTS = (1 << 20) + 1;     // the C-ABI allows s + w + k <= 2^20
constexpr int DEC_MAX_CHUNKS = (DEC_MAX_SLOTS + DEC_CHUNK - 1) / DEC_CHUNK;

__device__ __forceinline__ uint64_t decode_key(float sc, int t) {
  if (sc != sc) sc = -INFINITY;
  if (sc == 0.f) sc = 0.f;
  const uint32_t u = __float_as_uint(sc);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)(~ord) << 32) | (uint32_t)t;
}

static int decode_ring(int w) { return w > 0 ? w + 1 : 0; }
static int decode_slots(const DecodeShapeInfo &s) { return s.sinks + decode_ring(s.window) + s.topk; }

struct DecodeState {
  void *k, *v;
  int *pos;
  uint64_t *key;
  int *count;      // [BH][2]
  int *wslot;      // [BH][2]
  uint64_t *wkey;  // [BH][2]
  float *part;     // [B*Hq][nchunk][D + 2]
};

static DecodeState decode_state_view(const DecodeShapeInfo &s, void *base, size_t *total = nullptr) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t BH = (size_t)s.B * s.Hkv, C = (size_t)decode_slots(s);
  const size_t es = s.dtype == 0 ? 2 : 4;
  const size_t nch = (C + DEC_CHUNK - 1) / DEC_CHUNK;
  const uintptr_t p = reinterpret_cast<uintptr_t>(base);
  DecodeState st{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    void *q = reinterpret_cast<void *>(p + off);
    off = al(off + bytes);
    return q;
  };
  st.k = take(BH * C * s.D * es);
  st.v = take(BH * C * s.D * es);
  st.pos = reinterpret_cast<int *>(take(BH * C * 4));
  st.key = reinterpret_cast<uint64_t *>(take(BH * C * 8));
  st.count = reinterpret_cast<int *>(take(BH * 2 * 4));
  st.wslot = reinterpret_cast<int *>(take(BH * 2 * 4));
  st.wkey = reinterpret_cast<uint64_t *>(take(BH * 2 * 8));
  st.part = reinterpret_cast<float *>(take((size_t)s.B * s.Hq * nch * (s.D + 2) * 4));
  if (total) *total = off;
  return st;
}

size_t decode_state_bytes(const DecodeShapeInfo &s) {
  size_t total = 0;
  decode_state_view(s, nullptr, &total);
  return total;
}

struct DecParams {
  DecodeState st;
  const void *q, *k, *v;
  const float *score;
  void *o;
  float *lse;
  int B, Hq, Hkv, G, D, C, R, sinks, window, topk, d, nchunk, dtype;
  float scale_log2;
};

__global__ void __launch_bounds__(256) decode_init_kernel(DecParams p) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t n = (size_t)p.B * p.Hkv * p.C;
  if (i < n) {
    p.st.pos[i] = -1;
    p.st.key[i] = ~0ull;
  }
  if (i < (size_t)p.B * p.Hkv * 2) {
    p.st.count[i] = 0;
    p.st.wslot[i] = -1;
    p.st.wkey[i] = 0ull;
  }
}

// Eight consecutive elements of a slot row, moved with 16-byte accesses.
template <typename T>
struct Row8;
template <>
struct Row8<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16 *src) { v = *reinterpret_cast<const bf16x8 *>(src); }
  __device__ __forceinline__ void store(bf16 *dst) const { *reinterpret_cast<bf16x8 *>(dst) = v; }
  __device__ __forceinline__ float operator[](int e) const { return (float)v[e]; }
};
template <>
struct Row8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float *src) {
    a = *reinterpret_cast<const f32x4 *>(src);
    b = *reinterpret_cast<const f32x4 *>(src + 4);
  }
  __device__ __forceinline__ void store(float *dst) const {
    *reinterpret_cast<f32x4 *>(dst) = a;
    *reinterpret_cast<f32x4 *>(dst + 4) = b;
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

// The decision of step d for one (b, h), the same in every workgroup: the
// ring slot of the leaving token e = d - w, whether e enters the top-k and
// where, and the slot of the new token.
struct DecStep {
  int e, ring_e;  // leaving token and its ring slot (-1 if none)
  int n;          // top-k count before the step
  uint64_t ke;    // order key of e
  int target;     // top-k slot that receives e (-1: e does not enter)
  int slot_new;   // slot of the new token d (-1: with w = 0 it only competes)
};

__device__ __forceinline__ DecStep decode_decide(const DecParams &p, int bh) {
  DecStep x;
  const int s = p.sinks, w = p.window, k = p.topk, d = p.d, cur = d & 1;
  const uint64_t *key = p.st.key + (size_t)bh * p.C;
  x.e = d - w;
  const bool compete = k > 0 && x.e >= s;
  x.ring_e = (w > 0 && x.e >= s) ? s + x.e % p.R : -1;
  x.n = p.st.count[bh * 2 + cur];
  x.ke = compete ? (w > 0 ? key[x.ring_e] : decode_key(p.score[bh], d)) : 0ull;
  x.target = -1;
  if (compete) {
    if (x.n < k) x.target = s + p.R + x.n;
    else if (x.ke < p.st.wkey[bh * 2 + cur]) x.target = p.st.wslot[bh * 2 + cur];
  }
  x.slot_new = d < s ? d : (w > 0 ? s + d % p.R : -1);
  return x;
}

// Workgroup (chunk, b*Hkv + h): the G query heads of KV head h against slots
// [chunk*DEC_CHUNK, +DEC_CHUNK) of the state after this step's update.  The
// attention is bound by latency, not by bandwidth or arithmetic, so the chunk
// is spread over dec_waves(G) waves of DEC_ROWS rows each, and every wave issues
// all of its K, V and position loads before it computes anything.  Lane l
// covers 8 elements at 8*(l % LPR) of a slot row (LPR = D/8 lanes per row,
// RPW = 64/LPR rows per load instruction).  Phases:
//   1. logits: per-lane partial dot products finished by a DPP sum over the
//      LPR lanes of a row, written to LDS (-inf for empty slots);
//   2. one wave per query head reduces that head's maximum and sum of
//      exponentials over the chunk;
//   3. each wave forms its rows' probabilities and partial PV sums, reduced
//      over the rows of the wave, then over the waves through LDS;
//   4. the slots of this chunk that change in this step are written, and
//      chunk 0 writes the next step's count and worst retained token.
// G (query heads per KV head) and D are template parameters so that register
// arrays are indexed statically and every reduction is unrolled.
template <typename T, int G, int D>
__global__ void __launch_bounds__(dec_waves(G) * 64) decode_step_kernel(DecParams p) {
  constexpr int DEC_WAVES = dec_waves(G);
  constexpr int DEC_ROWS = DEC_CHUNK / DEC_WAVES;  // slot rows per wave
  constexpr int EPL = 8;               // elements per lane and row
  constexpr int LPR = D / EPL;         // lanes per row: 16 (D=128) or 8 (D=64)
  constexpr int RPW = 64 / LPR;        // rows per load instruction: 4 or 8
  constexpr int NRG = DEC_ROWS / RPW;  // row groups per wave
  static_assert(DEC_ROWS % RPW == 0, "whole row groups per wave");
  static_assert(G <= DEC_WAVES, "one wave per query head in phase 2");
  __shared__ float lg[G][DEC_CHUNK];
  __shared__ float ml[G][2];  // per head: maximum (log2 units) and sum
  __shared__ float osum[DEC_WAVES][G][D];
  __shared__ uint64_t red_key[DEC_WAVES];
  __shared__ int red_slot[DEC_WAVES];
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.Hkv, h = bh % p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r_in = lane / LPR, c = lane % LPR;
  T *sk = reinterpret_cast<T *>(p.st.k) + (size_t)bh * p.C * D;
  T *sv = reinterpret_cast<T *>(p.st.v) + (size_t)bh * p.C * D;
  int *pos = p.st.pos + (size_t)bh * p.C;
  uint64_t *key = p.st.key + (size_t)bh * p.C;
  const T *knew = reinterpret_cast<const T *>(p.k) + (size_t)bh * D;
  const T *vnew = reinterpret_cast<const T *>(p.v) + (size_t)bh * D;
  const int j0 = chunk * DEC_CHUNK;
  const int nslots = min(DEC_CHUNK, p.C - j0);
  // Every load of this wave is issued before anything waits on one: the
  // chunk's slot rows and positions, the two rows a step can substitute (the
  // leaving token's, from its ring slot, and the new token's), and the
  // decision's inputs.  The decision then picks, per row, which data is the
  // slot's after this step.  Rows past the chunk's end re-read its last row
  // and are masked.
  const int ring_e = (p.window > 0 && p.d - p.window >= p.sinks) ? p.sinks + (p.d - p.window) % p.R : -1;
  const T *ek = ring_e >= 0 ? sk + (size_t)ring_e * D : knew;  // source of the token entering the top-k
  const T *ev = ring_e >= 0 ? sv + (size_t)ring_e * D : vnew;
  Row8<T> kr[NRG], vr[NRG], ke8, ve8, kn8, vn8;
  int pj[NRG];
#pragma unroll
  for (int i = 0; i < NRG; ++i) {
    const int j = wave * DEC_ROWS + i * RPW + r_in;
    const int jj = j0 + min(j, nslots - 1);
    kr[i].load(sk + (size_t)jj * D + c * EPL);
    vr[i].load(sv + (size_t)jj * D + c * EPL);
    pj[i] = pos[jj];
  }
  ke8.load(ek + c * EPL);
  ve8.load(ev + c * EPL);
  kn8.load(knew + c * EPL);
  vn8.load(vnew + c * EPL);
  // chunk 0 keeps the top-k's worst key up to date for the next step.  The
  // only slot an eviction can empty is the current worst W, so the largest
  // key of the other slots is all it needs besides the entering key; its
  // loads go out here with the rest.
  constexpr int SCAN = 4;  // keys per thread in flight (4096 slots per pass)
  const int cur = p.d & 1, kb = p.sinks + p.R;
  const int w_cur = p.st.wslot[bh * 2 + cur];
  uint64_t ex_best = 0;
  int ex_slot = -1;
  auto scan_pass = [&](int base) {
    uint64_t kk[SCAN];
#pragma unroll
    for (int u = 0; u < SCAN; ++u) {
      const int j = base + tid + u * DEC_WAVES * 64;
      kk[u] = j < p.topk ? key[kb + j] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < SCAN; ++u) {
      const int j = base + tid + u * DEC_WAVES * 64;
      if (j < p.topk && kb + j != w_cur && (ex_slot < 0 || kk[u] > ex_best)) {
        ex_best = kk[u];
        ex_slot = kb + j;
      }
    }
  };
  const bool full_topk = p.topk > 0 && p.st.count[bh * 2 + cur] == p.topk;
  if (chunk == 0 && full_topk) scan_pass(0);
  const DecStep x = decode_decide(p, bh);
  bool ok[NRG];
#pragma unroll
  for (int i = 0; i < NRG; ++i) {
    const int j = wave * DEC_ROWS + i * RPW + r_in;
    const int jj = j0 + min(j, nslots - 1);
    bool valid = pj[i] >= 0 && jj != x.ring_e;
    if (jj == x.target) {
      kr[i] = ke8;
      vr[i] = ve8;
      valid = true;
    }
    if (jj == x.slot_new) {
      kr[i] = kn8;
      vr[i] = vn8;
      valid = true;
    }
    ok[i] = j < nslots && valid;
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
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) s += qv[g][e] * kr[i][e];
      s = lane_group_sum<LPR>(s);
      if (c == 0) lg[g][j] = ok[i] ? s * p.scale_log2 : -INFINITY;
    }
  }
  __syncthreads();

  // 2. wave g: maximum and sum of exponentials of head g over the chunk
  if (wave < G) {
    const int g = wave;
    constexpr int PER = DEC_CHUNK / 64;  // logits per lane
    float xs[PER];
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      xs[u] = lg[g][lane + 64 * u];
      m = fmaxf(m, xs[u]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float mu = m == -INFINITY ? 0.f : m;
    float l = 0.f;
#pragma unroll
    for (int u = 0; u < PER; ++u) l += exp2f(xs[u] - mu);  // -inf: 0
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
      const float pg = ok[i] ? exp2f(lg[g][j] - ml[g][0]) : 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] += pg * vf[e];
    }
  }
  // reduce over the row groups of the wave (lanes with the same c)
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float s = acc[g][e];
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) s += __shfl_xor(s, o);
      acc[g][e] = s;
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

  // 4. the slots of this chunk that change; only this workgroup read their
  // rows above, and the entering token's source row is not written in this
  // step
  if (x.target >= j0 && x.target < j0 + nslots) {
    for (int e0 = tid * EPL; e0 < D; e0 += DEC_WAVES * 64 * EPL) {
      Row8<T> r;
      r.load(ek + e0);
      r.store(sk + (size_t)x.target * D + e0);
      r.load(ev + e0);
      r.store(sv + (size_t)x.target * D + e0);
    }
    if (tid == 0) {
      pos[x.target] = x.e;
      key[x.target] = x.ke;
    }
  }
  if (x.slot_new >= j0 && x.slot_new < j0 + nslots) {
    for (int e0 = tid * EPL; e0 < D; e0 += DEC_WAVES * 64 * EPL) {
      Row8<T> r;
      r.load(knew + e0);
      r.store(sk + (size_t)x.slot_new * D + e0);
      r.load(vnew + e0);
      r.store(sv + (size_t)x.slot_new * D + e0);
    }
    if (tid == 0) {
      pos[x.slot_new] = p.d;
      key[x.slot_new] = decode_key(p.score[bh], p.d);
    }
  }
  // the next step's count and worst retained token (chunk 0 of (b, h)); no
  // key read here is written in this step
  if (chunk == 0) {
    const int nxt = cur ^ 1;
    const int k = p.topk;
    int ws = w_cur;
    uint64_t wk = p.st.wkey[bh * 2 + cur];
    if (x.target >= 0 && x.n < k) {  // filling: the worst is the largest key so far
      if (x.n == 0 || x.ke > wk) {
        ws = x.target;
        wk = x.ke;
      }
    } else if (x.target >= 0) {  // W was evicted: the larger of the others' maximum and e's key
      for (int base = SCAN * DEC_WAVES * 64; base < k; base += SCAN * DEC_WAVES * 64) scan_pass(base);
      for (int o = 32; o > 0; o >>= 1) {
        const uint64_t ob = __shfl_xor(ex_best, o);
        const int os = __shfl_xor(ex_slot, o);
        if (os >= 0 && (ex_slot < 0 || ob > ex_best)) {
          ex_best = ob;
          ex_slot = os;
        }
      }
      if (lane == 0) {
        red_key[wave] = ex_best;
        red_slot[wave] = ex_slot;
      }
      __syncthreads();
      ws = x.target;
      wk = x.ke;
      for (int q = 0; q < DEC_WAVES; ++q)
        if (red_slot[q] >= 0 && red_key[q] > wk) {
          wk = red_key[q];
          ws = red_slot[q];
        }
    }
    if (tid == 0) {
      p.st.count[bh * 2 + nxt] = x.n + ((x.target >= 0 && x.n < k) ? 1 : 0);
      p.st.wslot[bh * 2 + nxt] = ws;
      p.st.wkey[bh * 2 + nxt] = wk;
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
  p.R = decode_ring(s.window);
  p.C = decode_slots(s);
  p.sinks = s.sinks;
  p.window = s.window;
  p.topk = s.topk;
  p.nchunk = (p.C + DEC_CHUNK - 1) / DEC_CHUNK;
  p.dtype = s.dtype;
  p.scale_log2 = s.scale * kLog2e;
  return p;
}

hipError_t launch_decode_init(const DecodeShapeInfo &s, void *state, hipStream_t st) {
  DecParams p = decode_params(s, state);
  const size_t slots = (size_t)p.B * p.Hkv * p.C, books = (size_t)p.B * p.Hkv * 2;
  const size_t n = slots > books ? slots : books;
  hipLaunchKernelGGL(decode_init_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <typename T, int D>
static bool launch_step_g(const DecParams &p, dim3 grid, hipStream_t st) {
  const dim3 block(dec_waves(p.G) * 64);
  switch (p.G) {
    case 1: hipLaunchKernelGGL((decode_step_kernel<T, 1, D>), grid, block, 0, st, p); return true;
    case 2: hipLaunchKernelGGL((decode_step_kernel<T, 2, D>), grid, block, 0, st, p); return true;
    case 3: hipLaunchKernelGGL((decode_step_kernel<T, 3, D>), grid, block, 0, st, p); return true;
    case 4: hipLaunchKernelGGL((decode_step_kernel<T, 4, D>), grid, block, 0, st, p); return true;
    case 5: hipLaunchKernelGGL((decode_step_kernel<T, 5, D>), grid, block, 0, st, p); return true;
    case 6: hipLaunchKernelGGL((decode_step_kernel<T, 6, D>), grid, block, 0, st, p); return true;
    case 7: hipLaunchKernelGGL((decode_step_kernel<T, 7, D>), grid, block, 0, st, p); return true;
    case 8: hipLaunchKernelGGL((decode_step_kernel<T, 8, D>), grid, block, 0, st, p); return true;
    default: return false;
  }
}

template <typename T>
static hipError_t run_decode(DecParams &p, hipStream_t st) {
  const dim3 grid(p.nchunk, p.B * p.Hkv);
  const bool ok = p.D == 128 ? launch_step_g<T, 128>(p, grid, st)
                : p.D == 64  ? launch_step_g<T, 64>(p, grid, st)
                             : false;
  if (!ok) return hipErrorInvalidValue;
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
