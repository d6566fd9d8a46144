// Device-side building blocks shared by the gfx950 kernels of libkvpop.
//
// Matrix-core convention used everywhere (CDNA4 v_mfma_f32_32x32x16_bf16 and
// v_mfma_f32_32x32x2_f32):
//   * A operand: lane l supplies row (l % 32) of a 32 x 16 slice, the eight
//     contraction indices 8*(l/32) .. 8*(l/32)+7 ("k-chunk" of that lane half);
//   * B operand: lane l supplies column (l % 32), same eight contraction
//     indices;
//   * C/D: lane l, register i holds element
//       row 8*(i/4) + 4*(l/32) + (i%4), column l % 32.
// A k-chunk is eight consecutive elements of a row in memory, so one 16-byte
// load (bf16) or two (fp32) fill it.  For fp32 the 16-wide k-step is issued
// as eight 32x32x2 instructions, one per element of the chunk; the logical
// layout is the same, so every kernel is written once for both types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace kvpop {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

template <typename T> struct Frag;
template <> struct Frag<bf16> {
  bf16x8 v;
};
template <> struct Frag<float> {
  f32x4 lo, hi;
};

__device__ __forceinline__ void mma(f32x16 &acc, const Frag<bf16> &a, const Frag<bf16> &b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16 &acc, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[e], b.lo[e], acc, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[e], b.hi[e], acc, 0, 0, 0);
}
// d = a * b + c with a separate addend tile (c is not overwritten).
__device__ __forceinline__ f32x16 mma_add(const Frag<bf16> &a, const Frag<bf16> &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma_add(const Frag<float> &a, const Frag<float> &b, const f32x16 &c) {
  f32x16 d = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[0], b.lo[0], c, 0, 0, 0);
#pragma unroll
  for (int e = 1; e < 4; ++e) d = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[e], b.lo[e], d, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) d = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[e], b.hi[e], d, 0, 0, 0);
  return d;
}

// Multiplies a fragment by x, rounding each element back to the fragment type
// (round to nearest even for bf16).

// Eight consecutive elements starting at p (16-byte aligned).
__device__ __forceinline__ void load_frag(Frag<bf16> &f, const bf16 *p) {
  f.v = *reinterpret_cast<const bf16x8 *>(p);
}
__device__ __forceinline__ void load_frag(Frag<float> &f, const float *p) {
  f.lo = *reinterpret_cast<const f32x4 *>(p);
  f.hi = *reinterpret_cast<const f32x4 *>(p + 4);
}

// Row i of an MFMA C/D tile held by lane-half `hf` in register i.
__device__ __forceinline__ constexpr int c_row(int i, int hf) { return 8 * (i / 4) + 4 * hf + (i % 4); }

// ---------------------------------------------------------------------------
// LDS tiles of ROWS x D elements of T, stored in 16-byte chunks with an XOR
// swizzle so that 16 lanes reading the same column chunk of 16 different rows
// hit 16 different bank groups (64 banks x 4 bytes).
template <typename T, int D>
struct SwizzledTile {
  static constexpr int kRowBytes = D * (int)sizeof(T);
  static constexpr int kChunks = kRowBytes / 16;
  __device__ static __forceinline__ int swz(int r) {
    return kRowBytes == 128 ? ((r >> 1) & 7) : (r & 15);
  }
  // byte offset of chunk c of row r
  __device__ static __forceinline__ int off(int r, int c) { return r * kRowBytes + ((c ^ swz(r)) << 4); }
  // bf16 k-chunk stored at byte offset o (a value of off())
  __device__ static __forceinline__ void read_at(Frag<bf16> &f, const char *base, int o) {
    f.v = *reinterpret_cast<const bf16x8 *>(base + o);
  }
  // k-chunk (8 elements starting at element e0, a multiple of 8) of row r
  __device__ static __forceinline__ void read(Frag<T> &f, const char *base, int r, int e0) {
    constexpr int kChunkElems = 16 / (int)sizeof(T);
    const int c = e0 / kChunkElems;
    if constexpr (sizeof(T) == 2) {
      f.v = *reinterpret_cast<const bf16x8 *>(base + off(r, c));
    } else {
      f.lo = *reinterpret_cast<const f32x4 *>(base + off(r, c));
      f.hi = *reinterpret_cast<const f32x4 *>(base + off(r, c + 1));
    }
  }
};

// ---------------------------------------------------------------------------
// Document of position pos: the last m with cu[m] <= pos (cu rises strictly
// from 0 to S).  Without offsets the whole row is one document.
struct Doc {
  int start, end;
};
__device__ __forceinline__ Doc find_doc(const int *cu, int n_docs, int S, int pos) {
  if (cu == nullptr) return Doc{0, S};
  int lo = 0, hi = n_docs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (__ldg(cu + mid) <= pos) lo = mid; else hi = mid - 1;
  }
  return Doc{__ldg(cu + lo), __ldg(cu + lo + 1)};
}

// Raw buffer resource over [base, base + bytes) (gfx9 descriptor, no
// swizzle, stride 0): a load at an offset >= bytes returns zero instead of
// touching memory, so tile loads need no per-lane clamping.
constexpr int kBufferDword3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, kBufferDword3);
}

// Buffer loads that write straight into LDS: lane l stores its `bytes`
// (4 or 16) at lds + l * bytes.  Out-of-range lanes store zeros.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, void *lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, void *lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4, voff, 0, 0, 0);
}

// f(std::integral_constant<int, i>{}) for i = 0 .. N-1, in order
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace kvpop
