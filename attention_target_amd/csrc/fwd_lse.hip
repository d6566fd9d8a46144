// Dense causal attention forward with LSE (kvpop_attn_fwd_lse).
#include "attn_fwd.h"
#include "launch.h"

namespace kvpop {

template <typename T, int D, bool WO>
static hipError_t run_fwd(const FwdParams &fp, int grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, WO, false>), dim3(grid), dim3(256), 0, st, fp);
  return hipGetLastError();
}

long long fwd_grid_blocks(const ShapeInfo &s) {
  const int G = s.Hq / s.Hkv, HG = fwd_heads_per_block(G);
  const long long QB = 32 * (4 / HG);
  return (s.S + QB - 1) / QB * s.B * s.Hkv * (G / HG);
}

hipError_t launch_fwd(const ShapeInfo &s, const void *q, const void *k, const void *v, void *o,
                      float *lse, hipStream_t st) {
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
  const int QB = 32 * (4 / fp.HG);
  const int nqb = (s.S + QB - 1) / QB;
  const int grid = nqb * s.B * s.Hkv * (fp.G / fp.HG);
  const bool wo = (o != nullptr);
  if (s.dtype == 0 && s.D == 128) return wo ? run_fwd<bf16, 128, true>(fp, grid, st) : run_fwd<bf16, 128, false>(fp, grid, st);
  if (s.dtype == 0 && s.D == 64) return wo ? run_fwd<bf16, 64, true>(fp, grid, st) : run_fwd<bf16, 64, false>(fp, grid, st);
  if (s.dtype == 1 && s.D == 64) return wo ? run_fwd<float, 64, true>(fp, grid, st) : run_fwd<float, 64, false>(fp, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace kvpop
