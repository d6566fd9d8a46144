// Host-side launchers of libkvpop (internal; the public ABI is include/kvpop.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kvpop {

// A validated problem description (see kvpop_shape in include/kvpop.h).
struct ShapeInfo {
  int B, S, Hq, Hkv, D, dtype;  // dtype: 0 = bf16, 1 = fp32
  float scale;                  // softmax scale (already defaulted)
  const int *cu;                // device offsets or nullptr
  const int *cu_host;           // host offsets or nullptr
  int n_docs;                   // documents per sequence (1 without offsets)
  int max_doc;                  // longest document
};

// Workgroups a launch may use: grid sizes are ints on the device side.
constexpr long long kMaxGridBlocks = 2147483647ll - 64;

// Workgroups of the forward (dense and budget-masked) and of the target pass
// for a validated shape, counted in 64 bits.
long long fwd_grid_blocks(const ShapeInfo &s);
long long tgt_grid_blocks(const ShapeInfo &s, int window);

hipError_t launch_fwd(const ShapeInfo &s, const void *q, const void *k, const void *v, void *o,
                      float *lse, hipStream_t st);

size_t tgt_workspace_bytes(const ShapeInfo &s);             // enough for every aggregation
size_t tgt_workspace_bytes_for(const ShapeInfo &s, int agg);  // what one aggregation uses
// The no-allocation target's scratch: a fixed array per device, and its
// address on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
constexpr int kMaxScratchDevices = 64;
hipError_t noalloc_scratch(void **out);
hipError_t launch_future_target(const ShapeInfo &s, const void *q, const void *k, const float *lse,
                                int window, int agg, int mean, float eps, float *target, void *ws,
                                hipStream_t st);

size_t budget_workspace_bytes(const ShapeInfo &s, int sinks, int window, int topk);
// Where kvpop_budget_mask_fwd leaves its per-query-block key lists in the
// workspace (byte offsets) and how they are shaped.
struct BudgetListsInfo {
  size_t lists, spans, lens, lens_full, status;
  int nqb, QB, cap, tile;
};
BudgetListsInfo budget_lists_info(const ShapeInfo &s, int sinks, int window, int topk);
hipError_t launch_budget(const ShapeInfo &s, const void *q, const void *k, const void *v,
                         const float *scores, int sinks, int window, int topk, void *o, float *lse,
                         int *rank_out, int *cutoff_out, void *ws, hipStream_t st);

size_t teacher_workspace_bytes(int B, int Hkv, int S);
hipError_t launch_teacher(int B, int Hkv, int S, const float *y, const float *lam, int delta, int sinks, int window,
                          int topk, int *label, int *boundary, int *rank_out, int *brank_out, void *ws,
                          hipStream_t st);
size_t boundary_loss_workspace_bytes(int B, int Hkv, int S);
hipError_t launch_boundary_loss(int B, int Hkv, int S, const float *pred, const int *label, const int *boundary,
                                int sinks, int window, int topk, float tau, const float *weight, float *loss,
                                float *grad, void *ws, hipStream_t st);

// Fixed-budget decoding (see kvpop_decode_shape in include/kvpop.h).
struct DecodeShapeInfo {
  int B, Hq, Hkv, D, dtype;
  float scale;
  int sinks, window, topk, C;  // C = sinks + window + topk slots
};
size_t decode_state_bytes(const DecodeShapeInfo &s);
hipError_t launch_decode_init(const DecodeShapeInfo &s, void *state, hipStream_t st);
hipError_t launch_decode_step(const DecodeShapeInfo &s, void *state, int position, const void *q, const void *k,
                              const void *v, const float *score, void *o, float *lse, hipStream_t st);

// Query heads of one GQA group handled by one forward workgroup.
inline int fwd_heads_per_block(int G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }

}  // namespace kvpop
