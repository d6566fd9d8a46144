// C ABI of libkvpop.so (declared in include/kvpop.h): host-side validation,
// workspace sizing and dispatch to the gfx950 kernels.  Every argument check
// runs before the first HIP call, so invalid calls never touch the device.
#include "kvpop.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_last_error;

kvpop_status fail(kvpop_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

kvpop_status ok() {
  g_last_error.clear();
  return KVPOP_OK;
}

// Validates the shape and fills the internal description.
kvpop_status check_shape(const kvpop_shape *sh, kvpop::ShapeInfo &s) {
  if (sh == nullptr) return fail(KVPOP_EINVAL, "shape is NULL");
  if (sh->batch < 1 || sh->seqlen < 1 || sh->n_q_heads < 1 || sh->n_kv_heads < 1)
    return fail(KVPOP_EINVAL, "batch, seqlen, n_q_heads and n_kv_heads must be >= 1");
  if (sh->n_q_heads % sh->n_kv_heads != 0)
    return fail(KVPOP_EINVAL, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", sh->n_q_heads,
                sh->n_kv_heads);
  if (sh->head_dim != 64 && sh->head_dim != 128)
    return fail(KVPOP_EUNSUPPORTED, "head_dim %d is not supported (64 or 128)", sh->head_dim);
  if (sh->dtype != KVPOP_BF16 && sh->dtype != KVPOP_F32)
    return fail(KVPOP_EUNSUPPORTED, "dtype %d is not supported", sh->dtype);
  if (sh->seqlen > (1 << 24)) return fail(KVPOP_EUNSUPPORTED, "seqlen %d exceeds 2^24", sh->seqlen);
  const double elems = (double)sh->batch * sh->n_q_heads * sh->seqlen * sh->head_dim;
  if (elems > 9.0e15) return fail(KVPOP_EUNSUPPORTED, "tensor too large");
  if ((sh->cu_seqlens == nullptr) != (sh->cu_seqlens_host == nullptr))
    return fail(KVPOP_EINVAL, "cu_seqlens and cu_seqlens_host must both be set or both be NULL");
  s.B = sh->batch;
  s.S = sh->seqlen;
  s.Hq = sh->n_q_heads;
  s.Hkv = sh->n_kv_heads;
  s.D = sh->head_dim;
  s.dtype = sh->dtype;
  s.scale = (sh->softmax_scale > 0.f) ? sh->softmax_scale : (float)(1.0 / std::sqrt((double)sh->head_dim));
  s.cu = sh->cu_seqlens;
  s.cu_host = sh->cu_seqlens_host;
  s.n_docs = 1;
  s.max_doc = sh->seqlen;
  if (sh->cu_seqlens != nullptr) {
    if (sh->batch != 1) return fail(KVPOP_EINVAL, "packed sequences (cu_seqlens) need batch == 1");
    if (sh->n_docs < 1) return fail(KVPOP_EINVAL, "n_docs must be >= 1 with cu_seqlens");
    const int32_t *c = sh->cu_seqlens_host;
    if (c[0] != 0) return fail(KVPOP_EINVAL, "cu_seqlens[0] must be 0 (got %d)", c[0]);
    int mx = 0;
    for (int m = 0; m < sh->n_docs; ++m) {
      if (c[m + 1] <= c[m])
        return fail(KVPOP_EINVAL, "cu_seqlens must rise strictly (index %d: %d -> %d)", m, c[m], c[m + 1]);
      if (c[m + 1] - c[m] > mx) mx = c[m + 1] - c[m];
    }
    if (c[sh->n_docs] != sh->seqlen)
      return fail(KVPOP_EINVAL, "cu_seqlens[n_docs] = %d but seqlen = %d", c[sh->n_docs], sh->seqlen);
    s.n_docs = sh->n_docs;
    s.max_doc = mx;
  }
  return KVPOP_OK;
}

// Alignment the kernels rely on: tensors read or written in 16-byte vectors
// (Q, K, V, O, workspaces, decode state) and 4-byte fp32/int32 arrays.  NULL
// entries are optional outputs and are skipped.
struct Aligned {
  const char *name;
  const void *ptr;
  size_t bytes;
};
kvpop_status check_alignment(std::initializer_list<Aligned> ptrs) {
  for (const Aligned &a : ptrs)
    if (a.ptr != nullptr && (reinterpret_cast<uintptr_t>(a.ptr) % a.bytes) != 0)
      return fail(KVPOP_EINVAL, "%s must be %zu-byte aligned", a.name, a.bytes);
  return KVPOP_OK;
}

kvpop_status check_device() {
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n == 0) {
    (void)hipGetLastError();
    return fail(KVPOP_EHIP, "no HIP device available (%s)", hipGetErrorString(e));
  }
  return KVPOP_OK;
}

kvpop_status from_hip(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  (void)hipGetLastError();
  return fail(KVPOP_EHIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char *kvpop_status_str(kvpop_status status) {
  switch (status) {
    case KVPOP_OK: return "ok";
    case KVPOP_EINVAL: return "invalid argument";
    case KVPOP_EUNSUPPORTED: return "unsupported configuration";
    case KVPOP_EWORKSPACE: return "workspace too small";
    case KVPOP_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *kvpop_last_error(void) { return g_last_error.c_str(); }

size_t kvpop_workspace_size(int32_t which, const kvpop_shape *shape, int32_t sinks, int32_t window,
                            int32_t topk) {
  kvpop::ShapeInfo s{};
  if (check_shape(shape, s) != KVPOP_OK) return 0;
  if (sinks < 0 || window < 0 || topk < 0) return 0;
  switch (which) {
    case KVPOP_CALL_FUTURE_TARGET: return kvpop::tgt_workspace_bytes(s);
    case KVPOP_CALL_BUDGET_MASK_FWD: return kvpop::budget_workspace_bytes(s, sinks, window, topk);
    default: return 0;
  }
}

kvpop_status kvpop_budget_lists_layout(const kvpop_shape *shape, int32_t sinks, int32_t window, int32_t topk,
                                       kvpop_lists_layout *layout) {
  kvpop::ShapeInfo s{};
  kvpop_status st = check_shape(shape, s);
  if (st != KVPOP_OK) return st;
  if (layout == nullptr) return fail(KVPOP_EINVAL, "layout is NULL");
  if (sinks < 0 || window < 0 || topk < 0)
    return fail(KVPOP_EINVAL, "sinks, window and topk must be >= 0 (got %d, %d, %d)", sinks, window, topk);
  const kvpop::BudgetListsInfo li = kvpop::budget_lists_info(s, sinks, window, topk);
  layout->lists_offset = li.lists;
  layout->spans_offset = li.spans;
  layout->lens_offset = li.lens;
  layout->lens_full_offset = li.lens_full;
  layout->status_offset = li.status;
  layout->n_query_blocks = li.nqb;
  layout->query_block = li.QB;
  layout->capacity = li.cap;
  layout->tile_keys = li.tile;
  return ok();
}

kvpop_status kvpop_attn_fwd_lse(const kvpop_shape *shape, const void *q, const void *k, const void *v,
                                void *o, float *lse, void *hip_stream) {
  kvpop::ShapeInfo s{};
  kvpop_status st = check_shape(shape, s);
  if (st != KVPOP_OK) return st;
  if (!q || !k || !v || !lse) return fail(KVPOP_EINVAL, "q, k, v and lse must be non-NULL");
  if ((st = check_alignment({{"q", q, 16}, {"k", k, 16}, {"v", v, 16}, {"o", o, 16}, {"lse", lse, 4},
                             {"cu_seqlens", s.cu, 4}})) != KVPOP_OK)
    return st;
  if (s.dtype == KVPOP_F32 && s.D != 64)
    return fail(KVPOP_EUNSUPPORTED, "the fp32 forward supports head_dim 64 only");
  if (kvpop::fwd_grid_blocks(s) > kvpop::kMaxGridBlocks)
    return fail(KVPOP_EUNSUPPORTED, "the forward would need %lld workgroups", kvpop::fwd_grid_blocks(s));
  if ((st = check_device()) != KVPOP_OK) return st;
  return from_hip(kvpop::launch_fwd(s, q, k, v, o, lse, (hipStream_t)hip_stream), "kvpop_attn_fwd_lse launch");
}

kvpop_status kvpop_future_target(const kvpop_shape *shape, const void *q, const void *k, const float *lse,
                                 int32_t window, int32_t agg, int32_t mean_over_queries, float eps,
                                 float *target, void *workspace, size_t ws_bytes, void *hip_stream) {
  kvpop::ShapeInfo s{};
  kvpop_status st = check_shape(shape, s);
  if (st != KVPOP_OK) return st;
  if (!q || !k || !lse || !target) return fail(KVPOP_EINVAL, "q, k, lse and target must be non-NULL");
  if ((st = check_alignment({{"q", q, 16}, {"k", k, 16}, {"lse", lse, 4}, {"target", target, 4},
                             {"cu_seqlens", s.cu, 4}, {"workspace", workspace, 16}})) != KVPOP_OK)
    return st;
  if (window < 0) return fail(KVPOP_EINVAL, "window must be >= 0 (got %d)", window);
  if (agg != KVPOP_AGG_SUM && agg != KVPOP_AGG_MAX && agg != KVPOP_AGG_NONE)
    return fail(KVPOP_EINVAL, "agg must be KVPOP_AGG_SUM, _MAX or _NONE (got %d)", agg);
  if (!(eps >= 0.f) || std::isinf(eps)) return fail(KVPOP_EINVAL, "eps must be finite and >= 0");
  if (kvpop::tgt_grid_blocks(s, window) > kvpop::kMaxGridBlocks)
    return fail(KVPOP_EUNSUPPORTED, "the target pass would need %lld workgroups", kvpop::tgt_grid_blocks(s, window));
  const size_t need = kvpop::tgt_workspace_bytes(s);
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(KVPOP_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : (size_t)0);
  if ((st = check_device()) != KVPOP_OK) return st;
  return from_hip(kvpop::launch_future_target(s, q, k, lse, window, agg, mean_over_queries != 0, eps, target,
                                              workspace, (hipStream_t)hip_stream),
                  "kvpop_future_target launch");
}

kvpop_status kvpop_future_target_noalloc(const kvpop_shape *shape, const void *q, const void *k, const float *lse,
                                         int32_t window, int32_t agg, int32_t mean_over_queries, float eps,
                                         float *target, void *hip_stream) {
  static_assert(KVPOP_NOALLOC_SCRATCH_BYTES == kvpop::kNoAllocScratchBytes, "header and library agree");
  kvpop::ShapeInfo s{};
  kvpop_status st = check_shape(shape, s);
  if (st != KVPOP_OK) return st;
  if (!q || !k || !lse || !target) return fail(KVPOP_EINVAL, "q, k, lse and target must be non-NULL");
  if ((st = check_alignment({{"q", q, 16}, {"k", k, 16}, {"lse", lse, 4}, {"target", target, 4},
                             {"cu_seqlens", s.cu, 4}})) != KVPOP_OK)
    return st;
  if (window < 0) return fail(KVPOP_EINVAL, "window must be >= 0 (got %d)", window);
  if (agg != KVPOP_AGG_SUM && agg != KVPOP_AGG_MAX && agg != KVPOP_AGG_NONE)
    return fail(KVPOP_EINVAL, "agg must be KVPOP_AGG_SUM, _MAX or _NONE (got %d)", agg);
  if (!(eps >= 0.f) || std::isinf(eps)) return fail(KVPOP_EINVAL, "eps must be finite and >= 0");
  if (kvpop::tgt_grid_blocks(s, window) > kvpop::kMaxGridBlocks)
    return fail(KVPOP_EUNSUPPORTED, "the target pass would need %lld workgroups", kvpop::tgt_grid_blocks(s, window));
  const size_t need = kvpop::tgt_workspace_bytes_for(s, agg);
  if (need > kvpop::kNoAllocScratchBytes)
    return fail(KVPOP_EUNSUPPORTED,
                "this shape needs %zu bytes of scratch; the no-allocation target holds %zu (use "
                "kvpop_future_target with a workspace)",
                need, kvpop::kNoAllocScratchBytes);
  if ((st = check_device()) != KVPOP_OK) return st;
  void *scratch = nullptr;
  hipError_t e = kvpop::noalloc_scratch(&scratch);
  if (e != hipSuccess) return from_hip(e, "kvpop_future_target_noalloc scratch lookup");
  return from_hip(kvpop::launch_future_target(s, q, k, lse, window, agg, mean_over_queries != 0, eps, target,
                                              scratch, (hipStream_t)hip_stream),
                  "kvpop_future_target_noalloc launch");
}

kvpop_status kvpop_budget_mask_fwd(const kvpop_shape *shape, const void *q, const void *k, const void *v,
                                   const float *scores, int32_t sinks, int32_t window, int32_t topk, void *o,
                                   float *lse, int32_t *rank_out, int32_t *cutoff_out, void *workspace,
                                   size_t ws_bytes, void *hip_stream) {
  kvpop::ShapeInfo s{};
  kvpop_status st = check_shape(shape, s);
  if (st != KVPOP_OK) return st;
  if (!q || !k || !v || !scores) return fail(KVPOP_EINVAL, "q, k, v and scores must be non-NULL");
  if ((o == nullptr) != (lse == nullptr))
    return fail(KVPOP_EINVAL, "o and lse must both be set, or both be NULL for the mask alone");
  if ((st = check_alignment({{"q", q, 16}, {"k", k, 16}, {"v", v, 16}, {"o", o, 16}, {"scores", scores, 4},
                             {"lse", lse, 4}, {"rank_out", rank_out, 4}, {"cutoff_out", cutoff_out, 4},
                             {"workspace", workspace, 16}})) != KVPOP_OK)
    return st;
  if (sinks < 0 || window < 0 || topk < 0)
    return fail(KVPOP_EINVAL, "sinks, window and topk must be >= 0 (got %d, %d, %d)", sinks, window, topk);
  if (s.dtype == KVPOP_F32 && s.D != 64)
    return fail(KVPOP_EUNSUPPORTED, "the fp32 budget forward supports head_dim 64 only");
  if ((long long)s.S * s.D * (s.dtype == KVPOP_F32 ? 4 : 2) >= (1ll << 31))
    return fail(KVPOP_EUNSUPPORTED, "the budget forward gathers keys with 32-bit offsets: seqlen * head_dim * "
                                    "element size must stay below 2^31 bytes");
  if (kvpop::fwd_grid_blocks(s) > kvpop::kMaxGridBlocks)
    return fail(KVPOP_EUNSUPPORTED, "the budget forward would need %lld workgroups", kvpop::fwd_grid_blocks(s));
  const size_t need = kvpop::budget_workspace_bytes(s, sinks, window, topk);
  if (workspace == nullptr || ws_bytes < need)
    return fail(KVPOP_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : (size_t)0);
  if ((st = check_device()) != KVPOP_OK) return st;
  return from_hip(kvpop::launch_budget(s, q, k, v, scores, sinks, window, topk, o, lse, rank_out, cutoff_out,
                                       workspace, (hipStream_t)hip_stream),
                  "kvpop_budget_mask_fwd launch");
}


static kvpop_status check_seq(int32_t batch, int32_t n_kv_heads, int32_t seqlen) {
  if (batch < 1 || n_kv_heads < 1 || seqlen < 1)
    return fail(KVPOP_EINVAL, "batch, n_kv_heads and seqlen must be >= 1");
  if (seqlen > (1 << 24)) return fail(KVPOP_EUNSUPPORTED, "seqlen %d exceeds 2^24", seqlen);
  if ((double)batch * n_kv_heads * seqlen > 2.0e9) return fail(KVPOP_EUNSUPPORTED, "tensor too large");
  return KVPOP_OK;
}

size_t kvpop_teacher_workspace_size(int32_t batch, int32_t n_kv_heads, int32_t seqlen) {
  if (check_seq(batch, n_kv_heads, seqlen) != KVPOP_OK) return 0;
  return kvpop::teacher_workspace_bytes(batch, n_kv_heads, seqlen);
}

size_t kvpop_boundary_loss_workspace_size(int32_t batch, int32_t n_kv_heads, int32_t seqlen) {
  if (check_seq(batch, n_kv_heads, seqlen) != KVPOP_OK) return 0;
  return kvpop::boundary_loss_workspace_bytes(batch, n_kv_heads, seqlen);
}

kvpop_status kvpop_teacher_labels(int32_t batch, int32_t n_kv_heads, int32_t seqlen, const float *target,
                                  const float *decay_lambda, int32_t decay_step, int32_t sinks, int32_t window,
                                  int32_t topk, int32_t *label, int32_t *boundary, int32_t *rank_out,
                                  int32_t *brank_out, void *workspace, size_t ws_bytes, void *hip_stream) {
  kvpop_status st = check_seq(batch, n_kv_heads, seqlen);
  if (st != KVPOP_OK) return st;
  if (!target || !label || !boundary) return fail(KVPOP_EINVAL, "target, label and boundary must be non-NULL");
  if ((st = check_alignment({{"target", target, 4}, {"decay_lambda", decay_lambda, 4}, {"label", label, 4},
                             {"boundary", boundary, 4}, {"rank_out", rank_out, 4}, {"brank_out", brank_out, 4},
                             {"workspace", workspace, 16}})) != KVPOP_OK)
    return st;
  if (sinks < 0 || window < 0 || topk < 0)
    return fail(KVPOP_EINVAL, "sinks, window and topk must be >= 0 (got %d, %d, %d)", sinks, window, topk);
  if (decay_step < 1) return fail(KVPOP_EINVAL, "decay_step must be >= 1 (got %d)", decay_step);
  const size_t need = kvpop::teacher_workspace_bytes(batch, n_kv_heads, seqlen);
  if (workspace == nullptr || ws_bytes < need)
    return fail(KVPOP_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : (size_t)0);
  if ((st = check_device()) != KVPOP_OK) return st;
  return from_hip(kvpop::launch_teacher(batch, n_kv_heads, seqlen, target, decay_lambda, decay_step, sinks, window,
                                        topk, label, boundary, rank_out, brank_out, workspace,
                                        (hipStream_t)hip_stream),
                  "kvpop_teacher_labels launch");
}

kvpop_status kvpop_boundary_loss(int32_t batch, int32_t n_kv_heads, int32_t seqlen, const float *pred,
                                 const int32_t *label, const int32_t *boundary, int32_t sinks, int32_t window,
                                 int32_t topk, float tau, const float *weight, float *loss, float *grad,
                                 void *workspace, size_t ws_bytes, void *hip_stream) {
  kvpop_status st = check_seq(batch, n_kv_heads, seqlen);
  if (st != KVPOP_OK) return st;
  if (!pred || !label || !boundary || !loss || !grad)
    return fail(KVPOP_EINVAL, "pred, label, boundary, loss and grad must be non-NULL");
  if ((st = check_alignment({{"pred", pred, 4}, {"label", label, 4}, {"boundary", boundary, 4},
                             {"weight", weight, 4}, {"loss", loss, 4}, {"grad", grad, 4},
                             {"workspace", workspace, 16}})) != KVPOP_OK)
    return st;
  if (sinks < 0 || window < 0 || topk < 0)
    return fail(KVPOP_EINVAL, "sinks, window and topk must be >= 0 (got %d, %d, %d)", sinks, window, topk);
  if (!(tau > 0.f) || std::isinf(tau)) return fail(KVPOP_EINVAL, "tau must be finite and > 0");
  const size_t need = kvpop::boundary_loss_workspace_bytes(batch, n_kv_heads, seqlen);
  if (workspace == nullptr || ws_bytes < need)
    return fail(KVPOP_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : (size_t)0);
  if ((st = check_device()) != KVPOP_OK) return st;
  return from_hip(kvpop::launch_boundary_loss(batch, n_kv_heads, seqlen, pred, label, boundary, sinks, window, topk,
                                              tau, weight, loss, grad, workspace, (hipStream_t)hip_stream),
                  "kvpop_boundary_loss launch");
}


static kvpop_status check_decode_shape(const kvpop_decode_shape *sh, kvpop::DecodeShapeInfo &s) {
  if (sh == nullptr) return fail(KVPOP_EINVAL, "shape is NULL");
  if (sh->batch < 1 || sh->n_q_heads < 1 || sh->n_kv_heads < 1)
    return fail(KVPOP_EINVAL, "batch, n_q_heads and n_kv_heads must be >= 1");
  if (sh->n_q_heads % sh->n_kv_heads != 0)
    return fail(KVPOP_EINVAL, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", sh->n_q_heads, sh->n_kv_heads);
  if (sh->n_q_heads / sh->n_kv_heads > 8)
    return fail(KVPOP_EUNSUPPORTED, "decoding supports at most 8 query heads per KV head");
  if (sh->head_dim != 64 && sh->head_dim != 128)
    return fail(KVPOP_EUNSUPPORTED, "head_dim %d is not supported (64 or 128)", sh->head_dim);
  if (sh->dtype != KVPOP_BF16 && sh->dtype != KVPOP_F32)
    return fail(KVPOP_EUNSUPPORTED, "dtype %d is not supported", sh->dtype);
  if (sh->sinks < 0 || sh->window < 0 || sh->topk < 0)
    return fail(KVPOP_EINVAL, "sinks, window and topk must be >= 0");
  const long long C = (long long)sh->sinks + sh->window + sh->topk;
  if (C < 1) return fail(KVPOP_EINVAL, "the cache needs at least one slot (sinks + window + topk >= 1)");
  if (C > (1 << 20)) return fail(KVPOP_EUNSUPPORTED, "cache of %lld slots exceeds 2^20", C);
  s.B = sh->batch;
  s.Hq = sh->n_q_heads;
  s.Hkv = sh->n_kv_heads;
  s.D = sh->head_dim;
  s.dtype = sh->dtype;
  s.scale = (sh->softmax_scale > 0.f) ? sh->softmax_scale : (float)(1.0 / std::sqrt((double)sh->head_dim));
  s.sinks = sh->sinks;
  s.window = sh->window;
  s.topk = sh->topk;
  s.C = (int)C;
  return KVPOP_OK;
}

size_t kvpop_decode_state_size(const kvpop_decode_shape *shape) {
  kvpop::DecodeShapeInfo s{};
  if (check_decode_shape(shape, s) != KVPOP_OK) return 0;
  return kvpop::decode_state_bytes(s);
}

kvpop_status kvpop_decode_init(const kvpop_decode_shape *shape, void *state, size_t state_bytes, void *hip_stream) {
  kvpop::DecodeShapeInfo s{};
  kvpop_status st = check_decode_shape(shape, s);
  if (st != KVPOP_OK) return st;
  if (state == nullptr || state_bytes < kvpop::decode_state_bytes(s))
    return fail(KVPOP_EWORKSPACE, "decode state of %zu bytes needed", kvpop::decode_state_bytes(s));
  if ((st = check_alignment({{"state", state, 16}})) != KVPOP_OK) return st;
  if ((st = check_device()) != KVPOP_OK) return st;
  return from_hip(kvpop::launch_decode_init(s, state, (hipStream_t)hip_stream), "kvpop_decode_init launch");
}

kvpop_status kvpop_decode_step(const kvpop_decode_shape *shape, void *state, size_t state_bytes, int32_t position,
                               const void *q, const void *k, const void *v, const float *score, void *o, float *lse,
                               void *hip_stream) {
  kvpop::DecodeShapeInfo s{};
  kvpop_status st = check_decode_shape(shape, s);
  if (st != KVPOP_OK) return st;
  if (!q || !k || !v || !score || !o || !lse)
    return fail(KVPOP_EINVAL, "q, k, v, score, o and lse must be non-NULL");
  if (position < 0) return fail(KVPOP_EINVAL, "position must be >= 0 (got %d)", position);
  if (state == nullptr || state_bytes < kvpop::decode_state_bytes(s))
    return fail(KVPOP_EWORKSPACE, "decode state of %zu bytes needed", kvpop::decode_state_bytes(s));
  if ((st = check_alignment({{"q", q, 16}, {"k", k, 16}, {"v", v, 16}, {"o", o, 16}, {"score", score, 4},
                             {"lse", lse, 4}, {"state", state, 16}})) != KVPOP_OK)
    return st;
  if ((st = check_device()) != KVPOP_OK) return st;
  return from_hip(kvpop::launch_decode_step(s, state, position, q, k, v, score, o, lse, (hipStream_t)hip_stream),
                  "kvpop_decode_step launch");
}

}  // extern "C"
