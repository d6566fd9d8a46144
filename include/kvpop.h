/*
 * kvpop.h -- C ABI of libkvpop.so: the training-time hot path of KVpop
 * (future-attention target and fixed-budget sparse attention) on AMD
 * Instinct MI355X (gfx950).
 *
 * Sources: "KVpop -- Key-Value Cache Compression with Predictive Online
 * Pruning" (paper text): Section 3 (fixed per-KV-head budget of sinks,
 * protected window and long-range top-k), Section 3.1 (future-attention
 * target, Eqs. 2-4), Section 3.2 (transposed-attention target computation,
 * Eq. 8; running top-k sparse attention), Section 4 (packed training
 * sequences).  The Korean technical summary of the same paper (gist.science),
 * Section 2.1, writes the budget as B = s + w + k and Section 2.2 the target
 * condition d >= t + w.
 *
 * Conventions shared by every entry point
 *  - Layout: contiguous, heads-major.  Q and O are [B, Hq, S, D]; K and V are
 *    [B, Hkv, S, D]; LSE is [B, Hq, S]; scores are [B, Hkv, S].  A packed
 *    batch of documents is one sequence (B = 1) with document offsets
 *    cu_seqlens[0..n_docs] (0 = first, S = last); attention never crosses a
 *    document boundary.
 *  - GQA: query head g reads KV head g / (Hq / Hkv).
 *  - Logit s_{d,t} = softmax_scale * q_d . k_t (softmax_scale <= 0 selects
 *    1/sqrt(D)).  All logarithms returned are natural logarithms.
 *  - dtype: KVPOP_BF16 (bfloat16 Q/K/V/O, fp32 accumulation) or KVPOP_F32.
 *    head_dim must be 64 or 128, except that kvpop_attn_fwd_lse and
 *    kvpop_budget_mask_fwd take fp32 inputs at head_dim 64 only
 *    (KVPOP_EUNSUPPORTED otherwise).
 *  - Every pointer is device memory owned by the caller, except
 *    cu_seqlens_host (host memory, read synchronously during the call).
 *    Q, K, V, O, workspaces and the decode state must be 16-byte aligned,
 *    every fp32 or int32 array 4-byte aligned (KVPOP_EINVAL otherwise).  The
 *    library allocates nothing; workspace is caller-provided and sized by
 *    kvpop_workspace_size().  The stream is a hipStream_t passed as void*
 *    (NULL = the default stream); work is enqueued asynchronously.
 *  - Errors: arguments are validated on the host before anything is
 *    enqueued; a failed validation returns a non-zero status and leaves the
 *    outputs untouched.  kvpop_last_error() returns a thread-local message
 *    for the last failure.  Device faults surface at the caller's next
 *    synchronisation, as in HIP.  No exception crosses the ABI.
 *  - No global atomics: results are bitwise reproducible for a fixed shape.
 */
#ifndef KVPOP_H
#define KVPOP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvpop_status;
#define KVPOP_OK 0
#define KVPOP_EINVAL 1        /* bad argument (null pointer, bad shape, bad offsets) */
#define KVPOP_EUNSUPPORTED 2  /* unsupported head_dim, dtype or combination */
#define KVPOP_EWORKSPACE 3    /* workspace smaller than kvpop_workspace_size() */
#define KVPOP_EHIP 4          /* HIP runtime error, including "no device" */

enum { KVPOP_BF16 = 0, KVPOP_F32 = 1 };
enum { KVPOP_AGG_SUM = 0, KVPOP_AGG_MAX = 1, KVPOP_AGG_NONE = 2 };
enum { KVPOP_CALL_FWD_LSE = 0, KVPOP_CALL_FUTURE_TARGET = 1, KVPOP_CALL_BUDGET_MASK_FWD = 2 };

/* cutoff_out sentinels of kvpop_budget_mask_fwd */
#define KVPOP_CUTOFF_ALL 2147483647 /* fewer than k eligible tokens: all kept */
#define KVPOP_CUTOFF_NONE (-1)      /* k == 0: no eligible token kept */

typedef struct {
  int32_t batch;       /* B >= 1 (must be 1 when cu_seqlens is given) */
  int32_t seqlen;      /* S >= 1 (total packed length with cu_seqlens) */
  int32_t n_q_heads;   /* Hq >= 1, multiple of n_kv_heads */
  int32_t n_kv_heads;  /* Hkv >= 1 */
  int32_t head_dim;    /* D: 64 or 128 */
  int32_t dtype;       /* KVPOP_BF16 or KVPOP_F32: element type of Q, K, V, O */
  float softmax_scale; /* <= 0: 1/sqrt(D) */
  const int32_t *cu_seqlens;      /* device [n_docs+1] or NULL (one document per batch row) */
  const int32_t *cu_seqlens_host; /* the same offsets in host memory (NULL iff cu_seqlens is NULL) */
  int32_t n_docs;                 /* number of documents when packed, else ignored */
} kvpop_shape;

/*
 * Causal attention forward with per-query log-sum-exp.
 *
 * For every batch row b, query head g and query d:
 *   L_d = ln sum_{t <= d, same document} exp(s_{d,t})
 *   O_d = sum_t exp(s_{d,t} - L_d) v_t
 * The paper's target is defined through these dense causal probabilities
 * and its transposed identity is exact with this L (Section 3.2).
 *
 *  q [B,Hq,S,D], k, v [B,Hkv,S,D]  inputs (dtype)
 *  o [B,Hq,S,D]                    output (dtype); may be NULL: LSE only
 *  lse [B,Hq,S] fp32               output
 */
kvpop_status kvpop_attn_fwd_lse(const kvpop_shape *shape, const void *q, const void *k,
                                const void *v, void *o, float *lse, void *hip_stream);

/*
 * Future-attention target by one transposed-attention pass (Section 3.2,
 * Eq. 8): key tiles stay resident, query tiles stream past them, the logits
 * are recomputed and the given per-query normaliser is subtracted; nothing
 * of size S x S is stored.  For key t of KV head h and query head g of its
 * group:
 *   mass_g(t) = sum_{d >= t + window, same document} exp(s_{d,t} - lse_d)
 * With mean_over_queries != 0 the mass is divided by N_t, the number of such
 * queries (the mean of Eq. 2; an empty set gives 0).  Then
 *   KVPOP_AGG_SUM : target[b,h,t] = ln(sum_g mass_g(t) + eps)
 *   KVPOP_AGG_MAX : target[b,h,t] = max_g ln(mass_g(t) + eps)   (Eq. 3, max)
 *   KVPOP_AGG_NONE: target[b,g,t] = ln(mass_g(t) + eps)
 * An empty set with eps = 0 gives -inf.
 *
 *  q [B,Hq,S,D], k [B,Hkv,S,D]      inputs (dtype)
 *  lse [B,Hq,S] fp32                natural-log normaliser per query: the
 *                                   dense one from kvpop_attn_fwd_lse makes
 *                                   the identity exact; the sparse one from
 *                                   kvpop_budget_mask_fwd is the paper's
 *                                   approximation.  The masses are summed
 *                                   in fp32 without a running maximum, so a
 *                                   key whose summed mass exceeds FLT_MAX
 *                                   (ln = 88.72, before any mean; possible
 *                                   only when s_{d,t} - lse_d exceeds ~88 for
 *                                   some d, never with the dense normaliser,
 *                                   which bounds every logit of its row)
 *                                   saturates to +inf, never NaN; keys below
 *                                   are unaffected.
 *  window >= 0, eps >= 0
 *  target [B,Hkv,S] fp32 (SUM, MAX) or [B,Hq,S] fp32 (NONE)  output
 *  workspace, ws_bytes             >= kvpop_workspace_size(KVPOP_CALL_FUTURE_TARGET, ...)
 */
kvpop_status kvpop_future_target(const kvpop_shape *shape, const void *q, const void *k,
                                 const float *lse, int32_t window, int32_t agg,
                                 int32_t mean_over_queries, float eps, float *target,
                                 void *workspace, size_t ws_bytes, void *hip_stream);

/*
 * kvpop_future_target without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, layouts,
 * results (bit for bit) and errors as kvpop_future_target, minus the
 * workspace: the call uses a fixed scratch array of
 * KVPOP_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends, and calls no allocator.  A shape whose scratch
 * need (the partial sums [B, Hkv (SUM) or Hq, chunks, S] fp32 plus
 * [B, Hq, S] fp32) exceeds it returns KVPOP_EUNSUPPORTED with the sizes in
 * kvpop_last_error().  Every call on a GPU shares that GPU's array, so calls
 * that overlap on one GPU (other streams, other threads) race and must be
 * ordered by the caller.  Call with the stream's device current.
 */
#define KVPOP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kvpop_status kvpop_future_target_noalloc(const kvpop_shape *shape, const void *q, const void *k,
                                         const float *lse, int32_t window, int32_t agg,
                                         int32_t mean_over_queries, float eps, float *target,
                                         void *hip_stream);

/*
 * Fixed-budget sparse attention forward (Section 3 budget; Section 3.2
 * "Running top-k sparse attention").  Per KV head (shared by its query
 * heads), query d keeps
 *   - the sinks t < sinks,
 *   - the protected window d - window < t <= d,
 *   - among the eligible tokens E_d = [sinks, d - window] (Eq. 4), the topk
 *     best by static priority: rank(t) orders scores descending, ties (and
 *     -0.0 vs +0.0) to the lower index, NaN as -inf; with
 *     c_d = the topk-th smallest rank in E_d, token t in E_d is kept iff
 *     rank(t) <= c_d.
 * It returns the attention output and natural-log LSE under that mask (the
 * sparse normaliser the paper reuses for its target).  A row with nothing
 * kept (sinks = window = topk = 0) gets lse = -inf and O = 0.  Packed
 * documents (cu_seqlens, Section 4 trains on packed sequences): every
 * document keeps what it would keep on its own, with positions counted from
 * its first token a: sinks [a, a + sinks), the window clipped at a, and
 * E_d = [a + sinks, d - window].  rank_out then ranks the whole packed
 * sequence (restricted to a document it orders that document's tokens as
 * the document's own ranks would) and cutoff_out is in those ranks.
 *
 *  q, k, v                          inputs as for kvpop_attn_fwd_lse (seqlen * head_dim *
 *                                   element size < 2^31 bytes, else KVPOP_EUNSUPPORTED)
 *  scores [B,Hkv,S] fp32            static priorities
 *  sinks, window, topk >= 0
 *  o [B,Hq,S,D] (dtype), lse [B,Hq,S] fp32   outputs; both NULL: the mask alone (ranks,
 *                                   cutoffs and the key lists in the workspace), no attention
 *  rank_out [B,Hkv,S] int32         optional (NULL): rank(t), a permutation of 0..S-1
 *  cutoff_out [B,Hkv,S] int32       optional (NULL): c_d, or KVPOP_CUTOFF_ALL
 *                                   when |E_d| < topk, or KVPOP_CUTOFF_NONE
 *                                   when topk == 0
 *  workspace, ws_bytes              >= kvpop_workspace_size(KVPOP_CALL_BUDGET_MASK_FWD, ...)
 */
kvpop_status kvpop_budget_mask_fwd(const kvpop_shape *shape, const void *q, const void *k,
                                   const void *v, const float *scores, int32_t sinks,
                                   int32_t window, int32_t topk, void *o, float *lse,
                                   int32_t *rank_out, int32_t *cutoff_out, void *workspace,
                                   size_t ws_bytes, void *hip_stream);

/*
 * Where a kvpop_budget_mask_fwd call with this shape and these budget
 * parameters leaves its per-query-block key lists in its workspace, for
 * inspection once the call has completed (every call rebuilds them).  Query
 * block m covers positions [m * query_block, min(S, (m + 1) * query_block)).
 * For batch row b, KV head h and block m, with i = (b * Hkv + h) *
 * n_query_blocks + m, the workspace holds, at the given byte offsets:
 *   int32 lists[i * capacity + j], j < lens[i]: the positions of the keys the
 *     block's queries may keep; the first lens_full[i] are kept by every
 *     query of the block, and whole tiles of tile_keys of them are attended
 *     without a per-element mask; the list is padded to whole tiles with
 *     position S;
 *   int32 spans[2 * (i * capacity + j)], [... + 1] for j from
 *     (lens_full[i] / tile_keys) * tile_keys on: lo and hi, the query
 *     positions d with lo <= d < hi keep that key (the element mask of the
 *     masked tiles); padding keeps none;
 *   int32 lens[i], lens_full[i];
 *   int32 status[i]: 0 when the list is whole; bit 0 set when entries past
 *     the capacity were dropped; bit 1 set when the number of keys kept by
 *     every query differs from the count the list was laid out for.
 * Returns KVPOP_EINVAL for an invalid shape or negative budget parameters.
 */
typedef struct {
  size_t lists_offset, spans_offset, lens_offset, lens_full_offset, status_offset;
  int32_t n_query_blocks, query_block, capacity, tile_keys;
} kvpop_lists_layout;
kvpop_status kvpop_budget_lists_layout(const kvpop_shape *shape, int32_t sinks, int32_t window,
                                       int32_t topk, kvpop_lists_layout *layout);

/*
 * Bytes of workspace the call `which` (KVPOP_CALL_*) needs for this shape
 * and these budget parameters (sinks, window and topk matter only for
 * KVPOP_CALL_BUDGET_MASK_FWD; pass 0 otherwise).  Returns 0 for an invalid
 * shape and for calls that need none (KVPOP_CALL_FWD_LSE).
 */
size_t kvpop_workspace_size(int32_t which, const kvpop_shape *shape, int32_t sinks,
                            int32_t window, int32_t topk);

/*
 * Teacher labels at the eviction boundary (Section 3.1, Eqs. 4-6).  For each
 * (batch row, KV head) the teacher ranks the eligible tokens
 * E_d = [sinks, d - window] by effective scores, the target y(t) minus a
 * per-head decay of lambda per decay_step positions of age (Eq. 5), and
 * keeps the top `topk`.  Section 3.2's running threshold over static
 * priorities is used: pi(t) = y(t) + (lambda / decay_step) * t, computed in
 * fp32 as c = lambda / decay_step, then y + c * t, each operation rounded
 * (exact for lambda = 0 or decay_step = 1; otherwise the pages' own
 * approximation: it ranks like Eq. 5 except between tokens whose static
 * priorities lie within lambda (decay_step - 1) / decay_step, where the
 * whole-step decay can swap them).  Order: priority
 * descending, ties (and -0.0 vs +0.0) to the lower index, NaN as -inf.
 *
 *  target [B,Hkv,S] fp32            y, e.g. kvpop_future_target's output (AGG_MAX, mean)
 *  decay_lambda [Hkv] fp32          per-head decay, or NULL for none
 *  decay_step >= 1, sinks, window, topk >= 0
 *  label [B,Hkv,S] int32            label[d] = 1 if the teacher keeps the newly eligible
 *                                   token d - window at query d, 0 if not, -1 when
 *                                   d - window < sinks or topk == 0
 *  boundary [B,Hkv,S] int32         the last kept token at query d (-1 if none): the token
 *                                   of rank b_d = the min(topk, |E_d|)-th smallest rank of E_d
 *  rank_out [B,Hkv,S] int32         optional (NULL): rank(t) under the priorities
 *  brank_out [B,Hkv,S] int32        optional (NULL): b_d (-1 if none)
 *  workspace, ws_bytes              >= kvpop_teacher_workspace_size()
 */
kvpop_status kvpop_teacher_labels(int32_t batch, int32_t n_kv_heads, int32_t seqlen, const float *target,
                                  const float *decay_lambda, int32_t decay_step, int32_t sinks, int32_t window,
                                  int32_t topk, int32_t *label, int32_t *boundary, int32_t *rank_out,
                                  int32_t *brank_out, void *workspace, size_t ws_bytes, void *hip_stream);
size_t kvpop_teacher_workspace_size(int32_t batch, int32_t n_kv_heads, int32_t seqlen);

/*
 * Boundary-aware retention loss (Section 3.1, Eq. 7) and its gradient.  For
 * every query position d with a label and a boundary token b = boundary[d]:
 *   x_d = (pred[d - window] - pred[b]) / tau,  sign_d = +1 (kept) or -1,
 *   loss[d] = weight[d] * ln(1 + exp(-sign_d * x_d))     (0 elsewhere)
 * and grad = d(sum_d loss[d]) / d pred, per token.  The decay term is shared
 * by the two tokens compared at one d, so raw predicted scores are compared.
 *
 *  pred [B,Hkv,S] fp32              raw predicted scores
 *  label, boundary [B,Hkv,S] int32  from kvpop_teacher_labels with the same sinks, window
 *                                   and topk (the deterministic gradient reduction relies
 *                                   on their structure: the positions sharing a boundary
 *                                   token form at most one run before d = sinks + window +
 *                                   topk - 1 and one from there on)
 *  tau > 0; weight [B,Hkv,S] fp32 per query position, or NULL for 1
 *  loss, grad [B,Hkv,S] fp32        outputs
 *  workspace, ws_bytes              >= kvpop_boundary_loss_workspace_size()
 */
kvpop_status kvpop_boundary_loss(int32_t batch, int32_t n_kv_heads, int32_t seqlen, const float *pred,
                                 const int32_t *label, const int32_t *boundary, int32_t sinks, int32_t window,
                                 int32_t topk, float tau, const float *weight, float *loss, float *grad,
                                 void *workspace, size_t ws_bytes, void *hip_stream);
size_t kvpop_boundary_loss_workspace_size(int32_t batch, int32_t n_kv_heads, int32_t seqlen);

/*
 * Fixed-budget decoding (Section 3: sinks, protected window and top-k;
 * Section 3.2, "Running top-k sparse attention"; the paper text's results
 * section, Inference efficiency and Fig. 4, and Section 4.3 of the Korean
 * summary measure the resulting bounded cache).  The state holds, per (batch row, KV head),
 * sinks + window + topk slots of K and V plus bookkeeping; it is
 * caller-owned device memory of kvpop_decode_state_size() bytes, set up by
 * kvpop_decode_init().  kvpop_decode_step() appends token `position` (which
 * must be 0, 1, 2, ... in order after init; the state does not check it):
 * token position - window leaves the window and competes for the top-k by
 * its static priority (score descending, ties to the lower index); if the
 * top-k is full and it beats the worst retained token, that token is
 * evicted for good.  The query of the new token then attends over the
 * retained slots, which are exactly the budget mask's row `position` of
 * kvpop_budget_mask_fwd with the same scores.
 *
 *  q [B,Hq,D], k, v [B,Hkv,D]   the new token (dtype)
 *  score [B,Hkv] fp32           its static priority
 *  o [B,Hq,D] (dtype), lse [B,Hq] fp32   outputs
 * At most 8 query heads per KV head (else KVPOP_EUNSUPPORTED); head_dim 64
 * or 128; 1 <= sinks + window + topk <= 2^20 slots (more: KVPOP_EUNSUPPORTED).
 * A state too small for the shape gives KVPOP_EWORKSPACE.  Steps on one
 * state must be ordered (one stream); concurrent steps on one state race.
 */
typedef struct {
  int32_t batch, n_q_heads, n_kv_heads, head_dim;
  int32_t dtype;        /* KVPOP_BF16 or KVPOP_F32 */
  float softmax_scale;  /* <= 0: 1/sqrt(head_dim) */
  int32_t sinks, window, topk;
} kvpop_decode_shape;
size_t kvpop_decode_state_size(const kvpop_decode_shape *shape);
kvpop_status kvpop_decode_init(const kvpop_decode_shape *shape, void *state, size_t state_bytes, void *hip_stream);
kvpop_status kvpop_decode_step(const kvpop_decode_shape *shape, void *state, size_t state_bytes, int32_t position,
                               const void *q, const void *k, const void *v, const float *score, void *o,
                               float *lse, void *hip_stream);

/* Static description of a status code. */
const char *kvpop_status_str(kvpop_status status);

/* Thread-local detail of the last failed call on this thread ("" if none). */
const char *kvpop_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVPOP_H */
