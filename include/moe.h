/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE dispatch / grouped-FFN / combine
 * library.
 *
 * One MoE expert layer, forward and backward, on one GPU: top-k softmax
 * routing, dropless token dispatch into expert-contiguous rows, a grouped
 * SwiGLU expert FFN, and the weighted combine back to source order.
 *
 * The pages this follows name the hot path as "EP token dispatch" plus
 * "grouped expert compute" ("Add MoE expert parallel training runtime",
 * Major changes), and require that uneven or empty work neither
 * desynchronises nor crashes it, that callers never pad, that outputs come
 * back in full source order and that gradients accumulate ("Support combined
 * expert and data parallelism in TrainerRank", Desired behavior and
 * Acceptance). Unsupported configurations fail loudly and up front, and every
 * argument is validated before any is used (same page, Current behavior;
 * review note on "Add MoE expert parallel training runtime").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor is a device pointer to contiguous row-major memory, owned
 *    by the caller. The library never allocates, frees or keeps device
 *    memory; scratch memory is passed in as a workspace whose size
 *    moe_workspace_size() reports.
 *  - "s" below is the layer dtype: MOE_DTYPE_BF16 (bf16 storage, fp32
 *    accumulation, results rounded to nearest-even once) or MOE_DTYPE_F32.
 *    Routing tensors (logits, weights, their gradients) and weight gradients
 *    are always fp32; index tensors are int32.
 *  - Weights use the [out, in] convention: w_gu is [E, 2F, d] with the gate
 *    projection in rows [0, F) and the up projection in rows [F, 2F) of each
 *    expert; w_down is [E, d, F].
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default
 *    stream). The host never waits for the device and never reads device
 *    data; per-expert row counts stay on the device.
 *  - T == 0 (an empty microbatch) returns MOE_OK, launches nothing and writes
 *    nothing; NULL is then accepted for every tensor. The one exception is
 *    moe_aux_loss, which writes the zero losses of the empty microbatch.
 *  - Validation happens on the host before the first launch. A NULL pointer
 *    that must be read or written, a pointer not aligned to 16 bytes, a
 *    shape outside the supported matrix or a short workspace is reported
 *    with a status code and nothing is launched. No C++ exception crosses
 *    this interface.
 *  - Supported matrix: T >= 0, 1 <= k <= E <= 256, k <= 16, d and F
 *    positive multiples of 64, d <= 65536, F <= 65536, T*k < 2^31,
 *    dtype bf16 or fp32, and every launch within 2^32 threads per grid
 *    dimension: T < 2^24 and T*d < 2^35 (bf16) or 2^34 (fp32), and the
 *    weight-gradient grid of the grouped GEMM within that bound too.
 *    Anything else returns MOE_ERR_UNSUPPORTED.
 *  - Calls that overlap on one stream are ordered; calls on different
 *    streams that share buffers race, as with any HIP kernel.
 *
 * Numbering used in the comments: R = T*k routed rows; M_e = counts[e].
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1, /* NULL where data is needed, negative size, k > E, ... */
  MOE_ERR_UNSUPPORTED = 2,      /* outside the supported matrix above */
  MOE_ERR_WORKSPACE = 3,        /* workspace NULL or smaller than required */
  MOE_ERR_MISALIGNED = 4,       /* a tensor pointer not 16-byte aligned */
  MOE_ERR_HIP = 5               /* a HIP launch failed; see moe_last_error() */
} moe_status;

enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 };

/* MOE_FLAG_RENORM: renormalise the k selected weights so that they sum to
 * one. Without it the weights are the full-softmax probabilities of the
 * selected experts.
 *
 * MOE_FLAG_RECOMPUTE: keep no FFN activations between forward and backward
 * (activation checkpointing of the expert FFN: Add MoE expert parallel
 * training runtime, Major changes; no-grad execution: Support pipeline parallelism
 * in TrainerRank without exposing stage scheduling to callers, Acceptance).
 * moe_grouped_gemm_fwd then takes h = a = NULL, never writes h and keeps a
 * only in its workspace; it is also the forward to use when no backward
 * follows. moe_grouped_gemm_bwd takes h = a = NULL and first recomputes h and
 * a from x_perm into its workspace (one more gate/up product, bit-identical
 * to the forward's), then writes dH over the recomputed h. Results equal
 * those without the flag bit for bit. */
enum { MOE_FLAG_RENORM = 1u, MOE_FLAG_RECOMPUTE = 2u, MOE_FLAG_ACCUMULATE_DLOGITS = 4u };
/* MOE_FLAG_ACCUMULATE_DLOGITS: moe_route_bwd adds the routing-weight
 * gradient to what dlogits already holds (typically the auxiliary losses'
 * gradient from moe_aux_loss) instead of overwriting it, and with a router
 * back-propagates the sum into dx_router and dw_router. */

typedef struct moe_shape {
  int64_t T;      /* tokens in this microbatch (>= 0) */
  int32_t d;      /* hidden size */
  int32_t E;      /* experts held by this GPU */
  int32_t k;      /* experts per token */
  int32_t F;      /* SwiGLU hidden size of one expert */
  int32_t dtype;  /* MOE_DTYPE_F32 or MOE_DTYPE_BF16 */
  uint32_t flags; /* MOE_FLAG_* */
} moe_shape;

/* Opaque stream handle: a hipStream_t, or NULL for the default stream. */
typedef void *moe_stream_t;

/*
 * Workspace sizes in bytes for a shape: route_ws serves moe_route and
 * moe_route_bwd and moe_aux_loss, gemm_fwd_ws serves moe_grouped_gemm_fwd and gemm_bwd_ws
 * serves moe_grouped_gemm_bwd. A workspace sized for some T serves every
 * smaller T of the same (d, E, k, F, dtype), so one buffer sized for the
 * largest microbatch can be reused across microbatches of any size
 * ("live-graph/buffer-capacity transitions", Support combined expert and
 * data parallelism in TrainerRank, Acceptance). Any output pointer may be
 * NULL. Pure host function.
 */
moe_status moe_workspace_size(const moe_shape *shape, size_t *route_ws, size_t *gemm_fwd_ws,
                              size_t *gemm_bwd_ws);

/*
 * Routing and dispatch tables (the routing half of "EP token dispatch", Add
 * MoE expert parallel training runtime, Major changes; any per-expert count,
 * zero included, without padding by the caller: Support combined expert and
 * data parallelism in TrainerRank, Desired behavior).
 *
 * If w_router is non-NULL the logits are computed first,
 *   logits[t,e] = <x[t], w_router[e]> + bias[e]   (fp32 accumulation),
 * with x [T,d] s, w_router [E,d] s and bias [E] fp32 (NULL means zero), and
 * written to `logits`. Otherwise x, w_router and bias must be NULL and
 * `logits` [T,E] fp32 is read.
 *
 * Then, per token: topk_idx[t,:] [T,k] int32 holds the k largest logits in
 * descending order, equal logits going to the lower expert id (NaN ranks
 * below -inf; -0.0 equals +0.0); topk_w[t,j] [T,k] fp32 is
 * softmax(logits[t,:])[topk_idx[t,j]], divided by the sum over j when
 * MOE_FLAG_RENORM is set. Every token needs at least one finite logit.
 *
 * Dispatch tables: counts[e] [E] int32 rows per expert; offsets [E+1] int32
 * the exclusive prefix sum (offsets[E] = R); row_of_slot[t,j] [T,k] int32 the
 * row of the expert-contiguous buffers that receives slot (t,j); and
 * src_of_row[r] [R] int32 = t*k+j, its inverse. Rows of one expert follow
 * ascending source token (a stable counting sort); the order is decided
 * without atomics, so the tables are identical run to run.
 *
 * ws: route workspace of at least route_ws bytes.
 */
moe_status moe_route(const moe_shape *shape, const void *x, const void *w_router, const float *bias,
                     float *logits, int32_t *topk_idx, float *topk_w, int32_t *counts,
                     int32_t *offsets, int32_t *row_of_slot, int32_t *src_of_row, void *ws,
                     size_t ws_bytes, moe_stream_t stream);

/*
 * moe_route without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). Arguments, results and errors are those of moe_route;
 * the per-workgroup histograms go to a static scratch array of 16 MiB per GPU
 * instead (held by each GPU the library runs on until the process ends), so
 * ceil(T / 64) * E * 4 bytes must fit in it: T up to 1,048,576 tokens at
 * E = 256, 8,388,608 at E = 32. Larger shapes return MOE_ERR_UNSUPPORTED
 * before anything is launched. The call allocates no device memory. Every
 * call on one GPU shares that GPU's scratch: calls that overlap in time on
 * one GPU (different streams, or different threads) race and may return
 * wrong tables; calls ordered on one stream do not.
 */
moe_status moe_route_noalloc(const moe_shape *shape, const void *x, const void *w_router, const float *bias,
                             float *logits, int32_t *topk_idx, float *topk_w, int32_t *counts,
                             int32_t *offsets, int32_t *row_of_slot, int32_t *src_of_row,
                             moe_stream_t stream);

/*
 * Token dispatch (the data-moving half of "EP token dispatch", Add MoE expert
 * parallel training runtime, Major changes):
 *   x_perm[row_of_slot[t,j]] = x[t]     x [T,d] s -> x_perm [R,d] s.
 * Each source row is read once and written k times. No padding rows exist:
 * the buffers hold exactly R rows.
 */
moe_status moe_permute(const moe_shape *shape, const void *x, const int32_t *row_of_slot,
                       void *x_perm, moe_stream_t stream);

/*
 * Grouped SwiGLU expert FFN ("grouped expert compute", Add MoE expert parallel
 * training runtime, Major changes), expert by expert over
 * the rows [offsets[e], offsets[e+1]) of x_perm:
 *   h = X_e W_gu[e]^T         [R,2F] s   (saved for the backward)
 *   a = silu(h[:, :F]) * h[:, F:]  [R,F] s   (saved)
 *   y = a W_down[e]^T         [R,d] s   (unweighted expert output)
 * silu(z) = z / (1 + exp(-z)). The gate/up products feed the SwiGLU in fp32
 * before h and a are rounded. An expert with no rows costs nothing: tiles
 * are laid out on the device from `offsets`, which the host never reads.
 * With MOE_FLAG_RECOMPUTE, h and a must be NULL: h is not written and a
 * lives in ws. ws: at least gemm_fwd_ws bytes (may be NULL when that size
 * is 0; it is R*F*s bytes with MOE_FLAG_RECOMPUTE).
 */
moe_status moe_grouped_gemm_fwd(const moe_shape *shape, const void *x_perm, const void *w_gu,
                                const void *w_down, const int32_t *offsets, void *h, void *a,
                                void *y, void *ws, size_t ws_bytes, moe_stream_t stream);

/*
 * Weighted combine back to full source order (outputs are returned in full
 * source order: Support combined expert and data parallelism in TrainerRank,
 * Desired behavior):
 *   out[t] = sum_{j<k} topk_w[t,j] * y[row_of_slot[t,j]]    out [T,d] s,
 * summed in fp32 in increasing j and rounded once.
 */
moe_status moe_unpermute_combine(const moe_shape *shape, const void *y, const float *topk_w,
                                 const int32_t *row_of_slot, void *out, moe_stream_t stream);

/*
 * Backward of the combine (the backward every microbatch of the canary runs,
 * whose gradients are compared with a matched reference: Support combined
 * expert and data parallelism in TrainerRank, Acceptance):
 *   dy[row_of_slot[t,j]] = topk_w[t,j] * dout[t]     dy [R,d] s
 *   dtopk_w[t,j] = <dout[t], y[row_of_slot[t,j]]>   dtopk_w [T,k] fp32
 * Every row of dy is written (the rows are a permutation of the slots).
 */
moe_status moe_unpermute_combine_bwd(const moe_shape *shape, const void *dout, const void *y,
                                     const float *topk_w, const int32_t *row_of_slot, void *dy,
                                     float *dtopk_w, moe_stream_t stream);

/*
 * Backward of the routing weights (part of the backward whose model and
 * expert gradients the canary compares with a matched reference: Support
 * combined expert and data parallelism in TrainerRank, Acceptance; the router
 * gradient accumulates like every other: same page, Desired behavior).
 * Selection is piecewise constant, so only the weights carry gradient. With g = dtopk_w and p = softmax(logits[t,:]):
 *   no renorm: dlogits[t,m] = p_m * (G_m - sum_j topk_w[t,j] g[t,j]),
 *              G_m = g[t,j] if m == topk_idx[t,j] for some j, else 0;
 *   renorm:    dlogits[t,topk_idx[t,j]] = topk_w[t,j] (g[t,j] - sum_j' topk_w g),
 *              zero for unselected experts.
 * dlogits [T,E] fp32 is overwritten.
 *
 * If w_router is non-NULL (the logits came from the router inside
 * moe_route), x [T,d] s and w_router [E,d] s are read and
 *   dx_router = dlogits w_router   [T,d] fp32 (overwritten),
 *   dw_router += dlogits^T x       [E,d] fp32 (accumulated; zero it once),
 * both required; otherwise x, dx_router and dw_router must be NULL. The
 * router weight gradient is reduced in a fixed order (no atomics).
 * With MOE_FLAG_ACCUMULATE_DLOGITS the result is added to dlogits (and the
 * router backward, if any, uses the sum).
 * ws: route workspace of at least route_ws bytes.
 */
moe_status moe_route_bwd(const moe_shape *shape, const float *dtopk_w, const float *logits,
                         const int32_t *topk_idx, const float *topk_w, const void *x,
                         const void *w_router, float *dlogits, float *dx_router, float *dw_router,
                         void *ws, size_t ws_bytes, moe_stream_t stream);

/*
 * Backward of the grouped SwiGLU FFN, expert by expert:
 *   dA      = dY_e W_down[e]
 *   dH_gate = dA * h_up * sig(h_gate) * (1 + h_gate (1 - sig(h_gate)))
 *   dH_up   = dA * silu(h_gate)                   (dH kept in ws, dtype s)
 *   dx_perm = dH W_gu[e]                          [R,d] s   (overwritten)
 *   dw_down[e] += dY_e^T a_e                      [E,d,F] fp32
 *   dw_gu[e]   += dH^T X_e                        [E,2F,d] fp32
 * The weight gradients accumulate across calls (gradient accumulation across
 * microbatches and repeated forwards: Support pipeline parallelism in
 * TrainerRank without exposing stage scheduling to callers, Acceptance); the
 * caller zeroes them once. An expert with no rows leaves its dw slices
 * bit-identical. Each dw element is reduced by one workgroup in a fixed
 * order, so results are identical run to run.
 * With MOE_FLAG_RECOMPUTE, h and a must be NULL; h and a are recomputed from
 * x_perm into ws before the steps above, and dH overwrites the recomputed h.
 * ws: at least gemm_bwd_ws bytes; dH occupies its first R*2F*s bytes.
 */
moe_status moe_grouped_gemm_bwd(const moe_shape *shape, const void *dy, const void *x_perm,
                                const void *h, const void *a, const void *w_gu, const void *w_down,
                                const int32_t *offsets, void *dx_perm, float *dw_gu, float *dw_down,
                                void *ws, size_t ws_bytes, moe_stream_t stream);

/*
 * Backward of the dispatch, returning the token gradient in full source order
 * (Support combined expert and data parallelism in TrainerRank, Desired
 * behavior):
 *   dx[t] = sum_j dx_perm[row_of_slot[t,j]] (+ dx_extra[t])    dx [T,d] s,
 * summed in fp32 and rounded once. dx_extra [T,d] fp32 (the router's
 * contribution from moe_route_bwd) may be NULL.
 */
moe_status moe_permute_bwd(const moe_shape *shape, const void *dx_perm, const int32_t *row_of_slot,
                           const float *dx_extra, void *dx, moe_stream_t stream);

/*
 * MoE auxiliary losses and routing metrics ("MoE metrics" and the "MoE
 * losses" covered by its regression tests, Add MoE expert parallel training
 * runtime, Major changes; its test_moe_losses module, Validation; the pages
 * name them without a definition). From the fp32 logits [T,E] of a
 * microbatch and the counts [E] moe_route produced, with p the softmax over
 * all E experts (whatever MOE_FLAG_RENORM says):
 *   f_e   = counts[e] / (T k),   P_e = (1/T) sum_t p[t,e]
 *   L_bal = E sum_e f_e P_e      load balancing (Switch Transformers, 2.2)
 *   L_z   = (1/T) sum_t lse_t^2, lse_t = log sum_e exp(logits[t,e])
 *                                router z-loss (ST-MoE, 3.1)
 * losses [2] fp32 (NULL: not written) receives (L_bal, L_z), unweighted.
 * metrics [MOE_METRIC_SCALARS + 2E] fp32 (NULL: not written) receives the
 * scalars indexed by MOE_METRIC_*, then f_e for every e, then P_e.
 * dlogits [T,E] fp32 (NULL: not written) receives the gradient of
 *   balance_coef L_bal + z_coef L_z
 * with respect to the logits, f held constant (it is piecewise constant):
 *   dlogits[t,i] = p_i (G_i - sum_e p_e G_e) + (2 z_coef / T) lse_t p_i,
 *   G_e = balance_coef E f_e / T,
 * overwriting dlogits, or added to it with MOE_AUX_ACCUMULATE. To train a
 * router through moe_route_bwd, call this first and set
 * MOE_FLAG_ACCUMULATE_DLOGITS on the shape. Every token needs a finite
 * logit. All sums run in a fixed order (no atomics). T == 0 (the empty-work
 * case, which must contribute zero) writes losses = (0, 0) and metrics all
 * zero except MOE_METRIC_EMPTY_EXPERTS = E, and no dlogits row; logits,
 * counts and dlogits may then be NULL.
 * ws: route workspace of at least route_ws bytes.
 * Errors: cfg NULL or a non-finite coefficient -> MOE_ERR_INVALID_ARGUMENT;
 * unknown cfg flag bits -> MOE_ERR_UNSUPPORTED.
 */
enum { MOE_AUX_ACCUMULATE = 1u };
enum {
  MOE_METRIC_IMBALANCE = 0,     /* max_e counts[e] / (T k / E) */
  MOE_METRIC_EMPTY_EXPERTS = 1, /* experts with no rows */
  MOE_METRIC_COUNT_CV = 2,      /* population std / mean of counts */
  MOE_METRIC_ENTROPY = 3,       /* mean over tokens of -sum_e p log p (nats) */
  MOE_METRIC_MAX_PROB = 4,      /* mean over tokens of max_e p */
  MOE_METRIC_SCALARS = 5        /* number of scalars before the per-expert arrays */
};

typedef struct moe_aux_config {
  float balance_coef; /* weight of L_bal in the gradient */
  float z_coef;       /* weight of L_z in the gradient */
  uint32_t flags;     /* MOE_AUX_* */
} moe_aux_config;

moe_status moe_aux_loss(const moe_shape *shape, const float *logits, const int32_t *counts,
                        const moe_aux_config *cfg, float *losses, float *metrics, float *dlogits,
                        void *ws, size_t ws_bytes, moe_stream_t stream);

/*
 * Optimizer update of the expert weights (the "optimizer update" step the
 * canary of Support combined expert and data parallelism in TrainerRank,
 * Acceptance, completes after forward and backward). The pages do not name
 * the optimizer; this is AdamW (Adam with decoupled weight decay), computed
 * element by element on fp32 master weights as PyTorch's AdamW does:
 *   g     = grad_scale * grad
 *   m     = beta1 m + (1 - beta1) g            (exp_avg, fp32, in place)
 *   v     = beta2 v + (1 - beta2) g^2          (exp_avg_sq, fp32, in place)
 *   param = param (1 - lr weight_decay)
 *           - lr / (1 - beta1^step) * m / (sqrt(v) / sqrt(1 - beta2^step) + eps)
 * If param_bf16 is non-NULL, the updated param rounded to bf16 (nearest-even)
 * is also written there, e.g. straight into the w_gu / w_down the grouped
 * GEMMs read. With MOE_ADAMW_ZERO_GRAD, grad is set to zero in the same pass,
 * ready for the next accumulation. grad_scale turns the summed gradients of
 * several microbatches into a mean if the caller wants one.
 * All arrays hold n elements, contiguous, 16-byte aligned, not overlapping;
 * n == 0 is a no-op that accepts NULLs. The update of an element reads and
 * writes that element only: results do not depend on n or on launch layout.
 * Errors: cfg NULL, lr < 0, a beta outside [0, 1), eps <= 0, weight_decay < 0,
 * a non-finite scalar, step < 1 or n < 0 -> MOE_ERR_INVALID_ARGUMENT; unknown
 * flag bits or n >= 2^35 (a launch of 2^32 threads) -> MOE_ERR_UNSUPPORTED.
 */
enum { MOE_ADAMW_ZERO_GRAD = 1u };

typedef struct moe_adamw_config {
  float lr;           /* learning rate */
  float beta1;        /* first-moment decay */
  float beta2;        /* second-moment decay */
  float eps;          /* added to the bias-corrected sqrt(v) */
  float weight_decay; /* decoupled weight decay */
  float grad_scale;   /* gradient multiplier applied first */
  int64_t step;       /* step number of this update, 1 for the first */
  uint32_t flags;     /* MOE_ADAMW_* */
} moe_adamw_config;

moe_status moe_adamw_step(const moe_adamw_config *cfg, int64_t n, float *param, float *grad,
                          float *exp_avg, float *exp_avg_sq, void *param_bf16, moe_stream_t stream);

/*
 * Expert parallelism: the token exchange between EP ranks around the grouped
 * FFN, for EP combined with data parallelism where ranks hold different token
 * counts, uneven work or none, and the runtime (not the caller) coordinates
 * expert communication, its order and its buffer capacities (Support combined
 * expert and data parallelism in TrainerRank, Desired behavior; an EP=2 run on
 * unequal batches with an empty-work case: same page, Acceptance).
 *
 * Global expert g = r*E_local + e is local expert e of rank r (EP ranks,
 * E = EP*E_local experts in all). A source rank routes its tokens over all E
 * experts with moe_route and dispatches them with moe_permute: its x_perm is
 * then one contiguous segment per destination rank, ordered by local expert,
 * then source token. A destination numbers the rows it receives
 * source-major (all of source 0's segment, then source 1's, ...) and runs
 * the grouped FFN on them regrouped by local expert, then source, then their
 * order in the segment. Every count stays on the device; the host passes
 * capacities only. 1 <= EP <= MOE_EP_MAX_RANKS, EP*E_local <= 256, every
 * row capacity below 2^24 (one 256-thread workgroup per row; larger
 * capacities return MOE_ERR_UNSUPPORTED).
 */
enum { MOE_EP_MAX_RANKS = 8 };

/*
 * Send plan of one source rank (shape->E = EP*E_local global experts), from
 * the counts [E] and offsets [E+1] moe_route wrote:
 *   send_counts[r*E_local + e] = counts[r*E_local + e]    [EP*E_local] int32
 *   send_offsets[r] = offsets[r*E_local], send_offsets[EP] = offsets[E]
 *                                                          [EP+1] int32
 * (rows [send_offsets[r], send_offsets[r+1]) of x_perm go to rank r). With
 * T == 0 both tables are written as zeros and counts/offsets may be NULL: a
 * rank with no work still takes part in the counts exchange. This is the
 * second exception to "T == 0 writes nothing".
 * Errors: ep outside [1, MOE_EP_MAX_RANKS] or not dividing E ->
 * MOE_ERR_UNSUPPORTED; plus the shape and pointer rules of the other calls.
 */
moe_status moe_ep_send_plan(const moe_shape *shape, int32_t ep, const int32_t *counts, const int32_t *offsets,
                            int32_t *send_counts, int32_t *send_offsets, moe_stream_t stream);

/*
 * Receive plan of one destination rank from recv_counts [EP*E_local] int32
 * (entry s*E_local + e: rows of local expert e that source s sends):
 *   local_counts[e] = sum_s recv_counts[s*E_local + e]        [E_local]
 *   local_offsets = exclusive scan of local_counts             [E_local+1]
 *   recv_offsets[s] = first received row of source s           [EP+1]
 *   regroup_row[i] = grouped row of received row i, for i < recv_offsets[EP]
 *                                                              [rows_cap]
 * rows_cap is the capacity of the receive and grouped buffers (rows the
 * host sized them for, e.g. EP * T_max * k); entries of regroup_row at or past
 * the received total are not written. local_offsets is the `offsets` of the
 * grouped FFN calls on the grouped rows (shape T = rows_cap, k = 1,
 * E = E_local).
 */
moe_status moe_ep_recv_plan(int32_t ep, int32_t e_local, int64_t rows_cap, const int32_t *recv_counts,
                            int32_t *local_counts, int32_t *local_offsets, int32_t *recv_offsets,
                            int32_t *regroup_row, moe_stream_t stream);

/*
 * Regroup of the received rows i < recv_offsets[EP] (d columns of dtype):
 *   reverse == 0: dst[regroup_row[i]] = src[i]   (received -> grouped)
 *   reverse != 0: dst[i] = src[regroup_row[i]]   (grouped -> received)
 * src and dst hold rows_cap rows and do not overlap.
 */
moe_status moe_ep_regroup(int32_t d, int32_t dtype, int64_t rows_cap, int32_t ep, const int32_t *recv_offsets,
                          const int32_t *regroup_row, const void *src, void *dst, int32_t reverse,
                          moe_stream_t stream);

/*
 * One-GPU stand-ins for the two exchanges between the EP ranks, for EP
 * ranks simulated on one device (the multi-GPU path replaces them with an
 * all-to-all of the counts tables and an all-to-allv of the rows). Arrays of
 * EP device pointers are host arrays indexed by rank.
 *
 * Counts: recv_counts[r][s*E_local + e] = send_counts[s][r*E_local + e].
 *
 * Rows (reverse == 0): for every source s and destination r, rows
 * [send_offsets[s][r], send_offsets[s][r+1]) of send_bufs[s] are received by
 * r as rows recv_offsets[r][s] .. and land there in recv_bufs[r], or, if
 * regroup_rows is non-NULL, straight at their grouped rows
 * regroup_rows[r][received row] (the exchange and moe_ep_regroup in one
 * copy). reverse != 0 copies the same rows back into send_bufs from the same
 * places. send_caps[s] / recv_caps[r]: rows each buffer holds (a source with
 * T = 0 has capacity 0 and sends nothing). d columns of dtype.
 */
moe_status moe_ep_exchange_counts_loopback(int32_t ep, int32_t e_local, const int32_t *const *send_counts,
                                           int32_t *const *recv_counts, moe_stream_t stream);
moe_status moe_ep_exchange_loopback(int32_t ep, int32_t d, int32_t dtype, void *const *send_bufs,
                                    const int64_t *send_caps, const int32_t *const *send_offsets,
                                    void *const *recv_bufs, const int64_t *recv_caps,
                                    const int32_t *const *recv_offsets, const int32_t *const *regroup_rows,
                                    int32_t reverse, moe_stream_t stream);

/* Static English text for a status code. */
const char *moe_status_string(moe_status status);

/* Detail of the last error reported on the calling thread ("" if none). */
const char *moe_last_error(void);

/*
 * Per-kernel timing with HIP events, for measurement. When enabled, every
 * kernel the library launches is bracketed by two events recorded on the
 * launch stream; moe_profiler_read() waits for them and returns, per kernel
 * name, the number of launches and the summed elapsed milliseconds since the
 * last moe_profiler_reset(). Process-wide host-side state guarded by a
 * mutex: launches from several threads are timed together, and a read blocks
 * until the events of its entry have completed. Meant for measurement;
 * disabled by default.
 */
moe_status moe_profiler_enable(int on);
moe_status moe_profiler_reset(void);
/* Number of distinct kernel names recorded so far. */
int moe_profiler_count(void);
/* Entry i: name (static string), launches, total ms. Blocks until the events
 * of that entry have completed. */
moe_status moe_profiler_read(int i, const char **name, int64_t *launches, double *total_ms);

/* Library version string. */
const char *moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
