/*
 * moe.h -- C ABI of libmoe.so, the gfx950 (MI355X) local MoE forward chain.
 *
 * The chain and its contract come from the ruDNN User Guide (ruDNN 0.1.5 on
 * docs.rs, and the same text in the 0.1.13 Chinese README and the RUDA
 * Japanese guide):
 *   section 3 "MoE workflow":       logits -> softmax/top-k -> compact
 *                                    dispatch -> SwiGLU experts -> weighted
 *                                    combine, run locally on one device;
 *   section 4 "Routing contract":    [T,E] F32/F16/BF16 logits, 1 <= top_k <= E,
 *                                    FP32 softmax over all experts before top-k,
 *                                    ties to the lower expert id, optional
 *                                    renormalisation, weights cast to the logits
 *                                    dtype, NaN kept for NaN/+inf/all -inf rows,
 *                                    [T,top_k] U32 indices;
 *   section 5 "Expert weights and dispatch": x [T,H], gate/up [E,I,H],
 *                                    down [E,H,I], one float dtype and device,
 *                                    no capacity drop, unspecified order inside
 *                                    an expert, a saved mapping restores order;
 *   section 6 "Call MoE":            the fused forward and the split
 *                                    route / dispatch / forward_dispatched /
 *                                    combine stages; shape, dtype and device
 *                                    mismatches are reported as errors.
 *
 * Conventions shared by every call:
 *   - Tensors are dense row-major device buffers (hipMalloc'd memory of the
 *     device the stream belongs to).  The caller owns every buffer; the
 *     library never allocates or frees device memory and keeps no pointer
 *     after a call returns.  Expert weights are only read, so one set can
 *     serve any number of batches.
 *   - `stream` is a hipStream_t (NULL: the null stream of the current
 *     device).  Every call only enqueues kernels and returns; it never waits
 *     for the device and never reads device memory on the host.
 *   - Arguments are checked before anything is enqueued; on any error
 *     nothing is written.  Check order: null pointers / negative extents,
 *     dtypes, shapes, top_k, limits of this implementation, workspace size,
 *     device residency, then the launches.
 *   - A tensor with zero elements may have data == NULL.  T = 0 is a valid
 *     no-op.
 *   - Results are bitwise reproducible run to run, although the row order
 *     inside an expert (which follows device atomics) is not.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_dtype {
    MOE_F32 = 0,
    MOE_F16 = 1,
    MOE_BF16 = 2,
    MOE_U32 = 3,
    MOE_I32 = 4, /* router-training indices only */
    MOE_I64 = 5  /* router-training indices only */
} moe_dtype;

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative extent, bad ndim */
    MOE_ERR_DTYPE = 2,            /* a dtype the contract does not allow */
    MOE_ERR_SHAPE = 3,            /* extents that disagree with each other */
    MOE_ERR_TOP_K = 4,            /* top_k < 1 or top_k > E */
    MOE_ERR_DEVICE = 5,           /* a buffer not on the stream's device */
    MOE_ERR_WORKSPACE = 6,        /* workspace missing or too small */
    MOE_ERR_LAUNCH = 7,           /* a HIP error; never hidden */
    MOE_ERR_UNSUPPORTED = 8       /* outside this implementation's limits */
} moe_status;

/* A dense row-major tensor: ndim in 1..3 extents in dims[0..ndim-1]. */
typedef struct moe_tensor {
    void* data;
    int32_t dtype; /* moe_dtype */
    int32_t ndim;
    int64_t dims[3];
} moe_tensor;

/* Routing contract options: 1 <= top_k <= E; renormalize is 0 or 1. */
typedef struct moe_routing_options {
    int32_t top_k;
    int32_t renormalize;
} moe_routing_options;

/* Group-limited sigmoid routing options (section 10):
 *   top_k 1..64; groups 1..128 dividing E; selected_groups 1..groups;
 *   top_k <= selected_groups * (E / groups); group_top_two 0 or 1 (1 needs
 *   E / groups >= 2); renormalize 0 or 1; scale finite and > 0. */
typedef struct moe_group_routing_options {
    int32_t top_k;
    int32_t groups;
    int32_t selected_groups;
    int32_t group_top_two;
    int32_t renormalize;
    float scale;
} moe_group_routing_options;

/* Router-weight options of the training calls (RUDA guide, section 12):
 *   scoring MOE_SCORING_SOFTMAX (FP32 softmax over all E experts) or
 *   MOE_SCORING_SIGMOID (sigmoid of each logit); renormalize 0 or 1; scale
 *   finite and > 0, applied last. */
typedef enum moe_router_scoring {
    MOE_SCORING_SOFTMAX = 0,
    MOE_SCORING_SIGMOID = 1
} moe_router_scoring;
typedef struct moe_router_weight_options {
    int32_t scoring;
    int32_t renormalize;
    float scale;
} moe_router_weight_options;

/* Limits of this implementation (beyond them: MOE_ERR_UNSUPPORTED). */
#define MOE_MAX_EXPERTS 4096   /* E */
#define MOE_DIM_MULTIPLE 8     /* H and I of the expert products */

/*
 * moe_route -- routing contract (section 4).
 *   logits  [T,E]  F32 | F16 | BF16, read only.
 *   indices [T,k]  U32, written: per token the k experts with the largest
 *                  FP32 softmax probability, largest first, ties to the
 *                  lower id.  A row holding a NaN or +inf, or only -inf,
 *                  gets indices 0..k-1.
 *   weights [T,k]  logits dtype, written: the selected probabilities,
 *                  divided by their FP32 sum when renormalize is set, then
 *                  rounded to nearest even; NaN for the rows above.
 */
moe_status moe_route(const moe_tensor* logits, moe_routing_options options,
                     moe_tensor* indices, moe_tensor* weights, void* stream);

/*
 * moe_route_sigmoid_grouped -- group-limited sigmoid routing (section 10).
 *   logits  [T,E]  F32 | F16 | BF16, read only; E 1..1024 (beyond:
 *                  MOE_ERR_UNSUPPORTED).
 *   bias    [E]    F32 correction, read only, or NULL for none.  It steers
 *                  the choice only: corrected score c = sigmoid(l) + bias.
 *   indices [T,k]  U32, written: the experts chosen as follows, in order
 *                  of decreasing c, ties to the lower id.  The experts form
 *                  `groups` contiguous groups of E/groups; a group scores
 *                  its largest c (or, with group_top_two, the sum of its two
 *                  largest); the selected_groups best groups are kept (ties
 *                  to the lower group id); the top_k experts of the kept
 *                  groups by c are chosen.
 *   weights [T,k]  logits dtype, written: sigmoid(l) of the chosen experts
 *                  (not c), divided by their FP32 sum when renormalize is
 *                  set, times scale, rounded to nearest even.
 * A row with a NaN in c (a NaN logit or bias) gets indices 0..k-1 and NaN
 * weights.  Bad options: MOE_ERR_INVALID_ARGUMENT; top_k outside its range:
 * MOE_ERR_TOP_K.
 */
moe_status moe_route_sigmoid_grouped(const moe_tensor* logits, const moe_tensor* bias,
                                     moe_group_routing_options options, moe_tensor* indices,
                                     moe_tensor* weights, void* stream);

/* Workspace bytes moe_dispatch needs for T tokens, E experts, top_k. */
size_t moe_dispatch_workspace_bytes(int64_t T, int64_t E, int32_t top_k);

/*
 * moe_dispatch -- compact, drop-free dispatch (section 5).
 *   input          [T,H]   F32 | F16 | BF16, read only.
 *   indices        [T,k]   U32 expert ids, read only.  An id >= E is not
 *                          checked on the host (that would need a sync): its
 *                          slot is not copied, its row_of_slot is 0xFFFFFFFF,
 *                          and moe_combine turns that token's row into NaN.
 *   num_experts    E, 1..MOE_MAX_EXPERTS.
 *   dispatched     [T*k,H] input dtype, written: rows grouped by expert in
 *                          ascending expert id; each row is a bit copy of its
 *                          token.  Rows past expert_offsets[E] are untouched.
 *                          May be NULL: then no row is copied and only the
 *                          three mapping outputs are written (for
 *                          moe_experts_gate_up_gathered, which reads the
 *                          tokens in place).
 *   expert_offsets [E+1]   U32, written: rows of expert e are
 *                          [expert_offsets[e], expert_offsets[e+1]).
 *   row_of_slot    [T*k]   U32, written: dispatched row of slot t*k+j.
 *   token_of_row   [T*k]   U32, written: token of each dispatched row.
 *   workspace      >= moe_dispatch_workspace_bytes(T,E,k) device bytes.
 * The order of rows inside an expert follows device atomics and is not
 * fixed from run to run.
 */
moe_status moe_dispatch(const moe_tensor* input, const moe_tensor* indices, int64_t num_experts,
                        moe_tensor* dispatched, moe_tensor* expert_offsets,
                        moe_tensor* row_of_slot, moe_tensor* token_of_row,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes moe_experts_forward needs for N dispatched rows. */
size_t moe_experts_workspace_bytes(int64_t N, int64_t H, int64_t I, int64_t E, int32_t dtype);

/*
 * moe_experts_forward -- SwiGLU experts on dispatched rows (section 5):
 * for every row r of expert e, y_r = down_e (silu(gate_e x_r) * up_e x_r),
 * silu(z) = z / (1 + exp(-z)), FP32 accumulation, the activation stored in
 * the weight dtype between the two products.
 *   gate, up       [E,I,H]  F32 | F16 | BF16 (one dtype), read only.
 *   down           [E,H,I]  same dtype, read only.
 *   dispatched     [N,H]    same dtype, read only.
 *   expert_offsets [E+1]    U32 (as written by moe_dispatch), read only;
 *                           offsets past N or out of order are clamped, so
 *                           no access leaves the buffers.
 *   expert_out     [N,H]    same dtype, written for rows < expert_offsets[E].
 *   workspace      >= moe_experts_workspace_bytes(N,H,I,E,dtype) bytes.
 * H and I must be multiples of MOE_DIM_MULTIPLE.
 */
moe_status moe_experts_forward(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* down,
                               const moe_tensor* dispatched, const moe_tensor* expert_offsets,
                               moe_tensor* expert_out, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * moe_experts_gate_up / moe_experts_down -- the two halves of
 * moe_experts_forward, for callers that want the activation or time the
 * products separately.  Together they compute exactly what
 * moe_experts_forward computes (the same kernels, bit for bit).
 *   moe_experts_gate_up: h [N,I] (weight dtype) written for rows <
 *     expert_offsets[E]: h_r = silu(gate_e x_r) * up_e x_r, FP32 accumulation,
 *     rounded once to the weight dtype.
 *   moe_experts_down: expert_out [N,H] written for rows < expert_offsets[E]:
 *     y_r = down_e h_r, FP32 accumulation.
 *   Other arguments as for moe_experts_forward; the workspace of
 *   moe_experts_workspace_bytes is enough for either.
 */
moe_status moe_experts_gate_up(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* dispatched,
                               const moe_tensor* expert_offsets, moe_tensor* h, void* workspace,
                               size_t workspace_bytes, void* stream);
moe_status moe_experts_down(const moe_tensor* down, const moe_tensor* h, const moe_tensor* expert_offsets,
                            moe_tensor* expert_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_experts_gate_up_gathered -- moe_experts_gate_up with the dispatch
 * gather folded in (section 5: the saved token<->row mapping): product row r
 * reads token row input[token_of_row[r]] in place instead of a dispatched
 * copy.  Bit for bit the result of moe_experts_gate_up on the rows that
 * moe_dispatch would copy; moe_forward runs its products this way.
 *   input        [T,H]  weight dtype, read only.
 *   token_of_row [N]    U32 as written by moe_dispatch, read only; an entry
 *                       >= T is clamped to T-1, so no access leaves input.
 *   h            [N,I]  written for rows < expert_offsets[E].
 *   Other arguments as for moe_experts_gate_up (workspace of
 *   moe_experts_workspace_bytes(N, ...)).
 */
moe_status moe_experts_gate_up_gathered(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* input,
                                        const moe_tensor* token_of_row, const moe_tensor* expert_offsets,
                                        moe_tensor* h, void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_combine -- weighted combine in token order (sections 5 and 6):
 * out[t] = sum over j < k, in order, of weights[t,j] * expert_out[row_of_slot[t*k+j]],
 * accumulated in FP32 and rounded once to the input dtype.
 *   expert_out  [N,H]  F32 | F16 | BF16, read only.
 *   row_of_slot [T*k]  U32, read only; a row >= N (e.g. 0xFFFFFFFF) makes
 *                      the token's output row NaN.
 *   weights     [T,k]  F32 | F16 | BF16, read only.
 *   output      [T,H]  expert_out dtype, written.
 */
moe_status moe_combine(const moe_tensor* expert_out, const moe_tensor* row_of_slot,
                       const moe_tensor* weights, moe_tensor* output, void* stream);

/* Workspace bytes moe_forward needs. */
size_t moe_forward_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int32_t top_k,
                                   int32_t dtype);

/*
 * moe_forward -- the whole local chain (section 6, SwiGluExperts::forward):
 * route, dispatch, experts and combine on one stream.
 *   gate, up [E,I,H]; down [E,H,I]; input [T,H]: one float dtype.
 *   logits [T,E]: F32 | F16 | BF16, independent of the input dtype.
 *   output [T,H]: input dtype, written.
 *   workspace >= moe_forward_workspace_bytes(T,H,I,E,k,dtype) bytes.
 */
moe_status moe_forward(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* down,
                       const moe_tensor* input, const moe_tensor* logits,
                       moe_routing_options options, moe_tensor* output,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_forward_sigmoid_grouped -- moe_forward with group-limited sigmoid
 * routing (section 10, forward_sigmoid_grouped): moe_route_sigmoid_grouped,
 * then dispatch, experts and combine as moe_forward does them.
 *   bias [E] F32 or NULL; options as for moe_route_sigmoid_grouped; the
 *   other arguments as for moe_forward, with the workspace of
 *   moe_forward_workspace_bytes(T, H, I, E, options.top_k, dtype).
 */
moe_status moe_forward_sigmoid_grouped(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* down,
                                       const moe_tensor* input, const moe_tensor* logits, const moe_tensor* bias,
                                       moe_group_routing_options options, moe_tensor* output,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_forward_no_alloc -- moe_forward for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  It takes no workspace: the library
 * keeps a static device array of 64 MiB (67108864 bytes) per device, held
 * from the library's load until the process ends, and runs moe_forward's
 * kernels with that array as their workspace.  It calls no hipMalloc,
 * hipFree or allocating library routine.
 *   Arguments as for moe_forward, without workspace and workspace_bytes.
 *   Limit: moe_forward_workspace_bytes(T, H, I, E, top_k, dtype) must not
 *   exceed 67108864 (e.g. T*top_k rows of H = 4096, I = 1536 in BF16 up to
 *   about 5900 rows); larger batches get MOE_ERR_WORKSPACE and nothing is
 *   enqueued.
 *   The first call on a device looks up that device's array (a host-side
 *   symbol lookup, no allocation); make one call before capturing a graph
 *   if that lookup must stay outside the capture.  A device error of the
 *   stream is reported before shape errors.
 *   Every call on one device uses the same array, so calls that overlap on
 *   one device (two streams, or two host threads) race and give undefined
 *   results: serialise them.  Every value the chain needs zeroed is cleared
 *   by its own kernels, so the contents left by an earlier call do not
 *   matter.
 */
moe_status moe_forward_no_alloc(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* down,
                                const moe_tensor* input, const moe_tensor* logits,
                                moe_routing_options options, moe_tensor* output, void* stream);

/* ------------------------------------------------------------------ */
/* First-order training (RUDA ruDNN library guide, section 12).          */
/* The forward keeps what the backward needs (the FP32 pre-activations   */
/* and the activation); the backward then runs, in this order:           */
/* moe_combine_backward, moe_experts_backward, moe_dispatch_backward and */
/* moe_router_backward.  Only the weights of the fixed selection are     */
/* differentiated: not the top-k choice, the group choice or a           */
/* correction bias.  The saved inputs must not change before the         */
/* backward.                                                             */
/* ------------------------------------------------------------------ */

/*
 * moe_router_weights -- selected_router_weights: the weights of a fixed
 * selection.
 *   logits  [T,E]  F32 | F16 | BF16, read only.
 *   indices [T,k]  U32 | I32 | I64, read only; 1 <= k <= min(E, 64).  A
 *                  repeated index is gathered again.  An index outside
 *                  [0, E) is not checked on the host: it makes the token's
 *                  row NaN, with no access outside the logits.
 *   weights [T,k]  F32, written: w_j = scale * q_j / S, with q_j the score
 *                  (softmax probability or sigmoid) of expert indices[t,j]
 *                  and S the FP32 sum of the row's q in slot order when
 *                  renormalize is set (else w_j = scale * q_j).
 */
moe_status moe_router_weights(const moe_tensor* logits, const moe_tensor* indices,
                              moe_router_weight_options options, moe_tensor* weights, void* stream);

/*
 * moe_router_backward -- selected_router_backward: d loss / d logits from
 * the FP32 weight gradients, for the same selection and options.
 *   grad_weights [T,k]  F32, read only.
 *   grad_logits  [T,E]  logits dtype, written (every element; NaN rows for
 *                       tokens with an index outside [0, E)).
 *   Other arguments as for moe_router_weights.
 */
moe_status moe_router_backward(const moe_tensor* logits, const moe_tensor* indices,
                               const moe_tensor* grad_weights, moe_router_weight_options options,
                               moe_tensor* grad_logits, void* stream);

/*
 * moe_combine_backward -- step 1: the backward of moe_combine.
 *   expert_out      [N,H]  F32 | F16 | BF16, read only (the forward's).
 *   row_of_slot     [T*k]  U32, read only (moe_dispatch's).
 *   weights         [T,k]  F32 | F16 | BF16, read only (the combine's).
 *   grad_output     [T,H]  expert_out dtype, read only.
 *   grad_expert_out [N,H]  expert_out dtype, written for every row some slot
 *                          names: row_of_slot[t*k+j] gets weights[t,j] *
 *                          grad_output[t], rounded once.
 *   grad_weights    [T,k]  F32, written: <expert_out[row_of_slot[t*k+j]],
 *                          grad_output[t]>, FP32 sums in a fixed order; NaN
 *                          for every slot of a token with a row >= N.
 */
moe_status moe_combine_backward(const moe_tensor* expert_out, const moe_tensor* row_of_slot,
                                const moe_tensor* weights, const moe_tensor* grad_output,
                                moe_tensor* grad_expert_out, moe_tensor* grad_weights, void* stream);

/*
 * moe_experts_forward_training -- forward_dispatched_training: the experts
 * forward (bit for bit moe_experts_forward's output) that also keeps the
 * cache of the backward.
 *   rows           [R,H]   weight dtype, read only: the N dispatched rows
 *                          (token_of_row NULL, R = N), or the T token rows
 *                          read in place through token_of_row.
 *   token_of_row   [N]     U32 (moe_dispatch's) or NULL; an entry >= R is
 *                          clamped to R-1.
 *   expert_out     [N,H]   written for rows < expert_offsets[E].
 *   preact         [N,2I]  F32, written: g = gate_e x in columns [0, I),
 *                          u = up_e x in [I, 2I), FP32 accumulations.
 *   h              [N,I]   weight dtype, written: silu(g) * u, rounded once.
 *   workspace      >= moe_experts_workspace_bytes(N,H,I,E,dtype) bytes.
 *   Other arguments as for moe_experts_forward.
 */
moe_status moe_experts_forward_training(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* down,
                                        const moe_tensor* rows, const moe_tensor* token_of_row,
                                        const moe_tensor* expert_offsets, moe_tensor* expert_out,
                                        moe_tensor* preact, moe_tensor* h, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* Workspace bytes moe_experts_backward needs for N dispatched rows. */
size_t moe_experts_backward_workspace_bytes(int64_t N, int64_t H, int64_t I, int64_t E, int32_t dtype);

/*
 * moe_experts_backward -- step 2 (cache.backward): for the rows r of expert
 * e, with dh = grad_expert_out_r down_e, s = 1/(1+exp(-g)):
 *   du = dh * g * s and dg = dh * u * s * (1 + g * (1 - s)), each rounded
 *   to the weight dtype;
 *   grad_rows_r = gate_e^T dg + up_e^T du   [N,H] weight dtype, written for
 *                                            rows < expert_offsets[E];
 *   grad_gate_e = sum_r dg x_r^T, grad_up_e = sum_r du x_r^T   [E,I,H] F32;
 *   grad_down_e = sum_r grad_expert_out_r h_r^T                [E,H,I] F32;
 *   FP32 accumulation; an expert without rows gets zero gradients.
 *   rows, token_of_row, expert_offsets, preact, h: as given to (and written
 *   by) moe_experts_forward_training; grad_expert_out [N,H] weight dtype.
 *   workspace >= moe_experts_backward_workspace_bytes(N,H,I,E,dtype) bytes.
 */
moe_status moe_experts_backward(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* down,
                                const moe_tensor* rows, const moe_tensor* token_of_row,
                                const moe_tensor* expert_offsets, const moe_tensor* preact, const moe_tensor* h,
                                const moe_tensor* grad_expert_out, moe_tensor* grad_rows, moe_tensor* grad_gate,
                                moe_tensor* grad_up, moe_tensor* grad_down, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * moe_dispatch_backward -- step 3: grad_input[t] = the FP32 sum, in slot
 * order, of grad_rows[row_of_slot[t*k+j]] over j < top_k, rounded once; the
 * routing weights are not applied again.
 *   grad_rows   [N,H]      F32 | F16 | BF16, read only.
 *   row_of_slot [T*top_k]  U32, read only; a row >= N makes the token's
 *                          grad_input row NaN.
 *   grad_input  [T,H]      grad_rows dtype, written.
 */
moe_status moe_dispatch_backward(const moe_tensor* grad_rows, const moe_tensor* row_of_slot, int32_t top_k,
                                 moe_tensor* grad_input, void* stream);

/* Static text of a status code. */
const char* moe_status_string(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
