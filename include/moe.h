/*
 * moe.h - C ABI of a single-GPU Mixture-of-Experts layer forward for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer is the pipeline the DWDP-Triton-MoE-Inference-Engine README lays
 * out ("Runtime Integration Layer"): a router (router logits, routing
 * probabilities, top-k expert ids, normalised routing weights), a dispatcher
 * (token-major assignments -> expert-major layout), an executor (grouped
 * SwiGLU experts over the expert ranges) and a merger (weighted combine back
 * to token order).  The comms planner of that pipeline has no role on one GPU.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  - Every tensor argument is a DEVICE pointer to a contiguous row-major
 *    array owned by the caller; the library never allocates, frees or keeps
 *    a pointer after the call returns.  Pointers to activations, weights and
 *    outputs must be 16-byte aligned.
 *  - `dtype` (moe_dtype) is the storage type of the hidden states and of every
 *    weight.  Logits, routing weights, router bias and shared-gate logits are
 *    always float32; the packed expert outputs are float32 or, for bf16
 *    layers, bf16 (an explicit argument says which); expert ids and every
 *    dispatch array are int32.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    call only enqueues work on that stream: it does not synchronise and does
 *    not copy anything to the host.
 *  - Shapes: T = num_tokens, H = hidden_size, E = num_experts, k = top_k,
 *    I = intermediate_size, P = T*k (number of (token, expert) assignments).
 *  - Assignments are indexed token-major, a = t*k + j (row-major [T, k]), as
 *    build_ep_routing_table in metrale's ep_dispatch.rs reads its gate arrays.
 *  - Errors: every argument check runs on the host before anything is
 *    enqueued; on any status other than MOE_OK nothing was enqueued, except
 *    for MOE_ERR_HIP, which reports a failed launch.  moe_last_error_message()
 *    returns a per-thread text naming the offending argument (for example
 *    "topk_ids is NULL" or "workspace too small").  num_tokens == 0 is a valid
 *    no-op that returns MOE_OK.
 *  - Device-side preconditions that the host cannot see (expert ids in
 *    [0, E), offsets consistent with P) are the caller's contract; the plan
 *    produced by moe_dispatch_plan always satisfies them.
 *  - Limits: 1 <= E <= 512, 1 <= k <= E, T*k < 2^31, H a multiple of 8.
 *    I (and the shared expert's I) a multiple of 16, which admits the expert
 *    widths of 8-way tensor-parallel slices (768 / 8 = 96, 1408 / 8 = 176).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5
#define MOE_MAX_EXPERTS 512

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* NULL pointer, bad size, k out of range, length mismatch */
  MOE_ERR_UNSUPPORTED = 2, /* valid but not supported: E > 512, H/I alignment, misaligned pointer */
  MOE_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than the *_workspace_size() result */
  MOE_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} moe_status;

typedef enum moe_dtype {
  MOE_DTYPE_F32 = 0,
  MOE_DTYPE_BF16 = 1,
  /* a bf16 layer whose expert weights (w13, w2 and the shared expert's
   * shared_w13, shared_w2) are in the K-blocked layout that moe_pack_weights
   * writes; activations, the router weight and the shared gate stay
   * row-major.  Accepted wherever a bf16 layer is. */
  MOE_DTYPE_BF16_KB32 = 2
} moe_dtype;

/* Projection of one expert, as a per-expert checkpoint names it. */
typedef enum moe_proj {
  MOE_PROJ_GATE = 0, /* gate_proj (w1) [I, H] */
  MOE_PROJ_UP = 1,   /* up_proj (w3)   [I, H] */
  MOE_PROJ_DOWN = 2  /* down_proj (w2) [H, I] */
} moe_proj;

/* MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);

/* Static text of a status code ("MOE_OK", ...). Never NULL. */
const char* moe_status_string(int status);

/* Per-thread text of the last error raised by a call on this thread, "" if
 * the last call succeeded. Valid until the next call on the same thread. */
const char* moe_last_error_message(void);

/*
 * Router: logits, softmax, top-k, routing weights.
 * [DWDP README "Router Module"; diffulex.moe "diffulex.moe.topk": a standard
 *  top-k router]
 *
 *   router_logits[t,e] = sum_h hidden_states[t,h] * router_weight[e,h]
 *                        (+ router_bias[e])                          (fp32 accumulate)
 *   topk_ids[t,:]      = the k experts with the largest logits, in descending
 *                        logit order; equal fp32 logits go to the lower id first,
 *                        -0.0 counts as equal to +0.0
 *   topk_weights[t,j]  = softmax(router_logits[t])[topk_ids[t,j]], divided by the
 *                        sum over the k chosen experts when renormalize != 0
 *                        (so each token's weights sum to one)
 *   routing_probs[t,e] = softmax(router_logits[t])[e]
 *   shared_gate_logit[t] = sum_h hidden_states[t,h] * shared_gate[h]
 *
 * hidden_states [T,H] dtype; router_weight [E,H] dtype; router_bias [E] f32 or
 * NULL (added before the softmax, so it moves the selection and the weights);
 * shared_gate [H] dtype or NULL; router_logits [T,E] f32 (required, never
 * NULL: the top-k stage reads the logits back from this buffer, and the
 * library allocates no memory of its own to hold them); routing_probs [T,E]
 * f32 or NULL; topk_ids [T,k] int32 (required);
 * topk_weights [T,k] f32 (required); shared_gate_logit [T] f32, required iff
 * shared_gate != NULL.
 * Errors: INVALID_ARG for a NULL required pointer, k < 1 or k > E, negative
 * sizes, shared_gate without shared_gate_logit (or the reverse);
 * UNSUPPORTED for E > 512, alignment.
 */
moe_status moe_router_topk(const void* hidden_states, const void* router_weight,
                           const float* router_bias, const void* shared_gate,
                           int64_t num_tokens, int64_t hidden_size, int64_t num_experts,
                           int64_t top_k, int renormalize, int dtype,
                           float* router_logits, float* routing_probs,
                           int32_t* topk_ids, float* topk_weights,
                           float* shared_gate_logit, void* stream);

/*
 * Router with group-limited expert selection.
 * [diffulex.moe "diffulex.moe.topk": GroupLimitedTopKRouter, a router with
 *  group-limited expert selection; the steps below are this library's
 *  reading, the page gives none]
 *
 * As moe_router_topk (no shared gate), except for the choice of experts:
 *   group g holds experts [g*E/n_group, (g+1)*E/n_group); its score is its
 *   largest logit; the topk_group highest-scoring groups are kept (equal
 *   scores: the lower group first); topk_ids[t,:] are the k largest logits
 *   among the kept groups' experts, with the ordering and tie rule of
 *   moe_router_topk.  Weights and routing_probs are defined as there (the
 *   softmax runs over all E experts).  n_group == 1 is moe_router_topk.
 * Errors: as moe_router_topk, plus INVALID_ARG unless 1 <= n_group <= 64,
 * n_group divides E, 1 <= topk_group <= n_group and
 * k <= topk_group * E / n_group.
 */
moe_status moe_router_topk_grouped(const void* hidden_states, const void* router_weight,
                                   const float* router_bias, int64_t num_tokens, int64_t hidden_size,
                                   int64_t num_experts, int64_t top_k, int64_t n_group,
                                   int64_t topk_group, int renormalize, int dtype,
                                   float* router_logits, float* routing_probs,
                                   int32_t* topk_ids, float* topk_weights, void* stream);

/*
 * Dispatch plan: token-major assignments -> expert-major layout.
 * [DWDP README "Dispatcher Module": expert-major grouping, per-expert counts,
 *  expert offsets, token permutation, inverse permutation, packed token
 *  indices, packed routing weights; metrale ep_dispatch.rs EpRoutingTable:
 *  assignments kept in the order given]
 *
 *   expert_counts[e]          = #{a : topk_ids[a] == e}                        [E]
 *   expert_offsets[e]         = sum_{e' < e} expert_counts[e'], offsets[E] = P  [E+1]
 *   token_permutation[p]      = a, listing the assignments sorted stably by
 *                               (expert id, a)                                 [P]
 *   inverse_permutation[a]    = p with token_permutation[p] == a               [P]
 *   packed_token_indices[p]   = token_permutation[p] / k                       [P]
 *   packed_routing_weights[p] = topk_weights[token_permutation[p]]             [P] f32
 *
 * The plan is deterministic: positions come from counts and prefix sums, never
 * from the order of atomic operations.  topk_weights may be NULL, then
 * packed_routing_weights must be NULL too.
 * workspace: at least moe_dispatch_workspace_size(T, k, E) bytes of device
 * memory, 256-byte aligned; its contents are scratch.
 * Errors: INVALID_ARG for NULL outputs or k/E out of range; WORKSPACE.
 */
size_t moe_dispatch_workspace_size(int64_t num_tokens, int64_t top_k, int64_t num_experts);
moe_status moe_dispatch_plan(const int32_t* topk_ids, const float* topk_weights,
                             int64_t num_tokens, int64_t top_k, int64_t num_experts,
                             int32_t* expert_counts, int32_t* expert_offsets,
                             int32_t* token_permutation, int32_t* inverse_permutation,
                             int32_t* packed_token_indices, float* packed_routing_weights,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dispatch plan without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).
 *
 * Same arguments, outputs, determinism and errors as moe_dispatch_plan, minus
 * the workspace: the plan's scratch (per-segment expert counts and bases) is a
 * fixed device array inside the library, moe_dispatch_noalloc_max_workspace()
 * bytes (8 MiB) per GPU, held by each GPU the library runs on until the
 * process ends.  The call allocates and frees nothing.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (different
 * streams, or different host threads without ordering) race on it and must
 * not be issued.  Nothing in it needs clearing: each call writes every entry
 * it later reads.
 * Errors: as moe_dispatch_plan; UNSUPPORTED when the plan's scratch,
 * moe_dispatch_workspace_size(T, k, E), exceeds the fixed size (for example
 * E = 128 allows up to T*k = 2^20 assignments); MOE_ERR_HIP when the array's
 * device address cannot be looked up.
 */
size_t moe_dispatch_noalloc_max_workspace(void);
moe_status moe_dispatch_plan_noalloc(const int32_t* topk_ids, const float* topk_weights,
                                     int64_t num_tokens, int64_t top_k, int64_t num_experts,
                                     int32_t* expert_counts, int32_t* expert_offsets,
                                     int32_t* token_permutation, int32_t* inverse_permutation,
                                     int32_t* packed_token_indices, float* packed_routing_weights,
                                     void* stream);

/*
 * Expert-parallel routing table: the assignments split into this rank's
 * experts and the rest.
 * [metrale_model_layers ep_dispatch.rs: build_ep_routing_table,
 *  EpRoutingTable; its tests print the expected tables]
 *
 * Assignment a = t*k + j of the row-major [T,k] gate arrays is local when
 * local_expert_start <= gate_indices[a] < local_expert_end, the ids compared
 * as unsigned 32-bit values (the page's expert ids are u32; a negative int32
 * is a large id and therefore remote).  Each bucket lists its entries in
 * assignment order; entry i is the triple
 *   (*_token_indices[i] = a / k, *_expert_ids[i] = gate_indices[a] (global,
 *    not rank-relative), *_weights[i] = gate_weights[a]).
 * counts[0] = local entries, counts[1] = remote entries; their sum is T*k.
 *
 * gate_indices [gate_indices_len] int32, gate_weights [gate_weights_len] f32;
 * each of the six outputs must hold T*k entries (device, caller-owned; only
 * the first counts[0] / counts[1] are written); counts [2] int32 device.
 * Errors: INVALID_ARG "gate_indices length mismatch" /
 * "gate_weights length mismatch" when a length is not num_tokens * top_k
 * (the page's function panics with these texts), NULL pointers, negative
 * range bounds, top_k < 1; WORKSPACE.  num_tokens == 0 writes counts = {0, 0}.
 * Deterministic (prefix sums, no atomics).
 * workspace: moe_ep_routing_table_workspace_size(T, k) bytes of device memory.
 */
size_t moe_ep_routing_table_workspace_size(int64_t num_tokens, int64_t top_k);
moe_status moe_ep_routing_table(const int32_t* gate_indices, int64_t gate_indices_len, const float* gate_weights,
                                int64_t gate_weights_len, int64_t num_tokens, int64_t top_k,
                                int64_t local_expert_start, int64_t local_expert_end,
                                int32_t* local_token_indices, int32_t* local_expert_ids, float* local_weights,
                                int32_t* remote_token_indices, int32_t* remote_expert_ids, float* remote_weights,
                                int32_t* counts, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Expert-parallel send counts: how many rows of the expert-major packed order
 * (the dispatch plan) go to each of num_ranks ranks that own contiguous
 * expert ranges, and where each rank's segment starts.
 * [metrale_model_layers ep_dispatch.rs: one rank's local_expert_start and
 *  local_expert_end; DWDP README "Dispatcher Module": expert-major layout
 *  with per-expert offsets]
 *
 * Rank r owns experts [floor(r*E/G), floor((r+1)*E/G)) (G = num_ranks; the
 * pages fix one rank's range, not how ranges are chosen: contiguous, every
 * expert once, sizes within one of each other).  Then
 *   send_counts[r]  = expert_offsets[(r+1)*E/G] - expert_offsets[r*E/G]   [G] int32
 *   send_offsets[r] = expert_offsets[r*E/G],  send_offsets[G] = expert_offsets[E]   [G+1] int32
 * which are the all-to-all-v send counts and displacements of the packed rows.
 * expert_offsets [E+1] int32 (device, as moe_dispatch_plan writes it);
 * send_counts [G] int32 device; send_offsets [G+1] int32 device or NULL.
 * Errors: INVALID_ARG for NULL pointers, num_experts outside [1, 512],
 * num_ranks outside [1, num_experts].
 */
moe_status moe_ep_rank_counts(const int32_t* expert_offsets, int64_t num_experts, int64_t num_ranks,
                              int32_t* send_counts, int32_t* send_offsets, void* stream);

/*
 * Grouped expert SwiGLU FFN over the expert-major layout.
 * [DWDP README "Executor Module": gather token activations per expert range,
 *  run the expert, write packed expert outputs; modelexpress refit test,
 *  FusedMoEModel: w13 holds the gate (w1) rows then the up (w3) rows of each
 *  expert slot]
 *
 * For every expert e and packed row p in [expert_offsets[e], expert_offsets[e+1]),
 * with x = hidden_states[packed_token_indices[p]]:
 *   g = w13[e, 0:I, :] . x,  u = w13[e, I:2I, :] . x
 *   h = silu(g) * u,  silu(z) = z / (1 + exp(-z))
 *   packed_expert_outputs[p] = w2[e] . h                          [P,H] expert_out_dtype
 * Routing weights are NOT applied here (moe_combine applies them).
 *
 * hidden_states [T,H] dtype; packed_token_indices [P] int32, or NULL meaning
 * row p reads token p (requires P <= T); expert_offsets [E+1] int32 device, or
 * NULL meaning a single expert (E must be 1) owning all P rows; w13 [E,2I,H]
 * dtype; w2 [E,H,I] dtype.  P = num_tokens * top_k.
 * Numerics (bf16): fp32 accumulation, h rounded once to bf16 (it is the
 * operand of the second bf16 GEMM), outputs fp32 or rounded once to bf16
 * (expert_out_dtype MOE_DTYPE_F32 or MOE_DTYPE_BF16; bf16 halves the bytes
 * the down projection writes and the combine reads).  f32 layers: fp32
 * throughout, expert_out_dtype must be MOE_DTYPE_F32.
 * Experts with no rows are skipped and their weights are not read.
 * workspace: moe_grouped_ffn_workspace_size(...) bytes (tile counters, h,
 * and for few rows per expert the fp32 partial sums of a split K loop).
 */
size_t moe_grouped_ffn_workspace_size(int64_t num_tokens, int64_t hidden_size, int64_t top_k,
                                      int64_t num_experts, int64_t intermediate_size, int dtype);
moe_status moe_grouped_ffn(const void* hidden_states, const int32_t* packed_token_indices,
                           const int32_t* expert_offsets, const void* w13, const void* w2,
                           int64_t num_tokens, int64_t hidden_size, int64_t num_experts,
                           int64_t top_k, int64_t intermediate_size, int dtype,
                           int expert_out_dtype, void* packed_expert_outputs,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Weighted combine back to token order.
 * [DWDP README "Merger Module": restore token-major assignment order,
 *  accumulate the top-k expert outputs, apply routing weights]
 *
 *   output[t] = sum_{j=0..k-1} topk_weights[t,j] * packed_expert_outputs[inverse_permutation[t*k+j]]
 *               (+ sigmoid(shared_gate_logit[t]) * shared_output[t])
 * summed in ascending j in fp32, the shared term added last.
 *
 * packed_expert_outputs [P,H] and shared_output [T,H] (or NULL) are
 * expert_dtype (MOE_DTYPE_F32 or MOE_DTYPE_BF16; bf16 values are widened
 * exactly); inverse_permutation [P] int32; topk_weights [T,k] f32;
 * shared_gate_logit [T] f32 or NULL (NULL with a shared_output means a gate
 * of 1); out_dtype MOE_DTYPE_F32 or MOE_DTYPE_BF16 (round to nearest even);
 * output [T,H] out_dtype.
 */
moe_status moe_combine(const void* packed_expert_outputs, const int32_t* inverse_permutation,
                       const float* topk_weights, const void* shared_output,
                       const float* shared_gate_logit,
                       int64_t num_tokens, int64_t hidden_size, int64_t top_k,
                       int expert_dtype, int out_dtype, void* output, void* stream);

/*
 * Whole layer forward: router -> dispatch plan -> grouped FFN -> combine,
 * plus an optional sigmoid-gated shared expert.
 * [DWDP README "How To Use": build_reference binds one explicit layer of
 *  hidden_size, num_experts, top_k and expert weights; "Runtime Integration
 *  Layer": the runtime owns reusable workspaces; diffulex.moe
 *  "diffulex.moe.layer": SharedExpertMLP]
 *
 *   output = combine(grouped_ffn(dispatch(router(x))))
 *            + sigmoid(x . shared_gate) * W2s (silu(W13s[0:Is] x) * W13s[Is:2Is] x)
 *
 * shared_w13 [2*Is,H], shared_w2 [H,Is], shared_gate [H] (all dtype) are all
 * given or all NULL (then shared_intermediate_size is ignored).
 * Optional outputs (NULL to skip): topk_ids_out [T,k] int32, topk_weights_out
 * [T,k] f32, router_logits_out [T,E] f32.
 * workspace: moe_forward_workspace_size(...) bytes; it holds the routing, the
 * plan, h and the packed expert outputs y in a slot of P*H*4 bytes.  What y
 * holds there depends on the batch: fp32 values for f32 layers and for bf16
 * layers with fewer than 96 packed rows per expert on average (decode-sized
 * batches); for bf16 layers with at least 96 (prefill-sized batches) and H a
 * multiple of 64, fp16 values y*2^s (P*H*2 bytes) followed by one int32
 * exponent s per (row, 64 columns) (P*H/16 bytes), s chosen per segment from
 * its largest magnitude so the fp16 values keep 11 significant bits without
 * overflow.  Both carry about 8x the precision of bf16 storage, which would
 * about double the output error of a bf16 layer.  The y slot is internal to
 * the forward (moe_grouped_ffn returns fp32 or bf16 expert outputs).
 */
size_t moe_forward_workspace_size(int64_t num_tokens, int64_t hidden_size, int64_t num_experts,
                                  int64_t top_k, int64_t intermediate_size,
                                  int64_t shared_intermediate_size, int dtype);
moe_status moe_forward(const void* hidden_states, const void* router_weight,
                       const float* router_bias, const void* w13, const void* w2,
                       const void* shared_w13, const void* shared_w2, const void* shared_gate,
                       int64_t num_tokens, int64_t hidden_size, int64_t num_experts,
                       int64_t top_k, int64_t intermediate_size,
                       int64_t shared_intermediate_size, int renormalize, int dtype,
                       int out_dtype, void* output,
                       int32_t* topk_ids_out, float* topk_weights_out, float* router_logits_out,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Tensor-parallel expert weight loader: one projection of one expert, the
 * slice that rank tp_rank of tp_size owns, copied into the rank's fused
 * buffers (the w13 / w2 that moe_grouped_ffn and moe_forward read).
 * [modelexpress refit test "test_reshard_refit_moe_experts.py": the module
 *  docstring gives the destination w13 [local_experts, 2*inter_per_tp,
 *  hidden]; FusedMoEModel._expert_loader takes the rank's rows of the source
 *  and writes them to the member half of the expert's slot, gate (w1) low,
 *  up (w3) high]
 *
 * With Ip = intermediate_size / tp_size the rank owns the intermediate
 * indices [tp_rank*Ip, tp_rank*Ip + Ip):
 *   MOE_PROJ_GATE / MOE_PROJ_UP: src [I, H];
 *     w13[expert, m*Ip + i, :] = src[tp_rank*Ip + i, :]   (m = 0 gate, 1 up)
 *     dst is w13 [local_experts, 2*Ip, H].
 *   MOE_PROJ_DOWN: src [H, I];
 *     w2[expert, h, i] = src[h, tp_rank*Ip + i]
 *     dst is w2 [local_experts, H, Ip].  The pages print the w13 loader only;
 *     the down projection is split along the same intermediate index, its
 *     columns, which makes the ranks' layer outputs add up to the unsliced
 *     layer's output (the all-reduce of tensor parallelism).
 * Elements are copied bit for bit; dtype only gives their size.  Unlike every
 * other entry point, src may be host or device memory (contiguous row-major);
 * dst is device memory, caller-owned.  The copy is enqueued on `stream`; a
 * host src must stay valid until the stream has passed the copy.
 * Errors: INVALID_ARG for NULL pointers, sizes < 1, tp_size < 1, tp_rank not
 * in [0, tp_size), expert not in [0, local_experts), an unknown proj, or a
 * tp_size that does not divide intermediate_size; MOE_ERR_HIP when the copy
 * cannot be enqueued.
 */
moe_status moe_tp_load_expert(const void* src, int proj, int64_t hidden_size, int64_t intermediate_size,
                              int tp_size, int tp_rank, int64_t expert, int64_t local_experts, int dtype,
                              void* dst, void* stream);

/*
 * K-blocked expert weights for MOE_DTYPE_BF16_KB32 layers, written once when
 * a layer is loaded.
 * [DWDP README "Executor Module": the executor runs each expert's FFN from
 *  its weights; modelexpress refit test: the fused w13 [E, 2I, H] and w2
 *  [E, H, I] it reads]
 *
 *   dst[g][b][r][i] = src[g][r][32*b + i]   for b < ceil(k/32), i < 32
 *                     (0 where 32*b + i >= k)
 *
 * src [groups, rows, k] bf16, row-major: w13 (groups = E, rows = 2I, k = H),
 * w2 (E, H, I), or the shared expert's shared_w13 (1, 2Is, H) and shared_w2
 * (1, H, Is).  dst: moe_packed_weights_size(groups, rows, k) bytes.  A K step
 * of 32 of a block of rows is then one contiguous run of memory: the grouped
 * GEMMs fetch whole 128-byte lines from it where a row-major K step of 32
 * covers half a line of each row.
 * k a multiple of 8; src and dst 16-byte aligned and not overlapping; one
 * group's packed bytes under 2 GiB (UNSUPPORTED otherwise); NULL pointers or
 * sizes < 1: INVALID_ARG.  Enqueued on `stream`, nothing allocated.
 */
size_t moe_packed_weights_size(int64_t groups, int64_t rows, int64_t k);
moe_status moe_pack_weights(const void* src, void* dst, int64_t groups, int64_t rows, int64_t k, void* stream);

/*
 * Kernel timing for measurement tools.  While enabled, every kernel the
 * library launches is bracketed by two HIP events recorded on the stream the
 * kernel is launched on.  moe_profile_collect() waits for the recorded events,
 * adds each kernel's elapsed time to its name's total, and clears the record.
 * This is process-wide state guarded by a mutex; it is meant for benchmarks,
 * not for concurrent production calls.
 *   names   : receives up to `capacity` static kernel-name strings
 *   total_ms: summed duration per name; launches: launch count per name
 * Returns the number of distinct names recorded (may exceed capacity).
 */
void moe_profile_enable(int enable);
int moe_profile_collect(const char** names, double* total_ms, int64_t* launches, int capacity);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
