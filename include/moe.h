/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE expert layer: one GPU's share of
 * a DeepSeek-V3-style mixture-of-experts layer, in four calls:
 *
 *   moe_route       group-limited top-k routing of each token
 *   moe_dispatch    counting-sort permutation of token rows to local experts
 *                   (moe_dispatch_capacity: the same with a per-expert capacity;
 *                   moe_dispatch_masked: into fixed per-expert slots;
 *                   moe_dispatch_deferred: overflow deferred to later rounds)
 *   moe_expert_ffn  grouped SwiGLU expert FFN (fused gate_up GEMM, SiLU*up, down GEMM)
 *   moe_combine     router-weighted sum of the expert outputs, back in token order
 *
 * the FP8 variant of the expert FFN (moe_quantize_e4m3 for the token rows,
 * moe_expert_ffn_fp8), and, for placement across GPUs, moe_eplb_place (host
 * planner), moe_eplb_remap (logical to physical replica per routed slot) and
 * moe_eplb_remap_capacity (the same with a per-replica capacity).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every array argument is a DEVICE pointer owned by the caller (except
 *   those of moe_eplb_place and moe_expert_capacity, which are host
 *   pointers); the library keeps no pointer after a call returns and
 *   allocates no memory (moe_expert_ffn_noalloc uses a fixed device array of
 *   the library's own instead of a workspace argument).
 * - Calls are asynchronous on `stream` (0 = the default stream). They do not
 *   synchronise with the host, so a sequence of calls can be captured in a
 *   HIP graph.
 * - Every argument is validated on the host before anything is enqueued; a
 *   call that returns an error status has enqueued nothing, except
 *   MOE_ERR_LAUNCH, which reports a failed kernel launch (hipGetLastError).
 * - Layouts are row-major and dense. bf16 buffers hold bf16 bit patterns.
 *   Activations and weights are 16-byte aligned.
 * - Preconditions not checked on the device: scores are finite; with
 *   renormalisation the selected scores have a positive sum; outputs do not
 *   alias inputs; topk_ids hold values in [0, num_experts).
 *
 * Sources (web pages; sections as printed on them):
 * - "大规模 EP 部署：分层 EPLB、DP 注意力的负载与双 batch 重叠" (anrans.github.io,
 *   ai-infra-handbooks serving/moe/ep-deploy), section "EPLB 与路由约束":
 *   group-limited routing, its seeded simulation, and the EPLB strategies.
 * - "第十五章：多节点大模型推理——并行部署、解码优化与 MoE 路由"
 *   (se7en.mintlify.app ch15), sections 3.4 and 4.1: gating, dispatch, combine;
 *   section 4.3: the capacity factor and the overflow policies.
 * - "追踪一个 Token 在 MoE 推理中穿越 TP/CP/SP/EP/DP/PP 的路径" (attain.fans),
 *   hop 4: y = p5 E5(x) + p27 E27(x).
 * - "Lecture 6 · 并行" (semidirectx.com cs349d lecture06), section 2.2: the
 *   gated MLP with W_gate, W_up, W_down.
 * - "推理 INFRA 方法论（2）：分布式推理：TP、DP、EP、CP 与 PP" (johneyzheng.top):
 *   gate and up fused into one GEMM with N = 2I; experts that no token hits
 *   are skipped; the fused gate_up grouped GEMM measured on FP8 weights.
 * - The EP deployment page above, section "双 batch 重叠": an expert's weights
 *   are 44 MB of FP8, and a dispatched token is FP8 plus 224 bytes of scales.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,      /* an argument is out of range or a required pointer is NULL */
  MOE_ERR_UNSUPPORTED = 2,  /* valid, but a shape this library does not implement */
  MOE_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than the *_workspace_size query */
  MOE_ERR_LAUNCH = 4,       /* a kernel launch failed */
  MOE_ERR_SCRATCH = 5       /* the sizes need more than the fixed scratch of moe_expert_ffn_noalloc */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

typedef enum {
  MOE_SCORE_SOFTMAX = 0,  /* scores are router logits: select on them, weight = softmax over all experts */
  MOE_SCORE_RAW = 1       /* scores are used as given: weight = the selected score */
} moe_score_mode_t;

/* Version of this ABI (incremented on any incompatible change). */
int32_t moe_abi_version(void);

/*
 * moe_eplb_place -- EPLB placement, on the HOST (page "大规模 EP 部署：分层 EPLB、
 * DP 注意力的负载与双 batch 重叠", section "EPLB 与路由约束"): logical experts,
 * with redundant replicas, onto num_gpus GPUs in num_nodes nodes.
 *   hierarchical != 0: the expert groups (contiguous, num_experts / num_groups
 *   each) are packed onto the nodes, balanced by load, the same number of
 *   groups per node; each node's hottest experts get extra replicas up to its
 *   share of num_physical; each node's physical experts are packed onto its
 *   GPUs, balanced, the same number per GPU.
 *   hierarchical == 0: the same over all experts and GPUs at once.
 * Balanced packing: items heaviest first (equal: lower index first), each into
 * the lightest pack with room (equal totals: lower pack). Replication: a
 * replica at a time to the expert with the highest load per replica (equal:
 * lower expert, in the node's expert order). float64 sums in placement order.
 *
 * load             [num_experts] float64, HOST: per-expert load (e.g. assignment
 *                  counts of a routed batch); finite and >= 0.
 * phys_to_logical  [num_physical] int32 HOST out: logical expert of each
 *                  physical slot; slot s sits on GPU s / (num_physical / num_gpus),
 *                  GPU g on node g / (num_gpus / num_nodes).
 * replica_offsets  [num_experts + 1] int32 HOST out, replica_slots
 *                  [num_physical] int32 HOST out: the slots holding expert e are
 *                  replica_slots[replica_offsets[e] .. replica_offsets[e + 1]),
 *                  ascending (the table moe_eplb_remap reads, once copied to the GPU).
 * Limits: num_experts % num_groups == 0; num_physical >= num_experts and a
 * multiple of num_gpus; num_gpus % num_nodes == 0; num_nodes <= 64;
 * hierarchical also needs num_groups and num_physical to be multiples of
 * num_nodes and the slots per node a multiple of the GPUs per node.
 * Synchronous; touches no device memory.
 */
moe_status_t moe_eplb_place(const double* load, int32_t num_experts, int32_t num_groups,
                            int32_t num_nodes, int32_t num_gpus, int32_t num_physical,
                            int32_t hierarchical, int32_t* phys_to_logical,
                            int32_t* replica_offsets, int32_t* replica_slots);

/*
 * moe_eplb_remap -- logical to physical expert per routed (token, slot), on
 * the GPU: the replica choice of the EPLB page's simulation. Per token, slots
 * in order: among the slots holding the expert that sit on a node the token
 * already goes to, the lowest; if none, the lowest slot on the lowest-numbered
 * node holding the expert, and that node is added to the token's nodes.
 *
 * topk_ids         [T, k] int32 (logical experts, from moe_route).
 * replica_offsets  [num_experts + 1], replica_slots [num_physical] int32: the
 *                  table moe_eplb_place writes, in device memory.
 * physical_ids     [T, k] int32 out: physical slots (GPU s / (num_physical /
 *                  num_gpus)); -1 for a slot whose expert id lies outside
 *                  [0, num_experts) or has no replica (no memory outside the
 *                  two tables is read for it).
 * Limits: as moe_eplb_place; the table holds slots in [0, num_physical)
 * (not checked on the device). T = 0 is a valid no-op.
 */
moe_status_t moe_eplb_remap(const int32_t* topk_ids, int32_t num_tokens, int32_t top_k,
                            const int32_t* replica_offsets, const int32_t* replica_slots,
                            int32_t num_experts, int32_t num_physical, int32_t num_gpus,
                            int32_t num_nodes, int32_t* physical_ids, hipStream_t stream);

/*
 * moe_dispatch_deferred -- dispatch with a per-expert capacity and the "defer
 * to a later round" overflow policy of ch15 section 4.3 (table of overflow
 * policies): an assignment past its expert's capacity keeps its expert and is
 * processed in a later round. The assignments of local expert e, in
 * assignment order a = t * k + j, fill round 0 up to expert_capacity = C, then
 * round 1, ...: the i-th (from 0) goes to round i / C; those past `rounds`
 * rounds (all, with C = 0) are dropped (assign_pos = -1). Rows are laid out
 * round after round and, inside a round, expert after expert in assignment
 * order, so round r is one moe_expert_ffn call with expert_offsets =
 * round_offsets + r * (E_loc + 1) (absolute rows), and one moe_combine over
 * assign_pos covers every round.
 *
 * round_counts   [rounds, E_loc] out: rows of expert e in round r.
 * round_offsets  [rounds, E_loc + 1] out: first row of expert e in round r;
 *                entry E_loc is the end of round r (= the start of round r + 1).
 * expert_demand  [E_loc] out, or NULL: assignments per local expert.
 * sorted_assign  [T * k] out: rows [0, end of the last round) written.
 * assign_pos     [T * k] out: row, or -1 (dropped or not local).
 * x, x_sorted    as moe_dispatch (both NULL, or the gather of the kept rows).
 * workspace      moe_dispatch_deferred_workspace_size bytes, 16-byte aligned;
 *                contents need not be initialised.
 * Limits: those of moe_dispatch; rounds >= 1. Errors as moe_dispatch;
 * MOE_ERR_INVALID also for C < 0 or rounds < 1.
 */
size_t moe_dispatch_deferred_workspace_size(int32_t num_tokens, int32_t top_k, int32_t num_local_experts);
moe_status_t moe_dispatch_deferred(const int32_t* topk_ids, int32_t num_tokens, int32_t top_k,
                                   int32_t expert_begin, int32_t num_local_experts, int32_t expert_capacity,
                                   int32_t rounds, const void* x, int32_t hidden, int32_t dtype,
                                   int32_t* round_counts, int32_t* round_offsets, int32_t* expert_demand,
                                   int32_t* sorted_assign, int32_t* assign_pos, void* x_sorted,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_eplb_remap_capacity -- logical to physical expert per routed (token,
 * slot) with a per-replica capacity and the "send to a same-weight replica"
 * overflow policy of ch15 section 4.3 (table of overflow policies; section
 * 4.4: the gating picks a logical expert, the system one of its identical
 * replicas). Logical expert e's replicas are replica_slots[replica_offsets[e]
 * .. replica_offsets[e + 1]) in that order, each with room for
 * replica_capacity = C assignments; e's assignments, in assignment order
 * a = t * k + j, fill its first replica, then the next: the i-th (from 0)
 * goes to replica i / C.
 *
 * topk_ids         [T, k] int32 logical experts (moe_route).
 * replica_offsets  [num_experts + 1], replica_slots int32, device memory (the
 *                  table moe_eplb_place writes, or any other replica list).
 * physical_ids     [T, k] int32 out: the physical slot, or -1 past the room
 *                  of all e's replicas, for ids outside [0, num_experts) and
 *                  for experts without a replica.
 * workspace        moe_eplb_remap_capacity_workspace_size bytes, 16-byte
 *                  aligned; contents need not be initialised.
 * Limits: num_experts <= 1024 (the counting sort of moe_dispatch over all of
 * them gives the ranks). T = 0 is a valid no-op. Errors: MOE_ERR_INVALID for
 * negative sizes or C, or a NULL pointer; MOE_ERR_WORKSPACE; MOE_ERR_UNSUPPORTED
 * past the limits.
 */
size_t moe_eplb_remap_capacity_workspace_size(int32_t num_tokens, int32_t top_k, int32_t num_experts);
moe_status_t moe_eplb_remap_capacity(const int32_t* topk_ids, int32_t num_tokens, int32_t top_k,
                                     const int32_t* replica_offsets, const int32_t* replica_slots,
                                     int32_t num_experts, int32_t replica_capacity, int32_t* physical_ids,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static, NUL-terminated description of a status; host only, never NULL. */
const char* moe_status_string(moe_status_t status);

/*
 * moe_route -- top-k gating per token (ch15 section 4.1), group-limited as on
 * the EPLB page (section "EPLB 与路由约束").
 *
 * scores        [T, E] float32. RAW: used as given. SOFTMAX: router logits.
 * topk_ids      [T, k] int32 out: selected experts, in selection order.
 * topk_weights  [T, k] float32 out.
 *
 * Per token:
 * 1. With num_groups > 1 the E experts form num_groups contiguous groups of
 *    G = E / num_groups. A group's score is the float32 sum of its two highest
 *    scores (a duplicated maximum counts twice). The topk_groups groups with
 *    the highest group score are kept (ties: lower group index).
 * 2. Among the experts of the kept groups (all experts if num_groups == 1),
 *    the top_k highest scores are selected, in descending order; ties go to
 *    the lower expert index, and -0 ties with +0.
 * 3. RAW: weight = selected score. SOFTMAX: weight = softmax over all E
 *    logits, at the selected expert. With renormalize != 0 the k weights are
 *    divided by their sum.
 * Limits: 1 <= E <= 1024; 1 <= top_k <= min(64, topk_groups * G);
 * num_groups divides E; G >= 2 when num_groups > 1; SOFTMAX needs
 * num_groups == 1. T = 0 is a valid no-op.
 */
moe_status_t moe_route(const float* scores, int32_t num_tokens, int32_t num_experts,
                       int32_t top_k, int32_t num_groups, int32_t topk_groups,
                       int32_t score_mode, int32_t renormalize,
                       int32_t* topk_ids, float* topk_weights, hipStream_t stream);

/* Bytes of device workspace moe_route_reroute needs; 0 when the sizes are invalid. */
size_t moe_route_reroute_workspace_size(int32_t num_tokens, int32_t num_experts, int32_t top_k,
                                        int32_t num_groups, int32_t topk_groups);

/*
 * moe_route_reroute -- moe_route (RAW scores) with a per-expert capacity C and
 * the first overflow policy of the table in ch15 section 4.3 ("负载均衡",
 * capacity factor): an assignment over its expert's capacity goes to the
 * token's next-highest-scoring expert instead.
 * 1. Every token is ranked as in moe_route (kept groups, descending score,
 *    lower index first); ranks 0 .. k-1 are its choices, ranks k, k+1, ...
 *    (up to 2k in all, at most 64, within its kept groups) its spares.
 * 2. Each expert keeps its first C original assignments in assignment order
 *    a = t * k + j; the others overflow.
 * 3. In assignment order, the i-th overflowing slot of a token (slot order)
 *    takes the token's spare of rank k + i if that expert then holds fewer than
 *    C assignments (the originals count first); otherwise, or without such a
 *    spare, the slot is dropped: topk_ids = -1, weight 0 (moe_dispatch treats
 *    -1 as not local).
 * 4. Weight = the score of the slot's final expert, divided by the sum over
 *    the token's slots that were not dropped when renormalize != 0.
 * topk_ids, topk_weights [T, k] out; expert_load [E] int32 out or NULL:
 * assignments each expert ends with (<= C).
 * workspace  >= moe_route_reroute_workspace_size bytes; contents need not be
 *            initialised.
 * Limits: those of moe_route (RAW mode), C >= 0. T = 0 is a valid no-op
 * (expert_load is then not written).
 */
moe_status_t moe_route_reroute(const float* scores, int32_t num_tokens, int32_t num_experts,
                               int32_t top_k, int32_t num_groups, int32_t topk_groups,
                               int32_t renormalize, int32_t expert_capacity, int32_t* topk_ids,
                               float* topk_weights, int32_t* expert_load, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of device workspace moe_dispatch needs for T * k assignments and
 * num_local_experts experts (0 when T * k <= 8192: then workspace may be NULL).
 */
size_t moe_dispatch_workspace_size(int32_t num_tokens, int32_t top_k, int32_t num_local_experts);

/*
 * moe_dispatch -- the dispatch step of ch15 section 3.4 on one GPU: a stable
 * counting sort of the assignments a = t * k + j (token t, slot j) whose
 * expert lies in [expert_begin, expert_begin + num_local_experts), followed by
 * an optional gather of the token rows into expert order.
 *
 * topk_ids        [T, k] int32 (from moe_route).
 * expert_counts   [E_loc] int32 out: rows per local expert.
 * expert_offsets  [E_loc + 1] int32 out: exclusive prefix sum; offsets[E_loc] = M.
 * sorted_assign   [T * k] int32 out: entries [0, M) hold the local assignments
 *                 ordered by (local expert, a); entries >= M are not written.
 * assign_pos      [T * k] int32 out: position of assignment a in sorted_assign,
 *                 or -1 when its expert is not local.
 * x               [T, hidden] (dtype) or NULL: token rows to gather.
 * x_sorted        [T * k, hidden] (dtype) out, or NULL (only with x == NULL):
 *                 row i = x[sorted_assign[i] / k] for i < M (exact copy).
 * workspace       device buffer of moe_dispatch_workspace_size bytes, 16-byte
 *                 aligned (the multi-workgroup sort's per-(expert, block)
 *                 counts and rank bases); contents need not be set.
 * Limits: 1 <= num_local_experts <= 1024 (as moe_expert_ffn); T * k < 2^31;
 * hidden % 8 == 0 when x is given. T = 0 writes zero counts and offsets.
 */
moe_status_t moe_dispatch(const int32_t* topk_ids, int32_t num_tokens, int32_t top_k,
                          int32_t expert_begin, int32_t num_local_experts,
                          const void* x, int32_t hidden, int32_t dtype,
                          int32_t* expert_counts, int32_t* expert_offsets,
                          int32_t* sorted_assign, int32_t* assign_pos, void* x_sorted,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_dispatch_capacity -- moe_dispatch with a per-expert capacity and the
 * drop policy, the capacity factor of ch15 section 4.3 ("负载均衡" section,
 * "Capacity Factor": C = ceil(c * T * k / E), and its table of overflow
 * policies). expert_capacity = C, computed by the caller (>= 0).
 *
 * Each local expert keeps its first C assignments in assignment order
 * a = t * k + j; the others are dropped: not in sorted_assign, assign_pos = -1
 * (so moe_combine leaves them out, as it does non-local ones).
 * expert_counts   [E_loc] out: rows kept, min(assignments, C).
 * expert_offsets  [E_loc + 1] out: exclusive prefix sum of expert_counts.
 * expert_demand   [E_loc] int32 out, or NULL: assignments per local expert
 *                 before the cap (demand - counts were dropped).
 * Every other argument, the workspace and the limits are those of
 * moe_dispatch; with C >= T * k the result equals moe_dispatch's.
 * Errors: as moe_dispatch; MOE_ERR_INVALID also for expert_capacity < 0.
 */
moe_status_t moe_dispatch_capacity(const int32_t* topk_ids, int32_t num_tokens, int32_t top_k,
                                   int32_t expert_begin, int32_t num_local_experts,
                                   int32_t expert_capacity, const void* x, int32_t hidden,
                                   int32_t dtype, int32_t* expert_counts, int32_t* expert_offsets,
                                   int32_t* expert_demand, int32_t* sorted_assign,
                                   int32_t* assign_pos, void* x_sorted, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * moe_expert_capacity -- the per-expert capacity of the capacity factor, ch15
 * section 4.3 ("负载均衡" section, "Capacity Factor"): C = ceil(c * T * k / E)
 * with c = factor_num / factor_den taken exactly (integer arithmetic, so a
 * factor such as 1.2 = 6/5 gives exactly 120 for T = 5600, k = 16, E = 896,
 * where a binary floating-point product lands just above 120). HOST only;
 * touches no device memory.
 * capacity  HOST out: C, the value moe_dispatch_capacity takes.
 * Errors: MOE_ERR_INVALID for T < 0, k < 1, E < 1, factor_num < 0,
 * factor_den < 1 or a NULL capacity; MOE_ERR_UNSUPPORTED when C does not fit
 * in int32 or factor_num, factor_den >= 2^31.
 */
moe_status_t moe_expert_capacity(int32_t num_tokens, int32_t top_k, int32_t num_experts,
                                 int64_t factor_num, int64_t factor_den, int32_t* capacity);

/*
 * Bytes of device workspace moe_expert_ffn needs for these sizes; 0 when the
 * sizes are invalid.
 */
size_t moe_expert_ffn_workspace_size(int32_t num_local_experts, int32_t hidden, int32_t inter,
                                     int32_t row_capacity, int32_t dtype);

/*
 * moe_expert_ffn -- the gated MLP of lecture 6 section 2.2 per local expert,
 * with gate and up fused into one GEMM of N = 2I (the INFRA page), over the
 * permuted rows: for each local expert e with rows [off[e], off[e+1]):
 *   [g | u] = X_e * W_gate_up[e]^T,  h = silu(g) * u,  o = h * W_down[e]^T,
 * silu(z) = z / (1 + exp(-z)). Experts without rows read no weights.
 *
 * x               the permuted activations, in one of two forms:
 *                 row_index == NULL: x_sorted [row_capacity, hidden] (moe_dispatch);
 *                 row_index != NULL: token rows [T, hidden], and permuted row i is
 *                 x[row_index[i] / row_index_div] -- pass sorted_assign and top_k to
 *                 fuse the dispatch gather into the first GEMM's loads.
 * expert_offsets  [E_loc + 1] int32 (moe_dispatch); read on the device only.
 * w_gate_up       [E_loc, 2 * inter, hidden] (dtype): rows [0, I) gate, [I, 2I) up.
 * w_down          [E_loc, hidden, inter] (dtype).
 * o_sorted        [row_capacity, hidden] (dtype) out: rows [0, M) written.
 * workspace       device buffer of at least moe_expert_ffn_workspace_size bytes
 *                 (holds h); contents need not be initialised.
 * bf16: float32 accumulation; h and o are rounded to bf16.
 * Limits (bf16): hidden % 256 == 0, inter % 64 == 0; row_capacity * max(hidden,
 * inter) < 2^31, and the caller keeps x below 2^32 bytes (the kernels address
 * rows with 32-bit byte offsets). f32: hidden % 4 == 0, inter % 4 == 0,
 * E_loc * ceil(row_capacity / 16) <= 65535. M = offsets[E_loc] must not exceed
 * row_capacity (rows past row_capacity are ignored on the device).
 */
moe_status_t moe_expert_ffn(const void* x, const int32_t* row_index, int32_t row_index_div,
                            const int32_t* expert_offsets, const void* w_gate_up,
                            const void* w_down, int32_t num_local_experts, int32_t hidden,
                            int32_t inter, int32_t row_capacity, int32_t dtype, void* o_sorted,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_dispatch_masked -- the capped dispatch of moe_dispatch_capacity into
 * fixed per-expert slots: the "masked" layout of the grouped GEMM that the
 * INFRA page measures (H20 paragraph, DeepGEMM masked). Local expert e owns
 * slot rows [e * C, (e + 1) * C); its first C assignments in assignment order
 * a = t * k + j take rows e * C, e * C + 1, ...; the others are dropped
 * (ch15 section 4.3, capacity factor, drop policy). C = expert_capacity.
 * expert_counts   [E_loc] out: rows used per expert, min(assignments, C).
 * expert_demand   [E_loc] out, or NULL: assignments per expert before the cap.
 * slot_assign     [E_loc * C] out: the assignment in each used slot row; rows
 *                 at or past their expert's count are not written (may be
 *                 NULL when C = 0).
 * assign_pos      [T * k] out: slot row of each assignment, -1 when dropped or
 *                 not local (moe_combine reads the slot-layout outputs with it).
 * x, x_slots      as in moe_dispatch, x_slots [E_loc * C, hidden]: used rows
 *                 are exact copies of their token's row, the others untouched.
 * Workspace and other limits: those of moe_dispatch; E_loc * C < 2^31.
 */
moe_status_t moe_dispatch_masked(const int32_t* topk_ids, int32_t num_tokens, int32_t top_k,
                                 int32_t expert_begin, int32_t num_local_experts,
                                 int32_t expert_capacity, const void* x, int32_t hidden,
                                 int32_t dtype, int32_t* expert_counts, int32_t* expert_demand,
                                 int32_t* slot_assign, int32_t* assign_pos, void* x_slots,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace moe_expert_ffn_masked needs; 0 when the sizes are invalid. */
size_t moe_expert_ffn_masked_workspace_size(int32_t num_local_experts, int32_t hidden,
                                            int32_t inter, int32_t expert_capacity, int32_t dtype);

/*
 * moe_expert_ffn_masked -- moe_expert_ffn on the masked layout: for each local
 * expert e only its valid slot rows [e * C, e * C + min(counts[e], C)) of
 * x_slots go through the expert, and their outputs go to the same rows of
 * o_slots; every other row of o_slots is left untouched, and no expert does
 * any work for its padding rows.
 * x_slots         [E_loc * C, hidden] (dtype), e.g. from moe_dispatch_masked.
 * expert_counts   [E_loc] int32, read on the device (negative counts count as 0).
 * w_gate_up, w_down, dtype, hidden, inter: as in moe_expert_ffn.
 * o_slots         [E_loc * C, hidden] (dtype) out.
 * workspace       >= moe_expert_ffn_masked_workspace_size bytes (compact
 *                 offsets, the row index, compact outputs and h); contents
 *                 need not be initialised.
 * Limits: those of moe_expert_ffn with row_capacity = E_loc * C.
 */
moe_status_t moe_expert_ffn_masked(const void* x_slots, const int32_t* expert_counts,
                                   int32_t expert_capacity, const void* w_gate_up,
                                   const void* w_down, int32_t num_local_experts, int32_t hidden,
                                   int32_t inter, int32_t dtype, void* o_slots, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * moe_expert_ffn_noalloc -- moe_expert_ffn for callers that cannot allocate
 * device memory at all (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation and kernels, with no
 * workspace argument; h and the kernels' partial sums live in a fixed scratch
 * array of MOE_FFN_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on
 * every GPU it runs on until the process ends. The call allocates nothing
 * (no hipMalloc, no hipFree); its first call on a device looks up that
 * device's copy of the array.
 * Arguments, layouts, limits and errors: those of moe_expert_ffn, and
 * MOE_ERR_SCRATCH (nothing enqueued) when moe_expert_ffn_workspace_size of
 * the sizes exceeds the scratch; MOE_ERR_LAUNCH also when the device address
 * of the scratch cannot be obtained (e.g. bf16 decode: 4096 rows x I = 2048 take 16 MiB; 512
 * tokens x 8 slots over 256 experts with I = 64 take 36 MiB).
 * Every call on one GPU shares that GPU's scratch, whatever the stream: two
 * calls that may overlap in time on one GPU (different streams, different
 * host threads) race and must be ordered by the caller. Nothing in the
 * scratch needs clearing between calls (every byte a call reads, the same
 * call wrote first).
 */
#define MOE_FFN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status_t moe_expert_ffn_noalloc(const void* x, const int32_t* row_index, int32_t row_index_div,
                                    const int32_t* expert_offsets, const void* w_gate_up,
                                    const void* w_down, int32_t num_local_experts, int32_t hidden,
                                    int32_t inter, int32_t row_capacity, int32_t dtype,
                                    void* o_sorted, hipStream_t stream);

/*
 * FP8 operands (moe_quantize_e4m3, moe_expert_ffn_fp8). Values are OCP FP8
 * E4M3 codes (1 byte: sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * largest finite 448; 0x7F and 0xFF are NaN) with float32 scales; a value is
 * code * scale. Token rows take one scale per row and 128 consecutive
 * features (224 B for 7168 features, the EP page's per-token count); weights
 * one per 128 x 128 block. The block shapes are this library's reading: the
 * pages give only the byte counts.
 */

/*
 * moe_quantize_e4m3 -- token rows to FP8, the form in which the EP page
 * dispatches them. For each row r and block b of 128 features:
 *   scale[r, b] = amax / 448 (float32; 1.0 for an all-zero block),
 *   code[r, c]  = the e4m3 value nearest to x[r, c] / scale[r, b] (float32
 *                 division), ties to the even code, magnitudes above 448
 *                 saturating to 448; the sign bit is x's sign bit.
 * x       [rows, cols] (dtype: MOE_F32 or MOE_BF16); finite values.
 * codes   [rows, cols] uint8 out.
 * scales  [rows, cols / 128] float32 out.
 * Limits: cols % 128 == 0; x, codes and scales 16-byte aligned. rows = 0
 * does nothing.
 */
moe_status_t moe_quantize_e4m3(const void* x, int32_t rows, int32_t cols, int32_t dtype, void* codes,
                               float* scales, hipStream_t stream);

/*
 * Bytes of device workspace moe_expert_ffn_fp8 needs; 0 when the sizes are
 * invalid.
 */
size_t moe_expert_ffn_fp8_workspace_size(int32_t num_local_experts, int32_t hidden, int32_t inter,
                                         int32_t row_capacity);

/*
 * moe_expert_ffn_fp8 -- moe_expert_ffn on FP8 operands. For each local
 * expert e with rows [off[e], off[e+1]):
 *   [g | u] = X_e * W_gate_up[e]^T   (dequantised operands, float32 accumulation)
 *   h       = silu(g) * u            (float32)
 *   (hq, hs)= h quantised per row and 128 columns exactly as moe_quantize_e4m3
 *   o       = dequant(hq, hs) * W_down[e]^T, rounded to bf16.
 *
 * x_codes, x_scales  the permuted rows in FP8 (moe_quantize_e4m3 layout), in
 *                 one of two forms as in moe_expert_ffn: row_index == NULL:
 *                 [row_capacity, hidden] permuted rows; else token rows, with
 *                 permuted row i = row row_index[i] / row_index_div (pass
 *                 sorted_assign and top_k to fuse the dispatch gather).
 * expert_offsets  [E_loc + 1] int32 (moe_dispatch); read on the device only.
 * w_gate_up       [E_loc, 2 * inter, hidden] e4m3: rows [0, I) gate, [I, 2I) up.
 * w_gate_up_scales [E_loc, 2 * inter / 128, hidden / 128] float32.
 * w_down          [E_loc, hidden, inter] e4m3.
 * w_down_scales   [E_loc, hidden / 128, inter / 128] float32.
 * o_sorted        [row_capacity, hidden] bf16 out: rows [0, M) written.
 * workspace       >= moe_expert_ffn_fp8_workspace_size bytes (holds h in
 *                 float32 and in FP8); contents need not be initialised.
 * Limits: hidden % 512 == 0, inter % 256 == 0; E_loc <= 1024;
 * row_capacity * inter * 4 < 2^31; the caller keeps x_codes below 2^32
 * bytes. M = offsets[E_loc] must not exceed row_capacity. Experts with at
 * most 64 rows stream their weights once per call (decode); larger ones are
 * multiplied in tiles of 128 rows x 128 weight rows (prefill), so their
 * weights are read once per 128 rows.
 */
moe_status_t moe_expert_ffn_fp8(const void* x_codes, const float* x_scales, const int32_t* row_index,
                                int32_t row_index_div, const int32_t* expert_offsets,
                                const void* w_gate_up, const float* w_gate_up_scales, const void* w_down,
                                const float* w_down_scales, int32_t num_local_experts, int32_t hidden,
                                int32_t inter, int32_t row_capacity, void* o_sorted, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * moe_combine -- the combine step (ch15 section 3.4; attain.fans hop 4):
 *   y[t] = sum over slots j = 0..k-1 with assign_pos[t*k+j] >= 0 of
 *          topk_weights[t, j] * o_sorted[assign_pos[t*k+j]],
 * summed in slot order in float32. Tokens with no local slot get a zero row
 * (y is this GPU's partial sum of the layer output).
 *
 * o_sorted      [>= M, hidden] (dtype).
 * assign_pos    [T * k] int32 (moe_dispatch).
 * topk_weights  [T, k] float32 (moe_route).
 * y             [T, hidden] (out_dtype) out.
 * Limits: hidden % 8 == 0; 1 <= top_k <= 64.
 */
moe_status_t moe_combine(const void* o_sorted, const int32_t* assign_pos,
                         const float* topk_weights, int32_t num_tokens, int32_t top_k,
                         int32_t hidden, int32_t dtype, int32_t out_dtype, void* y,
                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
