// Internal launchers of the HIP kernels; the public entry points in api.hip
// validate arguments and then call these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

struct RouteArgs {
  const float* scores;
  int T, E, k, num_groups, topk_groups, softmax, renormalize;
  int* ids;
  float* weights;
};
hipError_t launch_route(const RouteArgs& a, hipStream_t s);

// Routing with a per-expert capacity and the next-best expert overflow policy.
struct RerouteArgs {
  const float* scores;
  int T, E, k, num_groups, topk_groups, renormalize, cap;
  int* ids;        // [T, k] out
  float* weights;  // [T, k] out
  int* load;       // [E] out or null: assignments each expert ends with
  void* workspace;
};
int reroute_ranks(int E, int k, int num_groups, int topk_groups);
size_t reroute_workspace_size(int T, int E, int k, int num_groups, int topk_groups);
hipError_t launch_route_reroute(const RerouteArgs& a, hipStream_t s);

struct DispatchArgs {
  const int* ids;
  int n;  // T * k assignments
  int k, expert_begin, num_local;
  int* counts;
  int* offsets;
  int* sorted_assign;
  int* assign_pos;
  const void* x;
  void* x_sorted;
  int row_bytes;  // hidden * element size; 0 = no gather
  void* workspace;
  int capacity;   // rows kept per expert (first come, first served); INT32_MAX = no limit
  int* demand;    // null, or [num_local] out: assignments per expert before the cap
  int fixed_slots = 0;  // rows of expert e start at e * capacity (offsets may be null)
};
size_t dispatch_workspace_size(int n, int num_local);
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);
constexpr int kDispatchMaxLocal = 1024;  // per-(wave, expert) counters and offsets: 68 KiB of LDS at most
// Rows [0, end[num_local]) of x_sorted gathered from x through sorted_assign (row i = x[sorted_assign[i] / k]).
hipError_t launch_gather_rows(const void* x, const int* sorted_assign, const int* end, int num_local, int k,
                              int n, int row_bytes, void* x_sorted, hipStream_t s);

// Dispatch with the "defer to a later round" overflow policy (policies.hip):
// the i-th assignment of local expert e (assignment order) goes to round
// i / capacity; rounds are laid out one after another.
struct DeferredArgs {
  const int* ids;
  int n, k, expert_begin, num_local, capacity, rounds;
  const void* x;
  void* x_sorted;
  int row_bytes;       // 0 = no gather
  int* round_counts;   // [rounds][num_local]
  int* round_offsets;  // [rounds][num_local + 1], absolute rows
  int* demand;         // null, or [num_local]
  int* sorted_assign;
  int* assign_pos;
  void* workspace;
};
size_t deferred_workspace_size(int n, int num_local);
hipError_t launch_dispatch_deferred(const DeferredArgs& a, hipStream_t s);

// Logical -> physical expert with the "send to a same-weight replica" overflow
// policy (policies.hip): the i-th assignment of logical expert e goes to its
// replica i / capacity, or -1 past them.
struct RemapCapacityArgs {
  const int* ids;
  int n, num_experts, capacity;
  const int* rep_offsets;  // [num_experts + 1]
  const int* rep_slots;
  int* phys;
  void* workspace;
};
size_t remap_capacity_workspace_size(int n, int num_experts);
hipError_t launch_remap_capacity(const RemapCapacityArgs& a, hipStream_t s);

struct FfnArgs {
  const void* x;         // permuted rows, or token rows read through row_index
  const int* row_index;  // null, or sorted_assign (row i = x[row_index[i] / row_div])
  int row_div;
  const int* offsets;
  const void* w_gate_up;
  const void* w_down;
  int num_local, hidden, inter, capacity;
  bool bf16;
  void* o_sorted;
  void* workspace;
  // Masked layout (bf16, every expert streamed): rows per expert from these
  // counts (clamped to [0, slot_cap]) instead of offsets; x and o_sorted hold
  // expert e's r-th row at row e * slot_cap + r.
  const int* slot_counts = nullptr;
  int slot_cap = 0;
};
size_t ffn_workspace_size(int num_local, int hidden, int inter, int capacity, bool bf16);
hipError_t launch_ffn(const FfnArgs& a, hipStream_t s);

// The expert FFN on fixed per-expert slots of `cap` rows with a valid count per
// expert (the masked layout): when every expert is streamed the grouped FFN
// takes the counts and works on the slot rows directly; else a plan kernel, the
// grouped FFN through a row index, and a scatter of the outputs back to the
// slot rows.
struct FfnMaskedArgs {
  const void* x_slots;   // [num_local * cap, hidden]
  const int* counts;     // [num_local] valid rows per expert (clamped to [0, cap])
  int cap;
  const void* w_gate_up;
  const void* w_down;
  int num_local, hidden, inter;
  bool bf16;
  void* o_slots;         // [num_local * cap, hidden] out: valid rows written
  void* workspace;
};
size_t ffn_masked_workspace_size(int num_local, int hidden, int inter, int cap, bool bf16);
hipError_t launch_ffn_masked(const FfnMaskedArgs& a, hipStream_t s);

// FP8 (e4m3 codes, float32 block scales) expert FFN and row quantiser.
struct FfnFp8Args {
  const void* x_codes;     // [rows, hidden] e4m3: permuted rows, or token rows read through row_index
  const float* x_scales;   // [rows, hidden / 128]
  const int* row_index;
  int row_div;
  const int* offsets;
  const void* w_gate_up;   // [nloc, 2 * inter, hidden] e4m3
  const float* w_gate_up_scales;  // [nloc, 2 * inter / 128, hidden / 128]
  const void* w_down;      // [nloc, hidden, inter] e4m3
  const float* w_down_scales;     // [nloc, hidden / 128, inter / 128]
  int num_local, hidden, inter, capacity;
  void* o_sorted;          // [capacity, hidden] bf16
  void* workspace;
};
size_t ffn_fp8_workspace_size(int hidden, int inter, int capacity);
hipError_t launch_ffn_fp8(const FfnFp8Args& a, hipStream_t s);
hipError_t launch_quantize_rows(const void* x, int rows, int cols, bool bf16_in, uint8_t* codes, float* scales,
                                hipStream_t s);

struct CombineArgs {
  const void* o_sorted;
  const int* assign_pos;
  const float* weights;
  int T, k, hidden;
  bool o_bf16, y_bf16;
  void* y;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

// EPLB replica choice (device); the placement planner is host code (host_plan.h).
hipError_t launch_eplb_remap(const int* ids, int T, int k, const int* offsets, const int* slots,
                             int num_experts, int slots_per_gpu, int gpus_per_node, int* phys,
                             hipStream_t s);

}  // namespace moe
