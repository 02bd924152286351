// Public C entry points (include/moe.h): host-side argument validation, then
// the kernel launchers. Nothing is enqueued when validation fails, and no C++
// exception crosses the ABI.
#include "../../include/moe.h"

#include <stdint.h>

#include <cmath>
#include <mutex>

#include "host_plan.h"
#include "launch.h"

namespace {

constexpr int kAbiVersion = 9;

// The fixed scratch of moe_expert_ffn_noalloc (h and partial sums). In host
// code `scratch` names a host-side stand-in, not device memory: kernels get
// the per-device address that hipGetSymbolAddress returns (scratch_ptr).
static __device__ __align__(256) char scratch[MOE_FFN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device (with that
// device current, as the calling thread has it); null on failure.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

moe_status_t from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return kAbiVersion; }

const char* moe_status_string(moe_status_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_SCRATCH: return "sizes exceed the fixed scratch of moe_expert_ffn_noalloc";
  }
  return "unknown status";
}

static moe_status_t check_route_args(int32_t num_tokens, int32_t num_experts, int32_t top_k,
                                     int32_t num_groups, int32_t topk_groups, int32_t score_mode) {
  if (num_tokens < 0 || num_experts < 1 || top_k < 1 || num_groups < 1 || topk_groups < 1)
    return MOE_ERR_INVALID;
  if (score_mode != MOE_SCORE_SOFTMAX && score_mode != MOE_SCORE_RAW) return MOE_ERR_INVALID;
  if (num_experts % num_groups != 0 || topk_groups > num_groups) return MOE_ERR_INVALID;
  const int G = num_experts / num_groups;
  if (num_groups > 1 && G < 2) return MOE_ERR_INVALID;
  if ((int64_t)top_k > (int64_t)topk_groups * G) return MOE_ERR_INVALID;
  if (score_mode == MOE_SCORE_SOFTMAX && num_groups != 1) return MOE_ERR_INVALID;
  if (num_experts > 1024 || top_k > 64 || num_groups > 64) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)num_tokens * num_experts >= ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status_t moe_route(const float* scores, int32_t num_tokens, int32_t num_experts,
                       int32_t top_k, int32_t num_groups, int32_t topk_groups,
                       int32_t score_mode, int32_t renormalize, int32_t* topk_ids,
                       float* topk_weights, hipStream_t stream) {
  const moe_status_t st = check_route_args(num_tokens, num_experts, top_k, num_groups, topk_groups,
                                           score_mode);
  if (st != MOE_OK) return st;
  if (num_tokens == 0) return MOE_OK;
  if (!scores || !topk_ids || !topk_weights) return MOE_ERR_INVALID;
  moe::RouteArgs a{scores,      num_tokens,  num_experts, top_k,   num_groups, topk_groups,
                   score_mode == MOE_SCORE_SOFTMAX ? 1 : 0, renormalize ? 1 : 0, topk_ids,
                   topk_weights};
  return from_hip(moe::launch_route(a, stream));
}

size_t moe_route_reroute_workspace_size(int32_t num_tokens, int32_t num_experts, int32_t top_k,
                                        int32_t num_groups, int32_t topk_groups) {
  if (check_route_args(num_tokens, num_experts, top_k, num_groups, topk_groups, MOE_SCORE_RAW) != MOE_OK)
    return 0;
  if ((int64_t)num_tokens * 64 >= ((int64_t)1 << 31) - 65536) return 0;
  return moe::reroute_workspace_size(num_tokens, num_experts, top_k, num_groups, topk_groups);
}

moe_status_t moe_route_reroute(const float* scores, int32_t num_tokens, int32_t num_experts,
                               int32_t top_k, int32_t num_groups, int32_t topk_groups,
                               int32_t renormalize, int32_t expert_capacity, int32_t* topk_ids,
                               float* topk_weights, int32_t* expert_load, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  const moe_status_t st = check_route_args(num_tokens, num_experts, top_k, num_groups, topk_groups,
                                           MOE_SCORE_RAW);
  if (st != MOE_OK) return st;
  if (expert_capacity < 0) return MOE_ERR_INVALID;
  // the ranking and both counting sorts hold T * 2k assignments in 32-bit ints
  if ((int64_t)num_tokens * 64 >= ((int64_t)1 << 31) - 65536) return MOE_ERR_UNSUPPORTED;
  if (num_tokens == 0) return MOE_OK;
  if (!scores || !topk_ids || !topk_weights) return MOE_ERR_INVALID;
  const size_t need = moe::reroute_workspace_size(num_tokens, num_experts, top_k, num_groups, topk_groups);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return MOE_ERR_WORKSPACE;
  moe::RerouteArgs a{scores, num_tokens, num_experts, top_k, num_groups, topk_groups,
                     renormalize ? 1 : 0, expert_capacity, topk_ids, topk_weights, expert_load, workspace};
  return from_hip(moe::launch_route_reroute(a, stream));
}

size_t moe_dispatch_workspace_size(int32_t num_tokens, int32_t top_k, int32_t num_local_experts) {
  if (num_tokens < 0 || top_k < 1 || num_local_experts < 1) return 0;
  const int64_t n = (int64_t)num_tokens * top_k;
  if (n >= ((int64_t)1 << 31) - 65536) return 0;
  return moe::dispatch_workspace_size((int)n, num_local_experts);
}

static moe_status_t dispatch_impl(const int32_t* topk_ids, int32_t num_tokens, int32_t top_k,
                                  int32_t expert_begin, int32_t num_local_experts, const void* x,
                                  int32_t hidden, int32_t dtype, int32_t* expert_counts,
                                  int32_t* expert_offsets, int32_t* sorted_assign,
                                  int32_t* assign_pos, void* x_sorted, void* workspace,
                                  size_t workspace_bytes, int32_t capacity, int32_t* demand,
                                  int fixed, hipStream_t stream) {
  if (num_tokens < 0 || top_k < 1 || expert_begin < 0 || num_local_experts < 1 || capacity < 0)
    return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (num_local_experts > moe::kDispatchMaxLocal) return MOE_ERR_UNSUPPORTED;
  const int64_t n = (int64_t)num_tokens * top_k;
  if (n >= ((int64_t)1 << 31) - 65536) return MOE_ERR_UNSUPPORTED;
  // fixed slots: rows e * C + r are addressed with 32-bit ints
  if (fixed && (int64_t)num_local_experts * capacity >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (!expert_counts || (!fixed && !expert_offsets)) return MOE_ERR_INVALID;
  if (n > 0 && (!topk_ids || !assign_pos)) return MOE_ERR_INVALID;
  if (n > 0 && !sorted_assign && !(fixed && capacity == 0)) return MOE_ERR_INVALID;
  if ((x == nullptr) != (x_sorted == nullptr)) return MOE_ERR_INVALID;
  int row_bytes = 0;
  if (x) {
    if (hidden < 8 || hidden % 8 != 0) return MOE_ERR_INVALID;
    if (!aligned16(x) || !aligned16(x_sorted)) return MOE_ERR_INVALID;
    const int64_t rb = (int64_t)hidden * (dtype == MOE_BF16 ? 2 : 4);
    if (rb > (1 << 30)) return MOE_ERR_UNSUPPORTED;
    row_bytes = (int)rb;
  }
  const size_t need = moe::dispatch_workspace_size((int)n, num_local_experts);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return MOE_ERR_WORKSPACE;
  moe::DispatchArgs a{topk_ids, (int)n, top_k, expert_begin, num_local_experts, expert_counts,
                      fixed ? nullptr : expert_offsets, sorted_assign, assign_pos, x, x_sorted,
                      row_bytes, workspace, capacity, demand, fixed ? 1 : 0};
  return from_hip(moe::launch_dispatch(a, stream));
}

moe_status_t moe_dispatch(const int32_t* topk_ids, int32_t num_tokens, int32_t top_k,
                          int32_t expert_begin, int32_t num_local_experts, const void* x,
                          int32_t hidden, int32_t dtype, int32_t* expert_counts,
                          int32_t* expert_offsets, int32_t* sorted_assign, int32_t* assign_pos,
                          void* x_sorted, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  return dispatch_impl(topk_ids, num_tokens, top_k, expert_begin, num_local_experts, x, hidden,
                       dtype, expert_counts, expert_offsets, sorted_assign, assign_pos, x_sorted,
                       workspace, workspace_bytes, INT32_MAX, nullptr, 0, stream);
}

moe_status_t moe_dispatch_capacity(const int32_t* topk_ids, int32_t num_tokens, int32_t top_k,
                                   int32_t expert_begin, int32_t num_local_experts,
                                   int32_t expert_capacity, const void* x, int32_t hidden,
                                   int32_t dtype, int32_t* expert_counts, int32_t* expert_offsets,
                                   int32_t* expert_demand, int32_t* sorted_assign,
                                   int32_t* assign_pos, void* x_sorted, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  return dispatch_impl(topk_ids, num_tokens, top_k, expert_begin, num_local_experts, x, hidden,
                       dtype, expert_counts, expert_offsets, sorted_assign, assign_pos, x_sorted,
                       workspace, workspace_bytes, expert_capacity, expert_demand, 0, stream);
}

moe_status_t moe_dispatch_masked(const int32_t* topk_ids, int32_t num_tokens, int32_t top_k,
                                 int32_t expert_begin, int32_t num_local_experts,
                                 int32_t expert_capacity, const void* x, int32_t hidden,
                                 int32_t dtype, int32_t* expert_counts, int32_t* expert_demand,
                                 int32_t* slot_assign, int32_t* assign_pos, void* x_slots,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return dispatch_impl(topk_ids, num_tokens, top_k, expert_begin, num_local_experts, x, hidden,
                       dtype, expert_counts, nullptr, slot_assign, assign_pos, x_slots, workspace,
                       workspace_bytes, expert_capacity, expert_demand, 1, stream);
}

moe_status_t moe_expert_capacity(int32_t num_tokens, int32_t top_k, int32_t num_experts,
                                 int64_t factor_num, int64_t factor_den, int32_t* capacity) {
  if (num_tokens < 0 || top_k < 1 || num_experts < 1 || factor_num < 0 || factor_den < 1 || !capacity)
    return MOE_ERR_INVALID;
  const int64_t lim = (int64_t)1 << 31;
  if (factor_num >= lim || factor_den >= lim) return MOE_ERR_UNSUPPORTED;
  const int64_t tk = (int64_t)num_tokens * top_k;
  if (tk >= lim) return MOE_ERR_UNSUPPORTED;
  const int64_t c = moe::expert_capacity(tk, factor_num, factor_den, num_experts);
  if (c > (int64_t)INT32_MAX) return MOE_ERR_UNSUPPORTED;
  *capacity = (int32_t)c;
  return MOE_OK;
}

static moe_status_t check_ffn_sizes(int32_t num_local_experts, int32_t hidden, int32_t inter,
                                    int32_t row_capacity, int32_t dtype) {
  if (num_local_experts < 1 || hidden < 1 || inter < 1 || row_capacity < 0) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (num_local_experts > 1024) return MOE_ERR_UNSUPPORTED;
  if (dtype == MOE_BF16) {
    if (hidden % 256 != 0 || inter % 64 != 0) return MOE_ERR_UNSUPPORTED;
  } else {
    if (hidden % 4 != 0 || inter % 4 != 0) return MOE_ERR_UNSUPPORTED;
    // the float32 kernels index (expert, 16-row tile) along one grid dimension
    if ((int64_t)num_local_experts * ((row_capacity + 15) / 16) > 65535) return MOE_ERR_UNSUPPORTED;
  }
  if ((int64_t)2 * inter * hidden >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  // the bf16 kernels address an expert's weights and the activation rows with
  // 32-bit byte offsets
  if ((int64_t)row_capacity * (hidden > inter ? hidden : inter) >= ((int64_t)1 << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t moe_expert_ffn_workspace_size(int32_t num_local_experts, int32_t hidden, int32_t inter,
                                     int32_t row_capacity, int32_t dtype) {
  if (check_ffn_sizes(num_local_experts, hidden, inter, row_capacity, dtype) != MOE_OK) return 0;
  return moe::ffn_workspace_size(num_local_experts, hidden, inter, row_capacity,
                                 dtype == MOE_BF16);
}

// Validation of moe_expert_ffn's arguments other than the workspace.
static moe_status_t check_ffn_args(const void* x, const int32_t* row_index, int32_t row_index_div,
                                   const int32_t* expert_offsets, const void* w_gate_up,
                                   const void* w_down, int32_t num_local_experts, int32_t hidden,
                                   int32_t inter, int32_t row_capacity, int32_t dtype,
                                   const void* o_sorted) {
  const moe_status_t st = check_ffn_sizes(num_local_experts, hidden, inter, row_capacity, dtype);
  if (st != MOE_OK) return st;
  if (!expert_offsets || !w_gate_up || !w_down) return MOE_ERR_INVALID;
  if (row_index && row_index_div < 1) return MOE_ERR_INVALID;
  if (row_capacity > 0 && (!x || !o_sorted)) return MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(o_sorted) || !aligned16(w_gate_up) || !aligned16(w_down))
    return MOE_ERR_INVALID;
  return MOE_OK;
}

moe_status_t moe_expert_ffn(const void* x, const int32_t* row_index, int32_t row_index_div,
                            const int32_t* expert_offsets, const void* w_gate_up,
                            const void* w_down, int32_t num_local_experts, int32_t hidden,
                            int32_t inter, int32_t row_capacity, int32_t dtype, void* o_sorted,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const moe_status_t st = check_ffn_args(x, row_index, row_index_div, expert_offsets, w_gate_up,
                                         w_down, num_local_experts, hidden, inter, row_capacity,
                                         dtype, o_sorted);
  if (st != MOE_OK) return st;
  const size_t need = moe::ffn_workspace_size(num_local_experts, hidden, inter, row_capacity,
                                              dtype == MOE_BF16);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return MOE_ERR_WORKSPACE;
  moe::FfnArgs a{x, row_index, row_index ? row_index_div : 1, expert_offsets, w_gate_up, w_down,
                 num_local_experts, hidden, inter, row_capacity, dtype == MOE_BF16, o_sorted,
                 workspace};
  return from_hip(moe::launch_ffn(a, stream));
}

moe_status_t moe_expert_ffn_noalloc(const void* x, const int32_t* row_index, int32_t row_index_div,
                                    const int32_t* expert_offsets, const void* w_gate_up,
                                    const void* w_down, int32_t num_local_experts, int32_t hidden,
                                    int32_t inter, int32_t row_capacity, int32_t dtype,
                                    void* o_sorted, hipStream_t stream) {
  const moe_status_t st = check_ffn_args(x, row_index, row_index_div, expert_offsets, w_gate_up,
                                         w_down, num_local_experts, hidden, inter, row_capacity,
                                         dtype, o_sorted);
  if (st != MOE_OK) return st;
  const size_t need = moe::ffn_workspace_size(num_local_experts, hidden, inter, row_capacity,
                                              dtype == MOE_BF16);
  if (need > MOE_FFN_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  void* ws = scratch_ptr();
  if (!ws) return MOE_ERR_LAUNCH;
  moe::FfnArgs a{x, row_index, row_index ? row_index_div : 1, expert_offsets, w_gate_up, w_down,
                 num_local_experts, hidden, inter, row_capacity, dtype == MOE_BF16, o_sorted, ws};
  return from_hip(moe::launch_ffn(a, stream));
}

size_t moe_expert_ffn_masked_workspace_size(int32_t num_local_experts, int32_t hidden,
                                            int32_t inter, int32_t expert_capacity, int32_t dtype) {
  if (expert_capacity < 0 || num_local_experts < 1) return 0;
  const int64_t rows = (int64_t)num_local_experts * expert_capacity;
  if (rows >= ((int64_t)1 << 31)) return 0;
  if (check_ffn_sizes(num_local_experts, hidden, inter, (int32_t)rows, dtype) != MOE_OK) return 0;
  return moe::ffn_masked_workspace_size(num_local_experts, hidden, inter, expert_capacity,
                                        dtype == MOE_BF16);
}

moe_status_t moe_expert_ffn_masked(const void* x_slots, const int32_t* expert_counts,
                                   int32_t expert_capacity, const void* w_gate_up,
                                   const void* w_down, int32_t num_local_experts, int32_t hidden,
                                   int32_t inter, int32_t dtype, void* o_slots, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  if (expert_capacity < 0 || num_local_experts < 1) return MOE_ERR_INVALID;
  const int64_t rows = (int64_t)num_local_experts * expert_capacity;
  if (rows >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  const moe_status_t st = check_ffn_args(x_slots, nullptr, 1, expert_counts, w_gate_up, w_down,
                                         num_local_experts, hidden, inter, (int32_t)rows, dtype,
                                         o_slots);
  if (st != MOE_OK) return st;
  const size_t need = moe::ffn_masked_workspace_size(num_local_experts, hidden, inter,
                                                     expert_capacity, dtype == MOE_BF16);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return MOE_ERR_WORKSPACE;
  if (rows == 0) return MOE_OK;
  moe::FfnMaskedArgs a{x_slots, expert_counts, expert_capacity, w_gate_up, w_down,
                       num_local_experts, hidden, inter, dtype == MOE_BF16, o_slots, workspace};
  return from_hip(moe::launch_ffn_masked(a, stream));
}

moe_status_t moe_quantize_e4m3(const void* x, int32_t rows, int32_t cols, int32_t dtype, void* codes,
                               float* scales, hipStream_t stream) {
  if (rows < 0 || cols < 128 || cols % 128 != 0) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID;
  if ((int64_t)rows * cols >= ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!x || !codes || !scales) return MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return MOE_ERR_INVALID;
  return from_hip(moe::launch_quantize_rows(x, rows, cols, dtype == MOE_BF16, (uint8_t*)codes, scales, stream));
}

static moe_status_t check_ffn_fp8_sizes(int32_t num_local_experts, int32_t hidden, int32_t inter,
                                        int32_t row_capacity) {
  if (num_local_experts < 1 || hidden < 1 || inter < 1 || row_capacity < 0) return MOE_ERR_INVALID;
  if (num_local_experts > 1024) return MOE_ERR_UNSUPPORTED;
  if (hidden % 512 != 0 || inter % 256 != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)2 * inter * hidden >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  // h (float32) and the permuted rows are addressed with 32-bit byte offsets
  if ((int64_t)row_capacity * inter * 4 >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t moe_expert_ffn_fp8_workspace_size(int32_t num_local_experts, int32_t hidden, int32_t inter,
                                         int32_t row_capacity) {
  if (check_ffn_fp8_sizes(num_local_experts, hidden, inter, row_capacity) != MOE_OK) return 0;
  return moe::ffn_fp8_workspace_size(hidden, inter, row_capacity);
}

moe_status_t moe_expert_ffn_fp8(const void* x_codes, const float* x_scales, const int32_t* row_index,
                                int32_t row_index_div, const int32_t* expert_offsets,
                                const void* w_gate_up, const float* w_gate_up_scales, const void* w_down,
                                const float* w_down_scales, int32_t num_local_experts, int32_t hidden,
                                int32_t inter, int32_t row_capacity, void* o_sorted, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  const moe_status_t st = check_ffn_fp8_sizes(num_local_experts, hidden, inter, row_capacity);
  if (st != MOE_OK) return st;
  if (!expert_offsets || !w_gate_up || !w_gate_up_scales || !w_down || !w_down_scales) return MOE_ERR_INVALID;
  if (row_index && row_index_div < 1) return MOE_ERR_INVALID;
  if (row_capacity > 0 && (!x_codes || !x_scales || !o_sorted)) return MOE_ERR_INVALID;
  if (!aligned16(x_codes) || !aligned16(x_scales) || !aligned16(o_sorted) || !aligned16(w_gate_up) ||
      !aligned16(w_down) || !aligned16(w_gate_up_scales) || !aligned16(w_down_scales))
    return MOE_ERR_INVALID;
  const size_t need = moe::ffn_fp8_workspace_size(hidden, inter, row_capacity);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return MOE_ERR_WORKSPACE;
  moe::FfnFp8Args a{x_codes, x_scales, row_index, row_index ? row_index_div : 1, expert_offsets,
                    w_gate_up, w_gate_up_scales, w_down, w_down_scales, num_local_experts, hidden, inter,
                    row_capacity, o_sorted, workspace};
  return from_hip(moe::launch_ffn_fp8(a, stream));
}

moe_status_t moe_combine(const void* o_sorted, const int32_t* assign_pos,
                         const float* topk_weights, int32_t num_tokens, int32_t top_k,
                         int32_t hidden, int32_t dtype, int32_t out_dtype, void* y,
                         hipStream_t stream) {
  if (num_tokens < 0 || top_k < 1 || hidden < 8 || hidden % 8 != 0) return MOE_ERR_INVALID;
  if ((dtype != MOE_F32 && dtype != MOE_BF16) || (out_dtype != MOE_F32 && out_dtype != MOE_BF16))
    return MOE_ERR_INVALID;
  if (top_k > 64) return MOE_ERR_UNSUPPORTED;
  if (num_tokens == 0) return MOE_OK;
  if (!o_sorted || !assign_pos || !topk_weights || !y) return MOE_ERR_INVALID;
  if (!aligned16(o_sorted) || !aligned16(y)) return MOE_ERR_INVALID;
  moe::CombineArgs a{o_sorted, assign_pos, topk_weights, num_tokens, top_k, hidden,
                     dtype == MOE_BF16, out_dtype == MOE_BF16, y};
  return from_hip(moe::launch_combine(a, stream));
}

moe_status_t moe_eplb_place(const double* load, int32_t num_experts, int32_t num_groups,
                            int32_t num_nodes, int32_t num_gpus, int32_t num_physical,
                            int32_t hierarchical, int32_t* phys_to_logical,
                            int32_t* replica_offsets, int32_t* replica_slots) {
  if (num_experts < 1 || num_groups < 1 || num_nodes < 1 || num_gpus < 1) return MOE_ERR_INVALID;
  if (num_experts % num_groups != 0 || num_gpus % num_nodes != 0) return MOE_ERR_INVALID;
  if (num_physical < num_experts || num_physical % num_gpus != 0) return MOE_ERR_INVALID;
  if (num_nodes > 64) return MOE_ERR_UNSUPPORTED;
  if (hierarchical) {   // whole groups per node, whole per-node slot and GPU counts
    if (num_groups % num_nodes != 0 || num_physical % num_nodes != 0) return MOE_ERR_INVALID;
    if ((num_physical / num_nodes) % (num_gpus / num_nodes) != 0) return MOE_ERR_INVALID;
  }
  if ((int64_t)num_physical >= ((int64_t)1 << 30)) return MOE_ERR_UNSUPPORTED;
  if (!load || !phys_to_logical || !replica_offsets || !replica_slots) return MOE_ERR_INVALID;
  for (int32_t e = 0; e < num_experts; ++e)
    if (!std::isfinite(load[e]) || load[e] < 0.0) return MOE_ERR_INVALID;
  const int n = moe::eplb_place(load, num_experts, num_groups, num_nodes, num_gpus, num_physical,
                                hierarchical != 0, phys_to_logical, replica_offsets, replica_slots);
  return n == num_physical ? MOE_OK : MOE_ERR_INVALID;
}

moe_status_t moe_eplb_remap(const int32_t* topk_ids, int32_t num_tokens, int32_t top_k,
                            const int32_t* replica_offsets, const int32_t* replica_slots,
                            int32_t num_experts, int32_t num_physical, int32_t num_gpus,
                            int32_t num_nodes, int32_t* physical_ids, hipStream_t stream) {
  if (num_tokens < 0 || top_k < 1 || num_experts < 1 || num_gpus < 1 || num_nodes < 1)
    return MOE_ERR_INVALID;
  if (num_physical < num_experts || num_physical % num_gpus != 0 || num_gpus % num_nodes != 0)
    return MOE_ERR_INVALID;
  if (num_nodes > 64) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)num_tokens * top_k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (num_tokens == 0) return MOE_OK;
  if (!topk_ids || !replica_offsets || !replica_slots || !physical_ids) return MOE_ERR_INVALID;
  return from_hip(moe::launch_eplb_remap(topk_ids, num_tokens, top_k, replica_offsets, replica_slots,
                                         num_experts, num_physical / num_gpus, num_gpus / num_nodes,
                                         physical_ids, stream));
}

size_t moe_dispatch_deferred_workspace_size(int32_t num_tokens, int32_t top_k, int32_t num_local_experts) {
  if (num_tokens < 0 || top_k < 1 || num_local_experts < 1 || num_local_experts > moe::kDispatchMaxLocal)
    return 0;
  const int64_t n = (int64_t)num_tokens * top_k;
  if (n >= ((int64_t)1 << 31) - 65536) return 0;
  return moe::deferred_workspace_size((int)n, num_local_experts);
}

moe_status_t moe_dispatch_deferred(const int32_t* topk_ids, int32_t num_tokens, int32_t top_k,
                                   int32_t expert_begin, int32_t num_local_experts, int32_t expert_capacity,
                                   int32_t rounds, const void* x, int32_t hidden, int32_t dtype,
                                   int32_t* round_counts, int32_t* round_offsets, int32_t* expert_demand,
                                   int32_t* sorted_assign, int32_t* assign_pos, void* x_sorted,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (num_tokens < 0 || top_k < 1 || expert_begin < 0 || num_local_experts < 1 || expert_capacity < 0 ||
      rounds < 1)
    return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (num_local_experts > moe::kDispatchMaxLocal) return MOE_ERR_UNSUPPORTED;
  const int64_t n = (int64_t)num_tokens * top_k;
  if (n >= ((int64_t)1 << 31) - 65536) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)rounds * (num_local_experts + 1) >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (!round_counts || !round_offsets) return MOE_ERR_INVALID;
  if (n > 0 && (!topk_ids || !assign_pos || !sorted_assign)) return MOE_ERR_INVALID;
  if ((x == nullptr) != (x_sorted == nullptr)) return MOE_ERR_INVALID;
  int row_bytes = 0;
  if (x) {
    if (hidden < 8 || hidden % 8 != 0) return MOE_ERR_INVALID;
    if (!aligned16(x) || !aligned16(x_sorted)) return MOE_ERR_INVALID;
    const int64_t rb = (int64_t)hidden * (dtype == MOE_BF16 ? 2 : 4);
    if (rb > (1 << 30)) return MOE_ERR_UNSUPPORTED;
    row_bytes = (int)rb;
  }
  const size_t need = moe::deferred_workspace_size((int)n, num_local_experts);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return MOE_ERR_WORKSPACE;
  moe::DeferredArgs a{topk_ids, (int)n, top_k, expert_begin, num_local_experts, expert_capacity, rounds,
                      x, x_sorted, row_bytes, round_counts, round_offsets, expert_demand, sorted_assign,
                      assign_pos, workspace};
  return from_hip(moe::launch_dispatch_deferred(a, stream));
}

size_t moe_eplb_remap_capacity_workspace_size(int32_t num_tokens, int32_t top_k, int32_t num_experts) {
  if (num_tokens < 0 || top_k < 1 || num_experts < 1 || num_experts > moe::kDispatchMaxLocal) return 0;
  const int64_t n = (int64_t)num_tokens * top_k;
  if (n >= ((int64_t)1 << 31) - 65536) return 0;
  return moe::remap_capacity_workspace_size((int)n, num_experts);
}

moe_status_t moe_eplb_remap_capacity(const int32_t* topk_ids, int32_t num_tokens, int32_t top_k,
                                     const int32_t* replica_offsets, const int32_t* replica_slots,
                                     int32_t num_experts, int32_t replica_capacity, int32_t* physical_ids,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (num_tokens < 0 || top_k < 1 || num_experts < 1 || replica_capacity < 0) return MOE_ERR_INVALID;
  if (num_experts > moe::kDispatchMaxLocal) return MOE_ERR_UNSUPPORTED;
  const int64_t n = (int64_t)num_tokens * top_k;
  if (n >= ((int64_t)1 << 31) - 65536) return MOE_ERR_UNSUPPORTED;
  if (n == 0) return MOE_OK;
  if (!topk_ids || !replica_offsets || !replica_slots || !physical_ids) return MOE_ERR_INVALID;
  const size_t need = moe::remap_capacity_workspace_size((int)n, num_experts);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return MOE_ERR_WORKSPACE;
  moe::RemapCapacityArgs a{topk_ids, (int)n, num_experts, replica_capacity, replica_offsets, replica_slots,
                           physical_ids, workspace};
  return from_hip(moe::launch_remap_capacity(a, stream));
}

}  // extern "C"
