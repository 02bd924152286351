// EPLB: placement of logical experts (with redundant replicas) on GPUs, and
// the choice of a physical replica for every routed (token, slot).
//
// From the page "大规模 EP 部署：分层 EPLB、DP 注意力的负载与双 batch 重叠"
// (anrans.github.io), section "EPLB 与路由约束". Hierarchical strategy: pack
// the expert groups onto the nodes, balanced by load with the same number of
// groups per node; inside each node give the hottest experts extra replicas;
// pack each node's physical experts onto its GPUs, balanced, the same number
// per GPU. Global strategy: the same over all experts and GPUs at once.
// Balanced packing takes items heaviest first (equal weights: lower index
// first) into the lightest pack that still has room (equal totals: lower
// pack); replication repeatedly adds a replica to the expert with the highest
// load per replica (equal: the expert listed first). Sums are float64 in
// placement order.
//
// The replica choice follows the page's simulation: a token slot uses a
// replica on a node the token already goes to when there is one (the lowest
// such slot), else the lowest slot on the lowest-numbered node holding one.
// The placement planner (host code) is in host_plan.cpp.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace moe {

namespace {

// One thread per token; its nodes so far in a 64-bit mask. An expert id
// outside [0, E), or one without a replica, gets -1 and reads nothing else.
__global__ __launch_bounds__(256) void remap_kernel(const int* __restrict__ ids, int T, int k,
                                                    const int* __restrict__ offsets,
                                                    const int* __restrict__ slots, int E,
                                                    int slots_per_gpu, int gpus_per_node,
                                                    int* __restrict__ phys) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  uint64_t used = 0;
  const int per_node = slots_per_gpu * gpus_per_node;
  for (int j = 0; j < k; ++j) {
    const int e = ids[(size_t)t * k + j];
    if ((unsigned)e >= (unsigned)E) {
      phys[(size_t)t * k + j] = -1;
      continue;
    }
    const int r0 = offsets[e], r1 = offsets[e + 1];
    if (r1 <= r0) {
      phys[(size_t)t * k + j] = -1;
      continue;
    }
    int on_used = -1, lowest = -1, lowest_node = 1 << 30;
    for (int r = r0; r < r1; ++r) {   // ascending slots
      const int s = slots[r];
      const int node = s / per_node;
      if (on_used < 0 && ((used >> node) & 1ull)) on_used = s;
      if (node < lowest_node) { lowest_node = node; lowest = s; }
    }
    if (on_used >= 0) {
      phys[(size_t)t * k + j] = on_used;
    } else {
      phys[(size_t)t * k + j] = lowest;
      used |= 1ull << lowest_node;
    }
  }
}

}  // namespace

hipError_t launch_eplb_remap(const int* ids, int T, int k, const int* offsets, const int* slots,
                             int num_experts, int slots_per_gpu, int gpus_per_node, int* phys,
                             hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(remap_kernel, dim3((T + 255) / 256), dim3(256), 0, s, ids, T, k, offsets, slots,
                     num_experts, slots_per_gpu, gpus_per_node, phys);
  return hipGetLastError();
}

}  // namespace moe
