// Routing with a per-expert capacity and the "next-best expert" overflow
// policy: the first row of the table of overflow policies in ch15 section 4.3
// ("第十五章：多节点大模型推理", se7en.mintlify.app; "负载均衡" section: an
// assignment over its expert's capacity goes to the token's next-highest-
// scoring expert instead). The routing itself is the group-limited top-k of
// the EPLB page (section "EPLB 与路由约束").
//
// Readings (the page names the policy only): capacity goes first to the
// original choices (each expert keeps its first C original assignments in
// assignment order a = t * k + j); then, in assignment order, the i-th
// overflowing slot of a token takes the token's spare candidate of rank k + i
// (the next experts of the same ranking, inside its kept groups) if that
// expert then holds fewer than C assignments; otherwise the slot is dropped
// (id -1). Weights are the final experts' scores, renormalised over the
// token's slots that were not dropped.
//
// Everything is parallel: the ranking is moe_route's top-2k; the originals'
// ranks come from the capped counting sort; each overflowing slot's candidate
// is fixed by its token alone; the candidates' ranks among all rerouted slots
// of their expert (assignment order) come from a second counting sort, and a
// rerouted slot is kept when that rank is below the room the originals left.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

// ids2 [T, k2] -> the original choices [T, k] (the first k ranks).
__global__ __launch_bounds__(256) void reroute_originals_kernel(const int* __restrict__ ids2, int T, int k,
                                                                int k2, int* __restrict__ ids) {
  const long n = (long)T * k;
  for (long a = (long)blockIdx.x * blockDim.x + threadIdx.x; a < n; a += (long)gridDim.x * blockDim.x) {
    const long t = a / k;
    ids[a] = ids2[t * k2 + (a - t * k)];
  }
}

// One wavefront per token, lane j = slot j (k <= 64): the i-th overflowing slot
// (pos1 < 0; i = overflowing slots before it, a ballot prefix) takes spare
// rank k + i, or -1 when the token has no such candidate; kept slots get -1
// (not rerouted).
__global__ __launch_bounds__(256) void reroute_candidates_kernel(const int* __restrict__ ids2,
                                                                 const int* __restrict__ pos1, int T, int k,
                                                                 int k2, int* __restrict__ rid) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;   // uniform per wave
  const long a = (long)t * k + lane;
  const bool over = lane < k && pos1[a] < 0;
  const int i = __popcll(__ballot(over) & ((1ull << lane) - 1ull));
  if (lane < k) rid[a] = (over && k + i < k2) ? ids2[(long)t * k2 + k + i] : -1;
}

// One wavefront per token, lane j = slot j: final experts and weights. A
// rerouted slot is kept when its rank among its expert's rerouted slots is
// below C - counts1[e]. The scores of the final experts are summed in slot
// order (the weights' normaliser). Threads of the grid also write the final
// load of every expert.
__global__ __launch_bounds__(256) void reroute_finalize_kernel(
    const float* __restrict__ scores, const int* __restrict__ ids2, const int* __restrict__ pos1,
    const int* __restrict__ counts1, const int* __restrict__ rid, const int* __restrict__ pos2,
    const int* __restrict__ offsets2, const int* __restrict__ counts2, int T, int E, int k, int k2, int cap,
    int renormalize, int* __restrict__ ids, float* __restrict__ weights, int* __restrict__ load) {
  if (load)
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < E; e += gridDim.x * blockDim.x)
      load[e] = counts1[e] + min(counts2[e], cap - counts1[e]);
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;   // uniform per wave
  const long a = (long)t * k + lane;
  int e = -1;
  if (lane < k) {
    if (pos1[a] >= 0) {
      e = ids2[(long)t * k2 + lane];
    } else {
      const int r = rid[a];
      if (r >= 0 && pos2[a] - offsets2[r] < cap - counts1[r]) e = r;
    }
    ids[a] = e;
  }
  const float w = e >= 0 ? scores[(long)t * E + e] : 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
  if (lane < k) weights[a] = renormalize ? (sum > 0.0f ? w / sum : 0.0f) : w;
}

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

int reroute_ranks(int E, int k, int num_groups, int topk_groups) {
  const int G = E / num_groups;
  return std::min(std::min(2 * k, topk_groups * G), 64);
}

size_t reroute_workspace_size(int T, int E, int k, int num_groups, int topk_groups) {
  const size_t n = (size_t)T * k, n2 = (size_t)T * reroute_ranks(E, k, num_groups, topk_groups);
  return 2 * al256(n2 * 4) + 5 * al256(n * 4) + 2 * al256((size_t)E * 4) + 2 * al256((size_t)(E + 1) * 4) +
         al256(dispatch_workspace_size((int)n, E));
}

hipError_t launch_route_reroute(const RerouteArgs& a, hipStream_t s) {
  const int k2 = reroute_ranks(a.E, a.k, a.num_groups, a.topk_groups);
  const size_t n = (size_t)a.T * a.k, n2 = (size_t)a.T * k2;
  char* p = (char*)a.workspace;
  auto take = [&](size_t bytes) { char* q = p; p += al256(bytes); return q; };
  int* ids2 = (int*)take(n2 * 4);
  float* w2 = (float*)take(n2 * 4);
  int* pos1 = (int*)take(n * 4);
  int* sa1 = (int*)take(n * 4);
  int* rid = (int*)take(n * 4);
  int* pos2 = (int*)take(n * 4);
  int* sa2 = (int*)take(n * 4);
  int* counts1 = (int*)take((size_t)a.E * 4);
  int* counts2 = (int*)take((size_t)a.E * 4);
  int* offsets1 = (int*)take((size_t)(a.E + 1) * 4);
  int* offsets2 = (int*)take((size_t)(a.E + 1) * 4);
  void* dws = p;
  // 1. ranking: the k choices and the spares
  RouteArgs r{a.scores, a.T, a.E, k2, a.num_groups, a.topk_groups, 0, 0, ids2, w2};
  hipError_t err = launch_route(r, s);
  if (err != hipSuccess) return err;
  const int blocks = (int)std::min<long>(((long)n + 255) / 256, 4096);
  hipLaunchKernelGGL(reroute_originals_kernel, dim3(blocks), dim3(256), 0, s, ids2, a.T, a.k, k2, a.ids);
  // 2. originals: each expert keeps its first C in assignment order
  DispatchArgs d1{a.ids, (int)n, a.k, 0, a.E, counts1, offsets1, sa1, pos1, nullptr, nullptr, 0, dws, a.cap,
                  nullptr};
  err = launch_dispatch(d1, s);
  if (err != hipSuccess) return err;
  // 3. each overflowing slot's candidate, then its rank among its expert's rerouted slots
  const int tb = (a.T + 3) / 4;   // a wavefront per token
  hipLaunchKernelGGL(reroute_candidates_kernel, dim3(tb), dim3(256), 0, s, ids2, pos1, a.T, a.k, k2, rid);
  DispatchArgs d2{rid, (int)n, a.k, 0, a.E, counts2, offsets2, sa2, pos2, nullptr, nullptr, 0, dws, INT32_MAX,
                  nullptr};
  err = launch_dispatch(d2, s);
  if (err != hipSuccess) return err;
  // 4. final experts, weights and loads
  hipLaunchKernelGGL(reroute_finalize_kernel, dim3(tb), dim3(256), 0, s, a.scores, ids2, pos1, counts1, rid, pos2,
                     offsets2, counts2, a.T, a.E, a.k, k2, a.cap, a.renormalize, a.ids, a.weights, a.load);
  return hipGetLastError();
}

}  // namespace moe
