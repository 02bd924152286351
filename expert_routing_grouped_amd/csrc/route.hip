// Router kernel: one wavefront per token.
//
// Group-limited top-k routing as stated on the page "大规模 EP 部署：分层 EPLB、
// DP 注意力的负载与双 batch 重叠" (anrans.github.io, section "EPLB 与路由约束"):
// group score = sum of the group's two highest scores, keep the best
// topk_groups groups, then select top_k experts inside them; and plain top-k
// gating with softmax weights (ch15 section 4.1) when there are no groups.
//
// Layout: lane l holds experts [l*V, l*V + V) of its token in registers
// (V = values per lane, a power of two, 64*V >= E). Selection runs k rounds
// of a wave-wide maximum over 64-bit keys (order-preserving float bits in the
// high word, the complemented expert index in the low word), so equal scores
// resolve to the lower expert index and the result does not depend on the
// reduction order.
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

// Insert v into the pair (a1 >= a2) of the two largest values seen so far; an
// equal value is kept twice, so a duplicated maximum fills both places.
__device__ __forceinline__ void top2_insert(float v, float& a1, float& a2) {
  const float hi = fmaxf(a1, v), lo = fminf(a1, v);
  a2 = fmaxf(a2, lo);
  a1 = hi;
}

// Merge two (first, second) pairs into the top two of the four values.
__device__ __forceinline__ void top2_merge(float& a1, float& a2, float b1, float b2) {
  float lo = fminf(a1, b1), hi = fmaxf(a1, b1);
  a2 = fmaxf(lo, fmaxf(a2, b2));
  a1 = hi;
}

template <int V, bool ALIGNED>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ scores, int T, int E,
                                                    int k, int num_groups, int topk_groups,
                                                    int softmax, int renormalize,
                                                    int* __restrict__ topk_ids,
                                                    float* __restrict__ topk_weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* row = scores + (size_t)t * E;

  float val[V];
  bool valid[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int idx = lane * V + v;
    valid[v] = idx < E;
    val[v] = valid[v] ? row[idx] : 0.0f;
  }

  float lmax = 0.0f, lsum = 1.0f;
  if (softmax) {
    float m = -INFINITY;
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (valid[v]) m = fmaxf(m, val[v]);
    lmax = wave_max_f32(m);
    float s = 0.0f;
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (valid[v]) s += expf(val[v] - lmax);
    lsum = wave_sum_f32(s);
  }

  // ---- group stage: which groups stay candidates
  uint64_t kept = ~0ull;
  int G = E;
  if (num_groups > 1) {
    G = E / num_groups;
    float gs = -INFINITY;  // lane g < num_groups ends up holding group g's score
    if (ALIGNED) {
      // Each lane's V experts lie in one group; a group spans G / V lanes.
      const int lpg = G / V;
      float a1 = -INFINITY, a2 = -INFINITY;
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (valid[v]) top2_insert(val[v], a1, a2);
      for (int m = 1; m < lpg; m <<= 1) {
        const float b1 = __shfl_xor(a1, m, MOE_WAVE);
        const float b2 = __shfl_xor(a2, m, MOE_WAVE);
        top2_merge(a1, a2, b1, b2);
      }
      const float mine = a1 + a2;
      const int src = (lane < num_groups ? lane : 0) * lpg;
      gs = __shfl(mine, src, MOE_WAVE);
    } else {
      for (int g = 0; g < num_groups; ++g) {
        float a1 = -INFINITY, a2 = -INFINITY;
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const int idx = lane * V + v;
          if (valid[v] && idx / G == g) top2_insert(val[v], a1, a2);
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
          const float b1 = __shfl_xor(a1, m, MOE_WAVE);
          const float b2 = __shfl_xor(a2, m, MOE_WAVE);
          top2_merge(a1, a2, b1, b2);
        }
        if (lane == g) gs = a1 + a2;
      }
    }
    // rank of group `lane` = number of groups ahead of it (higher score, or equal and lower index)
    int rank = 0;
    for (int g2 = 0; g2 < num_groups; ++g2) {
      const float o = __shfl(gs, g2, MOE_WAVE);
      rank += (o > gs) || (o == gs && g2 < lane);
    }
    kept = __ballot(lane < num_groups && rank < topk_groups);
  }

  // ---- candidate keys
  uint64_t key[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const uint32_t idx = (uint32_t)(lane * V + v);
    const bool cand = valid[v] && ((kept >> (idx / (uint32_t)G)) & 1ull);
    key[v] = cand ? (((uint64_t)ordered_key(val[v]) << 32) | (uint32_t)(~idx)) : 0ull;
  }

  // ---- k rounds of wave argmax
  int my_id = 0;
  float my_val = 0.0f;
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0ull;
    float bestv = 0.0f;
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (key[v] > best) { best = key[v]; bestv = val[v]; }
    const uint64_t win = wave_max_u64(best);
    const int idx = (int)(~(uint32_t)win);
    const int owner = idx / V;
    const float sv = __shfl(bestv, owner, MOE_WAVE);
    if (lane == owner) {
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (key[v] == win) key[v] = 0ull;
    }
    if (lane == r) { my_id = idx; my_val = sv; }
  }

  float w = softmax ? expf(my_val - lmax) / lsum : my_val;
  if (renormalize) {
    const float s = wave_sum_f32(lane < k ? w : 0.0f);
    w = w / s;
  }
  if (lane < k) {
    topk_ids[(size_t)t * k + lane] = my_id;
    topk_weights[(size_t)t * k + lane] = w;
  }
}

template <int V>
hipError_t launch_v(const RouteArgs& a, hipStream_t s) {
  const dim3 grid((a.T + 3) / 4), block(256);
  const int G = a.num_groups > 1 ? a.E / a.num_groups : a.E;
  const int lpg = G / V;
  const bool aligned = a.num_groups > 1 && G % V == 0 && lpg >= 1 && lpg <= 64 && (lpg & (lpg - 1)) == 0;
  if (aligned)
    hipLaunchKernelGGL((route_kernel<V, true>), grid, block, 0, s, a.scores, a.T, a.E, a.k,
                       a.num_groups, a.topk_groups, a.softmax, a.renormalize, a.ids, a.weights);
  else
    hipLaunchKernelGGL((route_kernel<V, false>), grid, block, 0, s, a.scores, a.T, a.E, a.k,
                       a.num_groups, a.topk_groups, a.softmax, a.renormalize, a.ids, a.weights);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  const int per_lane = (a.E + 63) / 64;
  if (per_lane <= 1) return launch_v<1>(a, s);
  if (per_lane <= 2) return launch_v<2>(a, s);
  if (per_lane <= 4) return launch_v<4>(a, s);
  if (per_lane <= 8) return launch_v<8>(a, s);
  return launch_v<16>(a, s);
}

}  // namespace moe
