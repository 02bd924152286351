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
// of a wave-wide maximum over order-preserving float keys (DPP within rows of
// 16 lanes, scalar reads across rows); among lanes holding the maximum the
// lowest one wins, so equal scores resolve to the lower expert index and the
// result does not depend on the reduction order.
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
                                                    int softmax, int renormalize, int vec4,
                                                    int* __restrict__ topk_ids,
                                                    float* __restrict__ topk_weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* row = scores + (size_t)t * E;

  float val[V];
  bool valid[V];
  if (V >= 4 && vec4) {
    // rows 16-byte aligned and E % 4 == 0: a lane's scores are V / 4 whole
    // 16-byte loads, each all valid or all past E
#pragma unroll
    for (int j = 0; j < (V >= 4 ? V / 4 : 1); ++j) {
      const int idx = lane * V + 4 * j;
      const float4 q = idx < E ? *(const float4*)(row + idx) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float qv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * j + i < V) {
          val[4 * j + i] = qv[i];
          valid[4 * j + i] = idx < E;
        }
      }
    }
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int idx = lane * V + v;
      valid[v] = idx < E;
      val[v] = valid[v] ? row[idx] : 0.0f;
    }
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

  // ---- group stage: which experts stay candidates
  bool cand[V];
#pragma unroll
  for (int v = 0; v < V; ++v) cand[v] = valid[v];
  if (num_groups > 1) {
    const int G = E / num_groups;
    if (ALIGNED) {
      // Each lane's V experts lie in one group; a group spans lpg = G / V lanes
      // (a power of two): merge the (first, second) pairs across the group's
      // lanes with DPP inside rows of 16 and shuffles across rows.
      const int lpg = G / V;
      float a1 = -INFINITY, a2 = -INFINITY;
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (valid[v]) top2_insert(val[v], a1, a2);
      if (lpg >= 2) top2_merge(a1, a2, dpp_f32<kDppQuadXor1>(a1), dpp_f32<kDppQuadXor1>(a2));
      if (lpg >= 4) top2_merge(a1, a2, dpp_f32<kDppQuadXor2>(a1), dpp_f32<kDppQuadXor2>(a2));
      if (lpg >= 8) top2_merge(a1, a2, dpp_f32<kDppHalfMirror>(a1), dpp_f32<kDppHalfMirror>(a2));
      if (lpg >= 16) top2_merge(a1, a2, dpp_f32<kDppRowMirror>(a1), dpp_f32<kDppRowMirror>(a2));
      for (int m = 16; m < lpg; m <<= 1)
        top2_merge(a1, a2, __shfl_xor(a1, m, MOE_WAVE), __shfl_xor(a2, m, MOE_WAVE));
      const float mine = a1 + a2;  // every lane of the group holds its group score
      const int gl = lane / lpg;
      // rank of this lane's group: groups ahead of it (higher score, or equal and lower index)
      int rank = 0;
      for (int g2 = 0; g2 < num_groups; ++g2) {
        const float o = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), g2 * lpg));
        rank += (o > mine) || (o == mine && g2 < gl);
      }
      const bool keep = rank < topk_groups;
#pragma unroll
      for (int v = 0; v < V; ++v) cand[v] = cand[v] && keep;
    } else {
      float gs = -INFINITY;  // lane g < num_groups ends up holding group g's score
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
      int rank = 0;
      for (int g2 = 0; g2 < num_groups; ++g2) {
        const float o = __shfl(gs, g2, MOE_WAVE);
        rank += (o > gs) || (o == gs && g2 < lane);
      }
      const uint64_t kept = __ballot(lane < num_groups && rank < topk_groups);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int idx = lane * V + v;
        cand[v] = cand[v] && ((kept >> (idx / G)) & 1ull);
      }
    }
  }

  // ---- k rounds of wave argmax. Keys are order-preserving float bits (0 =
  // not a candidate). The round's maximum comes from a DPP reduction; the
  // lowest lane holding it (a ballot) has the lowest expert index among equal
  // scores, and inside a lane the first v wins.
  uint32_t key[V];
#pragma unroll
  for (int v = 0; v < V; ++v) key[v] = cand[v] ? ordered_key(val[v]) : 0u;
  int my_id = 0;
  float my_val = 0.0f;
  if constexpr (V >= 8) {
    // Many values per lane: each lane sorts its (key, v) pairs once (bitonic
    // network on key << 32 | (V - 1 - v): larger key first, then lower v), parks
    // the sorted list and its values in its wavefront's LDS, and a round pops
    // only the winner's head -- O(1) instructions per round instead of a pass
    // over the V values. Same winners, same order, same values.
    __shared__ uint64_t s_pk[4][V][64];
    __shared__ float s_val[4][V][64];
    const int wv = threadIdx.x >> 6;
    uint64_t pk[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      pk[v] = ((uint64_t)key[v] << 32) | (uint32_t)(V - 1 - v);
      s_val[wv][v][lane] = val[v];
    }
#pragma unroll
    for (int size = 2; size <= V; size <<= 1)
#pragma unroll
      for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const int j = i ^ stride;
          if (j > i) {
            const uint64_t x = pk[i], y = pk[j];
            const bool sw = (i & size) == 0 ? x < y : x > y;   // descending runs first
            pk[i] = sw ? y : x;
            pk[j] = sw ? x : y;
          }
        }
#pragma unroll
    for (int v = 0; v < V; ++v) s_pk[wv][v][lane] = pk[v];
    uint64_t cur = pk[0], nxt = pk[1];
    int head = 1;   // position of nxt
    for (int r = 0; r < k; ++r) {
      const uint32_t ck = (uint32_t)(cur >> 32);
      const uint32_t win = wave_max_u32_dpp(ck);
      const uint64_t holders = __ballot(ck == win);
      const int owner = __ffsll((unsigned long long)holders) - 1;
      int vsel = 0;
      float sv = 0.0f;   // no candidate left anywhere: expert 0, value 0, as the plain pass gives
      if (win != 0u) {
        vsel = V - 1 - __builtin_amdgcn_readlane((int)(uint32_t)cur, owner);
        sv = s_val[wv][vsel][owner];
        if (lane == owner) {
          cur = nxt;
          ++head;
          nxt = head < V ? s_pk[wv][head][lane] : 0ull;
        }
      }
      if (lane == r) { my_id = owner * V + vsel; my_val = sv; }
    }
  } else {
  for (int r = 0; r < k; ++r) {
    uint32_t best = 0u;
    int bv = 0;
    float bval = 0.0f;
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (key[v] > best) { best = key[v]; bv = v; bval = val[v]; }
    const uint32_t win = wave_max_u32_dpp(best);
    const uint64_t holders = __ballot(best == win);
    const int owner = __ffsll((unsigned long long)holders) - 1;
    const int vsel = __builtin_amdgcn_readlane(bv, owner);
    const float sv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bval), owner));
    if (lane == owner) {
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (v == vsel) key[v] = 0u;
    }
    if (lane == r) { my_id = owner * V + vsel; my_val = sv; }
  }
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
  const int vec4 = (reinterpret_cast<uintptr_t>(a.scores) % 16 == 0 && a.E % 4 == 0) ? 1 : 0;
  if (aligned)
    hipLaunchKernelGGL((route_kernel<V, true>), grid, block, 0, s, a.scores, a.T, a.E, a.k,
                       a.num_groups, a.topk_groups, a.softmax, a.renormalize, vec4, a.ids, a.weights);
  else
    hipLaunchKernelGGL((route_kernel<V, false>), grid, block, 0, s, a.scores, a.T, a.E, a.k,
                       a.num_groups, a.topk_groups, a.softmax, a.renormalize, vec4, a.ids, a.weights);
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
