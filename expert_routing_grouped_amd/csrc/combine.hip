// Combine: y[t] = sum_j w[t, j] * o[pos[t*k + j]] over the token's local slots,
// in slot order, float32 accumulation.
//
// The combine step of ch15 section 3.4 ("第十五章：多节点大模型推理", se7en.mintlify.app)
// and the weighted sum y = p5 E5(x) + p27 E27(x) of hop 4 on the page
// "追踪一个 Token 在 MoE 推理中穿越 TP/CP/SP/EP/DP/PP 的路径" (attain.fans).
//
// One wavefront per token; each lane owns 8 consecutive elements per step
// (16-byte bf16 loads, or two 16-byte float32 loads) so every row of o is
// read with fully coalesced 1 KiB (or 2 KiB) wave accesses.
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

template <bool O_BF16>
__device__ __forceinline__ void load8(const void* base, size_t elem, float (&v)[8]) {
  if (O_BF16) {
    const uint4 q = *(const uint4*)((const uint16_t*)base + elem);
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
  } else {
    const float4 a = *(const float4*)((const float*)base + elem);
    const float4 b = *(const float4*)((const float*)base + elem + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool Y_BF16>
__device__ __forceinline__ void store8(void* base, size_t elem, const float (&v)[8]) {
  if (Y_BF16) {
    uint4 q;
    q.x = pack_bf16x2(v[0], v[1]); q.y = pack_bf16x2(v[2], v[3]);
    q.z = pack_bf16x2(v[4], v[5]); q.w = pack_bf16x2(v[6], v[7]);
    *(uint4*)((uint16_t*)base + elem) = q;
  } else {
    *(float4*)((float*)base + elem) = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)((float*)base + elem + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// Workgroup = 4 wavefronts on one token; wavefront = 512 consecutive
// elements (8 per lane). The token's slot positions and weights are read once
// (lane j holds slot j); a ballot lists the slots whose expert is local, and
// their rows are loaded four at a time (all four in flight) and added in slot
// order. Non-local slots cost nothing.
template <bool O_BF16, bool Y_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ o,
                                                      const int* __restrict__ assign_pos,
                                                      const float* __restrict__ weights, int T,
                                                      int k, int hidden, void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x;
  const int c0 = (blockIdx.y * 4 + (threadIdx.x >> 6)) * 512;
  if (c0 >= hidden) return;  // uniform per wave
  const int c = c0 + lane * 8;
  const bool active = c < hidden;
  const int cc = active ? c : 0;
  const int mypos = lane < k ? assign_pos[(size_t)t * k + lane] : -1;
  const float myw = lane < k ? weights[(size_t)t * k + lane] : 0.0f;
  uint64_t local = __ballot(mypos >= 0);  // slot j's bit is bit j
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  while (local) {
    int p[4];
    float w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      p[q] = -1;
      w[q] = 0.0f;
      if (local) {
        const int j = __ffsll((unsigned long long)local) - 1;
        local &= local - 1;
        p[q] = __builtin_amdgcn_readlane(mypos, j);
        w[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myw), j));
      }
    }
    float v[4][8];
#pragma unroll
    for (int q = 0; q < 4; ++q) load8<O_BF16>(o, (size_t)(p[q] >= 0 ? p[q] : p[0]) * hidden + cc, v[q]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (p[q] >= 0)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += w[q] * v[q][i];
  }
  if (active) store8<Y_BF16>(y, (size_t)t * hidden + c, acc);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid(a.T, (a.hidden + 2047) / 2048), block(256);
#define MOE_COMBINE(OB, YB)                                                                  \
  hipLaunchKernelGGL((combine_kernel<OB, YB>), grid, block, 0, s, a.o_sorted, a.assign_pos, \
                     a.weights, a.T, a.k, a.hidden, a.y)
  if (a.o_bf16 && a.y_bf16) MOE_COMBINE(true, true);
  else if (a.o_bf16) MOE_COMBINE(true, false);
  else if (a.y_bf16) MOE_COMBINE(false, true);
  else MOE_COMBINE(false, false);
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
