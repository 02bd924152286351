// Dispatch: stable counting sort of assignments to local experts, then a row
// gather of the token activations into expert order.
//
// The dispatch step of ch15 section 3.4 ("第十五章：多节点大模型推理", se7en.mintlify.app)
// on one GPU: each token's activation goes to the rows of its experts. Rows of
// one expert keep assignment order a = t * k + j, so the result is unique and
// equals a stable sort by expert.
//
// Sort kernel: one workgroup of 16 wavefronts. Wave w owns a contiguous chunk
// of assignments and walks it 64 at a time. Lanes holding the same expert are
// found with one ballot per key bit (a wave-wide "match"), which gives each
// lane its rank among equal keys in the step without atomics. Pass 1 counts
// per (wave, expert) in LDS; a scan turns the counts into per-(wave, expert)
// start positions; pass 2 re-walks the chunk and writes each assignment at
// start + rank. All integer, no atomics: bit-for-bit deterministic.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kSortWaves = 16;

// Bitmask of the lanes whose key equals this lane's key (only among active lanes).
__device__ __forceinline__ uint64_t match_key(int key, bool active, int nbits) {
  uint64_t m = __ballot(active);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bal = __ballot(active && bit);
    m &= bit ? bal : ~bal;
  }
  return active ? m : 0ull;
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, MOE_WAVE);
    if (lane >= d) v += o;
  }
  return v;
}

__global__ __launch_bounds__(1024) void sort_kernel(const int* __restrict__ ids, int n, int begin,
                                                    int nloc, int nbits, int* __restrict__ counts,
                                                    int* __restrict__ offsets,
                                                    int* __restrict__ sorted_assign,
                                                    int* __restrict__ assign_pos) {
  extern __shared__ int lds[];
  int* cnt = lds;                              // [kSortWaves][nloc]
  int* wbase = lds + kSortWaves * nloc;        // [kSortWaves]
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < kSortWaves * nloc; i += blockDim.x) cnt[i] = 0;
  __syncthreads();

  const int per_wave = (((n + kSortWaves - 1) / kSortWaves) + 63) & ~63;
  const int lo = min(n, w * per_wave), hi = min(n, lo + per_wave);
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  int* my_cnt = cnt + w * nloc;

  // pass 1: counts per (wave, expert)
  for (int base = lo; base < hi; base += 64) {
    const int a = base + lane;
    int e = -1;
    if (a < hi) {
      const int x = ids[a] - begin;
      if ((unsigned)x < (unsigned)nloc) e = x;
    }
    const uint64_t peers = match_key(e, e >= 0, nbits);
    if (e >= 0 && (peers & lt_mask) == 0ull) my_cnt[e] += __popcll(peers);
  }
  __syncthreads();

  // scan: per-expert column prefix over waves, then exclusive scan over experts
  int total = 0;
  for (int e = threadIdx.x; e < nloc; e += blockDim.x) {  // nloc <= blockDim.x: one expert per thread
    for (int ww = 0; ww < kSortWaves; ++ww) {
      const int c = cnt[ww * nloc + e];
      cnt[ww * nloc + e] = total;
      total += c;
    }
  }
  const int incl = wave_inclusive_scan(total);
  if (lane == 63) wbase[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int v = lane < kSortWaves ? wbase[lane] : 0;
    const int vi = wave_inclusive_scan(v);
    if (lane < kSortWaves) wbase[lane] = vi - v;
  }
  __syncthreads();
  {
    const int e = threadIdx.x;
    const int excl = incl - total + wbase[w];
    if (e < nloc) {
      counts[e] = total;
      offsets[e] = excl;
      for (int ww = 0; ww < kSortWaves; ++ww) cnt[ww * nloc + e] += excl;
      if (e == nloc - 1) offsets[nloc] = excl + total;
    }
  }
  __syncthreads();

  // pass 2: scatter in chunk order
  for (int base = lo; base < hi; base += 64) {
    const int a = base + lane;
    int e = -1;
    if (a < hi) {
      const int x = ids[a] - begin;
      if ((unsigned)x < (unsigned)nloc) e = x;
    }
    const uint64_t peers = match_key(e, e >= 0, nbits);
    if (a < hi) {
      if (e >= 0) {
        const int p = my_cnt[e] + __popcll(peers & lt_mask);
        sorted_assign[p] = a;
        assign_pos[a] = p;
      } else {
        assign_pos[a] = -1;
      }
    }
    // LDS operations of one wave execute in order: every lane has read the
    // running count above before the leader advances it here.
    if (e >= 0 && (peers & lt_mask) == 0ull) my_cnt[e] += __popcll(peers);
  }
}

__global__ void zero_counts_kernel(int nloc, int* counts, int* offsets) {
  for (int e = threadIdx.x; e <= nloc; e += blockDim.x) {
    if (e < nloc) counts[e] = 0;
    offsets[e] = 0;
  }
}

// One wavefront per permuted row; 16-byte vector copies.
__global__ __launch_bounds__(256) void gather_kernel(const uint4* __restrict__ x,
                                                     const int* __restrict__ sorted_assign,
                                                     const int* __restrict__ offsets, int nloc,
                                                     int k, int capacity, int row_vec,
                                                     uint4* __restrict__ x_sorted) {
  const int lane = threadIdx.x & 63;
  const int M = min(offsets[nloc], capacity);
  for (int r = blockIdx.x * 4 + (threadIdx.x >> 6); r < M; r += gridDim.x * 4) {
    const int t = sorted_assign[r] / k;
    const uint4* src = x + (size_t)t * row_vec;
    uint4* dst = x_sorted + (size_t)r * row_vec;
    for (int c = lane; c < row_vec; c += 64) dst[c] = src[c];
  }
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  if (a.n == 0) {
    hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(256), 0, s, a.num_local, a.counts,
                       a.offsets);
    return hipGetLastError();
  }
  int nbits = 1;
  while ((1 << nbits) < a.num_local) ++nbits;
  const size_t lds = (size_t)(kSortWaves * a.num_local + kSortWaves) * sizeof(int);
  hipLaunchKernelGGL(sort_kernel, dim3(1), dim3(kSortWaves * 64), lds, s, a.ids, a.n,
                     a.expert_begin, a.num_local, nbits, a.counts, a.offsets, a.sorted_assign,
                     a.assign_pos);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.row_bytes == 0) return err;
  const int row_vec = a.row_bytes / 16;
  const int blocks = (int)std::min<long>((a.n + 3) / 4, 2048);
  hipLaunchKernelGGL(gather_kernel, dim3(blocks), dim3(256), 0, s, (const uint4*)a.x,
                     a.sorted_assign, a.offsets, a.num_local, a.k, a.n, row_vec,
                     (uint4*)a.x_sorted);
  return hipGetLastError();
}

}  // namespace moe
