// Two overflow policies of the capacity factor beside drop and next-best
// expert, from the table of overflow policies in ch15 section 4.3
// ("第十五章：多节点大模型推理", se7en.mintlify.app) and its section 4.4 (expert
// replication):
//
// * defer to a later round -- an assignment past its expert's capacity keeps
//   its expert and is processed in a later round: the i-th assignment of
//   local expert e (assignment order a = t * k + j, from 0) goes to round
//   i / C; rounds past the last are dropped. Rows are laid out round after
//   round and, inside a round, expert after expert, so each round is one
//   grouped FFN call over its own offsets and one combine covers them all.
// * send to a same-weight replica -- the i-th assignment of logical expert e
//   goes to its replica i / C (the replicas in the order the placement lists
//   them, each with room for C), or is dropped past the last one.
//
// Both need the rank of each assignment among its expert's assignments: the
// stable dropless dispatch gives it (row - the expert's first row).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Block-wide exclusive scan of one int per thread (1024 threads); *total gets the sum.
__device__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, MOE_WAVE);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int i = 0; i < nw; ++i) {
    const int s = wsum[i];
    if (i < w) before += s;
    all += s;
  }
  __syncthreads();  // wsum is reused by the next scan
  *total = all;
  return before + incl - v;
}

// One workgroup of 1024 threads, thread e = local expert e (num_local <= 1024):
// round r takes min(max(demand_e - r C, 0), C) rows of expert e; offsets run
// over (round, expert) in that order.
__global__ __launch_bounds__(1024) void rounds_plan_kernel(const int* __restrict__ demand_in, int nloc, int cap,
                                                           int rounds, int* __restrict__ round_counts,
                                                           int* __restrict__ round_offsets,
                                                           int* __restrict__ demand_out) {
  __shared__ int wsum[16];
  const int e = threadIdx.x;
  const int dem = e < nloc ? demand_in[e] : 0;
  if (demand_out && e < nloc) demand_out[e] = dem;
  int base = 0;
  for (int r = 0; r < rounds; ++r) {
    const long left = (long)dem - (long)r * cap;
    const int c = (e < nloc && left > 0) ? (int)(left < cap ? left : cap) : 0;
    int total;
    const int excl = block_exclusive_scan(c, wsum, &total);
    if (e < nloc) {
      round_counts[(size_t)r * nloc + e] = c;
      round_offsets[(size_t)r * (nloc + 1) + e] = base + excl;
    }
    if (e == 0) round_offsets[(size_t)r * (nloc + 1) + nloc] = base + total;
    base += total;
  }
}

// One thread per row i of the dropless layout (rows [0, off_full[nloc])):
// its expert e (binary search in off_full, kept in LDS), rank r = i -
// off_full[e], round r / cap; the assignment moves to its row in that round,
// or is dropped past the last round.
__global__ __launch_bounds__(256) void rounds_scatter_kernel(const int* __restrict__ sorted_full,
                                                             const int* __restrict__ off_full, int nloc, int cap,
                                                             int rounds, const int* __restrict__ round_offsets,
                                                             int* __restrict__ sorted_assign,
                                                             int* __restrict__ assign_pos) {
  extern __shared__ int s_off[];  // [nloc + 1]
  for (int i = threadIdx.x; i <= nloc; i += blockDim.x) s_off[i] = off_full[i];
  __syncthreads();
  const int M = s_off[nloc];
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < M; i += gridDim.x * blockDim.x) {
    int lo = 0, hi = nloc - 1;  // the expert e with s_off[e] <= i < s_off[e + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int r = i - s_off[lo];
    const int round = cap > 0 ? r / cap : rounds;
    const int a = sorted_full[i];
    if (round < rounds) {
      const int row = round_offsets[(size_t)round * (nloc + 1) + lo] + (r - round * cap);
      sorted_assign[row] = a;
      assign_pos[a] = row;
    } else {
      assign_pos[a] = -1;
    }
  }
}

// One thread per assignment a: logical expert e = ids[a], its rank among e's
// assignments from the dropless dispatch over all experts, replica rank / cap.
__global__ __launch_bounds__(256) void remap_capacity_kernel(const int* __restrict__ ids, int n, int E, int cap,
                                                             const int* __restrict__ rep_off,
                                                             const int* __restrict__ rep_slots,
                                                             const int* __restrict__ off_full,
                                                             const int* __restrict__ pos_full,
                                                             int* __restrict__ phys) {
  for (int a = blockIdx.x * blockDim.x + threadIdx.x; a < n; a += gridDim.x * blockDim.x) {
    const int e = ids[a];
    int out = -1;
    if ((unsigned)e < (unsigned)E) {
      const int r0 = rep_off[e], nrep = rep_off[e + 1] - r0;
      const int rank = pos_full[a] - off_full[e];
      const int rep = cap > 0 ? rank / cap : nrep;
      if (rep < nrep) out = rep_slots[r0 + rep];
    }
    phys[a] = out;
  }
}

int grid_for(long items) { return (int)std::max<long>(1, std::min<long>((items + 255) / 256, 4096)); }

}  // namespace

// Workspace: the dropless dispatch's own, then its counts [nloc], offsets
// [nloc + 1] and rows [n].
size_t deferred_workspace_size(int n, int num_local) {
  return align256(dispatch_workspace_size(n, num_local)) + align256((size_t)num_local * 4) +
         align256((size_t)(num_local + 1) * 4) + align256((size_t)std::max(n, 1) * 4);
}

hipError_t launch_dispatch_deferred(const DeferredArgs& a, hipStream_t s) {
  char* ws = (char*)a.workspace;
  void* dws = ws;
  ws += align256(dispatch_workspace_size(a.n, a.num_local));
  int* counts_full = (int*)ws;
  ws += align256((size_t)a.num_local * 4);
  int* off_full = (int*)ws;
  ws += align256((size_t)(a.num_local + 1) * 4);
  int* sorted_full = (int*)ws;
  // the dropless dispatch writes assign_pos = -1 for the assignments of other
  // GPUs' experts; the scatter overwrites every local one
  DispatchArgs d{a.ids, a.n, a.k, a.expert_begin, a.num_local, counts_full, off_full, sorted_full,
                 a.assign_pos, nullptr, nullptr, 0, dws, INT32_MAX, nullptr, 0};
  hipError_t err = launch_dispatch(d, s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(rounds_plan_kernel, dim3(1), dim3(1024), 0, s, counts_full, a.num_local, a.capacity,
                     a.rounds, a.round_counts, a.round_offsets, a.demand);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.n > 0) {
    hipLaunchKernelGGL(rounds_scatter_kernel, dim3(grid_for(a.n)), dim3(256), (size_t)(a.num_local + 1) * 4,
                       s, sorted_full, off_full, a.num_local, a.capacity, a.rounds, a.round_offsets,
                       a.sorted_assign, a.assign_pos);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return launch_gather_rows(a.x, a.sorted_assign, a.round_offsets + (size_t)(a.rounds - 1) * (a.num_local + 1),
                            a.num_local, a.k, a.n, a.row_bytes, a.x_sorted, s);
}

// Workspace: the dropless dispatch's own, then its counts [E], offsets
// [E + 1], rows [n] and positions [n].
size_t remap_capacity_workspace_size(int n, int num_experts) {
  return align256(dispatch_workspace_size(n, num_experts)) + align256((size_t)num_experts * 4) +
         align256((size_t)(num_experts + 1) * 4) + 2 * align256((size_t)std::max(n, 1) * 4);
}

hipError_t launch_remap_capacity(const RemapCapacityArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  char* ws = (char*)a.workspace;
  void* dws = ws;
  ws += align256(dispatch_workspace_size(a.n, a.num_experts));
  int* counts = (int*)ws;
  ws += align256((size_t)a.num_experts * 4);
  int* off = (int*)ws;
  ws += align256((size_t)(a.num_experts + 1) * 4);
  int* sorted = (int*)ws;
  ws += align256((size_t)a.n * 4);
  int* pos = (int*)ws;
  DispatchArgs d{a.ids, a.n, 1, 0, a.num_experts, counts, off, sorted, pos, nullptr, nullptr, 0, dws,
                 INT32_MAX, nullptr, 0};
  hipError_t err = launch_dispatch(d, s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(remap_capacity_kernel, dim3(grid_for(a.n)), dim3(256), 0, s, a.ids, a.n, a.num_experts,
                     a.capacity, a.rep_offsets, a.rep_slots, off, pos, a.phys);
  return hipGetLastError();
}

}  // namespace moe
