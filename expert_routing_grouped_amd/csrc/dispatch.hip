// Dispatch: stable counting sort of assignments to local experts, then a row
// gather of the token activations into expert order.
//
// The dispatch step of ch15 section 3.4 ("第十五章：多节点大模型推理", se7en.mintlify.app)
// on one GPU: each token's activation goes to the rows of its experts. Rows of
// one expert keep assignment order a = t * k + j, so the result is unique and
// equals a stable sort by expert.
//
// Sort kernel: one workgroup of 16 wavefronts. Wave w owns a contiguous chunk
// of assignments and walks it 64 at a time. Pass 1 counts per (wave, expert)
// in LDS (an integer atomic add per assignment); a scan turns the counts into
// per-(wave, expert) rank bases (assignments of the expert in earlier waves)
// and per-expert offsets; pass 2 re-walks the chunk: lanes holding the same
// expert are found with ballots (a wave-wide "match": one ballot per distinct
// expert present when few lanes hold a local one, else one per key bit), which
// gives each lane its rank among equal keys in the step, and the lowest lane
// of each key group advances the wave's base for the next step. Each
// assignment goes to offset + rank. Integer arithmetic only, and the ranks
// follow assignment order: bit-for-bit deterministic.
//
// With a per-expert capacity C (the capacity factor of ch15 section 4.3,
// drop policy) an expert keeps the assignments of rank < C, i.e. its first C
// in assignment order; the offsets are the prefix sums of min(count, C) and a
// dropped assignment gets assign_pos = -1, like a non-local one. In the fixed
// slot ("masked") layout expert e's rows start at e * C instead of at the
// prefix sum, and no offsets are written.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kSortWaves = 16;
constexpr int kSingleBlockMax = 8192;  // larger T*k uses the multi-workgroup sort

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

// The same masks for the lanes of `act` (non-negative keys), one ballot per
// distinct key present: cheaper than a ballot per key bit when few lanes
// hold a local expert (under expert parallelism about E_loc / E of the
// assignments are local).
__device__ __forceinline__ uint64_t match_few(int key, uint64_t act) {
  uint64_t m = 0ull;
  while (act) {
    const int k = __builtin_amdgcn_readlane(key, __ffsll((unsigned long long)act) - 1);
    const uint64_t mk = __ballot(key == k) & act;
    if (key == k) m = mk;
    act &= ~mk;
  }
  return m;
}

constexpr int kFewKeys = 8;   // lanes with a local expert up to which match_few is used

// Masks of equal local experts (e >= 0) in one 64-id group.
__device__ __forceinline__ uint64_t match_local(int e, int nbits) {
  const uint64_t act = __ballot(e >= 0);
  return __popcll(act) <= kFewKeys ? match_few(e, act) : match_key(e, e >= 0, nbits);
}

// Inclusive prefix sum over the 64 lanes with DPP: row_shr 1, 2, 4, 8 inside
// each row of 16 lanes (lanes whose source lies before the row start add 0),
// then row_bcast:15 adds the last lane of rows 0 and 2 to rows 1 and 3, and
// row_bcast:31 adds lane 31 to rows 2 and 3 (gfx9 DPP controls).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  return v;
}

// Ids are read kBatch groups of 64 at a time: all of a batch's loads are in
// flight before the first is used.
constexpr int kBatch = 8;

// Local expert of assignment a (-1 if a >= hi or its expert is not local),
// for the kBatch groups of 64 starting at base.
__device__ __forceinline__ void load_batch(const int* __restrict__ ids, int base, int hi, int begin,
                                           int nloc, int (&ev)[kBatch]) {
  const int lane = threadIdx.x & 63;
  int raw[kBatch];
#pragma unroll
  for (int g = 0; g < kBatch; ++g) {
    const int a = base + g * 64 + lane;
    raw[g] = a < hi ? ids[a] - begin : -1;
  }
#pragma unroll
  for (int g = 0; g < kBatch; ++g) ev[g] = (unsigned)raw[g] < (unsigned)nloc ? raw[g] : -1;
}

// Counts one wavefront's assignments [lo, hi) per local expert into my_cnt
// (this wavefront's LDS row): each lane with a local expert adds 1 with an
// LDS atomic (integer sums: the result does not depend on their order).
__device__ __forceinline__ void wave_count(const int* __restrict__ ids, int lo, int hi, int begin,
                                           int nloc, int* my_cnt) {
  for (int base = lo; base < hi; base += 64 * kBatch) {
    int ev[kBatch];
    load_batch(ids, base, hi, begin, nloc, ev);
#pragma unroll
    for (int g = 0; g < kBatch; ++g)
      if (ev[g] >= 0) atomicAdd(&my_cnt[ev[g]], 1);
  }
}

// Writes one wavefront's assignments [lo, hi) in order: assignment a with
// local expert e has rank r = my_base[e] + (earlier assignments of e in this
// wavefront's range) and goes to ebase[e] + r when r < cap. Non-local and
// dropped assignments get assign_pos = -1. Per 64-id group the lowest lane of
// each key group advances my_base[e] by the group's size with an LDS atomic
// that returns the old value, and the other lanes of the key group read it
// from that lane. A wavefront's LDS operations execute in issue order, so the
// ranks follow assignment order; the batch's atomics are all issued before
// the first result is used.
__device__ __forceinline__ void wave_scatter(const int* __restrict__ ids, int lo, int hi, int begin,
                                             int nloc, int nbits, int* my_base, const int* ebase,
                                             int cap, int* __restrict__ sorted_assign,
                                             int* __restrict__ assign_pos) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  for (int base = lo; base < hi; base += 64 * kBatch) {
    int ev[kBatch];
    load_batch(ids, base, hi, begin, nloc, ev);
    uint64_t peers[kBatch];
    int old[kBatch];
#pragma unroll
    for (int g = 0; g < kBatch; ++g) {
      peers[g] = match_local(ev[g], nbits);
      old[g] = 0;
      if (ev[g] >= 0 && (peers[g] & lt_mask) == 0ull) old[g] = atomicAdd(&my_base[ev[g]], __popcll(peers[g]));
    }
#pragma unroll
    for (int g = 0; g < kBatch; ++g) {
      const int a = base + g * 64 + lane;
      const int e = ev[g];
      const int first = e >= 0 ? __ffsll((unsigned long long)peers[g]) - 1 : lane;
      const int b0 = __shfl(old[g], first, MOE_WAVE);
      if (a < hi) {
        const int r = e >= 0 ? b0 + __popcll(peers[g] & lt_mask) : cap;
        if (r < cap) {
          const int p = ebase[e] + r;
          sorted_assign[p] = a;
          assign_pos[a] = p;
        } else {
          assign_pos[a] = -1;
        }
      }
    }
  }
}

// ---- multi-workgroup sort (large T*k), three passes: block b owns
// assignments [b*per_block, (b+1)*per_block), wavefront w a quarter of that.
// per_block is 1024 until the block count reaches kMaxBlocks, then grows.
// ws holds [nblocks][nloc] ints, then the experts' totals [nloc].
// 1. block_count_kernel: per-block counts per local expert -> ws[b][e].
// 2. block_scan_kernel (a workgroup per 64 experts): ws[b][e] becomes the
//    expert's assignments in blocks before b; the totals are written.
// 3. block_scatter_kernel: each block reads its row of ws and the totals,
//    scans the kept rows over the experts (block 0 writes counts, offsets and
//    demand), recounts its wavefronts and scatters.
constexpr int kBlkWaves = 4;
constexpr int kBlkElems = kBlkWaves * 256;
constexpr int kMaxBlocks = 256;

__host__ __device__ inline int sort_blocks(int n) {
  const int b = (n + kBlkElems - 1) / kBlkElems;
  return b < kMaxBlocks ? b : kMaxBlocks;
}
// Assignments per block: a multiple of 256 so each wavefront's quarter is a
// whole number of 64-lane steps.
__host__ __device__ inline int sort_per_block(int n) {
  const int b = sort_blocks(n);
  const long per = ((long)n + b - 1) / b;
  return (int)((per + 255) & ~255L);
}

__global__ __launch_bounds__(256) void block_count_kernel(const int* __restrict__ ids, int n,
                                                          int per_block, int begin, int nloc,
                                                          int* __restrict__ ws) {
  extern __shared__ int lds[];
  int* cnt = lds;  // [kBlkWaves][nloc]
  const int w = threadIdx.x >> 6, b = blockIdx.x;
  for (int i = threadIdx.x; i < kBlkWaves * nloc; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  const int per_wave = per_block / kBlkWaves;
  const int lo = (int)min((long)n, (long)b * per_block + (long)w * per_wave);
  const int hi = (int)min((long)n, (long)lo + per_wave);
  wave_count(ids, lo, hi, begin, nloc, cnt + w * nloc);
  __syncthreads();
  for (int e = threadIdx.x; e < nloc; e += blockDim.x) {
    int c = 0;
    for (int ww = 0; ww < kBlkWaves; ++ww) c += cnt[ww * nloc + e];
    ws[(size_t)b * nloc + e] = c;
  }
}

// Workgroup j takes experts [64 j, 64 j + 64), lane = expert; wavefront q takes
// the q-th quarter of the blocks, so each load reads 64 consecutive experts of
// one block. Pass 1 sums a quarter (kScanBatch loads in flight), the quarter
// sums give each quarter's start, pass 2 re-reads the quarter and writes the
// exclusive prefix over the blocks in place.
constexpr int kScanBatch = 16;

__global__ __launch_bounds__(256) void block_scan_kernel(int* __restrict__ ws, int nblocks, int nloc) {
  __shared__ int qsum[kBlkWaves][64];
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int nq = (nblocks + kBlkWaves - 1) / kBlkWaves;
  const int b_lo = min(nblocks, q * nq), b_hi = min(nblocks, b_lo + nq);
  int sum = 0;
  if (e < nloc) {
    for (int b0 = b_lo; b0 < b_hi; b0 += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) c[i] = b0 + i < b_hi ? ws[(size_t)(b0 + i) * nloc + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) sum += c[i];
    }
  }
  qsum[q][lane] = sum;
  __syncthreads();
  int run = 0;
  for (int qq = 0; qq < q; ++qq) run += qsum[qq][lane];
  if (e < nloc) {
    for (int b0 = b_lo; b0 < b_hi; b0 += kScanBatch) {
      int c[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) c[i] = b0 + i < b_hi ? ws[(size_t)(b0 + i) * nloc + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) {
        if (b0 + i < b_hi) ws[(size_t)(b0 + i) * nloc + e] = run;
        run += c[i];
      }
    }
    if (q == kBlkWaves - 1) ws[(size_t)nblocks * nloc + e] = run;   // the expert's total
  }
}

// Rank bases per (wave, expert): the expert's assignments in earlier blocks
// (the scan) plus those in this block's earlier wavefronts (the recount). The
// expert offsets come from an exclusive scan of min(total, cap) over the
// experts, four per thread (the same sums in every block).
__global__ __launch_bounds__(256) void block_scatter_kernel(
    const int* __restrict__ ids, int n, int per_block, int begin, int nloc, int nbits,
    const int* __restrict__ ws, int nblocks, int cap, int fixed, int* __restrict__ counts,
    int* __restrict__ offsets, int* __restrict__ demand, int* __restrict__ sorted_assign,
    int* __restrict__ assign_pos) {
  extern __shared__ int lds[];
  int* cnt = lds;                          // [kBlkWaves][nloc]
  int* wsum = lds + kBlkWaves * nloc;      // [4]
  int* ebase = wsum + 4;                   // [nloc] expert first rows
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, b = blockIdx.x;
  for (int i = tid; i < kBlkWaves * nloc; i += blockDim.x) cnt[i] = 0;
  // this block's row of bases and the totals of experts tid*4 .. tid*4+3
  int tot[4], before[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    tot[q] = e < nloc ? ws[(size_t)nblocks * nloc + e] : 0;
    before[q] = e < nloc ? ws[(size_t)b * nloc + e] : 0;
  }
  __syncthreads();
  const int per_wave = per_block / kBlkWaves;
  const int lo = (int)min((long)n, (long)b * per_block + (long)w * per_wave);
  const int hi = (int)min((long)n, (long)lo + per_wave);
  wave_count(ids, lo, hi, begin, nloc, cnt + w * nloc);
#pragma unroll
  for (int q = 0; q < 4; ++q) sum += min(tot[q], cap);   // rows kept
  const int incl = wave_inclusive_scan(sum);
  if (lane == 63) wsum[w] = incl;
  __syncthreads();  // also orders the recount above before the reads below
  int run = incl - sum;
  for (int i = 0; i < w; ++i) run += wsum[i];
  int total = 0;
  for (int i = 0; i < 4; ++i) total += wsum[i];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    if (e < nloc) {
      if (b == 0) {
        counts[e] = min(tot[q], cap);
        if (offsets) offsets[e] = run;
        if (demand) demand[e] = tot[q];
      }
      ebase[e] = fixed ? e * cap : run;
      int c[kBlkWaves], s = before[q];
#pragma unroll
      for (int ww = 0; ww < kBlkWaves; ++ww) c[ww] = cnt[ww * nloc + e];
#pragma unroll
      for (int ww = 0; ww < kBlkWaves; ++ww) {
        cnt[ww * nloc + e] = s;
        s += c[ww];
      }
    }
    run += min(tot[q], cap);
  }
  if (b == 0 && tid == 0 && offsets) offsets[nloc] = total;
  __syncthreads();
  wave_scatter(ids, lo, hi, begin, nloc, nbits, cnt + w * nloc, ebase, cap, sorted_assign,
               assign_pos);
}

// Single-workgroup sort (n <= kSingleBlockMax): each wavefront's chunk is
// loaded once, all its 64-id groups at a time, and kept in registers (local
// expert and the mask of equal keys) for both the count and the scatter pass.
constexpr int kSortGroups = kSingleBlockMax / kSortWaves / 64;   // 64-id groups per wavefront

__global__ __launch_bounds__(1024) void sort_kernel(const int* __restrict__ ids, int n, int begin,
                                                    int nloc, int nbits, int cap, int fixed,
                                                    int* __restrict__ counts,
                                                    int* __restrict__ offsets,
                                                    int* __restrict__ demand,
                                                    int* __restrict__ sorted_assign,
                                                    int* __restrict__ assign_pos) {
  extern __shared__ int lds[];
  int* cnt = lds;                              // [kSortWaves][nloc]
  int* wbase = lds + kSortWaves * nloc;        // [kSortWaves]
  int* ebase = wbase + kSortWaves;             // [nloc] expert offsets
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  for (int i = threadIdx.x; i < kSortWaves * nloc; i += blockDim.x) cnt[i] = 0;

  const int per_wave = (((n + kSortWaves - 1) / kSortWaves) + 63) & ~63;   // <= 64 * kSortGroups
  const int lo = min(n, w * per_wave), hi = min(n, lo + per_wave);
  const int ng = (hi - lo + 63) >> 6;   // 64-id groups holding this wavefront's chunk (uniform)
  int* my_cnt = cnt + w * nloc;

  // load the chunk: one id per lane and group
  int raw[kSortGroups];
#pragma unroll
  for (int g = 0; g < kSortGroups; ++g) {
    const int a = lo + g * 64 + lane;
    raw[g] = a < hi ? ids[a] - begin : -1;
  }
  int ev[kSortGroups];
#pragma unroll
  for (int g = 0; g < kSortGroups; ++g) ev[g] = (unsigned)raw[g] < (unsigned)nloc ? raw[g] : -1;
  __syncthreads();  // counters cleared

  // pass 1: counts per (wave, expert), one LDS atomic add of 1 per lane with a
  // local expert (integer sums: the result does not depend on their order)
#pragma unroll
  for (int g = 0; g < kSortGroups; ++g) {
    if (g >= ng) break;
    if (ev[g] >= 0) atomicAdd(&my_cnt[ev[g]], 1);
  }
  __syncthreads();

  // scan: per-expert column prefix over waves (the wave rank bases; the
  // column is read into registers first), then an exclusive scan over
  // experts of the rows kept
  int total = 0;
  for (int e = threadIdx.x; e < nloc; e += blockDim.x) {  // nloc <= blockDim.x: one expert per thread
    int c[kSortWaves];
#pragma unroll
    for (int ww = 0; ww < kSortWaves; ++ww) c[ww] = cnt[ww * nloc + e];
#pragma unroll
    for (int ww = 0; ww < kSortWaves; ++ww) {
      cnt[ww * nloc + e] = total;
      total += c[ww];
    }
  }
  const int kept = min(total, cap);
  const int incl = wave_inclusive_scan(kept);
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
    const int excl = incl - kept + wbase[w];
    if (e < nloc) {
      counts[e] = kept;
      if (offsets) offsets[e] = excl;
      ebase[e] = fixed ? e * cap : excl;
      if (demand) demand[e] = total;
      if (e == nloc - 1 && offsets) offsets[nloc] = excl + kept;
    }
  }
  __syncthreads();

  // pass 2: scatter in chunk order. Per group the lowest lane of each key
  // group advances the wave's rank base with an LDS atomic that returns the
  // old value, which the key group's other lanes read from it; a wavefront's
  // LDS operations execute in issue order, so the ranks follow assignment
  // order. All groups' atomics go out before the first result is used.
  uint64_t peers[kSortGroups];
  int old[kSortGroups];
#pragma unroll
  for (int g = 0; g < kSortGroups; ++g) {
    if (g >= ng) break;
    peers[g] = match_local(ev[g], nbits);
    old[g] = 0;
    if (ev[g] >= 0 && (peers[g] & lt_mask) == 0ull) old[g] = atomicAdd(&my_cnt[ev[g]], __popcll(peers[g]));
  }
#pragma unroll
  for (int g = 0; g < kSortGroups; ++g) {
    if (g >= ng) break;
    const int a = lo + g * 64 + lane;
    const int e = ev[g];
    const int first = e >= 0 ? __ffsll((unsigned long long)peers[g]) - 1 : lane;
    const int b0 = __shfl(old[g], first, MOE_WAVE);
    if (a < hi) {
      const int r = e >= 0 ? b0 + __popcll(peers[g] & lt_mask) : cap;
      if (r < cap) {
        const int p = ebase[e] + r;
        sorted_assign[p] = a;
        assign_pos[a] = p;
      } else {
        assign_pos[a] = -1;
      }
    }
  }
}

__global__ void zero_counts_kernel(int nloc, int* counts, int* offsets, int* demand) {
  for (int e = threadIdx.x; e <= nloc; e += blockDim.x) {
    if (e < nloc) {
      counts[e] = 0;
      if (demand) demand[e] = 0;
    }
    if (offsets) offsets[e] = 0;
  }
}

// Fixed-slot layout: one wavefront per slot row r of the num_local x cap
// block; rows past their expert's count are left untouched.
__global__ __launch_bounds__(256) void gather_slots_kernel(const uint4* __restrict__ x,
                                                           const int* __restrict__ slot_assign,
                                                           const int* __restrict__ counts, int nloc,
                                                           int cap, int k, int row_vec,
                                                           uint4* __restrict__ x_slots) {
  const int lane = threadIdx.x & 63;
  const long rows = (long)nloc * cap;
  for (long r = (long)blockIdx.x * 4 + (threadIdx.x >> 6); r < rows; r += (long)gridDim.x * 4) {
    const int e = (int)(r / cap);
    if ((int)(r - (long)e * cap) >= counts[e]) continue;
    const int t = slot_assign[r] / k;
    const uint4* src = x + (size_t)t * row_vec;
    uint4* dst = x_slots + (size_t)r * row_vec;
    for (int c = lane; c < row_vec; c += 64) dst[c] = src[c];
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

size_t dispatch_workspace_size(int n, int num_local) {
  if (n <= kSingleBlockMax) return 0;
  return ((size_t)sort_blocks(n) + 1) * num_local * sizeof(int);
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  if (a.n == 0) {
    hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(256), 0, s, a.num_local, a.counts,
                       a.offsets, a.demand);
    return hipGetLastError();
  }
  int nbits = 1;
  while ((1 << nbits) < a.num_local) ++nbits;
  if (a.n <= kSingleBlockMax) {
    const size_t lds = (size_t)((kSortWaves + 1) * a.num_local + kSortWaves) * sizeof(int);
    hipLaunchKernelGGL(sort_kernel, dim3(1), dim3(kSortWaves * 64), lds, s, a.ids, a.n,
                       a.expert_begin, a.num_local, nbits, a.capacity, a.fixed_slots, a.counts,
                       a.offsets, a.demand, a.sorted_assign, a.assign_pos);
  } else {
    const int blocks = sort_blocks(a.n), per_block = sort_per_block(a.n);
    const size_t lds = (size_t)kBlkWaves * a.num_local * sizeof(int);
    hipLaunchKernelGGL(block_count_kernel, dim3(blocks), dim3(256), lds, s, a.ids, a.n, per_block,
                       a.expert_begin, a.num_local, (int*)a.workspace);
    hipLaunchKernelGGL(block_scan_kernel, dim3((a.num_local + 63) / 64), dim3(256), 0, s, (int*)a.workspace,
                       blocks, a.num_local);
    const size_t lds2 = lds + (size_t)(a.num_local + 4) * sizeof(int);
    hipLaunchKernelGGL(block_scatter_kernel, dim3(blocks), dim3(256), lds2, s, a.ids, a.n,
                       per_block, a.expert_begin, a.num_local, nbits, (const int*)a.workspace,
                       blocks, a.capacity, a.fixed_slots, a.counts, a.offsets, a.demand,
                       a.sorted_assign, a.assign_pos);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.row_bytes == 0) return err;
  const int row_vec = a.row_bytes / 16;
  if (a.fixed_slots) {
    const long rows = (long)a.num_local * a.capacity;
    if (rows == 0) return hipSuccess;
    const int blocks = (int)std::min<long>((rows + 3) / 4, 2048);
    hipLaunchKernelGGL(gather_slots_kernel, dim3(blocks), dim3(256), 0, s, (const uint4*)a.x,
                       a.sorted_assign, a.counts, a.num_local, a.capacity, a.k, row_vec,
                       (uint4*)a.x_sorted);
    return hipGetLastError();
  }
  const int blocks = (int)std::min<long>((a.n + 3) / 4, 2048);
  hipLaunchKernelGGL(gather_kernel, dim3(blocks), dim3(256), 0, s, (const uint4*)a.x,
                     a.sorted_assign, a.offsets, a.num_local, a.k, a.n, row_vec,
                     (uint4*)a.x_sorted);
  return hipGetLastError();
}

// Row gather for rows laid out by another pass (the deferred dispatch): rows
// [0, end[num_local]) of x_sorted from sorted_assign.
hipError_t launch_gather_rows(const void* x, const int* sorted_assign, const int* end, int num_local, int k,
                              int n, int row_bytes, void* x_sorted, hipStream_t s) {
  if (n == 0 || row_bytes == 0) return hipSuccess;
  const int blocks = (int)std::min<long>(((long)n + 3) / 4, 2048);
  hipLaunchKernelGGL(gather_kernel, dim3(blocks), dim3(256), 0, s, (const uint4*)x, sorted_assign, end,
                     num_local, k, n, row_bytes / 16, (uint4*)x_sorted);
  return hipGetLastError();
}

}  // namespace moe
