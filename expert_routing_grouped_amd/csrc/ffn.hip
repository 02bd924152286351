// Grouped SwiGLU expert FFN over the permuted rows.
//
// Per local expert e (rows [off[e], off[e+1]) of x_sorted):
//   [g | u] = X_e W_gate_up[e]^T      fused gate_up GEMM, N = 2I
//   h       = silu(g) * u             fused into the GEMM-1 epilogue
//   o       = h W_down[e]^T           GEMM-2
// The gated MLP (W_gate, W_up, W_down) is the one of section 2.2 of "Lecture 6
// · 并行" (semidirectx.com, cs349d lecture06); the fused gate_up GEMM with
// N = 2I and the skipping of experts that no token reaches come from the page
// "推理 INFRA 方法论（2）：分布式推理：TP、DP、EP、CP 与 PP" (johneyzheng.top).
//
// Scheduling: a one-workgroup plan kernel turns expert_offsets into a list of
// row tiles (expert, first row), so the number of rows never returns to the
// host; GEMM workgroups whose tile index is past the list end exit at once,
// and experts with no rows have no tiles, so their weights are never read.
//
// bf16 GEMMs use v_mfma_f32_16x16x32_bf16 (fp32 accumulate) on LDS tiles that
// are double-buffered through registers. Both operands are K-contiguous
// (activations [rows, K], weights [N, K]), so A and B fragments are the same
// kind of 16-byte LDS read. For GEMM-1 a workgroup's weight tile takes BN/2
// gate rows and the matching BN/2 up rows, arranged so that one lane holds
// g and u of the same output element; SiLU*up is applied before h is stored.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kBfBM = 64;   // rows per tile, bf16 path
constexpr int kF32BM = 16;  // rows per tile, f32 path

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------- plan

__global__ __launch_bounds__(1024) void plan_kernel(const int* __restrict__ offsets, int nloc,
                                                    int capacity, int bm,
                                                    int* __restrict__ num_tiles,
                                                    int* __restrict__ tile_expert,
                                                    int* __restrict__ tile_row0) {
  __shared__ int wsum[16];
  const int e = threadIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int lo = 0, n = 0;
  if (e < nloc) {
    lo = min(offsets[e], capacity);
    const int hi = min(offsets[e + 1], capacity);
    n = hi > lo ? (hi - lo + bm - 1) / bm : 0;
  }
  int incl = n;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, MOE_WAVE);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += wsum[i];
  const int start = base + incl - n;
  for (int i = 0; i < n; ++i) {
    tile_expert[start + i] = e;
    tile_row0[start + i] = lo + i * bm;
  }
  if (e == blockDim.x - 1) num_tiles[0] = base + incl;
}

// ---------------------------------------------------------------- bf16 MFMA GEMM

template <int BM, int BN, int BK, int WM, int WN, bool GATED>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const int* __restrict__ offsets, int capacity,
    const int* __restrict__ num_tiles, const int* __restrict__ tile_expert,
    const int* __restrict__ tile_row0, const uint16_t* __restrict__ W, int N, int K, int inter,
    uint16_t* __restrict__ C, int ldc) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  constexpr int LDK = BK + 8;  // padded LDS row (elements): spreads rows over banks
  constexpr int CPR = BK / 8;  // 16-byte chunks per tile row
  constexpr int A_CH = BM * CPR / NT, B_CH = BN * CPR / NT;
  static_assert(A_CH * NT == BM * CPR && B_CH * NT == BN * CPR, "tile/thread mismatch");
  static_assert(!GATED || TN % 2 == 0, "gated tiles pair gate and up fragments");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDK];

  const int tile = blockIdx.y;
  if (tile >= num_tiles[0]) return;
  const int e = tile_expert[tile];
  const int row0 = tile_row0[tile];
  const int rows = min(BM, min(offsets[e + 1], capacity) - row0);
  const uint16_t* We = W + (size_t)e * N * K;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  constexpr int HALF = TN * 8;  // gate (or up) columns per wave in a gated tile

  // Weight row held by LDS tile row r. Gated tiles: wave column ww owns HALF
  // gate rows followed by the HALF up rows of the same output columns.
  const int gate0 = blockIdx.x * (BN / 2);
  int b_row[B_CH], b_kc[B_CH], a_row[A_CH], a_kc[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + i * NT;
    a_row[i] = c / CPR;
    a_kc[i] = (c % CPR) * 8;
  }
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + i * NT, r = c / CPR;
    b_kc[i] = (c % CPR) * 8;
    if (GATED) {
      const int ww = r / (TN * 16), rem = r % (TN * 16);
      b_row[i] = rem < HALF ? gate0 + ww * HALF + rem : inter + gate0 + ww * HALF + rem - HALF;
    } else {
      b_row[i] = blockIdx.x * BN + r;
    }
  }

  u32x4_t ra[A_CH], rb[B_CH];
#define MOE_GLOAD(k0)                                                                         \
  do {                                                                                        \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i) ra[i] =                                  \
        a_row[i] < rows ? *(const u32x4_t*)(A + (size_t)(row0 + a_row[i]) * K + (k0) + a_kc[i]) \
                        : u32x4_t{0u, 0u, 0u, 0u};                                         \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i) rb[i] =                                  \
        *(const u32x4_t*)(We + (size_t)b_row[i] * K + (k0) + b_kc[i]);                          \
  } while (0)
#define MOE_SSTORE(buf)                                                                                  \
  do {                                                                                                   \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i) *(u32x4_t*)&As[buf][(tid + i * NT) / CPR * LDK + a_kc[i]] = ra[i]; \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i) *(u32x4_t*)&Bs[buf][(tid + i * NT) / CPR * LDK + b_kc[i]] = rb[i]; \
  } while (0)

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  MOE_GLOAD(0);
  MOE_SSTORE(0);
  __syncthreads();
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) MOE_GLOAD((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8_t a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *(const bf16x8_t*)&As[buf][(wm * TM * 16 + i * 16 + fr) * LDK + ks * 32 + fk];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *(const bf16x8_t*)&Bs[buf][(wn * TN * 16 + j * 16 + fr) * LDK + ks * 32 + fk];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) MOE_SSTORE(buf ^ 1);
    __syncthreads();
  }

#undef MOE_GLOAD
#undef MOE_SSTORE

  // Epilogue. Lane holds rows 4*(lane/16) + r, column lane % 16 of each 16x16 fragment.
  const int rq = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wm * TM * 16 + i * 16 + rq + r;
      if (row >= rows) continue;
      uint16_t* crow = C + (size_t)(row0 + row) * ldc;
      if (GATED) {
        const int n0 = blockIdx.x * (BN / 2) + wn * HALF;
#pragma unroll
        for (int j = 0; j < TN / 2; ++j) {
          const float g = acc[i][j][r], u = acc[i][j + TN / 2][r];
          crow[n0 + j * 16 + fr] = (uint16_t)f32_to_bf16_bits(silu(g) * u);
        }
      } else {
        const int n0 = blockIdx.x * BN + wn * TN * 16;
#pragma unroll
        for (int j = 0; j < TN; ++j) crow[n0 + j * 16 + fr] = (uint16_t)f32_to_bf16_bits(acc[i][j][r]);
      }
    }
  }
}

// ---------------------------------------------------------------- f32 GEMM (small shapes)

// 16 rows x 16 output columns per workgroup, plain FMA; bounds-checked in N and K.
template <bool GATED>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, const int* __restrict__ offsets, int capacity,
    const int* __restrict__ num_tiles, const int* __restrict__ tile_expert,
    const int* __restrict__ tile_row0, const float* __restrict__ W, int N, int K, int inter,
    float* __restrict__ C, int ldc) {
  __shared__ float As[16][17], Bg[16][17], Bu[16][17];
  const int tile = blockIdx.y;
  if (tile >= num_tiles[0]) return;
  const int e = tile_expert[tile];
  const int row0 = tile_row0[tile];
  const int rows = min(16, min(offsets[e + 1], capacity) - row0);
  const int n_out = GATED ? inter : N;
  const float* We = W + (size_t)e * N * K;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int col0 = blockIdx.x * 16;
  float g = 0.f, u = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int kk = k0 + tx;
    As[ty][tx] = (ty < rows && kk < K) ? A[(size_t)(row0 + ty) * K + kk] : 0.f;
    const int n = col0 + ty;
    Bg[ty][tx] = (n < n_out && kk < K) ? We[(size_t)n * K + kk] : 0.f;
    if (GATED) Bu[ty][tx] = (n < n_out && kk < K) ? We[(size_t)(inter + n) * K + kk] : 0.f;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      g += As[ty][q] * Bg[tx][q];
      if (GATED) u += As[ty][q] * Bu[tx][q];
    }
    __syncthreads();
  }
  const int col = col0 + tx;
  if (ty < rows && col < n_out) C[(size_t)(row0 + ty) * ldc + col] = GATED ? silu(g) * u : g;
}

// ---------------------------------------------------------------- workspace

struct Workspace {
  int* num_tiles;
  int* tile_expert;
  int* tile_row0;
  void* h;
  size_t bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Workspace carve(void* base, int num_local, int inter, int capacity, bool bf16) {
  const int bm = bf16 ? kBfBM : kF32BM;
  const size_t max_tiles = (size_t)(capacity + bm - 1) / bm + num_local;
  char* p = (char*)base;
  Workspace w;
  size_t off = 0;
  w.num_tiles = (int*)(p + off);
  off += 256;
  w.tile_expert = (int*)(p + off);
  off += align256(max_tiles * sizeof(int));
  w.tile_row0 = (int*)(p + off);
  off += align256(max_tiles * sizeof(int));
  w.h = p + off;
  off += align256((size_t)capacity * inter * (bf16 ? 2 : 4));
  w.bytes = off;
  return w;
}

}  // namespace

size_t ffn_workspace_size(int num_local, int hidden, int inter, int capacity, bool bf16) {
  (void)hidden;
  return carve(nullptr, num_local, inter, capacity, bf16).bytes;
}

hipError_t launch_ffn(const FfnArgs& a, hipStream_t s) {
  const Workspace ws = carve(a.workspace, a.num_local, a.inter, a.capacity, a.bf16);
  const int bm = a.bf16 ? kBfBM : kF32BM;
  const int max_tiles = (a.capacity + bm - 1) / bm + a.num_local;
  if (a.capacity == 0) return hipSuccess;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, a.offsets, a.num_local, a.capacity,
                     bm, ws.num_tiles, ws.tile_expert, ws.tile_row0);
  const int I = a.inter, d = a.hidden;
  if (a.bf16) {
    constexpr int BM = kBfBM, BN = 128, BK = 64;
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, 2, 2, true>), dim3(I / (BN / 2), max_tiles),
                       dim3(256), 0, s, (const uint16_t*)a.x_sorted, a.offsets, a.capacity,
                       ws.num_tiles, ws.tile_expert, ws.tile_row0, (const uint16_t*)a.w_gate_up,
                       2 * I, d, I, (uint16_t*)ws.h, I);
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, 2, 2, false>), dim3(d / BN, max_tiles),
                       dim3(256), 0, s, (const uint16_t*)ws.h, a.offsets, a.capacity,
                       ws.num_tiles, ws.tile_expert, ws.tile_row0, (const uint16_t*)a.w_down, d,
                       I, I, (uint16_t*)a.o_sorted, d);
  } else {
    hipLaunchKernelGGL((gemm_f32_kernel<true>), dim3((I + 15) / 16, max_tiles), dim3(256), 0, s,
                       (const float*)a.x_sorted, a.offsets, a.capacity, ws.num_tiles,
                       ws.tile_expert, ws.tile_row0, (const float*)a.w_gate_up, 2 * I, d, I,
                       (float*)ws.h, I);
    hipLaunchKernelGGL((gemm_f32_kernel<false>), dim3((d + 15) / 16, max_tiles), dim3(256), 0, s,
                       (const float*)ws.h, a.offsets, a.capacity, ws.num_tiles, ws.tile_expert,
                       ws.tile_row0, (const float*)a.w_down, d, I, I, (float*)a.o_sorted, d);
  }
  return hipGetLastError();
}

}  // namespace moe
