// Grouped SwiGLU expert FFN over the permuted rows.
//
// Per local expert e (rows [off[e], off[e+1]) of the permuted activations):
//   [g | u] = X_e W_gate_up[e]^T      fused gate_up GEMM, N = 2I
//   h       = silu(g) * u             fused into the GEMM-1 epilogue
//   o       = h W_down[e]^T           GEMM-2
// The gated MLP (W_gate, W_up, W_down) is the one of section 2.2 of "Lecture 6
// · 并行" (semidirectx.com, cs349d lecture06); the fused gate_up GEMM with
// N = 2I and the skipping of experts that no token reaches come from the page
// "推理 INFRA 方法论（2）：分布式推理：TP、DP、EP、CP 与 PP" (johneyzheng.top).
//
// The permuted activations are either a materialised x_sorted or, fused with
// the dispatch gather, the token rows x read through sorted_assign
// (row i = x[sorted_assign[i] / k]).
//
// Each GEMM is one persistent kernel that reads expert_offsets on the device
// (the row counts never return to the host) and builds its work lists in LDS:
// * streaming path -- experts with at most 256 rows (decode), in 64-row
//   chunks. Bound by the weight read: weight bytes go from HBM straight into
//   MFMA registers, with the next two K steps' loads in flight during the
//   current MFMAs.
// * tiled path -- experts with more rows (prefill): 128 x 128 tiles staged
//   through LDS on 32x32x16 bf16 MFMA.
// Experts with no rows appear in neither list, so their weights are not read.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kStreamMT = 4;                  // row tiles of 16 per streamed row chunk
constexpr int kChunkRows = kStreamMT * 16;    // rows per streamed chunk
constexpr int kStreamRows = 4 * kChunkRows;   // experts with more rows are tiled
constexpr int kTileBM = 128;                  // tokens per tile in the tiled path
constexpr int kMaxLocal = 1024;

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

struct GemmArgs {
  const uint16_t* A;      // activations: permuted rows, or token rows when row_index != null
  const int* row_index;   // null, or sorted_assign: permuted row i is A row row_index[i] / row_div
  int row_div;
  const int* offsets;     // [nloc + 1]
  int nloc, capacity;
  const uint16_t* W;      // [nloc, N, K], K contiguous
  int N, K, inter;        // gated GEMMs pair weight row n with row inter + n
  uint16_t* C;            // [capacity, ldc]
  int ldc;
};

__device__ __forceinline__ const uint16_t* a_row_ptr(const GemmArgs& a, int row) {
  const int src = a.row_index ? a.row_index[row] / a.row_div : row;
  return a.A + (size_t)src * a.K;
}

// ---------------------------------------------------------------- expert lists

// Splits the local experts by row count m, in expert order:
//   1 <= m <= kStreamRows: streamed, in ceil(m / kChunkRows) row chunks;
//                          s_first[e] = first chunk of expert e, s_first[nloc] = chunks
//   m > kStreamRows:       tiled, in ceil(m / bm) row tiles;
//                          t_first[e] = first tile of expert e, t_first[nloc] = tiles
// Every thread of the 256-thread workgroup calls this; 4 experts per thread.
__device__ void build_lists(const GemmArgs& a, int bm, int* s_first, int* t_first, int* wsum,
                            int& n_chunks, int& n_tiles) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int cc[4], tc[4], cs = 0, ct = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    int m = 0;
    if (e < a.nloc) {
      const int lo = min(a.offsets[e], a.capacity);
      m = max(0, min(a.offsets[e + 1], a.capacity) - lo);
    }
    cc[q] = (m > 0 && m <= kStreamRows) ? (m + kChunkRows - 1) / kChunkRows : 0;
    tc[q] = (m > kStreamRows) ? (m + bm - 1) / bm : 0;
    cs += cc[q];
    ct += tc[q];
  }
  int is = cs, it = ct;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int os = __shfl_up(is, d, MOE_WAVE), ot = __shfl_up(it, d, MOE_WAVE);
    if (lane >= d) { is += os; it += ot; }
  }
  if (lane == 63) { wsum[w] = is; wsum[4 + w] = it; }
  __syncthreads();
  int bs = 0, bt = 0, ts = 0, tt = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < w) { bs += wsum[i]; bt += wsum[4 + i]; }
    ts += wsum[i];
    tt += wsum[4 + i];
  }
  int ps = bs + is - cs, pt = bt + it - ct;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    if (e < a.nloc) {
      s_first[e] = ps;
      t_first[e] = pt;
      ps += cc[q];
      pt += tc[q];
    }
  }
  if (tid == 0) {
    s_first[a.nloc] = ts;
    t_first[a.nloc] = tt;
  }
  n_chunks = ts;
  n_tiles = tt;
  __syncthreads();
}

// The expert e with first[e] <= idx < first[e + 1] (first is non-decreasing).
__device__ __forceinline__ int find_expert(const int* first, int nloc, int idx) {
  int lo = 0, hi = nloc - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (first[mid] <= idx) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------- streaming path

// A work item is a row chunk (up to 64 rows) of one expert and a slab of
// output columns. The workgroup's 4 wavefronts split K into KS slices and
// (4 / KS) groups of NTW 16-row weight tiles. The weight tile is the MFMA A
// operand and the activations the B operand, so a lane ends up holding 4
// consecutive output columns of one row (one 8-byte store).
//
// In a K step of 32*U, load u of lane (r, g) = (lane % 16, lane / 16) reads 8
// bf16 of weight row r (or activation row r) at k = kk + 32u + 8g: one load
// instruction covers 64 contiguous bytes of each of 16 rows, and MFMA u
// consumes exactly the 32 k of load u for both operands. K slices are summed
// through LDS in slice order; then SiLU*up (gated) or the plain bf16 store.
template <int NTW, int KS, int U, bool GATED>
struct Stream {
  static constexpr int MT = kStreamMT;
  static constexpr int NWN = 4 / KS;
  static constexpr int HT = GATED ? NTW / 2 : NTW;  // output tiles per wavefront
  static constexpr int COLS = NWN * HT * 16;        // output columns per slab
  static constexpr int KSTEP = 32 * U;
  static constexpr int RED_BYTES = KS > 1 ? KS * NWN * MT * NTW * 64 * 16 : 0;
  static_assert(!GATED || NTW % 2 == 0, "gated slabs pair gate and up tiles");

  // MTA = active row tiles of the chunk (1..MT): the K loop has no branches,
  // so the only waits are on the registers an MFMA reads.
  template <int MTA>
  __device__ static void run_mt(const GemmArgs& a, int e, int lo, int m, int slab, f32x4_t* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ks = wave % KS, wn = wave / KS;
    const int fr = lane & 15, g = lane >> 4;
    const int col0 = (slab * NWN + wn) * HT * 16;  // first output column of this wavefront

    const uint16_t* wp[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int c = col0 + (t % HT) * 16 + fr;
      const int wrow = (GATED && t >= HT) ? a.inter + c : c;
      wp[t] = a.W + ((size_t)e * a.N + wrow) * a.K + g * 8;
    }
    // Rows past the chunk's end read its first row instead: an MFMA output
    // column depends only on its own activation row, and it is not stored.
    const uint16_t* ap[MTA];
#pragma unroll
    for (int i = 0; i < MTA; ++i) {
      const int r = i * 16 + fr;
      ap[i] = a_row_ptr(a, lo + (r < m ? r : 0)) + g * 8;
    }

    f32x4_t acc[MTA][NTW];
#pragma unroll
    for (int i = 0; i < MTA; ++i)
#pragma unroll
      for (int t = 0; t < NTW; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    bf16x8_t w0[NTW][U], w1[NTW][U], w2[NTW][U], a0[MTA][U], a1[MTA][U];
    auto load_w = [&](bf16x8_t (&w)[NTW][U], int kk) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < NTW; ++t) w[t][u] = *(const bf16x8_t*)(wp[t] + kk + u * 32);
    };
    auto load_a = [&](bf16x8_t (&av)[MTA][U], int kk) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < MTA; ++i) av[i][u] = *(const bf16x8_t*)(ap[i] + kk + u * 32);
    };
    auto mma = [&](const bf16x8_t (&w)[NTW][U], const bf16x8_t (&av)[MTA][U]) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < MTA; ++i)
#pragma unroll
          for (int t = 0; t < NTW; ++t)
            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[t][u], av[i][u], acc[i][t], 0, 0, 0);
    };

    // Software pipeline over K steps: weights two steps ahead (three register
    // sets), activations one step ahead (two sets). In step s the loads for
    // A(s+1) and then W(s+2) are issued before the MFMAs of step s. Loads
    // complete in issue order, so the oldest outstanding loads are exactly
    // W(s) and A(s): the MFMAs wait for those while W(s+1), A(s+1) and W(s+2)
    // stay in flight. Steps past the end reload the last chunk instead of
    // branching. The scheduling barriers keep this issue order.
    const int kw = a.K / KS, kbeg = ks * kw, klast = kbeg + kw - KSTEP;
    const int steps = kw / KSTEP;
    int kk = kbeg;
    load_w(w0, kk);
    load_a(a0, kk);
    load_w(w1, min(kk + KSTEP, klast));
#define MOE_STEP(WC, WN, AC, AN)           \
  load_a(AN, min(kk + KSTEP, klast));     \
  load_w(WN, min(kk + 2 * KSTEP, klast)); \
  __builtin_amdgcn_sched_barrier(0);      \
  mma(WC, AC);                            \
  __builtin_amdgcn_sched_barrier(0);      \
  kk += KSTEP;
    for (int s = 0; s < steps; s += 6) {
      MOE_STEP(w0, w2, a0, a1)
      if (s + 1 >= steps) break;
      MOE_STEP(w1, w0, a1, a0)
      if (s + 2 >= steps) break;
      MOE_STEP(w2, w1, a0, a1)
      if (s + 3 >= steps) break;
      MOE_STEP(w0, w2, a1, a0)
      if (s + 4 >= steps) break;
      MOE_STEP(w1, w0, a0, a1)
      if (s + 5 >= steps) break;
      MOE_STEP(w2, w1, a1, a0)
    }
#undef MOE_STEP

    if (KS > 1) {
      // red: [KS][NWN][MT][NTW][64] float4; slice ks finishes row tiles i with i % KS == ks
#pragma unroll
      for (int i = 0; i < MTA; ++i)
#pragma unroll
        for (int t = 0; t < NTW; ++t) red[(((ks * NWN + wn) * MT + i) * NTW + t) * 64 + lane] = acc[i][t];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MTA; ++i) {
        if (i % KS != ks) continue;
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          f32x4_t sum = red[(((0 * NWN + wn) * MT + i) * NTW + t) * 64 + lane];
#pragma unroll
          for (int q = 1; q < KS; ++q) sum += red[(((q * NWN + wn) * MT + i) * NTW + t) * 64 + lane];
          acc[i][t] = sum;
        }
      }
    }
    // Lane holds output row i*16 + lane % 16, columns col0 + t*16 + 4*(lane/16) + (0..3).
#pragma unroll
    for (int i = 0; i < MTA; ++i) {
      if (KS > 1 && i % KS != ks) continue;
      const int row = i * 16 + fr;
      if (row >= m) continue;
      uint16_t* crow = a.C + (size_t)(lo + row) * a.ldc + col0 + g * 4;
#pragma unroll
      for (int t = 0; t < HT; ++t) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          v[r] = GATED ? silu(acc[i][t][r]) * acc[i][t + HT][r] : acc[i][t][r];
        *(uint2*)(crow + t * 16) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
    if (KS > 1) __syncthreads();  // red is reused by the next work item
  }

  // Row chunk `chunk` (kChunkRows rows) of expert e, output slab `slab`.
  __device__ static void run(const GemmArgs& a, int e, int chunk, int slab, f32x4_t* red) {
    const int lo = min(a.offsets[e], a.capacity) + chunk * kChunkRows;
    const int m = min(kChunkRows, min(a.offsets[e + 1], a.capacity) - lo);
    switch ((m + 15) >> 4) {
      case 1: run_mt<1>(a, e, lo, m, slab, red); break;
      case 2: run_mt<2>(a, e, lo, m, slab, red); break;
      case 3: run_mt<3>(a, e, lo, m, slab, red); break;
      default: run_mt<4>(a, e, lo, m, slab, red); break;
    }
  }
};

// ---------------------------------------------------------------- tiled path

// Experts with more than kStreamRows rows (prefill): 128 weight rows x 128
// tokens per tile, K staged through LDS 64 at a time (double-buffered through
// registers), 4 wavefronts of 64 x 64 on v_mfma_f32_32x32x16_bf16 with
// float32 accumulators.
//
// The weight tile is the MFMA A operand (rows = output columns) and the token
// tile the B operand; a lane's 16 accumulators of a fragment are 4 runs of 4
// consecutive output columns of one token row (8-byte stores). A gated tile
// holds 64 gate rows and the 64 matching up rows, arranged so that fragment 0
// (gate) and fragment 1 (up) of a wavefront cover the same output columns.
//
// LDS rows are 64 bf16 (eight 16-byte chunks); chunk c of row r is stored at
// c ^ (r & 7), so the 32 rows one fragment read touches at one k are spread
// over the banks.
constexpr int kTileBN = 128;  // weight rows per tile
constexpr int kTileBK = 64;

template <bool GATED>
struct Tiled {
  static constexpr int COLS = GATED ? kTileBN / 2 : kTileBN;  // output columns per tile
  static constexpr int TILE = kTileBN * kTileBK;               // elements per operand tile
  static constexpr int LDS_BYTES = 2 * 2 * TILE * 2;           // [buffer][W | X], bf16
  static_assert(kTileBM == 128, "the tile holds 128 tokens");

  __device__ static __forceinline__ int swz(int row, int chunk) {
    return row * kTileBK + ((chunk ^ (row & 7)) << 3);
  }

  __device__ static void run(const GemmArgs& a, int e, int row0, int rows, int nb, uint16_t* lds) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;  // wavefront: weight rows wm*64.., tokens wn*64..
    const int K = a.K;
    const int kc = tid & 7;                   // 16-byte chunk this thread loads in every row
    const int rbase = tid >> 3;               // tile rows rbase + 32 i, i = 0..3

    // This thread's weight rows are wrow0 + woff[i]; its token rows are tok[i]
    // (rows past the tile's end read its first row; their outputs are not stored).
    int wrow0, woff[4];
    if (GATED) {
      // tile rows: [gate 32 | up 32] for wavefront row group 0, then for group 1
      wrow0 = nb * COLS + rbase;
      woff[0] = 0;
      woff[1] = a.inter;
      woff[2] = 32;
      woff[3] = a.inter + 32;
    } else {
      wrow0 = nb * kTileBN + rbase;
#pragma unroll
      for (int i = 0; i < 4; ++i) woff[i] = 32 * i;
    }
    const uint16_t* wsrc = a.W + ((size_t)e * a.N + wrow0) * K + kc * 8;
    int tok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rbase + 32 * i;
      const int row = row0 + (r < rows ? r : 0);
      tok[i] = a.row_index ? a.row_index[row] / a.row_div : row;
    }
    const uint16_t* xsrc = a.A + kc * 8;

    u32x4_t sw[4], sx[4];
    auto gload = [&](int k0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sw[i] = *(const u32x4_t*)(wsrc + (size_t)woff[i] * K + k0);
#pragma unroll
      for (int i = 0; i < 4; ++i) sx[i] = *(const u32x4_t*)(xsrc + (size_t)tok[i] * K + k0);
    };
    auto sstore = [&](int buf) {
      uint16_t* lw = lds + buf * 2 * TILE;
      uint16_t* lx = lw + TILE;
#pragma unroll
      for (int i = 0; i < 4; ++i) *(u32x4_t*)(lw + swz(rbase + 32 * i, kc)) = sw[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) *(u32x4_t*)(lx + swz(rbase + 32 * i, kc)) = sx[i];
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

    const int fr = lane & 31, fh = lane >> 5;  // fragment row, k half (8 of 16)
    const int nk = K / kTileBK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) gload((kt + 1) * kTileBK);
      const uint16_t* lw = lds + buf * 2 * TILE;
      const uint16_t* lx = lw + TILE;
#pragma unroll
      for (int kq = 0; kq < kTileBK / 16; ++kq) {
        const int chunk = kq * 2 + fh;
        bf16x8_t av[2], bv[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) av[i] = *(const bf16x8_t*)(lw + swz(wm * 64 + i * 32 + fr, chunk));
#pragma unroll
        for (int j = 0; j < 2; ++j) bv[j] = *(const bf16x8_t*)(lx + swz(wn * 64 + j * 32 + fr, chunk));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) sstore(buf ^ 1);
      __syncthreads();
    }

    // acc[i][j][r]: token wn*64 + j*32 + lane%32; weight tile row
    // wm*64 + i*32 + (r/4)*8 + (lane/32)*4 + r%4.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = wn * 64 + j * 32 + fr;
      if (t >= rows) continue;
      uint16_t* crow = a.C + (size_t)(row0 + t) * a.ldc;
      if (GATED) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = nb * COLS + wm * 32 + q * 8 + fh * 4;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = silu(acc[0][j][q * 4 + r]) * acc[1][j][q * 4 + r];
          *(uint2*)(crow + col) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = nb * COLS + wm * 64 + i * 32 + q * 8 + fh * 4;
            const f32x16_t& c = acc[i][j];
            *(uint2*)(crow + col) = make_uint2(pack_bf16x2(c[q * 4], c[q * 4 + 1]),
                                               pack_bf16x2(c[q * 4 + 2], c[q * 4 + 3]));
          }
      }
    }
  }
};

// ---------------------------------------------------------------- the GEMM kernel

// One persistent kernel per GEMM: first the streamed row chunks, then the row
// tiles of larger experts. The two paths share the LDS buffer.
template <int NTW, int KS, int U, bool GATED>
__global__ __launch_bounds__(256, 2) void ffn_gemm_kernel(GemmArgs a) {
  using S = Stream<NTW, KS, U, GATED>;
  using T = Tiled<GATED>;
  constexpr int SMEM = S::RED_BYTES > T::LDS_BYTES ? S::RED_BYTES : T::LDS_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  __shared__ int s_first[kMaxLocal + 1];
  __shared__ int t_first[kMaxLocal + 1];
  __shared__ int wsum[8];
  int n_chunks, n_tiles;
  build_lists(a, kTileBM, s_first, t_first, wsum, n_chunks, n_tiles);
  const int ncols = GATED ? a.inter : a.N;
  const int slabs = ncols / S::COLS, nblk = ncols / T::COLS;
  const int n_stream = n_chunks * slabs;
  const int total = n_stream + n_tiles * nblk;
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    if (w < n_stream) {
      const int c = w / slabs;
      const int e = find_expert(s_first, a.nloc, c);
      S::run(a, e, c - s_first[e], w % slabs, (f32x4_t*)smem);
    } else {
      const int tile = (w - n_stream) / nblk, nb = (w - n_stream) % nblk;
      const int e = find_expert(t_first, a.nloc, tile);
      const int row0 = min(a.offsets[e], a.capacity) + (tile - t_first[e]) * kTileBM;
      const int rows = min(kTileBM, min(a.offsets[e + 1], a.capacity) - row0);
      T::run(a, e, row0, rows, nb, (uint16_t*)smem);
      __syncthreads();  // the LDS buffer is reused by the next work item
    }
  }
}

// ---------------------------------------------------------------- f32 GEMM (small shapes)

struct GemmArgsF32 {
  const float* A;
  const int* row_index;
  int row_div;
  const int* offsets;
  int nloc, capacity, max_row_tiles;
  const float* W;
  int N, K, inter;
  float* C;
  int ldc;
};

// 16 rows x 16 output columns per workgroup, plain FMA, bounds-checked in N and K.
// blockIdx.y = expert * max_row_tiles + row tile; blockIdx.x = column block.
template <bool GATED>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgsF32 a) {
  __shared__ float As[16][17], Bg[16][17], Bu[16][17];
  const int e = blockIdx.y / a.max_row_tiles, tile = blockIdx.y % a.max_row_tiles;
  const int lo = min(a.offsets[e], a.capacity), hi = min(a.offsets[e + 1], a.capacity);
  const int row0 = lo + tile * 16;
  if (row0 >= hi) return;
  const int rows = min(16, hi - row0);
  const int n_out = GATED ? a.inter : a.N;
  const int K = a.K;
  const float* We = a.W + (size_t)e * a.N * K;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int col0 = blockIdx.x * 16;
  const float* arow = nullptr;
  if (ty < rows) {
    const int r = row0 + ty;
    arow = a.A + (size_t)(a.row_index ? a.row_index[r] / a.row_div : r) * K;
  }
  float gs = 0.f, us = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int kk = k0 + tx;
    As[ty][tx] = (arow && kk < K) ? arow[kk] : 0.f;
    const int n = col0 + ty;
    Bg[ty][tx] = (n < n_out && kk < K) ? We[(size_t)n * K + kk] : 0.f;
    if (GATED) Bu[ty][tx] = (n < n_out && kk < K) ? We[(size_t)(a.inter + n) * K + kk] : 0.f;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      gs += As[ty][q] * Bg[tx][q];
      if (GATED) us += As[ty][q] * Bu[tx][q];
    }
    __syncthreads();
  }
  const int col = col0 + tx;
  if (ty < rows && col < n_out) a.C[(size_t)(row0 + ty) * a.ldc + col] = GATED ? silu(gs) * us : gs;
}

// ---------------------------------------------------------------- host side

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int cu_count() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// Resident workgroups per CU of a kernel (queried once per kernel).
template <typename F>
int occupancy(F kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n <= 0)
    n = 1;
  return n;
}

// Shape of the streaming path per GEMM:
//   gate_up (gated): NTW = 2 (a gate and the matching up tile), U = 2
//   down (plain):    NTW = 4, U = 1
// and KS, the K slices of a workgroup: 4 when every slice still has at least
// 8 K steps, else 2 (gated: K = hidden is a multiple of 256), else 1.
template <bool GATED>
int stream_ks(int K) {
  constexpr int U = GATED ? 2 : 1;
  if (K % (4 * 32 * U) == 0 && K / 4 >= 8 * 32 * U) return 4;
  if (GATED || (K % (2 * 32 * U) == 0 && K / 2 >= 4 * 32 * U)) return 2;
  return 1;
}

template <bool GATED, int KS>
hipError_t launch_gemm_t(const GemmArgs& g, hipStream_t s) {
  constexpr int NTW = GATED ? 2 : 4, U = GATED ? 2 : 1;
  using S = Stream<NTW, KS, U, GATED>;
  using T = Tiled<GATED>;
  auto kernel = ffn_gemm_kernel<NTW, KS, U, GATED>;
  static const int occ = occupancy(kernel, 256);
  const int ncols = GATED ? g.inter : g.N;
  const long max_chunks = std::min<long>((long)g.nloc * (kStreamRows / kChunkRows),
                                         (long)(g.capacity + kChunkRows - 1) / kChunkRows + g.nloc);
  const long max_tiles = (long)(g.capacity + kTileBM - 1) / kTileBM + g.nloc;
  const long max_work = max_chunks * (ncols / S::COLS) + max_tiles * (ncols / T::COLS);
  const int grid = (int)std::max<long>(1, std::min<long>(max_work, (long)cu_count() * occ));
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, s, g);
  return hipGetLastError();
}

template <bool GATED>
hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  switch (stream_ks<GATED>(g.K)) {
    case 4: return launch_gemm_t<GATED, 4>(g, s);
    case 2: return launch_gemm_t<GATED, 2>(g, s);
    default: return GATED ? hipErrorInvalidValue : launch_gemm_t<false, 1>(g, s);
  }
}

}  // namespace

size_t ffn_workspace_size(int num_local, int hidden, int inter, int capacity, bool bf16) {
  (void)num_local;
  (void)hidden;
  return align256((size_t)capacity * inter * (bf16 ? 2 : 4));  // h
}

hipError_t launch_ffn(const FfnArgs& a, hipStream_t s) {
  if (a.capacity == 0) return hipSuccess;
  const int I = a.inter, d = a.hidden;
  if (a.bf16) {
    GemmArgs g1{(const uint16_t*)a.x, a.row_index, a.row_div, a.offsets, a.num_local,
                a.capacity, (const uint16_t*)a.w_gate_up, 2 * I, d, I,
                (uint16_t*)a.workspace, I};
    GemmArgs g2{(const uint16_t*)a.workspace, nullptr, 1, a.offsets, a.num_local, a.capacity,
                (const uint16_t*)a.w_down, d, I, I, (uint16_t*)a.o_sorted, d};
    const hipError_t err = launch_gemm<true>(g1, s);
    if (err != hipSuccess) return err;
    return launch_gemm<false>(g2, s);
  }
  const int mrt = (a.capacity + 15) / 16;
  GemmArgsF32 g1{(const float*)a.x, a.row_index, a.row_div, a.offsets, a.num_local, a.capacity,
                 mrt, (const float*)a.w_gate_up, 2 * I, d, I, (float*)a.workspace, I};
  GemmArgsF32 g2{(const float*)a.workspace, nullptr, 1, a.offsets, a.num_local, a.capacity, mrt,
                 (const float*)a.w_down, d, I, I, (float*)a.o_sorted, d};
  hipLaunchKernelGGL((gemm_f32_kernel<true>), dim3((I + 15) / 16, a.num_local * mrt), dim3(256),
                     0, s, g1);
  hipLaunchKernelGGL((gemm_f32_kernel<false>), dim3((d + 15) / 16, a.num_local * mrt), dim3(256),
                     0, s, g2);
  return hipGetLastError();
}

}  // namespace moe
