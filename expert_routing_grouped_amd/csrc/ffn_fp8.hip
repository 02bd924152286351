// FP8 variant of the grouped SwiGLU expert FFN, and the row quantiser.
//
// Operands are OCP e4m3 codes with float32 block scales: token rows (x, and
// h between the two GEMMs) take one scale per row and 128 consecutive
// features, weights one per 128 x 128 block; a value is code * scale. The
// pages count an expert's weights as 44 MB of FP8 and send a dispatched
// token as FP8 plus 224 bytes of scales ("大规模 EP 部署：分层 EPLB、DP 注意力的
// 负载与双 batch 重叠", anrans.github.io, section "双 batch 重叠"), and measure
// the fused gate_up grouped GEMM on FP8 weights ("推理 INFRA 方法论（2）",
// johneyzheng.top); the block shapes are this library's reading.
//
// Per local expert e (rows [off[e], off[e+1]) of the permuted rows):
//   [g | u] = X_e W_gate_up[e]^T      (float32 accumulation)
//   h       = silu(g) * u             float32, written to the workspace
//   (hq, hs)= quantise h per row and 128 columns
//   o       = hq W_down[e]^T          bf16 out
//
// Quantising a block of 128 values: scale = amax / 448 (1 for an all-zero
// block), code = the e4m3 value nearest to v / scale, ties to the even code,
// magnitudes above 448 saturate; both divisions are correctly rounded float32
// (the one by the scale computed as in div_by_scale).
//
// Experts with at most 64 rows (decode) stream the weights: a work item is
// the expert's rows and one slab of output columns. A K
// step is 128 k, one 128-byte line of each row, loaded coalesced (8 rows per
// instruction) into a wavefront-private XOR-swizzled LDS tile and read back
// as MFMA fragments for v_mfma_scale_f32_16x16x128_f8f6f4 (block scales of
// the instruction left at 1): one instruction covers exactly one scale block
// of k, so its float32 result is multiplied by (row scale x weight block
// scale) and added to the accumulator. Loads run two K steps ahead.
//
// Experts with more than 64 rows (prefill) are tiled instead: 128 weight rows
// x 128 tokens per work item, so the weights are read once per 128 rows and
// each loaded byte feeds 128 multiply-adds. A K step (128 k, one scale block)
// of both operands is staged through a double-buffered XOR-swizzled LDS tile;
// each wavefront multiplies 64 x 64 of the tile on
// v_mfma_scale_f32_32x32x64_f8f6f4 (two per K step and fragment pair, into a
// zeroed float32 partial that is then added with its scale factor). When
// their tiles fill the GPU (prefill) they take 256 x 256 tiles in
// ffn_fp8_big_kernel instead, whose gate_up also quantises its rows of h
// (128 output columns = one scale block per row), leaving the other rows to
// quantize_h_kernel.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kQBlock = 128;      // features per scale
constexpr int kF8Rows = 64;       // rows per chunk
constexpr int kF8MT = kF8Rows / 16;
constexpr int kF8Depth = 3;       // register sets: loads run kF8Depth - 1 steps ahead
constexpr int kF8MaxLocal = 1024;
constexpr int kF8Config = 0x00020000;   // buffer resource word 3 (raw buffer loads)
constexpr int kF8NonTemporal = 2;
constexpr int kT8Rows = 128;      // tokens per tile (experts with more than kF8Rows rows)
constexpr int kB8Rows = 256;      // tokens per large tile
constexpr int kB8MinCapacity = 16384;   // row capacity from which the large-tile kernel is launched

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

// e4m3 codes of four float32 values (value j in byte j): the nearest code,
// ties to the even code, saturating at +-448. The rounding is gfx950's packed
// float32 -> fp8 conversion (OCP e4m3): ties to even, subnormals below 2^-6
// as integers times 2^-9, the sign kept for -0; between 448 and 464 it rounds
// to 448 by itself, and the clamp keeps larger magnitudes there too. (Checked
// equal, on every float32 of magnitude up to 464 and both signs, to the code
// built from the bit pattern: the float32 mantissa rounded to 3 bits with a
// carry into the exponent, rebiased from 127 to 7, and below 2^-6 the integer
// nearest to |q| * 2^9.)
__device__ __forceinline__ float e4m3_clamp(float q) { return fmaxf(fminf(q, 448.0f), -448.0f); }

__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), w, true);
  return (uint32_t)w;
}

// v / s rounded to float32 -- the correctly rounded float32 quotient --
// from rs = 1 / s rounded to float64, as RN32(RN64(v * rs)). For float32 v
// and s the float64 product is within 2^-51.9 (relative) of v / s, while a
// quotient of two 24-bit significands that is not itself a float32 lies at
// least 2^-49 (relative) away from every float32 rounding midpoint (write
// v / s = (a / b) 2^e and a midpoint as M 2^f with a, b < 2^24 and M < 2^25
// odd: a 2^e - b M 2^f is a nonzero multiple of 2^f, and e > f), so both
// round to the same float32. One float64 multiply per value instead of a
// float32 division.
__device__ __forceinline__ float div_by_scale(float v, double rs) { return (float)((double)v * rs); }

// ---------------------------------------------------------------- quantiser

// A wavefront item is 4 consecutive blocks of one row (512 values): lane l
// holds 8 values of block l / 16, and the block's maximum is reduced over its
// 16 lanes. Lanes past the row's last block do nothing. A wavefront takes
// ITEMS items per pass (items w, w + stride, ...), all loads issued before
// the first is used: ITEMS = 1 when the grid has a wavefront for every item,
// else kQItems. The row count is rows, or min(rows, *rows_dev) when rows_dev
// is given.
constexpr int kQItems = 4;

template <bool BF16_IN, int ITEMS>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const void* in, int rows, const int* rows_dev,
                                                           int cols, uint8_t* codes, float* scales) {
  int n = rows;
  if (rows_dev) n = min(n, max(0, *rows_dev));
  const int nb = cols / kQBlock;
  const int groups = (nb + 3) / 4;
  const long total = (long)n * groups;
  const int lane = threadIdx.x & 63;
  const long stride = (long)gridDim.x * 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (long w0 = (long)blockIdx.x * 4 + wave; w0 < total; w0 += stride * ITEMS) {
    // items of this pass (the same for the whole wavefront): the others are
    // skipped, index arithmetic included
    const int cnt = ITEMS == 1 ? 1 : (int)min((long)ITEMS, (total - w0 + stride - 1) / stride);
    float v[ITEMS][8];
    size_t first[ITEMS];
    int row[ITEMS], blk[ITEMS];
    bool active[ITEMS];
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      active[u] = false;
      row[u] = blk[u] = 0;
      first[u] = 0;
      if (u < cnt) {
        const long w = w0 + u * stride;
        const int r = (int)(w / groups);
        row[u] = r;
        blk[u] = (int)(w - (long)r * groups) * 4 + (lane >> 4);
        active[u] = blk[u] < nb;
        first[u] = (size_t)r * cols + (size_t)blk[u] * kQBlock + (lane & 15) * 8;   // of 8 values
      }
      if (active[u]) {
        if (BF16_IN) {
          const u32x4_t p = *(const u32x4_t*)((const uint16_t*)in + first[u]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[u][2 * j] = bf16_lo(p[j]);
            v[u][2 * j + 1] = bf16_hi(p[j]);
          }
        } else {
          const f32x4_t p0 = *(const f32x4_t*)((const float*)in + first[u]);
          const f32x4_t p1 = *(const f32x4_t*)((const float*)in + first[u] + 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[u][j] = p0[j];
            v[u][4 + j] = p1[j];
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[u][j] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      if (u >= cnt) break;
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[u][j]));
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, MOE_WAVE));
      if (!active[u]) continue;
      const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
      const double rs = 1.0 / (double)s;
      float q[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) q[j] = div_by_scale(v[u][j], rs);
      const uint32_t lo = e4m3_pack4(q[0], q[1], q[2], q[3]), hi = e4m3_pack4(q[4], q[5], q[6], q[7]);
      *(uint2*)(codes + first[u]) = make_uint2(lo, hi);
      if ((lane & 15) == 0) scales[(size_t)row[u] * nb + blk[u]] = s;
    }
  }
}

// ---------------------------------------------------------------- GEMMs

struct F8Args {
  const uint8_t* A;       // activation codes: permuted rows, or token rows read through row_index
  const float* As;        // their scales, [rows, K / 128]
  const int* row_index;   // null, or sorted_assign: permuted row i is A row row_index[i] / row_div
  int row_div;
  const int* offsets;     // [nloc + 1]
  int nloc, capacity;
  const uint8_t* W;       // [nloc, N, K] codes, K contiguous
  const float* Ws;        // [nloc, N / 128, K / 128]
  int N, K, inter;        // gated GEMMs pair weight row n with row inter + n
  void* C;                // gated: float h [capacity, ldc]; plain: bf16 [capacity, ldc]
  int ldc;
  int big_ok;             // the large-tile kernel is launched too ...
  int big_min_items;      // ... and takes the tiled experts when it has at least this many items
  uint8_t* Cq;            // gated, large tiles: also h's e4m3 codes [capacity, ldc] ...
  float* Cs;              // ... and scales [capacity, ldc / 128]
};

struct F8QOut {
  uint8_t* q;
  float* s;
};

// F8Args in the kernel argument segment (constant memory: scalar loads).
typedef const __attribute__((address_space(4))) F8Args KernargF8Args;

__device__ __forceinline__ F8Args f8_args_copy(KernargF8Args* p) {
  F8Args r;
  r.A = p->A;
  r.As = p->As;
  r.row_index = p->row_index;
  r.row_div = p->row_div;
  r.offsets = p->offsets;
  r.nloc = p->nloc;
  r.capacity = p->capacity;
  r.W = p->W;
  r.Ws = p->Ws;
  r.N = p->N;
  r.K = p->K;
  r.inter = p->inter;
  r.C = p->C;
  r.ldc = p->ldc;
  r.big_ok = p->big_ok;
  r.big_min_items = p->big_min_items;
  r.Cq = p->Cq;
  r.Cs = p->Cs;
  return r;
}

// Work lists, in expert order, of the experts with rows: those with at most
// kF8Rows rows are one chunk each (c_first[e] = the chunk of expert e,
// c_first[nloc] = chunks), the others are cut into tiles of tile_rows rows
// (t_first[e] = first tile of expert e, t_first[nloc] = tiles). c_lo[e] =
// first row of expert e (clamped to the capacity), c_lo[nloc] = end of the
// last expert. n_big = the tiles of kB8Rows rows that the tiled experts
// need. Every thread of a workgroup of 256 calls this (4 experts per
// thread; a larger workgroup's other threads only take part in the
// barriers).
__device__ void f8_lists(const F8Args& a, int tile_rows, int* c_first, int* t_first, int* c_lo, int* wsum,
                         int& n_chunks, int& n_tiles, int& n_big) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int cc[4], tc[4], cs = 0, ct = 0, cb = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    int m = 0;
    if (e < a.nloc) {
      const int lo = min(a.offsets[e], a.capacity);
      const int hi = min(a.offsets[e + 1], a.capacity);
      m = max(0, hi - lo);
      c_lo[e] = lo;
      if (e == a.nloc - 1) c_lo[a.nloc] = max(lo, hi);
    }
    cc[q] = (m > 0 && m <= kF8Rows) ? 1 : 0;
    tc[q] = m > kF8Rows ? (m + tile_rows - 1) / tile_rows : 0;
    cs += cc[q];
    ct += tc[q];
    cb += m > kF8Rows ? (m + kB8Rows - 1) / kB8Rows : 0;
  }
  cb = wave_sum_i32(cb);
  int is = cs, it = ct;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int os = __shfl_up(is, d, MOE_WAVE), ot = __shfl_up(it, d, MOE_WAVE);
    if (lane >= d) { is += os; it += ot; }
  }
  if (lane == 63 && w < 4) { wsum[w] = is; wsum[4 + w] = it; wsum[8 + w] = cb; }
  __syncthreads();
  int bs = 0, bt = 0, ts = 0, tt = 0, tb = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < w) { bs += wsum[i]; bt += wsum[4 + i]; }
    ts += wsum[i];
    tt += wsum[4 + i];
    tb += wsum[8 + i];
  }
  int ps = bs + is - cs, pt = bt + it - ct;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    if (e < a.nloc) {
      c_first[e] = ps;
      t_first[e] = pt;
      ps += cc[q];
      pt += tc[q];
    }
  }
  if (tid == 0) {
    c_first[a.nloc] = ts;
    t_first[a.nloc] = tt;
  }
  __syncthreads();
  n_chunks = __builtin_amdgcn_readfirstlane(ts);
  n_tiles = __builtin_amdgcn_readfirstlane(tt);
  n_big = __builtin_amdgcn_readfirstlane(tb);
}

__device__ __forceinline__ int f8_find_expert(const int* first, int nloc, int idx) {
  int lo = 0, hi = nloc - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (first[mid] <= idx) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Permuted row numbers -> rows of A. The division by row_div is
// floor((v + 0.5) / row_div) in float64, exact for v < 2^31 (the error of the
// float64 quotient stays far below the distance 0.5 / row_div to an integer).
template <int N>
__device__ __forceinline__ void f8_rows(const F8Args& a, uint32_t* rows) {
  if (!a.row_index) return;
#pragma unroll
  for (int j = 0; j < N; ++j) rows[j] = (uint32_t)a.row_index[rows[j]];
  int div = a.row_div;
  asm volatile("" : "+s"(div));
  if (div != 1) {
    const double inv = 1.0 / (double)div;
#pragma unroll
    for (int j = 0; j < N; ++j) rows[j] = (uint32_t)(((double)rows[j] + 0.5) * inv);
  }
}

// A work item: a row chunk of expert e and a slab of output columns. The
// workgroup's 4 wavefronts split K into KS slices and (4 / KS) groups of NTW
// 16-row weight tiles (gated: a gate tile and the matching up tile). The
// weight tile is the MFMA A operand, the activations the B operand, so a
// lane holds 4 consecutive output columns of one row.
//
// Loads: lane l takes the 16-byte chunk l % 8 of row 8h + l / 8 of a 16-row
// tile (h = 0, 1) and writes it to row * 128 + ((chunk ^ row % 8) * 16) of its
// wavefront's LDS tile; fragments are read back with lane (r = l % 16,
// g = l / 16) taking chunks g and 4 + g of row r -- 32 bytes, the same k set
// for weights and activations, so the product sums each k once.
template <int NTW, int KS, bool GATED>
struct Stream8 {
  static constexpr int D = kF8Depth;
  static constexpr int MT = kF8MT;
  static constexpr int NWN = 4 / KS;
  static constexpr int HT = GATED ? NTW / 2 : NTW;
  static constexpr int COLS = NWN * HT * 16;        // output columns per slab
  static constexpr int KSTEP = 128;
  static constexpr int TILE_BYTES = 16 * 128;
  static constexpr int WAVE_LDS = (NTW + MT) * TILE_BYTES;
  static constexpr int LDS_BYTES = 4 * WAVE_LDS;
  static_assert(!GATED || NTW % 2 == 0, "gated slabs pair gate and up tiles");
  static_assert(MT * NTW * 1024 <= WAVE_LDS, "K-slice partial sums fit in the wavefront's tiles");
  static_assert(HT * 16 <= kQBlock && kQBlock % (HT * 16) == 0, "a wavefront's tiles share a weight scale block");

  template <int MTA, bool NT>
  __device__ static void run_mt(const F8Args& a, int e, int lo, int m, int slab, char* smem) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = wave % KS, wn = wave / KS;
    const int fr = lane & 15, g = lane >> 4;
    const int lr = lane >> 3, lc = lane & 7;
    const int col0 = (slab * NWN + wn) * HT * 16;
    const uint32_t pitch = (uint32_t)a.K;          // bytes per row
    const int KB = a.K / kQBlock;

    // Weights and their block scales: one buffer per expert.
    const __amdgpu_buffer_rsrc_t wbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.W + (size_t)e * a.N * a.K), 0, (int)(a.N * pitch), kF8Config);
    const __amdgpu_buffer_rsrc_t wsbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.Ws + (size_t)e * (a.N / kQBlock) * KB), 0, (a.N / kQBlock) * KB * 4, kF8Config);
    const uint32_t wv = (uint32_t)(col0 + lr) * pitch + lc * 16;
    int wso[NTW][2], wsc[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int n0 = col0 + (t % HT) * 16 + ((GATED && t >= HT) ? a.inter : 0);
      wsc[t] = (n0 / kQBlock - col0 / kQBlock) * KB * 4;   // relative to the wavefront's first block row
#pragma unroll
      for (int h = 0; h < 2; ++h) wso[t][h] = ((t % HT) * 16 + h * 8 + ((GATED && t >= HT) ? a.inter : 0)) * (int)pitch;
    }
    const uint32_t wsv = (uint32_t)(col0 / kQBlock) * KB * 4;
    // Activations: rows past the chunk's end read its first row (their output
    // column is not stored). av: the load rows; sv: the row of the lane's
    // MFMA column, for its scale.
    const __amdgpu_buffer_rsrc_t abuf = __builtin_amdgcn_make_buffer_rsrc((void*)a.A, 0, -1, kF8Config);
    const __amdgpu_buffer_rsrc_t asbuf = __builtin_amdgcn_make_buffer_rsrc((void*)a.As, 0, -1, kF8Config);
    uint32_t av[MTA][2], sv[MTA];
#pragma unroll
    for (int i = 0; i < MTA; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = i * 16 + h * 8 + lr;
        av[i][h] = lo + (r < m ? r : 0);
      }
      const int r = i * 16 + fr;
      sv[i] = lo + (r < m ? r : 0);
    }
    f8_rows<MTA * 2>(a, &av[0][0]);
    f8_rows<MTA>(a, sv);
#pragma unroll
    for (int i = 0; i < MTA; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) av[i][h] = av[i][h] * pitch + lc * 16;
      sv[i] = sv[i] * (uint32_t)KB * 4;
    }

    char* xs = smem + wave * WAVE_LDS;
    const int woff[2] = {lr * 128 + ((lc ^ lr) << 4), (8 + lr) * 128 + ((lc ^ lr) << 4)};
    const int roff[2] = {fr * 128 + ((g ^ (fr & 7)) << 4), fr * 128 + (((4 + g) ^ (fr & 7)) << 4)};

    f32x4_t acc[MTA][NTW];
#pragma unroll
    for (int i = 0; i < MTA; ++i)
#pragma unroll
      for (int t = 0; t < NTW; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t wr[D][NTW][2], ar[D][MTA][2];
    float wsr[D][NTW], asr[D][MTA];
    auto load = [&](int q, int kk) {
      const int kb4 = (kk / kQBlock) * 4;
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          wr[q][t][h] = __builtin_amdgcn_raw_buffer_load_b128(wbuf, wv, wso[t][h] + kk, NT ? kF8NonTemporal : 0);
        wsr[q][t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(wsbuf, wsv, wsc[t] + kb4, 0));
      }
#pragma unroll
      for (int i = 0; i < MTA; ++i) {
#pragma unroll
        for (int h = 0; h < 2; ++h) ar[q][i][h] = __builtin_amdgcn_raw_buffer_load_b128(abuf, av[i][h], kk, 0);
        asr[q][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(asbuf, sv[i], kb4, 0));
      }
    };
    auto mma = [&](int q) {
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) *(u32x4_t*)(xs + t * TILE_BYTES + woff[h]) = wr[q][t][h];
#pragma unroll
      for (int i = 0; i < MTA; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) *(u32x4_t*)(xs + (NTW + i) * TILE_BYTES + woff[h]) = ar[q][i][h];
      i32x8_t wf[NTW], af[MTA];
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const i32x4_t lo4 = *(const i32x4_t*)(xs + t * TILE_BYTES + roff[0]);
        const i32x4_t hi4 = *(const i32x4_t*)(xs + t * TILE_BYTES + roff[1]);
        wf[t] = i32x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      }
#pragma unroll
      for (int i = 0; i < MTA; ++i) {
        const i32x4_t lo4 = *(const i32x4_t*)(xs + (NTW + i) * TILE_BYTES + roff[0]);
        const i32x4_t hi4 = *(const i32x4_t*)(xs + (NTW + i) * TILE_BYTES + roff[1]);
        af[i] = i32x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      }
      f32x4_t p[MTA][NTW];
#pragma unroll
      for (int i = 0; i < MTA; ++i)
#pragma unroll
        for (int t = 0; t < NTW; ++t)
          p[i][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[t], af[i], f32x4_t{0.f, 0.f, 0.f, 0.f},
                                                                     0, 0, 0, 127, 0, 127);
#pragma unroll
      for (int i = 0; i < MTA; ++i)
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const float sc = asr[q][i] * wsr[q][t];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][t][r] = fmaf(p[i][t][r], sc, acc[i][t][r]);
        }
    };

    // Step s issues the loads of step s + D - 1 (steps past the end reload the
    // last one), then consumes step s; loads complete in issue order, so each
    // step waits only for its own data.
    const int kw = a.K / KS, kbeg = ks * kw, klast = kbeg + kw - KSTEP;
    const int steps = kw / KSTEP;
#pragma unroll
    for (int j = 0; j < D - 1; ++j) load(j, min(kbeg + j * KSTEP, klast));
    int kk = kbeg, s = 0;
#define MOE_F8_STEP(q)                                   \
  load(((q) + D - 1) % D, min(kk + (D - 1) * KSTEP, klast)); \
  __builtin_amdgcn_sched_barrier(0);                     \
  mma((q) % D);                                          \
  __builtin_amdgcn_sched_barrier(0);                     \
  kk += KSTEP;
    for (; s + D <= steps; s += D) {
#pragma unroll
      for (int q = 0; q < D; ++q) { MOE_F8_STEP(q) }
    }
#pragma unroll
    for (int q = 0; q < D - 1; ++q) {
      if (s + q >= steps) break;
      MOE_F8_STEP(q)
    }
#undef MOE_F8_STEP

    if (KS > 1) {
      f32x4_t* red = (f32x4_t*)xs;
#pragma unroll
      for (int i = 0; i < MTA; ++i)
#pragma unroll
        for (int t = 0; t < NTW; ++t) red[(i * NTW + t) * 64 + lane] = acc[i][t];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MTA; ++i) {
        if (i % KS != ks) continue;
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          f32x4_t sum = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int q = 0; q < KS; ++q)
            sum += ((const f32x4_t*)(smem + (wn * KS + q) * WAVE_LDS))[(i * NTW + t) * 64 + lane];
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
      if (GATED) {
        float* crow = (float*)a.C + (size_t)(lo + row) * a.ldc + col0 + g * 4;
#pragma unroll
        for (int t = 0; t < HT; ++t) {
          f32x4_t v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = silu_f(acc[i][t][r]) * acc[i][t + HT][r];
          *(f32x4_t*)(crow + t * 16) = v;
        }
      } else {
        uint16_t* crow = (uint16_t*)a.C + (size_t)(lo + row) * a.ldc + col0 + g * 4;
#pragma unroll
        for (int t = 0; t < HT; ++t) {
          const f32x4_t v = acc[i][t];
          *(uint2*)(crow + t * 16) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
      }
    }
  }

  // The rows of expert e (at most kF8Rows), output slab `slab`. The expert's
  // weights are read once per GEMM, non-temporally.
  __device__ static void run(const F8Args& a, const int* c_lo, int e, int slab, char* smem) {
    e = __builtin_amdgcn_readfirstlane(e);
    const int lo = __builtin_amdgcn_readfirstlane(c_lo[e]);
    const int m = __builtin_amdgcn_readfirstlane(min(kF8Rows, c_lo[e + 1] - lo));
    slab = __builtin_amdgcn_readfirstlane(slab);
    switch ((m + 15) >> 4) {
      case 1: run_mt<1, true>(a, e, lo, m, slab, smem); break;
      case 2: run_mt<2, true>(a, e, lo, m, slab, smem); break;
      case 3: run_mt<3, true>(a, e, lo, m, slab, smem); break;
      default: run_mt<4, true>(a, e, lo, m, slab, smem); break;
    }
  }
};

// ---------------------------------------------------------------- large-tile path

// Experts with more than kF8Rows rows when their 256-row tiles fill the GPU
// (prefill; f8_big_takes): 256 weight rows x 256 tokens per tile, one
// workgroup of 8 wavefronts per CU, two per SIMD, so that one wavefront's
// scale arithmetic runs while the other's MFMAs do. Wavefront w = 2 wm + wn
// multiplies tile weight rows wm*64 .. +63 (fragments i = 0..3 of 16 rows)
// by the token fragments 2j + wn (16 rows each, j = 0..7) on
// v_mfma_scale_f32_16x16x128_f8f6f4: one instruction per fragment pair and K
// step, i.e. per scale block, so its float32 result is added at once with
// the factor row scale x weight block scale (4 accumulators per pair, 128
// per lane). Only the token fragments that hold a valid row are multiplied
// (NJ of them, rounded up to even; a template argument so that the stage
// stays fully unrolled).
//
// K is staged 128 at a time (128 bytes of every row) in two 64 KB LDS
// buffers filled by LDS DMA: per stage each wavefront copies 4 blocks of 8
// weight rows and 4 blocks of 8 token rows (one instruction each, whole
// 128-byte lines), and wavefronts 0..3 copy the stage's 256 token scales
// (one dword instruction each), issued one per few MFMAs over the first half
// of the previous stage. Chunk c (16 bytes) of LDS row r sits at slot
// c ^ ((r >> 1) & 7): the 16 rows of a fragment read fall on 16 distinct
// 16-byte bank groups; the DMA writes 8 rows in lane order (lane l: row
// l / 8, slot l % 8), so in block b lane l fetches chunk
// (l % 8) ^ (4 (b % 2) + l / 16). A fragment read gives lane (r = l % 16,
// g = l / 16) chunks g and 4 + g of its row, the same bytes for weights and
// tokens.
//
// Gated tiles hold 128 output columns: wavefront row wm has the 32 gate rows
// of columns wm*32 .. +31 (fragments 0, 1) and then the 32 matching up rows
// (fragments 2, 3), so SiLU(gate) * up is formed from its own accumulators.
// Weight rows of a fragment lie in one 128-row scale block.
template <bool GATED>
struct Big8 {
  static constexpr int COLS = GATED ? 128 : 256;           // output columns per tile
  static constexpr int OP_BYTES = 256 * 128;                // one operand of one stage
  static constexpr int STAGE_BYTES = 2 * OP_BYTES;
  static constexpr int SCALE_OFF = 2 * STAGE_BYTES;         // token scales: [buffer][256] float
  static constexpr int AMAX_OFF = SCALE_OFF + 2 * 1024;     // gated: h's row maxima [wm][256] float
  static constexpr int LDS_BYTES = AMAX_OFF + (GATED ? 4 * 1024 : 0);
  static constexpr int DMA = 9;   // DMA instructions per wavefront per stage (wavefronts 4..7: 8)

  __device__ static void run(const F8Args& a, int e, int row0, int rows, int nb, char* lds, const F8QOut* qo,
                             int tid) {
    const int wn = __builtin_amdgcn_readfirstlane(tid >> 6) & 1;
    const int nf = (rows + 15) >> 4;   // token fragments holding a valid row
    const int nj = __builtin_amdgcn_readfirstlane(min(8, (((nf - wn + 1) >> 1) + 1) & ~1));
    switch (nj) {
      case 8: body<8>(a, e, row0, rows, nb, lds, qo, tid); break;
      case 6: body<6>(a, e, row0, rows, nb, lds, qo, tid); break;
      case 4: body<4>(a, e, row0, rows, nb, lds, qo, tid); break;
      case 2: body<2>(a, e, row0, rows, nb, lds, qo, tid); break;
      default: body<0>(a, e, row0, rows, nb, lds, qo, tid); break;
    }
  }

  // MFMA of a stage after which DMA instruction d of the next stage is
  // issued: spread evenly over the first half of the stage's 4 NJ MFMAs.
  template <int NJ>
  __device__ static constexpr int dma_after(int d) {
    const int m = (d + 1) * (2 * NJ) / DMA - 1;
    return m < 0 ? 0 : m;
  }

  template <int NJ>
  __device__ static void body(const F8Args& a, int e, int row0, int rows, int nb, char* lds, const F8QOut* qo,
                              int tid) {
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const uint32_t pitch = (uint32_t)a.K;
    const int KB = a.K / kQBlock;
    const int lrow = lane >> 3;                            // row within an 8-row DMA block
    const int lchunk = (lane & 7) ^ (lane >> 4);           // chunk fetched in even blocks
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);

    // DMA blocks b = 4 wave + d (d = 0..3) of both operands; odd blocks
    // fetch chunk lchunk ^ 4. Weights: the wavefront's 4 blocks are the 32
    // tile rows of group `wave` (gated: wavefront row wave / 2, gate rows for
    // even groups, up rows for odd ones), consecutive weight rows from the
    // first one: block d starts 8 d rows further.
    const i32x4_t wbuf = buffer_rsrc(a.W + (size_t)e * a.N * a.K, (uint32_t)(a.N * pitch));
    const int wfirst = GATED ? ((wave & 1) ? a.inter : 0) + nb * COLS + (wave >> 1) * 32 : nb * COLS + wave * 32;
    const int wso0 = __builtin_amdgcn_readfirstlane(wfirst * (int)pitch);
    const int wstep = __builtin_amdgcn_readfirstlane(8 * (int)pitch);
    const uint32_t wv[2] = {(uint32_t)lrow * pitch + lchunk * 16, (uint32_t)lrow * pitch + (lchunk ^ 4) * 16};
    // Tokens: rows past the tile's end read its first row (not stored).
    const i32x4_t xbuf = buffer_rsrc(a.A, 0xFFFFFFFFu);
    uint32_t xv[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int r = (wave * 4 + d) * 8 + lrow;
      xv[d] = row0 + (r < rows ? r : 0);
    }
    f8_rows<4>(a, xv);
#pragma unroll
    for (int d = 0; d < 4; ++d) xv[d] = xv[d] * pitch + (lchunk ^ ((d & 1) << 2)) * 16;

    // Scales. The stage's 256 token scales go to LDS with the operands:
    // wavefronts 0..3 copy them with one dword DMA each (lane l: token
    // 64 wave + l). Weight blocks of the wavefront's fragments (uniform):
    // gated gate and up, plain one block for all four; loaded a stage ahead
    // through per-lane addresses (the kernel has no scalar registers left
    // for another buffer resource).
    const int fr = lane & 15, fg = lane >> 4;
    uint32_t svoff = 0;
    if (wave < 4) {
      const int t = wave * 64 + lane;
      uint32_t r[1] = {(uint32_t)(row0 + (t < rows ? t : 0))};
      f8_rows<1>(a, r);
      svoff = r[0] * (uint32_t)KB * 4;
    }
    const i32x4_t asbuf = buffer_rsrc(a.As, 0xFFFFFFFFu);
    constexpr int NW = GATED ? 2 : 1;   // weight scale blocks per wavefront
    const float* wsp[NW];
    {
      const float* we = a.Ws + (size_t)e * (a.N / kQBlock) * KB;
      int blk0 = GATED ? (nb * COLS) / kQBlock : (nb * COLS + wm * 64) / kQBlock;
      asm volatile("" : "+v"(blk0));
      wsp[0] = we + (size_t)blk0 * KB;
      if (GATED) wsp[NW - 1] = wsp[0] + (size_t)(a.inter / kQBlock) * KB;
    }

    // DMA number d of this wavefront's share of stage kt: weight blocks
    // first, then token blocks, then (wavefronts 0..3) the token scales.
    auto issue_one = [&](int kt, int d) {
      // (opaque, so that the 9 LDS addresses of each buffer are formed at
      // their instructions rather than held in scalar registers)
      uint32_t ls = lds_base + (kt & 1) * STAGE_BYTES;
      asm volatile("" : "+s"(ls));
      const uint32_t ko = (uint32_t)kt * 128;
      if (d < 4) lds_dma16(ls + (wave * 4 + d) * 1024, wbuf, wv[d & 1], wso0 + d * wstep + ko);
      else if (d < 8) lds_dma16(ls + OP_BYTES + (wave * 4 + d - 4) * 1024, xbuf, xv[d - 4], ko);
      else if (wave < 4) lds_dma4(ls - (kt & 1) * STAGE_BYTES + SCALE_OFF + (kt & 1) * 1024 + wave * 256, asbuf, svoff,
                                  kt * 4);
    };
    float sw[NW];
    auto load_scales = [&](int kt) {
#pragma unroll
      for (int i = 0; i < NW; ++i) sw[i] = wsp[i][kt];
    };

    f32x4_t acc[4][NJ > 0 ? NJ : 1];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int fsw = (fr >> 1) & 7;
    const int off0 = (fg ^ fsw) << 4, off1 = ((4 + fg) ^ fsw) << 4;
    // Multiplies stage `slot` (its weight scales in sw, token scales in LDS):
    // takes the weight scales, loads stage knext's (if knext >= 0) in their
    // place, and issues the DMA of stage knext into the other buffers over
    // the MFMAs.
    auto compute = [&](int slot, int knext) {
      if (NJ == 0) {
        if (knext >= 0) {
#pragma unroll
          for (int d = 0; d < DMA; ++d) issue_one(knext, d);
        }
        return;
      }
      float swc[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) swc[w] = sw[w];
      if (knext >= 0) load_scales(knext);
      const float* ssa = (const float*)(lds + SCALE_OFF + slot * 1024) + wn * 16 + fr;
      const char* lw = lds + slot * STAGE_BYTES + (wm * 64 + fr) * 128;
      const char* lx = lds + slot * STAGE_BYTES + OP_BYTES + (wn * 16 + fr) * 128;
      i32x8_t af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x4_t lo4 = *(const i32x4_t*)(lw + i * 16 * 128 + off0);
        const i32x4_t hi4 = *(const i32x4_t*)(lw + i * 16 * 128 + off1);
        af[i] = i32x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float sa = ssa[j * 32];   // token (2j + wn)*16 + lane%16
        float sc[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) sc[w] = swc[w] * sa;
        i32x8_t bcur;
        {
          const i32x4_t lo4 = *(const i32x4_t*)(lx + j * 32 * 128 + off0);
          const i32x4_t hi4 = *(const i32x4_t*)(lx + j * 32 * 128 + off1);
          bcur = i32x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4_t p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af[i], bcur, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
          const float c = sc[GATED ? (i >> 1) : 0];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(p[r], c, acc[i][j][r]);
          const int m = j * 4 + i;   // MFMA number within the stage
#pragma unroll
          for (int d = 0; d < DMA; ++d) {
            if (dma_after<NJ>(d) == m) {
              __builtin_amdgcn_sched_barrier(0);
              if (knext >= 0) issue_one(knext, d);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      }
    };

    // Iteration kt: wait until this wavefront's DMA and scale loads of stage
    // kt have landed, barrier (every wavefront's share of stage kt is in LDS,
    // and every wavefront has finished stage kt - 1, whose buffers stage
    // kt + 1 reuses), multiply stage kt while loading stage kt + 1.
    const int nk = a.K / 128;
#pragma unroll
    for (int d = 0; d < DMA; ++d) issue_one(0, d);
    load_scales(0);
    for (int kt = 0; kt < nk; ++kt) {
      wait_vmcnt<0>();
      __syncthreads();
      compute(kt & 1, kt + 1 < nk ? kt + 1 : -1);
    }

    // acc[i][j][q]: token (2j + wn)*16 + lane%16; wavefront weight row
    // i*16 + 4*(lane/16) + q. C's rows are dense (ldc = inter for h, N for
    // o), which saves the kernel a scalar register.
    if (GATED) {
      // h = SiLU(gate) * up in float32, and its e4m3 codes: the tile's 128
      // output columns are one scale block of every token row, the four
      // wavefront rows (wm) each hold 32 of them, so the row maxima are
      // combined through LDS. The arithmetic is that of quantize_rows_kernel.
      float h[NJ > 0 ? NJ : 1][8];
      float* amax_part = (float*)(lds + AMAX_OFF);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int t = (2 * j + wn) * 16 + fr;
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            h[j][i * 4 + q] = silu_f(acc[i][j][q]) * acc[i + 2][j][q];
            m = fmaxf(m, fabsf(h[j][i * 4 + q]));
          }
        if (t < rows) {
          float* crow = (float*)a.C + (size_t)(row0 + t) * a.inter + nb * COLS + wm * 32 + fg * 4;
#pragma unroll
          for (int i = 0; i < 2; ++i)
            *(f32x4_t*)(crow + i * 16) = f32x4_t{h[j][i * 4], h[j][i * 4 + 1], h[j][i * 4 + 2], h[j][i * 4 + 3]};
        }
        m = fmaxf(m, __shfl_xor(m, 16, MOE_WAVE));
        m = fmaxf(m, __shfl_xor(m, 32, MOE_WAVE));
        if (fg == 0) amax_part[wm * 256 + t] = m;
      }
      {
        __syncthreads();   // every wavefront reaches it once (also with NJ = 0)
        uint8_t* const cq = qo->q;
        float* const cs = qo->s;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int t = (2 * j + wn) * 16 + fr;
          if (t >= rows) continue;
          const float amax = fmaxf(fmaxf(amax_part[t], amax_part[256 + t]),
                                   fmaxf(amax_part[512 + t], amax_part[768 + t]));
          const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
          const double rs = 1.0 / (double)sc;
          uint8_t* qrow = cq + (size_t)(row0 + t) * a.inter + nb * COLS + wm * 32 + fg * 4;
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const uint32_t c = e4m3_pack4(div_by_scale(h[j][i * 4], rs), div_by_scale(h[j][i * 4 + 1], rs),
                                          div_by_scale(h[j][i * 4 + 2], rs), div_by_scale(h[j][i * 4 + 3], rs));
            *(uint32_t*)(qrow + i * 16) = c;
          }
          if (wm == 0 && fg == 0) cs[(size_t)(row0 + t) * (a.inter / kQBlock) + nb] = sc;
        }
      }
    } else {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int t = (2 * j + wn) * 16 + fr;
      if (t >= rows) continue;
      {
        uint16_t* crow = (uint16_t*)a.C + (size_t)(row0 + t) * a.N + nb * COLS + wm * 64 + fg * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4_t& c = acc[i][j];
          *(uint2*)(crow + i * 16) = make_uint2(pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3]));
        }
      }
    }
    }
  }
};

// The large tiles take every expert with more than kF8Rows rows when their
// items (256-row tiles x N blocks) fill at least 3/4 of the CUs in the first
// round; else the 128 x 128 tiles of ffn_fp8_kernel do.
__device__ __forceinline__ bool f8_big_takes(int items, int cus) { return 4 * items >= 3 * cus; }

// The FFN's h quantiser at prefill sizes: when ffn_fp8_big_kernel takes the
// experts above kF8Rows rows (the same decision, from the same offsets) it
// has written their codes itself, so only the other experts' rows are
// quantised here; else every row. The rows to quantise are numbered
// expert after expert (q_first[e] = those before expert e); a wavefront item
// is 4 blocks of one of them (kQItems items per pass), as in
// quantize_rows_kernel.
__global__ __launch_bounds__(256) void quantize_h_kernel(const float* __restrict__ h, const int* __restrict__ offsets,
                                                         int nloc, int capacity, int cols, int big_ok, int cus,
                                                         uint8_t* __restrict__ codes, float* __restrict__ scales) {
  __shared__ int s_lo[kF8MaxLocal + 1];
  __shared__ int q_first[kF8MaxLocal + 1];
  __shared__ int wsum[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int m4[4], cb = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    m4[q] = 0;
    if (e < nloc) {
      const int lo = min(offsets[e], capacity);
      const int hi = min(offsets[e + 1], capacity);
      m4[q] = max(0, hi - lo);
      s_lo[e] = lo;
      if (e == nloc - 1) s_lo[nloc] = max(lo, hi);
      cb += m4[q] > kF8Rows ? (m4[q] + kB8Rows - 1) / kB8Rows : 0;
    }
  }
  cb = wave_sum_i32(cb);
  if (lane == 0) wsum[wave] = cb;
  __syncthreads();
  const bool big = big_ok && f8_big_takes((wsum[0] + wsum[1] + wsum[2] + wsum[3]) * (cols / Big8<true>::COLS), cus);
  int qc[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    qc[q] = (big && m4[q] > kF8Rows) ? 0 : m4[q];
    sum += qc[q];
  }
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, MOE_WAVE);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wsum[4 + wave] = incl;
  __syncthreads();
  int before = 0, n_q = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < wave) before += wsum[4 + i];
    n_q += wsum[4 + i];
  }
  int p = before + incl - sum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    if (e < nloc) q_first[e] = p;
    p += qc[q];
  }
  if (tid == 0) q_first[nloc] = n_q;
  __syncthreads();

  const int nb = cols / kQBlock;
  const int groups = (nb + 3) / 4;
  const long total = (long)n_q * groups;
  const long stride = (long)gridDim.x * 4;
  for (long w0 = (long)blockIdx.x * 4 + wave; w0 < total; w0 += stride * kQItems) {
    const int cnt = (int)min((long)kQItems, (total - w0 + stride - 1) / stride);
    float v[kQItems][8];
    size_t first[kQItems];
    int row[kQItems], blk[kQItems];
    bool active[kQItems];
#pragma unroll
    for (int u = 0; u < kQItems; ++u) {
      active[u] = false;
      row[u] = blk[u] = 0;
      first[u] = 0;
      if (u < cnt) {
        const long w = w0 + u * stride;
        const int qi = (int)(w / groups);
        int e = 0, hi = nloc - 1;   // the expert whose rows to quantise hold number qi
        while (e < hi) {
          const int mid = (e + hi + 1) >> 1;
          if (q_first[mid] <= qi) e = mid; else hi = mid - 1;
        }
        const int r = s_lo[e] + (qi - q_first[e]);
        row[u] = r;
        blk[u] = (int)(w - (long)qi * groups) * 4 + (lane >> 4);
        active[u] = blk[u] < nb;
        first[u] = (size_t)r * cols + (size_t)blk[u] * kQBlock + (lane & 15) * 8;
      }
      if (active[u]) {
        const f32x4_t p0 = *(const f32x4_t*)(h + first[u]);
        const f32x4_t p1 = *(const f32x4_t*)(h + first[u] + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[u][j] = p0[j];
          v[u][4 + j] = p1[j];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[u][j] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kQItems; ++u) {
      if (u >= cnt) break;
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[u][j]));
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, MOE_WAVE));
      if (!active[u]) continue;
      const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
      const double rs = 1.0 / (double)s;
      float q[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) q[j] = div_by_scale(v[u][j], rs);
      const uint32_t lo = e4m3_pack4(q[0], q[1], q[2], q[3]), hi = e4m3_pack4(q[4], q[5], q[6], q[7]);
      *(uint2*)(codes + first[u]) = make_uint2(lo, hi);
      if ((lane & 15) == 0) scales[(size_t)row[u] * nb + blk[u]] = s;
    }
  }
}

// Tile of kT8Rows tokens x 128 weight rows (experts with more than kF8Rows
// rows). Thread (rbase = tid / 8, kc = tid % 8) loads the 16-byte chunk kc
// of tile rows rbase + 32 i (i = 0..3) of both operands per K step; chunk c
// of LDS row r sits at slot c ^ (r % 8), so 8 threads store one row's 128
// bytes and the 32 rows a fragment read touches per chunk spread over the
// banks. Wavefront (wm, wn) multiplies weight rows wm*64.. by tokens wn*64..:
// 2 x 2 fragments of 32 x 32. MFMA u (0, 1) of a fragment pair takes chunks
// 4u + 2 fh and 4u + 2 fh + 1 of its row for lane half fh, the same bytes for
// weights and tokens, so the two instructions sum each k of the step once.
//
// A gated tile holds 64 output columns: tile rows [gate 32 | up 32] for
// wavefront row 0, then for row 1, so fragment 0 (gate) and fragment 1 (up)
// of a wavefront cover the same columns and SiLU(gate) * up is formed from
// its own accumulators. Weight rows of a fragment lie in one 128-row scale
// block (32 | 128), so a lane's partial of a step takes one factor: its
// token's row scale x the fragment's weight block scale.
template <bool GATED>
struct Tiled8 {
  static constexpr int COLS = GATED ? 64 : 128;     // output columns per tile
  static constexpr int OP = 128 * 128;               // bytes of one operand tile (128 rows x 128 k)
  static constexpr int LDS_BYTES = 2 * 2 * OP;       // [buffer][W | X]

  __device__ static __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

  __device__ static void run(const F8Args& a, int e, int row0, int rows, int nb, char* lds) {
    // the thread index passes through an empty asm statement, so the
    // compiler derives this item's lane offsets here instead of keeping them
    // in registers across the persistent loop (where the streaming path
    // needs them)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int kc = tid & 7, rbase = tid >> 3;
    const int fr = lane & 31, fh = lane >> 5;
    const uint32_t pitch = (uint32_t)a.K;
    const int KB = a.K / kQBlock;

    const __amdgpu_buffer_rsrc_t wbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.W + (size_t)e * a.N * a.K), 0, (int)(a.N * pitch), kF8Config);
    const __amdgpu_buffer_rsrc_t wsbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.Ws + (size_t)e * (a.N / kQBlock) * KB), 0, (a.N / kQBlock) * KB * 4, kF8Config);
    const __amdgpu_buffer_rsrc_t abuf = __builtin_amdgcn_make_buffer_rsrc((void*)a.A, 0, -1, kF8Config);
    const __amdgpu_buffer_rsrc_t asbuf = __builtin_amdgcn_make_buffer_rsrc((void*)a.As, 0, -1, kF8Config);

    // This thread's weight rows (loads) and token rows (rows past the tile's
    // end read its first row; their outputs are not stored).
    uint32_t wv[4], xv[4], sv[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int wr = GATED ? nb * COLS + rbase + ((i & 1) ? a.inter : 0) + (i >> 1) * 32
                           : nb * COLS + rbase + 32 * i;
      wv[i] = (uint32_t)wr * pitch + kc * 16;
      const int r = rbase + 32 * i;
      xv[i] = (uint32_t)(row0 + (r < rows ? r : 0));
    }
    // the rows of the lane's two MFMA columns, for their scales
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = wn * 64 + j * 32 + fr;
      sv[j] = (uint32_t)(row0 + (t < rows ? t : 0));
    }
    f8_rows<4>(a, xv);
    f8_rows<2>(a, sv);
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = xv[i] * pitch + kc * 16;
#pragma unroll
    for (int j = 0; j < 2; ++j) sv[j] = sv[j] * (uint32_t)KB * 4;
    // weight scale block of the wavefront's fragments (gated: gate, up)
    int wsb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int n0 = GATED ? nb * COLS + wm * 32 + (i ? a.inter : 0) : nb * COLS + wm * 64 + i * 32;
      wsb[i] = __builtin_amdgcn_readfirstlane((n0 / kQBlock) * KB * 4);
    }

    u32x4_t gw[4], gx[4];
    float gsa[2], gsw[2];
    auto gload = [&](int kt) {
      const int k0 = kt * 128;
#pragma unroll
      for (int i = 0; i < 4; ++i) gw[i] = __builtin_amdgcn_raw_buffer_load_b128(wbuf, wv[i], k0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) gx[i] = __builtin_amdgcn_raw_buffer_load_b128(abuf, xv[i], k0, 0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        gsa[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(asbuf, sv[j], kt * 4, 0));
#pragma unroll
      for (int i = 0; i < 2; ++i)
        gsw[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(wsbuf, 0, wsb[i] + kt * 4, 0));
    };
    auto sstore = [&](int buf) {
      char* lw = lds + buf * 2 * OP;
      char* lx = lw + OP;
#pragma unroll
      for (int i = 0; i < 4; ++i) *(u32x4_t*)(lw + swz(rbase + 32 * i, kc)) = gw[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) *(u32x4_t*)(lx + swz(rbase + 32 * i, kc)) = gx[i];
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

    const int nk = a.K / 128;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      float sc[2][2];   // this step's factors, taken before the next step's loads replace them
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) sc[i][j] = gsw[i] * gsa[j];
      if (kt + 1 < nk) gload(kt + 1);
      const char* lw = lds + buf * 2 * OP;
      const char* lx = lw + OP;
      f32x16_t p[2][2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c0 = 4 * u + 2 * fh;
        i32x8_t af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = wm * 64 + i * 32 + fr;
          const i32x4_t lo4 = *(const i32x4_t*)(lw + swz(r, c0));
          const i32x4_t hi4 = *(const i32x4_t*)(lw + swz(r, c0 + 1));
          af[i] = i32x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r = wn * 64 + j * 32 + fr;
          const i32x4_t lo4 = *(const i32x4_t*)(lx + swz(r, c0));
          const i32x4_t hi4 = *(const i32x4_t*)(lx + swz(r, c0 + 1));
          bfr[j] = i32x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            p[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bfr[j], u ? p[i][j] : f32x16_t{}, 0,
                                                                      0, 0, 127, 0, 127);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(p[i][j][r], sc[i][j], acc[i][j][r]);
      if (kt + 1 < nk) sstore(buf ^ 1);
      __syncthreads();
    }

    // acc[i][j][r]: token wn*64 + j*32 + lane%32; tile row wm*64 + i*32 +
    // (r/4)*8 + (lane/32)*4 + r%4.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = wn * 64 + j * 32 + fr;
      if (t >= rows) continue;
      if (GATED) {
        float* crow = (float*)a.C + (size_t)(row0 + t) * a.ldc;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = nb * COLS + wm * 32 + q * 8 + fh * 4;
          f32x4_t v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = silu_f(acc[0][j][q * 4 + r]) * acc[1][j][q * 4 + r];
          *(f32x4_t*)(crow + col) = v;
        }
      } else {
        uint16_t* crow = (uint16_t*)a.C + (size_t)(row0 + t) * a.ldc;
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

template <int NTW, int KS, bool GATED>
__global__ __launch_bounds__(256, 2) void ffn_fp8_kernel(F8Args a) {
  using S = Stream8<NTW, KS, GATED>;
  using T = Tiled8<GATED>;
  constexpr int SMEM = S::LDS_BYTES > T::LDS_BYTES ? S::LDS_BYTES : T::LDS_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  __shared__ int c_first[kF8MaxLocal + 1];
  __shared__ int t_first[kF8MaxLocal + 1];
  __shared__ int c_lo[kF8MaxLocal + 1];
  __shared__ int wsum[12];
  int chunks, tiles, n_big;
  f8_lists(a, kT8Rows, c_first, t_first, c_lo, wsum, chunks, tiles, n_big);
  const int ncols = GATED ? a.inter : a.N;
  const int slabs = ncols / S::COLS;
  const int nblk = ncols / T::COLS;
  const int n_stream = chunks * slabs;
  // the same decision as ffn_fp8_big_kernel's: when it takes the tiled
  // experts only the streamed ones are done here
  const bool big = a.big_ok && f8_big_takes(n_big * (ncols / Big8<GATED>::COLS), a.big_min_items);
  const int total = n_stream + (big ? 0 : tiles * nblk);
  // streamed chunks first, then the tiles with their N blocks fastest
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    if (w < n_stream) {
      const int c = w / slabs;
      const int e = f8_find_expert(c_first, a.nloc, c);
      S::run(a, c_lo, e, w % slabs, smem);
    } else {
      const int tile = (w - n_stream) / nblk, nb = (w - n_stream) % nblk;
      const int e = __builtin_amdgcn_readfirstlane(f8_find_expert(t_first, a.nloc, tile));
      const int row0 = __builtin_amdgcn_readfirstlane(c_lo[e] + (tile - t_first[e]) * kT8Rows);
      const int rows = __builtin_amdgcn_readfirstlane(min(kT8Rows, c_lo[e + 1] - row0));
      T::run(a, e, row0, rows, __builtin_amdgcn_readfirstlane(nb), smem);
    }
    __syncthreads();  // the LDS buffer is reused by the next work item
  }
}

// Tiles of the experts with more than kF8Rows rows, 256 tokens each; a
// persistent loop over them, one workgroup of 8 wavefronts per CU. Items are
// (token tile, N block) with N blocks fastest, taken round-robin by a grid
// that is a multiple of 8 (workgroup b runs on XCD b % 8), so the items of
// one N block -- the same weight rows for every tile of an expert -- share
// an XCD's L2 when the N blocks per tile are a multiple of 8; when all items
// fit in one round the N blocks are numbered up to a multiple of 8 (the
// padding items are skipped).
template <bool GATED>
__global__ __launch_bounds__(512, 1) void ffn_fp8_big_kernel(F8Args a) {
  using B = Big8<GATED>;
  __shared__ __attribute__((aligned(16))) char smem[B::LDS_BYTES];
  __shared__ int c_first[kF8MaxLocal + 1];
  __shared__ int t_first[kF8MaxLocal + 1];
  __shared__ int c_lo[kF8MaxLocal + 1];
  __shared__ int wsum[12];
  // the codes and scales outputs, read back from LDS in the epilogue only
  // (held in scalar registers they would not fit beside the K loop's)
  __shared__ F8QOut s_qout;
  if (threadIdx.x == 0) s_qout = F8QOut{a.Cq, a.Cs};
  int chunks, tiles, n_big;
  f8_lists(a, kB8Rows, c_first, t_first, c_lo, wsum, chunks, tiles, n_big);   // (its barriers publish s_qout)
  const int nblk = (GATED ? a.inter : a.N) / B::COLS;
  if (!f8_big_takes(n_big * nblk, a.big_min_items)) return;   // ffn_fp8_kernel does these experts
  const int nblk8 = (nblk + 7) & ~7;
  const int nbp = __builtin_amdgcn_readfirstlane(n_big * nblk8 <= (int)gridDim.x ? nblk8 : nblk);
  const int total = n_big * nbp;
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    if (w % nbp >= nblk) continue;
    const int tile = __builtin_amdgcn_readfirstlane(w / nbp);
    const int nb = __builtin_amdgcn_readfirstlane(w % nbp);
    int nloc = a.nloc;
    asm volatile("" : "+s"(nloc));
    const int e = __builtin_amdgcn_readfirstlane(f8_find_expert(t_first, nloc, tile));
    const int row0 = __builtin_amdgcn_readfirstlane(c_lo[e] + (tile - t_first[e]) * kB8Rows);
    const int rows = __builtin_amdgcn_readfirstlane(min(kB8Rows, c_lo[e + 1] - row0));
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));  // keeps per-thread setup inside the tile loop
    // likewise the arguments: read again per tile from the kernel argument
    // segment (the only argument is `a`, at its start) through an opaque
    // pointer, so that they and what is derived from them are not held in
    // scalar registers across the loop
    KernargF8Args* ka = (KernargF8Args*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(ka));
    const F8Args at = f8_args_copy(ka);
    B::run(at, e, row0, rows, nb, smem, &s_qout, tid);
    __syncthreads();  // the LDS buffers are reused by the next tile
  }
}

int f8_cu_count() {
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

// Tiled experts go to ffn_fp8_big_kernel when the row capacity is
// prefill-sized and (on the device) its tiles fill at least 3/4 of the CUs
// (f8_big_takes); else to the 128 x 128 tiles of ffn_fp8_kernel. Both paths
// are complete; the capacity test keeps decode-sized calls from paying for a
// second launch that finds no work.
template <bool GATED>
bool fp8_big_ok(const F8Args& g) {
  return g.capacity >= kB8MinCapacity && (GATED ? g.inter % 128 == 0 : g.N % 256 == 0);
}

template <int NTW, int KS, bool GATED>
hipError_t launch_fp8_gemm(const F8Args& g0, hipStream_t s) {
  using S = Stream8<NTW, KS, GATED>;
  F8Args g = g0;
  g.big_ok = fp8_big_ok<GATED>(g) ? 1 : 0;
  g.big_min_items = f8_cu_count();
  auto kernel = ffn_fp8_kernel<NTW, KS, GATED>;
  static const int occ = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, ffn_fp8_kernel<NTW, KS, GATED>, 256, 0) != hipSuccess ||
        n <= 0)
      n = 1;
    return n;
  }();
  const int ncols = GATED ? g.inter : g.N;
  // at most min(nloc, capacity) streamed experts, or capacity / kT8Rows + nloc tiles
  const long max_work = std::max<long>(std::min<long>(g.nloc, g.capacity) * (ncols / S::COLS),
                                       ((long)g.capacity / kT8Rows + g.nloc) * (ncols / Tiled8<GATED>::COLS));
  const int grid = (int)std::max<long>(1, std::min<long>(max_work, (long)f8_cu_count() * occ));
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, s, g);
  if (!g.big_ok) return hipGetLastError();
  // tiles <= ceil(capacity / 256) + (number of experts above kF8Rows rows)
  const long max_big = ((long)(g.capacity + kB8Rows - 1) / kB8Rows +
                        std::min<long>(g.nloc, (long)g.capacity / (kF8Rows + 1))) *
                       (ncols / Big8<GATED>::COLS);
  // persistent: one workgroup per CU (a multiple of 8, so each keeps its XCD)
  const long cus8 = std::max(8, f8_cu_count() / 8 * 8);
  const int grid_big = (int)std::max<long>(8, std::min<long>((max_big + 7) / 8 * 8, cus8));
  hipLaunchKernelGGL(ffn_fp8_big_kernel<GATED>, dim3(grid_big), dim3(512), 0, s, g);
  return hipGetLastError();
}

inline size_t f8_align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workgroups of 4 wavefronts for rows x ceil(cols / 512) wavefront items: one
// item per wavefront while they fit in max_per_cu workgroups per CU, else
// that many workgroups.
int quantize_grid(long rows, int cols, int max_per_cu) {
  const long items = rows * ((cols / kQBlock + 3) / 4);
  return (int)std::max<long>(1, std::min<long>((items + 3) / 4, (long)f8_cu_count() * max_per_cu));
}

// Launches the quantiser on `grid` workgroups: kQItems items per wavefront
// pass when rows (an upper bound with rows_dev) has more items than the grid
// has wavefronts, else one.
template <bool BF16_IN>
void launch_quantize(int grid, const void* in, int rows, const int* rows_dev, int cols, uint8_t* codes,
                     float* scales, hipStream_t s) {
  const long items = (long)rows * ((cols / kQBlock + 3) / 4);
  if (items > (long)grid * 4)
    hipLaunchKernelGGL((quantize_rows_kernel<BF16_IN, kQItems>), dim3(grid), dim3(256), 0, s, in, rows, rows_dev,
                       cols, codes, scales);
  else
    hipLaunchKernelGGL((quantize_rows_kernel<BF16_IN, 1>), dim3(grid), dim3(256), 0, s, in, rows, rows_dev, cols,
                       codes, scales);
}

}  // namespace

hipError_t launch_quantize_rows(const void* x, int rows, int cols, bool bf16_in, uint8_t* codes, float* scales,
                                hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int grid = quantize_grid(rows, cols, 16);
  if (bf16_in) launch_quantize<true>(grid, x, rows, nullptr, cols, codes, scales, s);
  else launch_quantize<false>(grid, x, rows, nullptr, cols, codes, scales, s);
  return hipGetLastError();
}

size_t ffn_fp8_workspace_size(int hidden, int inter, int capacity) {
  (void)hidden;
  return f8_align256((size_t)capacity * inter * 4) + f8_align256((size_t)capacity * inter) +
         f8_align256((size_t)capacity * (inter / kQBlock) * 4);
}

hipError_t launch_ffn_fp8(const FfnFp8Args& a, hipStream_t s) {
  if (a.capacity == 0) return hipSuccess;
  const int I = a.inter, d = a.hidden;
  char* ws = (char*)a.workspace;
  float* h = (float*)ws;
  uint8_t* hq = (uint8_t*)(ws + f8_align256((size_t)a.capacity * I * 4));
  float* hs = (float*)((char*)hq + f8_align256((size_t)a.capacity * I));
  F8Args g1{(const uint8_t*)a.x_codes, a.x_scales, a.row_index, a.row_div, a.offsets, a.num_local, a.capacity,
            (const uint8_t*)a.w_gate_up, a.w_gate_up_scales, 2 * I, d, I, h, I};
  const bool big_gu = fp8_big_ok<true>(g1);
  if (big_gu) {   // the large-tile gate_up quantises its rows of h (quantize_h_kernel the others)
    g1.Cq = hq;
    g1.Cs = hs;
  }
  F8Args g2{hq, hs, nullptr, 1, a.offsets, a.num_local, a.capacity,
            (const uint8_t*)a.w_down, a.w_down_scales, d, I, I, a.o_sorted, d};
  hipError_t err = launch_fp8_gemm<2, 4, true>(g1, s);
  if (err != hipSuccess) return err;
  // h has offsets[E_loc] rows, known on the device only: one workgroup per CU
  // covers a decode batch in one pass and loops over larger ones. From a
  // prefill-sized capacity on, the large-tile gate_up writes the codes of the
  // experts it takes, and the quantiser does the others.
  const int grid = quantize_grid(a.capacity, I, 1);
  if (big_gu)
    hipLaunchKernelGGL(quantize_h_kernel, dim3(grid), dim3(256), 0, s, (const float*)h, a.offsets, a.num_local,
                       a.capacity, I, 1, f8_cu_count(), hq, hs);
  else
    hipLaunchKernelGGL((quantize_rows_kernel<false, 1>), dim3(grid), dim3(256), 0, s, (const void*)h, a.capacity,
                       a.offsets + a.num_local, I, hq, hs);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_fp8_gemm<2, 2, false>(g2, s);
}

}  // namespace moe
