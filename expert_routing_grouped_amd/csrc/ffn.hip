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
// * streaming path -- experts with at most 64 rows (decode), one row chunk
//   each. Bound by the weight read: coalesced weight loads pass through a
//   wavefront-private LDS tile into MFMA registers, with the next two K
//   steps' loads in flight during the current MFMAs.
// * tiled path -- experts with more rows: 128 x 128 tiles staged through LDS
//   on 32x32x16 bf16 MFMA, or, when the experts above 256 rows fill the GPU
//   with them (prefill), 256 x 256 tiles in ffn_big_kernel.
// Experts with no rows appear in neither list, so their weights are not read.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kStreamMT = 4;                  // row tiles of 16 per streamed row chunk
constexpr int kChunkRows = kStreamMT * 16;    // rows per streamed chunk
constexpr int kTileBM = 128;                  // tokens per tile in the tiled path
constexpr int kBigBM = 256;                   // tokens per tile in the large-tile path
constexpr int kStreamDW = 3;                  // weight register sets of the streaming path
constexpr int kStreamDA = 3;                  // activation register sets
constexpr bool kUseBigTiles = true;           // 256 x 256 tiles for large experts
constexpr int kBigMinCapacity = 16384;        // row capacity from which they are used
constexpr int kMaxLocal = 1024;

constexpr int gcd_c(int x, int y) { return y == 0 ? x : gcd_c(y, x % y); }

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
  int big_ok;             // the large-tile kernel is launched too
  int big_min_items;      // ... and takes the tiled experts when it has at least this many tiles
  float* partials;        // shared-activation path: float32 partial sums of split K ranges
  int sk_grid;            // shared-activation path: workgroups that share out the K steps
  int sk_items;           // shared-activation path: finalize items (largest pair count x row blocks)
  int* chunk_desc;        // shared-activation path: [0] = pairs, then (lo, m, v0, v1) per (chunk, slab) pair
  // Masked layout (streaming path only): the rows per expert are min(max(count, 0), slot_cap)
  // from slot_counts instead of offsets, and expert e's r-th row is row e * slot_cap + r of A
  // (slot_a) or of C (slot_c) instead of its compact row.
  const int* slot_counts = nullptr;
  int slot_cap = 0, slot_a = 0, slot_c = 0;
};

// Replaces each permuted row number by the row of A that holds it. All index
// loads are issued before the first is used, so they cost one memory latency.
// The division by row_div is floor((v + 0.5) * (1 / row_div)) in float64: for
// v < 2^31 the rounding error stays below 2^-21 / row_div while (v + 0.5) /
// row_div is at least 0.5 / row_div away from any integer, so the truncation
// is exact; the reciprocal is a scalar, so nothing per lane outlives the call.
template <int N>
__device__ __forceinline__ void a_rows(const GemmArgs& a, uint32_t* rows) {
  if (a.row_index) {
#pragma unroll
    for (int j = 0; j < N; ++j) rows[j] = (uint32_t)a.row_index[rows[j]];
    int div = a.row_div;
    asm volatile("" : "+s"(div));  // computed here, not hoisted out of a caller's loop
    if (div != 1) {
      const double inv = 1.0 / (double)div;
#pragma unroll
      for (int j = 0; j < N; ++j) rows[j] = (uint32_t)(((double)rows[j] + 0.5) * inv);
    }
  }
}

// Buffer resource word 3 for raw (unformatted, unswizzled) buffer loads on gfx9.
constexpr int kBufferConfig = 0x00020000;
// Cache-policy operand of a buffer load: non-temporal (streamed once).
constexpr int kNonTemporal = 2;

// ---------------------------------------------------------------- expert lists

// Splits the local experts by row count m, in expert order (and leaves the
// clamped row bounds in s_lo: rows of expert e are [s_lo[e], s_lo[e] + m);
// n_big = the tiles of kBigBM rows that the tiled experts need; with
// all_chunks every expert is cut into chunks of chunk_rows rows):
//   1 <= m <= stream_max: streamed, in ceil(m / chunk_rows) row chunks;
//                         s_first[e] = first chunk of expert e, s_first[nloc] = chunks
//   m > stream_max:       tiled, in ceil(m / bm) row tiles;
//                         t_first[e] = first tile of expert e, t_first[nloc] = tiles
// Every thread of the 256-thread workgroup calls this; 4 experts per thread.
__device__ void build_lists(const GemmArgs& a, int bm, int* s_first, int* t_first, int* s_lo,
                            int* wsum, int& n_chunks, int& n_tiles, int& n_big,
                            bool all_chunks = false, int chunk_rows = kChunkRows,
                            int stream_max = kChunkRows) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int cc[4], tc[4], cs = 0, ct = 0, cb = 0;
  int ms[4] = {0, 0, 0, 0};
  if (a.slot_counts) {   // compact row bounds: the prefix sums of the clamped counts
    int rs = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      ms[q] = e < a.nloc ? min(max(a.slot_counts[e], 0), a.slot_cap) : 0;
      rs += ms[q];
    }
    int ir = rs;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(ir, d, MOE_WAVE);
      if (lane >= d) ir += o;
    }
    if (lane == 63) wsum[w] = ir;
    __syncthreads();
    int pr = ir - rs, tr = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < w) pr += wsum[i];
      tr += wsum[i];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      if (e < a.nloc) s_lo[e] = pr;
      pr += ms[q];
    }
    if (tid == 0) s_lo[a.nloc] = tr;
    __syncthreads();   // wsum is reused below
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    int m = ms[q];
    if (e < a.nloc && !a.slot_counts) {
      const int lo = min(a.offsets[e], a.capacity);
      const int hi = min(a.offsets[e + 1], a.capacity);
      m = max(0, hi - lo);
      s_lo[e] = lo;
      if (e == a.nloc - 1) s_lo[a.nloc] = max(lo, hi);
    }
    const bool chunked = all_chunks || m <= stream_max;
    cc[q] = (m > 0 && chunked) ? (m + chunk_rows - 1) / chunk_rows : 0;
    tc[q] = (m > 0 && !chunked) ? (m + bm - 1) / bm : 0;
    cs += cc[q];
    ct += tc[q];
    cb += (m > 0 && !chunked) ? (m + kBigBM - 1) / kBigBM : 0;
  }
  cb = wave_sum_i32(cb);
  int is = cs, it = ct;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int os = __shfl_up(is, d, MOE_WAVE), ot = __shfl_up(it, d, MOE_WAVE);
    if (lane >= d) { is += os; it += ot; }
  }
  if (lane == 63) { wsum[w] = is; wsum[4 + w] = it; wsum[8 + w] = cb; }
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
  // the totals are the same in every lane; say so, so that values derived
  // from them can live in scalar registers
  n_chunks = __builtin_amdgcn_readfirstlane(ts);
  n_tiles = __builtin_amdgcn_readfirstlane(tt);
  n_big = __builtin_amdgcn_readfirstlane(tb);
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
// A K step is 64 k: 128 bytes, one full cache line, of each row. Global loads
// are coalesced: load h of a 16-row tile gives lane l the 16-byte chunk l % 8
// of row 8h + l / 8, so each instruction reads 8 whole lines. (Loading
// directly in MFMA layout would touch 16 lines per instruction, 64 bytes each;
// the load pipeline then moves about a quarter of the bytes per clock.) The
// lane writes its chunk into its wavefront's LDS tile at row * 128 +
// ((chunk ^ row % 8) * 16), and MFMA fragments are read back with lane
// (r = l % 16, g = l / 16) taking chunk 4u + g of row r for MFMA u = 0, 1 --
// the same k order for weights and activations. The XOR keeps both the writes
// and the reads free of bank conflicts. Each wavefront has its own LDS tiles,
// so no barrier is needed inside the K loop.
//
// K slices are summed through LDS in slice order; then SiLU*up (gated) or the
// plain bf16 store.
template <int NTW, int KS, bool GATED, int DW, int DA>
struct Stream {
  static constexpr int PERIOD = DW * DA / gcd_c(DW, DA);  // register sets repeat every PERIOD steps
  static constexpr int MT = kStreamMT;
  static constexpr int NWN = 4 / KS;
  static constexpr int HT = GATED ? NTW / 2 : NTW;  // output tiles per wavefront
  static constexpr int COLS = NWN * HT * 16;        // output columns per slab
  static constexpr int KSTEP = 64;
  static constexpr int TILE_BYTES = 16 * 128;       // one 16-row tile of a K step
  static constexpr int WAVE_LDS = (NTW + MT) * TILE_BYTES;
  static constexpr int LDS_BYTES = 4 * WAVE_LDS;
  static_assert(!GATED || NTW % 2 == 0, "gated slabs pair gate and up tiles");
  static_assert(MT * NTW * 1024 <= WAVE_LDS, "K-slice partial sums fit in the wavefront's tiles");

  // MTA = active row tiles of the chunk (1..MT): the K loop has no branches,
  // so the only waits are on the registers an MFMA reads.
  template <int MTA, bool NT>
  __device__ static void run_mt(const GemmArgs& a, int e, int lo, int m, int slab, int shift, char* smem) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ks = wave % KS, wn = wave / KS;
    const int fr = lane & 15, g = lane >> 4;
    const int lr = lane >> 3, lc = lane & 7;       // load mapping: row lr (+8), chunk lc
    const int col0 = (slab * NWN + wn) * HT * 16;  // first output column of this wavefront
    const uint32_t pitch = (uint32_t)a.K * 2;      // row pitch in bytes

    // Weights: one buffer per expert; the lane's byte offset is fixed and the
    // tile/half/K-step offsets are wavefront-uniform.
    const __amdgpu_buffer_rsrc_t wbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.W + (size_t)e * a.N * a.K), 0, (int)(a.N * pitch), kBufferConfig);
    const uint32_t wv = (uint32_t)(col0 + lr) * pitch + lc * 16;
    int wso[NTW][2];
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        wso[t][h] = ((t % HT) * 16 + h * 8 + ((GATED && t >= HT) ? a.inter : 0)) * (int)pitch;
    // Activations: rows past the chunk's end read its first row instead: an
    // MFMA output column depends only on its own activation row, and it is not
    // stored.
    const __amdgpu_buffer_rsrc_t abuf = __builtin_amdgcn_make_buffer_rsrc((void*)a.A, 0, -1, kBufferConfig);
    uint32_t av[MTA][2];
#pragma unroll
    for (int i = 0; i < MTA; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = i * 16 + h * 8 + lr;
        av[i][h] = lo + (r < m ? r : 0) + (a.slot_a ? shift : 0);
      }
    a_rows<MTA * 2>(a, &av[0][0]);
#pragma unroll
    for (int i = 0; i < MTA; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) av[i][h] = av[i][h] * pitch + lc * 16;
    const int cshift = a.slot_c ? shift : 0;   // output rows: compact, or slot rows

    char* xs = smem + wave * WAVE_LDS;  // NTW weight tiles, then MT activation tiles
    const int woff[2] = {lr * 128 + ((lc ^ lr) << 4), (8 + lr) * 128 + ((lc ^ lr) << 4)};
    const int roff[2] = {fr * 128 + ((g ^ (fr & 7)) << 4), fr * 128 + (((4 + g) ^ (fr & 7)) << 4)};

    f32x4_t acc[MTA][NTW];
#pragma unroll
    for (int i = 0; i < MTA; ++i)
#pragma unroll
      for (int t = 0; t < NTW; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t wr[DW][NTW][2], ar[DA][MTA][2];
    auto load_w = [&](u32x4_t (&w)[NTW][2], int kk) {
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          w[t][h] = __builtin_amdgcn_raw_buffer_load_b128(wbuf, wv, wso[t][h] + kk * 2, NT ? kNonTemporal : 0);
    };
    auto load_a = [&](u32x4_t (&x)[MTA][2], int kk) {
#pragma unroll
      for (int i = 0; i < MTA; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) x[i][h] = __builtin_amdgcn_raw_buffer_load_b128(abuf, av[i][h], kk * 2, 0);
    };
    auto mma = [&](const u32x4_t (&w)[NTW][2], const u32x4_t (&av)[MTA][2]) {
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) *(u32x4_t*)(xs + t * TILE_BYTES + woff[h]) = w[t][h];
#pragma unroll
      for (int i = 0; i < MTA; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) *(u32x4_t*)(xs + (NTW + i) * TILE_BYTES + woff[h]) = av[i][h];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8_t wf[NTW], af[MTA];
#pragma unroll
        for (int t = 0; t < NTW; ++t) wf[t] = *(const bf16x8_t*)(xs + t * TILE_BYTES + roff[u]);
#pragma unroll
        for (int i = 0; i < MTA; ++i) af[i] = *(const bf16x8_t*)(xs + (NTW + i) * TILE_BYTES + roff[u]);
#pragma unroll
        for (int i = 0; i < MTA; ++i)
#pragma unroll
          for (int t = 0; t < NTW; ++t)
            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[t], af[i], acc[i][t], 0, 0, 0);
      }
    };

    // Software pipeline over K steps: weights DW - 1 steps ahead (DW register
    // sets), activations DA - 1 steps ahead (DA sets). Step s first issues the
    // loads of W(s + DW - 1) and A(s + DA - 1), then consumes W(s) and A(s).
    // Loads complete in issue order, so step s waits only for its own data
    // while the later steps stay in flight. Steps past the end reload the last
    // step instead of branching. The scheduling barriers keep this issue order.
    const int kw = a.K / KS, kbeg = ks * kw, klast = kbeg + kw - KSTEP;
    const int steps = kw / KSTEP;
#pragma unroll
    for (int j = 0; j < (DW > DA ? DW : DA) - 1; ++j) {
      if (j < DW - 1) load_w(wr[j], min(kbeg + j * KSTEP, klast));
      if (j < DA - 1) load_a(ar[j], min(kbeg + j * KSTEP, klast));
    }
    // The main loop runs whole periods with no exit inside, so the compiler's
    // wait counts stay exact across the back edge (an exit in the body makes
    // it drain every load at the loop head); the remainder runs after it.
    int kk = kbeg, s = 0;
#define MOE_STEP(q)                                                        \
  load_w(wr[((q) + DW - 1) % DW], min(kk + (DW - 1) * KSTEP, klast));      \
  load_a(ar[((q) + DA - 1) % DA], min(kk + (DA - 1) * KSTEP, klast));      \
  __builtin_amdgcn_sched_barrier(0);                                       \
  mma(wr[(q) % DW], ar[(q) % DA]);                                         \
  __builtin_amdgcn_sched_barrier(0);                                       \
  kk += KSTEP;
    for (; s + PERIOD <= steps; s += PERIOD) {
#pragma unroll
      for (int q = 0; q < PERIOD; ++q) { MOE_STEP(q) }
    }
#pragma unroll
    for (int q = 0; q < PERIOD - 1; ++q) {
      if (s + q >= steps) break;
      MOE_STEP(q)
    }
#undef MOE_STEP

    if (KS > 1) {
      // Each wavefront parks its partial sums in its own tiles ([MT][NTW][64]
      // float4); slice ks then finishes the row tiles i with i % KS == ks.
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
      uint16_t* crow = a.C + (size_t)(lo + row + cshift) * a.ldc + col0 + g * 4;
#pragma unroll
      for (int t = 0; t < HT; ++t) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          v[r] = GATED ? silu(acc[i][t][r]) * acc[i][t + HT][r] : acc[i][t][r];
        *(uint2*)(crow + t * 16) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
  }

  // Row chunk `chunk` (kChunkRows rows) of expert e, output slab `slab`. The
  // weights of an expert with a single chunk are read once per GEMM: with a
  // long K they are loaded non-temporally, which keeps the activation rows
  // that every slab re-reads in the caches.
  __device__ static void run(const GemmArgs& a, const int* s_lo, int e, int chunk, int slab, char* smem) {
    e = __builtin_amdgcn_readfirstlane(e);
    const int lo = __builtin_amdgcn_readfirstlane(s_lo[e] + chunk * kChunkRows);
    const int m = __builtin_amdgcn_readfirstlane(min(kChunkRows, s_lo[e + 1] - lo));
    const bool nt = __builtin_amdgcn_readfirstlane(s_lo[e + 1] - s_lo[e]) <= kChunkRows && a.K >= 512;
    slab = __builtin_amdgcn_readfirstlane(slab);
    // masked layout: slot row = e * slot_cap + (compact row - s_lo[e])
    const int shift = a.slot_counts ? __builtin_amdgcn_readfirstlane(e * a.slot_cap - s_lo[e]) : 0;
    switch (((m + 15) >> 4) * 2 + (nt ? 1 : 0)) {
      case 2: run_mt<1, false>(a, e, lo, m, slab, shift, smem); break;
      case 3: run_mt<1, true>(a, e, lo, m, slab, shift, smem); break;
      case 4: run_mt<2, false>(a, e, lo, m, slab, shift, smem); break;
      case 5: run_mt<2, true>(a, e, lo, m, slab, shift, smem); break;
      case 6: run_mt<3, false>(a, e, lo, m, slab, shift, smem); break;
      case 7: run_mt<3, true>(a, e, lo, m, slab, shift, smem); break;
      case 9: run_mt<4, true>(a, e, lo, m, slab, shift, smem); break;
      default: run_mt<4, false>(a, e, lo, m, slab, shift, smem); break;
    }
  }
};

// ---------------------------------------------------------------- walk path

// Plain GEMMs with a short K = 64 * KQ (KQ = 1, 2; the down projection of
// narrow experts): streaming K would give each work item a single K step, so
// here a wavefront keeps the chunk's activations (all of K) as MFMA fragments
// in registers and walks along N instead, one group of NTW 16-row weight
// tiles per step: load (two steps ahead, coalesced, through the same
// XOR-swizzled LDS tiles as the streaming path), multiply, store. A work item
// is a chunk and ITEM_COLS output columns, J steps per wavefront.
constexpr int kWalkDepth = 3;
constexpr int kWalkRows = 128;   // rows per chunk on the walk path

template <int KQ>
struct Walk {
  static constexpr int NTW = 2 / KQ;
  static constexpr int MT = kWalkRows / 16;
  static constexpr int STEP_COLS = NTW * 16;
  static constexpr int WD = kWalkDepth;               // weight register sets
  static constexpr int TILE_BYTES = 16 * 128;
  static constexpr int WAVE_LDS = (MT + NTW) * KQ * TILE_BYTES;
  static constexpr int LDS_BYTES = 4 * WAVE_LDS;

  template <int MTA>
  __device__ static void run_mt(const GemmArgs& a, int e, int lo, int m, int c0, int steps, char* smem) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int fr = lane & 15, g = lane >> 4;
    const int lr = lane >> 3, lc = lane & 7;
    const uint32_t pitch = (uint32_t)a.K * 2;

    char* xs = smem + wave * WAVE_LDS;   // MT * KQ activation tiles, then NTW * KQ weight tiles
    char* ws = xs + MT * KQ * TILE_BYTES;
    const int woff[2] = {lr * 128 + ((lc ^ lr) << 4), (8 + lr) * 128 + ((lc ^ lr) << 4)};
    const int roff[2] = {fr * 128 + ((g ^ (fr & 7)) << 4), fr * 128 + (((4 + g) ^ (fr & 7)) << 4)};

    // Activations: all K of the chunk's rows, once (rows past the end read row 0).
    const __amdgpu_buffer_rsrc_t abuf = __builtin_amdgcn_make_buffer_rsrc((void*)a.A, 0, -1, kBufferConfig);
    uint32_t av[MTA][2];
#pragma unroll
    for (int i = 0; i < MTA; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = i * 16 + h * 8 + lr;
        av[i][h] = lo + (r < m ? r : 0);
      }
    a_rows<MTA * 2>(a, &av[0][0]);
    {
      u32x4_t ax[MTA][KQ][2];
#pragma unroll
      for (int i = 0; i < MTA; ++i)
#pragma unroll
        for (int q = 0; q < KQ; ++q)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            ax[i][q][h] = __builtin_amdgcn_raw_buffer_load_b128(abuf, av[i][h] * pitch + lc * 16, q * 128, 0);
#pragma unroll
      for (int i = 0; i < MTA; ++i)
#pragma unroll
        for (int q = 0; q < KQ; ++q)
#pragma unroll
          for (int h = 0; h < 2; ++h) *(u32x4_t*)(xs + (i * KQ + q) * TILE_BYTES + woff[h]) = ax[i][q][h];
    }
    bf16x8_t af[MTA][KQ][2];
#pragma unroll
    for (int i = 0; i < MTA; ++i)
#pragma unroll
      for (int q = 0; q < KQ; ++q)
#pragma unroll
        for (int u = 0; u < 2; ++u) af[i][q][u] = *(const bf16x8_t*)(xs + (i * KQ + q) * TILE_BYTES + roff[u]);

    // Weights: step j, tile t, half h: rows c0 + j*STEP_COLS + t*16 + 8h + lr.
    const __amdgpu_buffer_rsrc_t wbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.W + (size_t)e * a.N * a.K), 0, (int)(a.N * pitch), kBufferConfig);
    const uint32_t wv = (uint32_t)(c0 + lr) * pitch + lc * 16;
    u32x4_t wr[WD][NTW][KQ][2];
    auto load_w = [&](u32x4_t (&w)[NTW][KQ][2], int j) {
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int q = 0; q < KQ; ++q)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            w[t][q][h] = __builtin_amdgcn_raw_buffer_load_b128(
                wbuf, wv, (j * STEP_COLS + t * 16 + h * 8) * (int)pitch + q * 128, kNonTemporal);
    };
    // Outputs go out in whole 128-byte row segments (64 columns): SEG steps
    // are staged in the activation tiles' LDS (free once the fragments are in
    // registers), XOR-swizzled by 16-byte chunk, then each store instruction
    // writes 8 rows x 128 bytes.
    constexpr int SEG = 64 / STEP_COLS;
    char* os = xs;  // [64 rows][128 bytes]
    auto step = [&](const u32x4_t (&w)[NTW][KQ][2], int j) {
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int q = 0; q < KQ; ++q)
#pragma unroll
          for (int h = 0; h < 2; ++h) *(u32x4_t*)(ws + (t * KQ + q) * TILE_BYTES + woff[h]) = w[t][q][h];
      f32x4_t acc[MTA][NTW];
#pragma unroll
      for (int i = 0; i < MTA; ++i)
#pragma unroll
        for (int t = 0; t < NTW; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < KQ; ++q)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          bf16x8_t wf[NTW];
#pragma unroll
          for (int t = 0; t < NTW; ++t) wf[t] = *(const bf16x8_t*)(ws + (t * KQ + q) * TILE_BYTES + roff[u]);
#pragma unroll
          for (int i = 0; i < MTA; ++i)
#pragma unroll
            for (int t = 0; t < NTW; ++t)
              acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[t], af[i][q][u], acc[i][t], 0, 0, 0);
        }
      // Lane holds output row i*16 + lane % 16, columns t*16 + 4*(lane/16) + (0..3)
      // of this step: staged at column (j % 2) * STEP_COLS + ... of the row segment.
#pragma unroll
      for (int i = 0; i < MTA; ++i) {
        const int row = i * 16 + fr;
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const int cb = ((j % SEG) * STEP_COLS + t * 16 + g * 4) * 2;   // byte in the row segment
          const int off = row * 128 + ((((cb >> 4) ^ (row & 7))) << 4) + (cb & 15);
          *(uint2*)(os + off) = make_uint2(pack_bf16x2(acc[i][t][0], acc[i][t][1]),
                                           pack_bf16x2(acc[i][t][2], acc[i][t][3]));
        }
      }
      if (j % SEG == SEG - 1 || j + 1 == steps) {
        // row segment of columns c0 + (j - j % SEG) * STEP_COLS .. + 64, of
        // which the walk filled the first chunks (all, unless it ended early)
        const int colb = c0 + (j - j % SEG) * STEP_COLS;
        const int chunks = (j % SEG + 1) * STEP_COLS / 8;
#pragma unroll
        for (int rr = 0; rr < MTA * 2; ++rr) {
          const int row = rr * 8 + lr;
          const u32x4_t v = *(const u32x4_t*)(os + row * 128 + ((lc ^ (row & 7)) << 4));
          if (row < m && lc < chunks)
            *(u32x4_t*)(a.C + (size_t)(lo + row) * a.ldc + colb + lc * 8) = v;
        }
      }
    };

    // Weights WD - 1 steps ahead in WD register sets (steps past the end
    // reload the last one); the main loop runs whole periods of WD.
#pragma unroll
    for (int q = 0; q < WD - 1; ++q) load_w(wr[q], min(q, steps - 1));
    int j = 0;
#define MOE_WALK(q)                                           \
  load_w(wr[((q) + WD - 1) % WD], min(j + WD - 1, steps - 1)); \
  __builtin_amdgcn_sched_barrier(0);                          \
  step(wr[(q) % WD], j);                                      \
  __builtin_amdgcn_sched_barrier(0);                          \
  ++j;
    for (; j + WD <= steps;) {
#pragma unroll
      for (int q = 0; q < WD; ++q) { MOE_WALK(q) }
    }
#pragma unroll
    for (int q = 0; q < WD - 1; ++q) {
      if (j >= steps) break;
      MOE_WALK(q)
    }
#undef MOE_WALK
  }

  // Columns [c0, c0 + steps * STEP_COLS) of chunk `chunk` of expert e, by
  // this wavefront alone (its own LDS region).
  __device__ static void run(const GemmArgs& a, const int* s_lo, int e, int chunk, int c0, int steps,
                             char* smem) {
    e = __builtin_amdgcn_readfirstlane(e);
    const int lo = __builtin_amdgcn_readfirstlane(s_lo[e] + chunk * kWalkRows);
    const int m = __builtin_amdgcn_readfirstlane(min(kWalkRows, s_lo[e + 1] - lo));
    c0 = __builtin_amdgcn_readfirstlane(c0);
    steps = __builtin_amdgcn_readfirstlane(steps);
    static_assert(kWalkRows == 128, "tile counts below");
    const int t = (m + 15) >> 4;   // 16-row tiles, rounded up to one of a few counts
    if (t <= 1) run_mt<1>(a, e, lo, m, c0, steps, smem);
    else if (t <= 2) run_mt<2>(a, e, lo, m, c0, steps, smem);
    else if (t <= 3) run_mt<3>(a, e, lo, m, c0, steps, smem);
    else if (t <= 4) run_mt<4>(a, e, lo, m, c0, steps, smem);
    else if (t <= 6) run_mt<6>(a, e, lo, m, c0, steps, smem);
    else run_mt<8>(a, e, lo, m, c0, steps, smem);
  }
};

// ---------------------------------------------------------------- shared-activation path

// Gated GEMMs of narrow experts (inter a multiple of 64, at most 128): a
// workgroup owns 64 output columns of one chunk -- 64 gate rows and the 64
// matching up rows of the weights, 16 + 16 per wavefront -- so all four
// wavefronts multiply the same activation K step. Each step's activation
// tile is loaded once, cooperatively, into a shared double-buffered LDS tile
// (one barrier per step) instead of once per 16-column slab, which cuts the
// activation traffic by the 4 slabs' repeat. With few columns per expert the
// work is then split over KP parts of K: each item writes float32 partial
// sums, and ffn_finalize_kernel adds the parts in order (deterministic) and
// applies SiLU(gate) * up. Every expert is cut into 64-row chunks here, large
// ones included.
constexpr int kShareCols = 64;   // output columns per item
constexpr int kShareRows = 128;  // rows per chunk: an expert's weights are read once per 128 rows

struct SharedA {
  static constexpr int NSET = 4;   // register sets: loads NSET - 1 steps ahead
  static constexpr int MT = kShareRows / 16;
  static constexpr int KSTEP = 64;
  static constexpr int TILE_BYTES = 16 * 128;
  static constexpr int A_BUF = MT * TILE_BYTES;                 // one step's activation tiles
  static constexpr int W_OFF = 2 * A_BUF;                       // after the two activation buffers
  static constexpr int DUMMY_OFF = W_OFF + 4 * 2 * TILE_BYTES;  // per-wave sink for unused shares
  static constexpr int LDS_BYTES = DUMMY_OFF + 4 * 1024;
  static constexpr int PART_FLOATS = kShareRows * 2 * kShareCols;   // one piece's partial sums

  template <int MTA>
  __device__ static void run_mt(const GemmArgs& a, int e, int lo, int m, int slab, int k0, int steps,
                                float* part, char* smem) {
    constexpr int HALVES = 2 * MTA;            // 8-row half tiles of one activation step
    constexpr int NSH = (HALVES + 3) / 4;      // shares per wavefront
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int fr = lane & 15, g = lane >> 4;
    const int lr = lane >> 3, lc = lane & 7;
    const uint32_t pitch = (uint32_t)a.K * 2;
    const int woff[2] = {lr * 128 + ((lc ^ lr) << 4), (8 + lr) * 128 + ((lc ^ lr) << 4)};
    const int roff[2] = {fr * 128 + ((g ^ (fr & 7)) << 4), fr * 128 + (((4 + g) ^ (fr & 7)) << 4)};

    // Weights: gate rows slab*64 + 16*wave + (8h + lr), up rows inter + the same.
    const __amdgpu_buffer_rsrc_t wbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.W + (size_t)e * a.N * a.K), 0, (int)(a.N * pitch), kBufferConfig);
    const uint32_t wv = (uint32_t)(slab * kShareCols + 16 * wave + lr) * pitch + lc * 16;
    // Activation share j of this wavefront: half tile hh = wave + 4j (tile hh / 2,
    // half hh % 2); shares past the step's half tiles load row 0 into a sink.
    const __amdgpu_buffer_rsrc_t abuf = __builtin_amdgcn_make_buffer_rsrc((void*)a.A, 0, -1, kBufferConfig);
    uint32_t av[NSH];
    int aoff[NSH];
#pragma unroll
    for (int j = 0; j < NSH; ++j) {
      const int hh = wave + 4 * j;
      const int r = (hh >> 1) * 16 + (hh & 1) * 8 + lr;
      av[j] = lo + ((hh < HALVES && r < m) ? r : 0);
      aoff[j] = hh < HALVES ? (hh >> 1) * TILE_BYTES + woff[hh & 1] : DUMMY_OFF + wave * 1024 + lane * 16;
    }
    a_rows<NSH>(a, av);
#pragma unroll
    for (int j = 0; j < NSH; ++j) av[j] = av[j] * pitch + lc * 16;

    const int kbeg = k0 * KSTEP, klast = kbeg + (steps - 1) * KSTEP;
    char* wl = smem + W_OFF + wave * 2 * TILE_BYTES;

    f32x4_t acc[MTA][2];
#pragma unroll
    for (int i = 0; i < MTA; ++i) acc[i][0] = acc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t wr[NSET][2][2], ar[NSET][NSH];
    auto load = [&](int set, int kk) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          wr[set][t][h] = __builtin_amdgcn_raw_buffer_load_b128(
              wbuf, wv, ((t ? a.inter : 0) + 8 * h) * (int)pitch + kk * 2, kNonTemporal);
#pragma unroll
      for (int j = 0; j < NSH; ++j) ar[set][j] = __builtin_amdgcn_raw_buffer_load_b128(abuf, av[j], kk * 2, 0);
    };
    auto step = [&](int set, int buf) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) *(u32x4_t*)(wl + t * TILE_BYTES + woff[h]) = wr[set][t][h];
#pragma unroll
      for (int j = 0; j < NSH; ++j) *(u32x4_t*)(smem + (aoff[j] < DUMMY_OFF ? buf * A_BUF : 0) + aoff[j]) = ar[set][j];
      __syncthreads();  // the step's activation tiles are complete
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8_t wf[2], xf[MTA];
#pragma unroll
        for (int t = 0; t < 2; ++t) wf[t] = *(const bf16x8_t*)(wl + t * TILE_BYTES + roff[u]);
#pragma unroll
        for (int i = 0; i < MTA; ++i) xf[i] = *(const bf16x8_t*)(smem + buf * A_BUF + i * TILE_BYTES + roff[u]);
#pragma unroll
        for (int i = 0; i < MTA; ++i)
#pragma unroll
          for (int t = 0; t < 2; ++t)
            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[t], xf[i], acc[i][t], 0, 0, 0);
      }
    };

    // Loads NSET - 1 steps ahead in NSET register sets. Step s writes
    // activation buffer s % 2, which every wavefront finished reading in step
    // s - 2, before the barrier of step s - 1. The main loop runs whole
    // periods of NSET steps (NSET even).
#pragma unroll
    for (int j = 0; j < NSET - 1; ++j) load(j, min(kbeg + j * KSTEP, klast));
    int kk = kbeg, st = 0;
#define MOE_SHARED(q)                                             \
  load(((q) + NSET - 1) % NSET, min(kk + (NSET - 1) * KSTEP, klast)); \
  __builtin_amdgcn_sched_barrier(0);                              \
  step((q) % NSET, (q) % 2);                                      \
  __builtin_amdgcn_sched_barrier(0);                              \
  kk += KSTEP;
    for (; st + NSET <= steps; st += NSET) {
#pragma unroll
      for (int q = 0; q < NSET; ++q) { MOE_SHARED(q) }
    }
#pragma unroll
    for (int q = 0; q < NSET - 1; ++q) {
      if (st + q >= steps) break;
      MOE_SHARED(q)
    }
#undef MOE_SHARED

    // Lane holds rows i*16 + lane % 16 and, per t (0 gate, 1 up), columns
    // 16*wave + 4*(lane/16) + (0..3) of the item's 64.
#pragma unroll
    for (int i = 0; i < MTA; ++i) {
      const int row = i * 16 + fr;
      if (row >= m) continue;
      const int col = 16 * wave + 4 * g;
      if (part) {
        float* prow = part + row * 2 * kShareCols;
        *(f32x4_t*)(prow + col) = acc[i][0];
        *(f32x4_t*)(prow + kShareCols + col) = acc[i][1];
      } else {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = silu(acc[i][0][r]) * acc[i][1][r];
        *(uint2*)(a.C + (size_t)(lo + row) * a.ldc + slab * kShareCols + col) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
  }

  __device__ static void run(const GemmArgs& a, const int* s_lo, int e, int chunk, int slab, int k0,
                             int steps, float* part, char* smem) {
    e = __builtin_amdgcn_readfirstlane(e);
    const int lo = __builtin_amdgcn_readfirstlane(s_lo[e] + chunk * kShareRows);
    const int m = __builtin_amdgcn_readfirstlane(min(kShareRows, s_lo[e + 1] - lo));
    // 16-row tiles, rounded up to one of a few counts
    const int t = (m + 15) >> 4;
    static_assert(kShareRows == 128, "tile counts below");
    if (t <= 1) run_mt<1>(a, e, lo, m, slab, k0, steps, part, smem);
    else if (t <= 2) run_mt<2>(a, e, lo, m, slab, k0, steps, part, smem);
    else if (t <= 3) run_mt<3>(a, e, lo, m, slab, k0, steps, part, smem);
    else if (t <= 4) run_mt<4>(a, e, lo, m, slab, k0, steps, part, smem);
    else if (t <= 6) run_mt<6>(a, e, lo, m, slab, k0, steps, part, smem);
    else run_mt<8>(a, e, lo, m, slab, k0, steps, part, smem);
  }
};

// Stream-K split: the K steps of all (chunk, slab) pairs, pair cs = chunk *
// slabs + slab, are laid end to end (nk steps each, global step index cs * nk
// + k) and shared out over the grid's G workgroups by cost, so that every
// workgroup moves about the same number of bytes: a step of a chunk with m
// rows loads 128 weight rows and m activation rows, cost 128 + m. With the
// step costs laid end to end (total C), workgroup v takes the steps whose
// starting cost lies in [ceil(C v / G), ceil(C (v+1) / G)), i.e. step owner
// = floor(start cost * G / C). A workgroup's range covers pieces of one or
// more pairs. A piece that is a whole pair writes h itself; any other piece
// writes its float32 partial sums, [64 rows][gate 64 | up 64], to slot v +
// cs (unique: along the sequence of pieces neither v nor cs decreases and one
// of them grows), and ffn_finalize_kernel adds a pair's pieces in K order.
// Workgroups of one XCD (b % 8) take consecutive ranges, so a pair's pieces
// and the chunks of one expert, which read the same weight rows, mostly share
// that XCD's L2. One workgroup per CU: with more, the workgroups sharing a CU
// get very unequal shares of its bandwidth and the last ones set the time.
// Only the first Ge = min(G, C / (128 + kShareRows)) workgroups take part: each range is then
// at least as wide as the costliest step, so every one of them owns a step
// and the pieces of a pair belong to a contiguous run of workgroups.
//
// Chunks (kShareRows rows, the last of an expert fewer) are contiguous in
// rows, so the steps before chunk c, starting at row lo_c, cost nk * slabs *
// (128 c + lo_c - lo_0).
struct SkCost {
  long long nks;   // nk * slabs
  int nk, slabs, lo0;
  int wrows;       // weight rows a step loads: 128 here, 64 on the walk path
  int crows;       // rows per chunk: kShareRows here, kWalkRows on the walk path
  __device__ long long chunk_start(int c, int lo_c) const { return nks * ((long long)wrows * c + lo_c - lo0); }
};

// First global step whose starting cost is >= x (x < C), from the expert lists:
// the last expert starting at or before x, then its chunk (all but the last
// are full), slab and step.
__device__ long long sk_step_at(const SkCost& q, long long x, const int* s_first, const int* s_lo, int nloc) {
  int lo = 0, hi = nloc - 1;   // last expert whose cost start is <= x
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (q.chunk_start(s_first[mid], s_lo[mid]) <= x) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const long long y = x - q.chunk_start(s_first[e], s_lo[e]);
  const int full = q.wrows + q.crows;   // step cost of a full chunk
  const int j = (int)(y / (q.nks * full));
  const int c = s_first[e] + j, lo_c = s_lo[e] + q.crows * j;
  const int u = q.wrows + min(q.crows, s_lo[e + 1] - lo_c);
  const long long y2 = y - q.nks * full * j;
  const int slab = (int)(y2 / ((long long)q.nk * u));
  const long long y3 = y2 - (long long)slab * q.nk * u;
  return ((long long)c * q.slabs + slab) * q.nk + (y3 + u - 1) / u;
}

__device__ __forceinline__ int sk_active(long long C, int grid) {
  return (int)max(1LL, min((long long)grid, C / (128 + kShareRows)));
}

__global__ __launch_bounds__(256, 1) void ffn_shared_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[SharedA::LDS_BYTES];
  __shared__ int s_first[kMaxLocal + 1];
  __shared__ int t_first[kMaxLocal + 1];
  __shared__ int s_lo[kMaxLocal + 1];
  __shared__ int wsum[12];
  int n_chunks, n_tiles, n_big;
  build_lists(a, kTileBM, s_first, t_first, s_lo, wsum, n_chunks, n_tiles, n_big, true, kShareRows);
  SkCost q;
  q.nk = a.K / SharedA::KSTEP;
  q.slabs = a.inter / kShareCols;
  q.nks = (long long)q.nk * q.slabs;
  q.lo0 = s_lo[0];
  q.wrows = 128;
  q.crows = kShareRows;
  const long long C = q.chunk_start(n_chunks, s_lo[a.nloc]);
  const long long total = (long long)n_chunks * q.nks;
  if (blockIdx.x == 0 && threadIdx.x == 0) a.chunk_desc[0] = n_chunks * (a.inter / kShareCols);
  if (C == 0) return;
  const int G = sk_active(C, a.sk_grid);
  const int v = (blockIdx.x % 8) * (a.sk_grid / 8) + blockIdx.x / 8;   // sk_grid == gridDim.x, a multiple of 8
  if (v >= G) return;
  const long long x0 = (C * v + G - 1) / G, x1 = (C * (v + 1) + G - 1) / G;
  long long st = x0 < C ? sk_step_at(q, x0, s_first, s_lo, a.nloc) : total;
  const long long s1 = x1 < C ? sk_step_at(q, x1, s_first, s_lo, a.nloc) : total;
  while (st < s1) {
    const int cs = __builtin_amdgcn_readfirstlane((int)(st / q.nk));
    const int k0 = __builtin_amdgcn_readfirstlane((int)(st - (long long)cs * q.nk));
    const int steps = __builtin_amdgcn_readfirstlane((int)min(s1 - st, (long long)(q.nk - k0)));
    const int c = cs / q.slabs, slab = cs % q.slabs;
    const int e = find_expert(s_first, a.nloc, c);
    if (k0 == 0 && threadIdx.x == 0) {  // the pair's record, for ffn_finalize_kernel
      const int lo = s_lo[e] + (c - s_first[e]) * kShareRows;
      const int m = min(kShareRows, s_lo[e + 1] - lo), u = q.wrows + m;
      const long long p = q.chunk_start(c, lo) + (long long)slab * q.nk * u;   // cost at the pair's step 0
      int4* rec = (int4*)(a.chunk_desc + 4) + cs;
      *rec = make_int4(lo, m, v, (int)((p + (long long)(q.nk - 1) * u) * G / C));
    }
    float* part = (k0 == 0 && steps == q.nk) ? nullptr : a.partials + (size_t)(v + cs) * SharedA::PART_FLOATS;
    SharedA::run(a, s_lo, e, c - s_first[e], slab, k0, steps, part, smem);
    __syncthreads();  // LDS is reused by the next piece
    st += steps;
  }
}

// h = SiLU(sum of gate pieces) * (sum of up pieces) for every (chunk, slab)
// pair that was split, pieces added in K order. ffn_shared_kernel leaves the
// pair count and, per pair, its rows and the workgroups v0..v1 that hold its
// pieces (slots v + pair).
__global__ __launch_bounds__(256) void ffn_finalize_kernel(GemmArgs a) {
  const int c16 = (threadIdx.x & 3) * 16;  // 64 rows x 4 column groups
  constexpr int RB = kShareRows / 64;     // 64-row blocks per chunk
  // items (pair, row block) up to the largest possible pair count; the pair
  // count and the pair's record are loaded together
  for (int it = blockIdx.x; it < a.sk_items; it += gridDim.x) {
    const int w = it / RB, rb = it % RB;
    const int pairs = a.chunk_desc[0];   // written by ffn_shared_kernel
    const int4 rec = ((const int4*)(a.chunk_desc + 4))[w];
    if (w >= pairs) continue;
    const int lo = rec.x, m = rec.y, v0 = rec.z, v1 = rec.w;
    const int slab = w % (a.inter / kShareCols);
    if (v0 == v1) continue;   // one piece: h written directly
    const int row = rb * 64 + (threadIdx.x >> 2);
    if (row < m) {
      f32x4_t gs[4], us[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) gs[i] = us[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // The pieces of workgroups v0..v1, in K order, four at a time: the loads
      // go out together, the sums are taken in order.
      for (int v = v0; v <= v1; v += 4) {
        const int nv = min(4, v1 + 1 - v);
        f32x4_t pg[4][4], pu[4][4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (b >= nv) break;
          const float* pk = a.partials + (size_t)(v + b + w) * SharedA::PART_FLOATS + row * 2 * kShareCols + c16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pg[b][i] = *(const f32x4_t*)(pk + 4 * i);
            pu[b][i] = *(const f32x4_t*)(pk + kShareCols + 4 * i);
          }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (b >= nv) break;
#pragma unroll
          for (int i = 0; i < 4; ++i) { gs[i] += pg[b][i]; us[i] += pu[b][i]; }
        }
      }
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] = pack_bf16x2(silu(gs[i][0]) * us[i][0], silu(gs[i][1]) * us[i][1]);
        o[2 * i + 1] = pack_bf16x2(silu(gs[i][2]) * us[i][2], silu(gs[i][3]) * us[i][3]);
      }
      uint4* dst = (uint4*)(a.C + (size_t)(lo + row) * a.ldc + slab * kShareCols + c16);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
}

// Plain GEMMs with K = 64 KQ on the walk path: every expert is cut into chunks
// of up to kWalkRows rows and each chunk's output columns into 64-column units (one 128-byte
// row segment); a unit loads 64 weight rows and stores m output rows, cost 64
// + m. The units of all chunks, laid end to end, are shared out by cost over
// all wavefronts of the grid (the same split as ffn_shared_kernel's, per
// wavefront; no K split, so no partial sums): every wavefront walks the
// columns of one or more chunk pieces on its own, in its own LDS region.
// Wavefronts of one XCD take consecutive ranges, so the chunks of one
// expert, which read the same weight rows, mostly share that XCD's L2.
template <int KQ>
__global__ __launch_bounds__(256, 1) void ffn_walk_kernel(GemmArgs a) {
  using Wk = Walk<KQ>;
  __shared__ __attribute__((aligned(16))) char smem[Wk::LDS_BYTES];
  __shared__ int s_first[kMaxLocal + 1];
  __shared__ int t_first[kMaxLocal + 1];
  __shared__ int s_lo[kMaxLocal + 1];
  __shared__ int wsum[12];
  int n_chunks, n_tiles, n_big;
  build_lists(a, kTileBM, s_first, t_first, s_lo, wsum, n_chunks, n_tiles, n_big, true, kWalkRows);
  SkCost q;
  q.nk = a.N / 64;   // units per chunk
  q.slabs = 1;
  q.nks = q.nk;
  q.lo0 = s_lo[0];
  q.wrows = 64;
  q.crows = kWalkRows;
  const long long C = q.chunk_start(n_chunks, s_lo[a.nloc]);
  if (C == 0) return;
  const long long total = (long long)n_chunks * q.nk;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NW = gridDim.x * 4;   // gridDim.x is a multiple of 8
  const int vw = ((blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8) * 4 + wave;
  const long long x0 = (C * vw + NW - 1) / NW, x1 = (C * (vw + 1) + NW - 1) / NW;
  long long st = x0 < C ? sk_step_at(q, x0, s_first, s_lo, a.nloc) : total;
  const long long s1 = x1 < C ? sk_step_at(q, x1, s_first, s_lo, a.nloc) : total;
  constexpr int SPU = 64 / Wk::STEP_COLS;   // walk steps per unit
  while (st < s1) {
    const int c = __builtin_amdgcn_readfirstlane((int)(st / q.nk));
    const int u0 = __builtin_amdgcn_readfirstlane((int)(st - (long long)c * q.nk));
    const int n = __builtin_amdgcn_readfirstlane((int)min(s1 - st, (long long)(q.nk - u0)));
    const int e = find_expert(s_first, a.nloc, c);
    Wk::run(a, s_lo, e, c - s_first[e], u0 * 64, n * SPU, smem);
    st += n;
  }
}

// ---------------------------------------------------------------- tiled path

// Experts with more than kChunkRows rows, when ffn_big_kernel does not take
// them: 128 weight rows x 128 tokens per tile, K staged through LDS 64 at a time (double-buffered through
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
    uint32_t tok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rbase + 32 * i;
      tok[i] = row0 + (r < rows ? r : 0);
    }
    a_rows<4>(a, tok);
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

// ---------------------------------------------------------------- large-tile path

// Experts with more than kChunkRows rows when their tiles fill the GPU
// (prefill; big_takes below), instead of the 128 x 128 tiles above: 256 weight rows x 256 tokens per tile, one workgroup
// of 4 wavefronts per CU, each wavefront 128 x 128 on v_mfma_f32_32x32x16_bf16
// (4 x 4 fragments, 256 float32 accumulators per lane). Per k16 step a
// wavefront reads 8 KB of fragments from LDS for 16 MFMAs, which leaves the
// LDS with headroom while the MFMA pipes are busy (a 128 x 128 wavefront
// tile is what makes that ratio work; 64 x 64 needs more LDS bandwidth than
// the CU has).
//
// K is staged 64 at a time in two LDS buffers filled by LDS DMA
// (buffer_load_dwordx4 ... lds: the data goes from memory to LDS without
// registers; lane l of one instruction writes 16 bytes at M0 + 16 l). Each
// DMA instruction covers 8 rows x 128 bytes, whole cache lines (from L2, an
// instruction over 16 half lines moved about half the bytes per clock of
// one over 8 whole lines). While one buffer is multiplied the next stage
// (64 KB) is loaded into the other. The DMA is issued from inline assembly
// and waited for explicitly: the compiler would otherwise wait for every
// outstanding LDS DMA at each barrier.
//
// LDS rows are 128 bytes (8 chunks of 16 bytes); chunk c of row r sits at
// slot c ^ ((r >> 1) & 7), so the 16 rows one fragment read touches per 16
// lanes fall on 16 distinct 16-byte bank groups. A DMA instruction writes 8
// rows in lane order (lane l: row l / 8, slot l % 8), so in block b (rows
// 8b..8b+7) lane l loads chunk (l % 8) ^ (4 (b % 2) + l / 16).
//
// Gated tiles hold, for 128 output columns, per wavefront row half: 64 gate
// rows then the 64 matching up rows, so SiLU(gate) * up is formed from the
// wavefront's own accumulators.
constexpr int kBigBK = 64;
constexpr int kBigStages = 2;

template <bool GATED>
struct Big {
  static constexpr int COLS = GATED ? 128 : 256;            // output columns per tile
  static constexpr int OP_BYTES = 256 * kBigBK * 2;          // one operand of one stage (32 KB)
  static constexpr int STAGE_BYTES = 2 * OP_BYTES;
  static constexpr int LDS_BYTES = kBigStages * STAGE_BYTES;  // 128 KB
  static constexpr int BLOCKS = 8;                            // 8-row DMA blocks per operand per wavefront

  // A wavefront multiplies its weight rows by token fragments 2j + wn (rows
  // (2j + wn) * 32 .. + 31, j = 0..3): the two wavefront columns take every
  // other 32-row fragment, so in an expert's last, partly filled tile they
  // keep about the same number of fragments. Only the fragments that hold a
  // valid row are multiplied (nj of them, a template argument so that the K
  // loop stays fully unrolled); all 256 token rows are still loaded (skipping
  // the blocks past the last row costs more scalar registers than the kernel
  // has).
  __device__ static void run(const GemmArgs& a, int e, int row0, int rows, int nb, char* lds, int tid) {
    const int wn = __builtin_amdgcn_readfirstlane(tid >> 6) & 1;
    const int nj = __builtin_amdgcn_readfirstlane(min(4, (((rows + 31) >> 5) - wn + 1) >> 1));
    switch (nj) {
      case 4: body<4>(a, e, row0, rows, nb, lds, tid); break;
      case 3: body<3>(a, e, row0, rows, nb, lds, tid); break;
      case 2: body<2>(a, e, row0, rows, nb, lds, tid); break;
      case 1: body<1>(a, e, row0, rows, nb, lds, tid); break;
      default: body<0>(a, e, row0, rows, nb, lds, tid); break;
    }
  }

  // MFMA of a stage after which DMA instruction d (0..15) of the next stage
  // is issued: the 16 instructions are spread evenly over the first half of
  // the stage's 16 NJ MFMAs.
  template <int NJ>
  __device__ static constexpr int dma_after(int d) {
    const int m = (d + 1) * (8 * NJ) / 16 - 1;
    return m < 0 ? 0 : m;
  }

  template <int NJ>
  __device__ static void body(const GemmArgs& a, int e, int row0, int rows, int nb, char* lds, int tid) {
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;   // weight rows wm*128.., token fragments 2j + wn
    const uint32_t pitch = (uint32_t)a.K * 2;
    const int lrow = lane >> 3;                               // row within an 8-row DMA block
    const int lchunk = (lane & 7) ^ (lane >> 4);              // chunk fetched in even blocks
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);

    // This wavefront fills 8-row blocks g = wave * 8 + i (i = 0..7) of both
    // operands; odd blocks fetch chunk lchunk ^ 4. Weights: block g -> first
    // weight row (uniform).
    const i32x4_t wbuf = buffer_rsrc(a.W + (size_t)e * a.N * a.K, (uint32_t)(a.N * pitch));
    int wso[BLOCKS];
#pragma unroll
    for (int i = 0; i < BLOCKS; ++i) {
      const int r = (wave * BLOCKS + i) * 8;   // first tile row of the block
      int base;
      if (GATED) {
        const int grp = r >> 5, wmi = grp >> 2, q = grp & 3;
        base = ((q < 2) ? 0 : a.inter) + nb * COLS + wmi * 64 + (q & 1) * 32 + (r & 31);
      } else {
        base = nb * 256 + r;
      }
      wso[i] = __builtin_amdgcn_readfirstlane(base * (int)pitch);
    }
    const uint32_t wv[2] = {(uint32_t)lrow * pitch + lchunk * 16, (uint32_t)lrow * pitch + (lchunk ^ 4) * 16};
    // Tokens: rows past the tile's end read its first row (not stored).
    const i32x4_t xbuf = buffer_rsrc(a.A, 0xFFFFFFFFu);
    uint32_t xv[BLOCKS];
#pragma unroll
    for (int i = 0; i < BLOCKS; ++i) {
      const int r = (wave * BLOCKS + i) * 8 + lrow;
      xv[i] = row0 + (r < rows ? r : 0);
    }
    a_rows<BLOCKS>(a, xv);
#pragma unroll
    for (int i = 0; i < BLOCKS; ++i) xv[i] = xv[i] * pitch + (lchunk ^ ((i & 1) << 2)) * 16;

    // DMA number d (0..15) of this wavefront's share of stage kt: weight
    // blocks first, then token blocks.
    auto issue_one = [&](int kt, int d) {
      const uint32_t lw = lds_base + (kt & 1) * STAGE_BYTES;
      const uint32_t ko = (uint32_t)kt * kBigBK * 2;
      if (d < BLOCKS) lds_dma16(lw + (wave * BLOCKS + d) * 1024, wbuf, wv[d & 1], wso[d] + ko);
      else lds_dma16(lw + OP_BYTES + (wave * BLOCKS + d - BLOCKS) * 1024, xbuf, xv[d - BLOCKS], ko);
    };

    f32x16_t acc[4][NJ > 0 ? NJ : 1];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16_t{};

    const int fr = lane & 31, fh = lane >> 5;  // fragment row, k half
    const int fsw = (fr >> 1) & 7;               // the swizzle of every row this lane reads
    // Multiplies stage `slot` and issues the DMA of stage knext (if >= 0) into
    // the other buffer, spread over the first half of the MFMAs. A wavefront
    // that issues a burst of vector-memory instructions stalls until the CU's
    // address unit has taken them, and with one wavefront per SIMD nothing
    // else keeps the SIMD's MFMA pipe busy meanwhile; spread out, they issue
    // without stalls, and the last one still has half a stage to land.
    // Fragments of the next 16 k are read while the current ones are
    // multiplied.
    auto compute = [&](int slot, int knext) {
      if (NJ == 0) {
        if (knext >= 0) {
#pragma unroll
          for (int d = 0; d < 2 * BLOCKS; ++d) issue_one(knext, d);
        }
        return;
      }
      const char* lw = lds + slot * STAGE_BYTES + (wm * 128 + fr) * 128;
      const char* lx = lds + slot * STAGE_BYTES + OP_BYTES + (wn * 32 + fr) * 128;
      constexpr int NQ = kBigBK / 16;
      bf16x8_t av[4], bv[NJ > 0 ? NJ : 1];
      {
        const int off = (fh ^ fsw) << 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = *(const bf16x8_t*)(lw + i * 32 * 128 + off);
#pragma unroll
        for (int j = 0; j < NJ; ++j) bv[j] = *(const bf16x8_t*)(lx + j * 64 * 128 + off);
      }
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int offn = (((q + 1) * 2 + fh) ^ fsw) << 4;
        bf16x8_t an[4], bn[NJ > 0 ? NJ : 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (q + 1 < NQ) {
            an[i] = *(const bf16x8_t*)(lw + i * 32 * 128 + offn);
            if (i < NJ) bn[i] = *(const bf16x8_t*)(lx + i * 64 * 128 + offn);
          }
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
            const int m = (q * 4 + i) * NJ + j;   // MFMA number within the stage
#pragma unroll
            for (int d = 0; d < 2 * BLOCKS; ++d) {
              if (dma_after<NJ>(d) == m) {
                __builtin_amdgcn_sched_barrier(0);
                if (knext >= 0) issue_one(knext, d);
                __builtin_amdgcn_sched_barrier(0);
              }
            }
          }
        }
        if (q + 1 < NQ) {
#pragma unroll
          for (int i = 0; i < 4; ++i) av[i] = an[i];
#pragma unroll
          for (int j = 0; j < NJ; ++j) bv[j] = bn[j];
        }
      }
    };

    // Iteration kt: wait until this wavefront's DMA of stage kt has landed,
    // barrier (every wavefront's share of stage kt is in LDS, and every
    // wavefront has finished stage kt - 1, whose buffer stage kt + 1 reuses),
    // multiply stage kt while issuing stage kt + 1.
    const int nk = a.K / kBigBK;
#pragma unroll
    for (int d = 0; d < 2 * BLOCKS; ++d) issue_one(0, d);
    for (int kt = 0; kt < nk; ++kt) {
      wait_vmcnt<0>();
      __syncthreads();
      compute(kt & 1, kt + 1 < nk ? kt + 1 : -1);
    }

    // One fragment column at a time (all lanes compute, only the store is
    // guarded), so the accumulators are read out piecewise.
    // acc[i][j][r]: token (2j + wn)*32 + lane%32; wavefront weight row
    // i*32 + (r/4)*8 + (lane/32)*4 + r%4.
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      const int t = (2 * j + wn) * 32 + fr;
      const bool ok = t < rows;
      uint16_t* crow = a.C + (size_t)(row0 + (ok ? t : 0)) * a.ldc;
      if (GATED) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = nb * COLS + wm * 64 + i * 32 + q * 8 + fh * 4;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = silu(acc[i][j][q * 4 + r]) * acc[i + 2][j][q * 4 + r];
            const uint2 pk = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            if (ok) *(uint2*)(crow + col) = pk;
          }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = nb * COLS + wm * 128 + i * 32 + q * 8 + fh * 4;
            const f32x16_t& c = acc[i][j];
            const uint2 pk = make_uint2(pack_bf16x2(c[q * 4], c[q * 4 + 1]),
                                        pack_bf16x2(c[q * 4 + 2], c[q * 4 + 3]));
            if (ok) *(uint2*)(crow + col) = pk;
          }
      }
    }
  }
};

// The large-tile kernel takes every expert with more than kChunkRows rows
// when its items (256-row tiles x N blocks) fill at least 3/4 of the CUs in
// their first round; else the persistent kernel's 128 x 128 tiles do (two
// workgroups per CU). The 256 x 256 tiles move half the bytes through L2, but
// a workgroup keeps only one 64 KB stage in flight, so on fewer CUs the
// aggregate L2 -> LDS rate of the smaller tiles wins. For an expert with 65
// .. 256 rows a row of (partly filled) 256 x 256 tiles costs less than
// streaming its weights once per 64-row chunk.
__device__ __forceinline__ bool big_takes(int items, int cus) { return 4 * items >= 3 * cus; }

// Tiles of the experts with more than kChunkRows rows, 256 tokens each; a
// persistent loop over them, one workgroup per CU.
template <bool GATED>
__global__ __launch_bounds__(256, 1) void ffn_big_kernel(GemmArgs a) {
  using B = Big<GATED>;
  __shared__ __attribute__((aligned(16))) char smem[B::LDS_BYTES];
  __shared__ int s_first[kMaxLocal + 1];
  __shared__ int t_first[kMaxLocal + 1];
  __shared__ int s_lo[kMaxLocal + 1];
  __shared__ int wsum[12];
  int n_chunks, n_tiles, n_big;
  build_lists(a, kBigBM, s_first, t_first, s_lo, wsum, n_chunks, n_tiles, n_big, false, kChunkRows,
              kChunkRows);
  const int nblk = (GATED ? a.inter : a.N) / B::COLS;
  if (!big_takes(n_tiles * nblk, a.big_min_items)) return;  // the persistent kernel does these experts
  // Items are (token tile, N block) with N blocks fastest, taken round-robin
  // by a grid that is a multiple of 8: workgroup b runs on XCD b % 8, so the
  // items of one N block -- the same weight block for every token tile of an
  // expert -- share that XCD's L2 when the N blocks per tile are a multiple
  // of 8, while the XCDs read the same token tiles at about the same time
  // (shared through the last-level cache). When all items fit in one round,
  // the N blocks per tile are padded to a multiple of 8 (the padding items
  // are skipped; the workgroups they would take are idle anyway), so that
  // holds for any nblk; with more rounds padding would leave whole
  // workgroups idle, so the numbering stays dense.
  // (The loop runs over a multiple of 8 items and skips the ones past the
  // end; this form compiles without register spills.)
  const int nblk8 = (nblk + 7) & ~7;
  const int nbp = __builtin_amdgcn_readfirstlane(n_tiles * nblk8 <= (int)gridDim.x ? nblk8 : nblk);
  const int total = n_tiles * nbp;
  const int per = (total + 7) / 8;
  for (int w = blockIdx.x; w < 8 * per; w += gridDim.x) {
    if (w >= total || w % nbp >= nblk) continue;
    const int tile = __builtin_amdgcn_readfirstlane(w / nbp);
    const int nb = __builtin_amdgcn_readfirstlane(w % nbp);
    const int e = __builtin_amdgcn_readfirstlane(find_expert(t_first, a.nloc, tile));
    const int row0 = __builtin_amdgcn_readfirstlane(s_lo[e] + (tile - t_first[e]) * kBigBM);
    const int rows = __builtin_amdgcn_readfirstlane(min(kBigBM, s_lo[e + 1] - row0));
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));  // keeps per-thread setup inside the tile loop
    B::run(a, e, row0, rows, nb, smem, tid);
    __syncthreads();  // the LDS buffers are reused by the next tile
  }
}

// ---------------------------------------------------------------- the GEMM kernel

// One persistent kernel per GEMM: first the streamed row chunks, then the row
// tiles of larger experts. The two paths share the LDS buffer.
template <int NTW, int KS, bool GATED>
__global__ __launch_bounds__(256, 2) void ffn_gemm_kernel(GemmArgs a) {
  using S = Stream<NTW, KS, GATED, kStreamDW, kStreamDA>;
  using T = Tiled<GATED>;
  constexpr int SL = S::LDS_BYTES;
  constexpr int SMEM = SL > T::LDS_BYTES ? SL : T::LDS_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  __shared__ int s_first[kMaxLocal + 1];
  __shared__ int t_first[kMaxLocal + 1];
  __shared__ int s_lo[kMaxLocal + 1];
  __shared__ int wsum[12];
  // Experts with more than kChunkRows rows are tiled (a tile reads the
  // weights once per kTileBM rows, a streamed chunk once per kChunkRows).
  int n_chunks, n_tiles, n_big;
  build_lists(a, kTileBM, s_first, t_first, s_lo, wsum, n_chunks, n_tiles, n_big, false, kChunkRows,
              kChunkRows);
  const int ncols = GATED ? a.inter : a.N;
  const int slabs = ncols / S::COLS;
  const int nblk = ncols / T::COLS;
  // Same decision as ffn_big_kernel (big_takes over the same tiles): when it
  // takes every tiled expert only the streamed ones are done here; else the
  // tiles are done here, 128 x 128.
  const bool big = a.big_ok && big_takes(n_big * (ncols / Big<GATED>::COLS), a.big_min_items);
  const int n_stream = n_chunks * slabs;
  const int total = n_stream + (big ? 0 : n_tiles * nblk);
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    if (w < n_stream) {
      const int c = w / slabs;
      const int e = find_expert(s_first, a.nloc, c);
      S::run(a, s_lo, e, c - s_first[e], w % slabs, smem);
      __syncthreads();  // the LDS buffer is reused by the next work item
    } else {
      const int tile = (w - n_stream) / nblk, nb = (w - n_stream) % nblk;
      const int e = find_expert(t_first, a.nloc, tile);
      const int row0 = s_lo[e] + (tile - t_first[e]) * kTileBM;
      const int rows = min(kTileBM, s_lo[e + 1] - row0);
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

// 16 rows x 16 output columns per workgroup, plain FMA, bounds-checked in N
// and K. K goes in chunks of 256: thread (ty, tx) loads elements tx + 16 j
// (j = 0..15) of the chunk for row ty of each operand (coalesced, all loads
// of a chunk in flight together), the next chunk's loads are issued before
// the current one is multiplied, and each output accumulates over k in
// ascending order. blockIdx.y = expert * max_row_tiles + row tile;
// blockIdx.x = column block.
constexpr int kF32KC = 256;
constexpr int kF32J = kF32KC / 16;   // elements per thread and operand of one chunk

template <bool GATED>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgsF32 a) {
  // rows padded by 4 floats: 16-byte aligned for float4 reads
  __shared__ __attribute__((aligned(16))) float As[16][kF32KC + 4], Bg[16][kF32KC + 4], Bu[16][kF32KC + 4];
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
  const int n = col0 + ty;   // the weight row this thread loads
  const float* grow = n < n_out ? We + (size_t)n * K : nullptr;
  const float* urow = (GATED && n < n_out) ? We + (size_t)(a.inter + n) * K : nullptr;
  float ra[kF32J], rg[kF32J], ru[kF32J];
  auto load = [&](int k0) {
#pragma unroll
    for (int j = 0; j < kF32J; ++j) {
      const int kk = k0 + tx + 16 * j;
      ra[j] = (arow && kk < K) ? arow[kk] : 0.f;
      rg[j] = (grow && kk < K) ? grow[kk] : 0.f;
      if (GATED) ru[j] = (urow && kk < K) ? urow[kk] : 0.f;
    }
  };
  float gs = 0.f, us = 0.f;
  load(0);
  for (int k0 = 0; k0 < K; k0 += kF32KC) {
#pragma unroll
    for (int j = 0; j < kF32J; ++j) {
      As[ty][tx + 16 * j] = ra[j];
      Bg[ty][tx + 16 * j] = rg[j];
      if (GATED) Bu[ty][tx + 16 * j] = ru[j];
    }
    __syncthreads();
    if (k0 + kF32KC < K) load(k0 + kF32KC);
#pragma unroll
    for (int q = 0; q < kF32KC; q += 4) {
      const float4 av = *(const float4*)&As[ty][q];
      const float4 gv = *(const float4*)&Bg[tx][q];
      gs = fmaf(av.x, gv.x, gs);
      gs = fmaf(av.y, gv.y, gs);
      gs = fmaf(av.z, gv.z, gs);
      gs = fmaf(av.w, gv.w, gs);
      if (GATED) {
        const float4 uv = *(const float4*)&Bu[tx][q];
        us = fmaf(av.x, uv.x, us);
        us = fmaf(av.y, uv.y, us);
        us = fmaf(av.z, uv.z, us);
        us = fmaf(av.w, uv.w, us);
      }
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

// Shape of the streaming path: NTW = 2 weight tiles per wavefront (gated: a
// gate tile and the matching up tile) and KS, the K slices of a workgroup.
// Gated GEMMs (K = hidden, a multiple of 256) take KS = 4 from K = 1024 on,
// else 2. Plain GEMMs take the largest KS that still leaves every slice at
// least 16 K steps, else 2 when K allows it, else 1.
template <bool GATED>
int stream_ks(int K) {
  if (GATED) return K >= 1024 ? 4 : 2;
  if (K % 256 == 0 && K / 4 >= 1024) return 4;
  if (K % 128 == 0) return 2;
  return 1;
}

// Tiled experts go to ffn_big_kernel when the output width allows its tiles,
// the row capacity is prefill-sized and (on the device) its tiles fill at
// least 3/4 of the CUs (big_takes); else to the 128 x 128 tiles of the
// persistent kernel. Both paths are complete; the capacity test keeps
// decode-sized calls from paying for a second launch that finds no work.
template <bool GATED>
bool use_big(const GemmArgs& g) {
  return kUseBigTiles && g.capacity >= kBigMinCapacity && g.K % kBigBK == 0 &&
         (GATED ? g.inter % 128 == 0 : g.N % 256 == 0);
}

template <bool GATED, int KS>
hipError_t launch_gemm_t(const GemmArgs& g0, hipStream_t s) {
  constexpr int NTW = 2;
  using S = Stream<NTW, KS, GATED, kStreamDW, kStreamDA>;
  using T = Tiled<GATED>;
  GemmArgs g = g0;
  g.big_ok = use_big<GATED>(g) ? 1 : 0;
  g.big_min_items = cu_count();
  auto kernel = ffn_gemm_kernel<NTW, KS, GATED>;
  static const int occ = occupancy(kernel, 256);
  const int ncols = GATED ? g.inter : g.N;
  const long max_chunks = g.nloc;   // streamed experts have at most kChunkRows rows: one chunk each
  const long max_tiles = (long)(g.capacity + kTileBM - 1) / kTileBM + g.nloc;
  const long per_chunk = ncols / S::COLS;
  const long max_work = max_chunks * per_chunk + max_tiles * (ncols / T::COLS);
  const int grid = (int)std::max<long>(1, std::min<long>(max_work, (long)cu_count() * occ));
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, s, g);
  if (!g.big_ok) return hipGetLastError();
  // tiles <= ceil(capacity / 256) + (number of experts above kChunkRows rows)
  const long max_big = ((long)(g.capacity + kBigBM - 1) / kBigBM +
                        std::min<long>(g.nloc, (long)g.capacity / (kChunkRows + 1))) *
                       (ncols / Big<GATED>::COLS);
  // persistent: one workgroup per CU (a multiple of 8, so each keeps its XCD's range)
  const long cus8 = std::max(8, cu_count() / 8 * 8);
  const int grid_big = (int)std::max<long>(8, std::min<long>((max_big + 7) / 8 * 8, cus8));
  hipLaunchKernelGGL(ffn_big_kernel<GATED>, dim3(grid_big), dim3(256), 0, s, g);
  return hipGetLastError();
}

// Walk path: all the wavefronts the grid can keep resident, the grid a multiple of 8.
template <int KQ>
hipError_t launch_walk(const GemmArgs& g, hipStream_t s) {
  static const int occ = occupancy(ffn_walk_kernel<KQ>, 256);
  const int grid = std::max(8, cu_count() * occ / 8 * 8);
  hipLaunchKernelGGL(ffn_walk_kernel<KQ>, dim3(grid), dim3(256), 0, s, g);
  return hipGetLastError();
}

template <bool GATED>
hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (!GATED && g.K == 64) return launch_walk<1>(g, s);
  if (!GATED && g.K == 128) return launch_walk<2>(g, s);
  switch (stream_ks<GATED>(g.K)) {
    case 4: return launch_gemm_t<GATED, 4>(g, s);
    case 2: return launch_gemm_t<GATED, 2>(g, s);
    default: return GATED ? hipErrorInvalidValue : launch_gemm_t<false, 1>(g, s);
  }
}

// The shared-activation path serves gated GEMMs of narrow experts (inter a
// multiple of 64, at most 128).
bool use_shared(int hidden, int inter) { return inter % kShareCols == 0 && inter <= 128 && hidden >= 1024; }
long shared_max_pairs(int num_local, int capacity, int inter) {
  return ((long)(capacity + kShareRows - 1) / kShareRows + num_local) * (inter / kShareCols);
}
// Workgroups of the shared-activation kernel: one per CU, a multiple of 8.
int shared_grid() { return std::max(8, cu_count() / 8 * 8); }

}  // namespace

size_t ffn_workspace_size(int num_local, int hidden, int inter, int capacity, bool bf16) {
  size_t bytes = align256((size_t)capacity * inter * (bf16 ? 2 : 4));  // h
  if (bf16 && use_shared(hidden, inter)) {  // partial sums (slots v + cs), chunk table
    const size_t pairs = (size_t)shared_max_pairs(num_local, capacity, inter);
    bytes += align256((pairs + shared_grid()) * SharedA::PART_FLOATS * sizeof(float));
    bytes += align256((4 + 4 * pairs) * sizeof(int));
  }
  return bytes;
}

namespace {

hipError_t launch_gate_up_shared(const GemmArgs& g0, size_t h_bytes, void* workspace, hipStream_t s) {
  GemmArgs g = g0;
  const long pairs = shared_max_pairs(g.nloc, g.capacity, g.inter);
  g.sk_grid = shared_grid();
  char* p = (char*)workspace + align256(h_bytes);
  g.partials = (float*)p;
  g.chunk_desc = (int*)(p + align256((size_t)(pairs + g.sk_grid) * SharedA::PART_FLOATS * sizeof(float)));
  hipLaunchKernelGGL(ffn_shared_kernel, dim3(g.sk_grid), dim3(256), 0, s, g);
  g.sk_items = (int)(pairs * (kShareRows / 64));
  const int grid_f = (int)std::max<long>(1, std::min<long>(g.sk_items, (long)cu_count() * 4));
  hipLaunchKernelGGL(ffn_finalize_kernel, dim3(grid_f), dim3(256), 0, s, g);
  return hipGetLastError();
}

// ---------------------------------------------------------------- masked layout

// Fixed per-expert slots of `cap` rows with a valid count per expert: one
// workgroup turns the counts into compact offsets (exclusive prefix sums of
// min(max(count, 0), cap)) and, for compact row i of expert e, row_index[i] =
// the slot row e * cap + (i - offsets[e]). nloc <= 1024: one expert per thread.
__global__ __launch_bounds__(1024) void masked_plan_kernel(const int* __restrict__ counts, int nloc, int cap,
                                                           int* __restrict__ offsets,
                                                           int* __restrict__ row_index) {
  __shared__ int s_off[kMaxLocal + 1];
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m = tid < nloc ? min(max(counts[tid], 0), cap) : 0;
  int incl = m;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, MOE_WAVE);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += wsum[i];
  const int excl = before + incl - m;
  if (tid < nloc) {
    s_off[tid] = excl;
    offsets[tid] = excl;
    if (tid == nloc - 1) {
      s_off[nloc] = excl + m;
      offsets[nloc] = excl + m;
    }
  }
  __syncthreads();
  for (int e = w; e < nloc; e += blockDim.x >> 6) {
    const int o = s_off[e], n = s_off[e + 1] - o;
    for (int r = lane; r < n; r += 64) row_index[o + r] = e * cap + r;
  }
}

// o_slots[row_index[i]] = o_compact[i] for the compact rows i < offsets[nloc]:
// one wavefront per row, 16-byte copies.
__global__ __launch_bounds__(256) void masked_scatter_kernel(const uint4* __restrict__ o_compact,
                                                             const int* __restrict__ row_index,
                                                             const int* __restrict__ offsets, int nloc,
                                                             int row_vec, uint4* __restrict__ o_slots) {
  const int lane = threadIdx.x & 63;
  const int M = offsets[nloc];
  for (int r = blockIdx.x * 4 + (threadIdx.x >> 6); r < M; r += gridDim.x * 4) {
    const uint4* src = o_compact + (size_t)r * row_vec;
    uint4* dst = o_slots + (size_t)row_index[r] * row_vec;
    for (int c = lane; c < row_vec; c += 64) dst[c] = src[c];
  }
}

}  // namespace

size_t ffn_masked_workspace_size(int num_local, int hidden, int inter, int cap, bool bf16) {
  const size_t rows = (size_t)num_local * cap;
  return align256((size_t)(num_local + 1) * sizeof(int)) + align256(rows * sizeof(int)) +
         align256(rows * hidden * (bf16 ? 2 : 4)) + ffn_workspace_size(num_local, hidden, inter, (int)rows, bf16);
}

hipError_t launch_ffn_masked(const FfnMaskedArgs& a, hipStream_t s) {
  const long rows = (long)a.num_local * a.cap;
  if (rows == 0) return hipSuccess;
  char* ws = (char*)a.workspace;
  // With at most kChunkRows rows per expert (and inter outside the shared and
  // walk paths' 64 and 128) every expert is streamed: the GEMMs take the counts
  // and read x and write o in slot rows themselves, so no plan, row index or
  // copy back is needed.
  if (a.bf16 && a.cap <= kChunkRows && a.inter != 64 && a.inter != 128) {
    ws += align256((size_t)(a.num_local + 1) * sizeof(int)) + align256((size_t)rows * sizeof(int)) +
          align256((size_t)rows * a.hidden * 2);
    FfnArgs f{a.x_slots, nullptr, 1, nullptr, a.w_gate_up, a.w_down, a.num_local, a.hidden, a.inter, (int)rows,
              true, a.o_slots, ws};
    f.slot_counts = a.counts;
    f.slot_cap = a.cap;
    return launch_ffn(f, s);
  }
  int* offsets = (int*)ws;
  ws += align256((size_t)(a.num_local + 1) * sizeof(int));
  int* row_index = (int*)ws;
  ws += align256((size_t)rows * sizeof(int));
  void* o_compact = ws;
  const size_t row_bytes = (size_t)a.hidden * (a.bf16 ? 2 : 4);
  ws += align256((size_t)rows * row_bytes);
  hipLaunchKernelGGL(masked_plan_kernel, dim3(1), dim3(1024), 0, s, a.counts, a.num_local, a.cap, offsets,
                     row_index);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  FfnArgs f{a.x_slots, row_index, 1, offsets, a.w_gate_up, a.w_down, a.num_local, a.hidden, a.inter, (int)rows,
            a.bf16, o_compact, ws};
  err = launch_ffn(f, s);
  if (err != hipSuccess) return err;
  const int blocks = (int)std::min<long>((rows + 3) / 4, 2048);
  hipLaunchKernelGGL(masked_scatter_kernel, dim3(blocks), dim3(256), 0, s, (const uint4*)o_compact, row_index,
                     offsets, a.num_local, (int)(row_bytes / 16), (uint4*)a.o_slots);
  return hipGetLastError();
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
    if (a.slot_counts) {   // masked layout: x and o in slot rows, h compact
      g1.slot_counts = g2.slot_counts = a.slot_counts;
      g1.slot_cap = g2.slot_cap = a.slot_cap;
      g1.slot_a = 1;
      g2.slot_c = 1;
    }
    const hipError_t err = use_shared(d, I)
        ? launch_gate_up_shared(g1, (size_t)a.capacity * I * 2, a.workspace, s)
        : launch_gemm<true>(g1, s);
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
