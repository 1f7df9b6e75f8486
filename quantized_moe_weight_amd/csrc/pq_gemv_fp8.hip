// Block-scaled FP8 weight-streaming GEMV / skinny GEMM (M <= 8) with the live
// FP8 activation quantisation fused in, K split inside the block where a row
// straddles waves, and an optional fused SiLU(gate)*up epilogue.
//
// [Sionic] §1: at batch 1 the weight-streaming GEMM must keep every compute
// unit issuing loads (split K when rows are too few) and the live FP8
// quantisation of the activation must overlap the first weight loads rather
// than run ahead of them.  [Sionic] §2: the per-K-block scale must not stall
// the load pipeline.  [Sionic] §4: quantisation lives inside the GEMM launch.
//
// gfx950 design
//   * each block owns a contiguous range of output rows; the (row, 1 KB
//     chunk) units of the block are dealt to its 8 waves in order, so K is
//     split wherever a row straddles two waves, and those cuts are reduced
//     through LDS after one barrier: no global partials, atomics or fences;
//   * lane l reads bytes [16l, 16l+16) of each chunk with one 128-bit
//     non-temporal buffer load, so every load instruction covers 8 full
//     128-byte lines, and the lane's 16 bytes lie inside one 128-wide scale
//     block: the block scale is one FMA per 16 weights, no barrier and no
//     cross-lane work inside the K loop;
//   * each wave keeps a ring of D chunk-steps of loads in flight, issued
//     without branches (out-of-range slots return zero without traffic); the
//     last D steps drain the ring without issuing;
//   * the activation is quantised once per block into LDS from loads issued
//     before the weight ring.
#include <stdlib.h>

#include "pq_quant_dev.h"

namespace {

constexpr int kThreads = 512;   // 8 waves; one block per CU
constexpr int kWaves = kThreads / pq::kWave;
constexpr int kMaxM = 8;
constexpr int kXPre = 2;        // activation loads issued ahead of the weight prefetch

constexpr int kRowsCap = 128;   // rows per block at most

struct GemvArgs {
  const uint16_t* x;
  const uint8_t* w;
  const float* wsc;
  uint16_t* y;
  uint8_t* xq_dbg;
  float* xs_dbg;
  int M, K, N;
  int R;            // output rows: N, or N/2 under the SiLU epilogue
  int nch;          // 1 KB chunks per row
};

// LDS layout of one block: [x codes M*K][x scales M*K/128][row partials]
__host__ __device__ inline size_t xs_offset(int M, int K) { return pqhost::align_up((size_t)M * K, 16); }
__host__ __device__ inline size_t part_offset(int M, int K) {
  return xs_offset(M, K) + pqhost::align_up((size_t)M * (K / pq::kBlock) * sizeof(float), 16);
}
__host__ __device__ inline size_t lds_bytes(int M, int K, int rows, int nrow) {
  return part_offset(M, K) + (size_t)(rows + kWaves) * M * nrow * sizeof(float);
}

// ---------------------------------------------------------------------------
// Live activation quantisation of x [M,K] (bf16) into LDS codes [M][K] and
// scales [M][K/128].  8 values per thread, 16 lanes per block.
// ---------------------------------------------------------------------------
struct XLoad {
  uint4 raw[kXPre];
};

__device__ __forceinline__ void xq_issue(const GemvArgs& a, pq::rsrc_t xr, XLoad& xl) {
#pragma unroll
  for (int it = 0; it < kXPre; ++it)
    xl.raw[it] = pq::buf_load16(xr, (uint32_t)(it * kThreads + threadIdx.x) * 16u);
}

__device__ __forceinline__ void xq_finish(const GemvArgs& a, pq::rsrc_t xr, const XLoad& xl, uint8_t* xq_s,
                                          float* xs_s) {
  const long total8 = (long)a.M * a.K / 8;
  const int iters = (int)((total8 + kThreads - 1) / kThreads);
  const bool dbg = blockIdx.x == 0 && a.xq_dbg != nullptr;
  for (int it = 0; it < iters; ++it) {
    const long t = (long)it * kThreads + threadIdx.x;
    const bool valid = t < total8;
    const uint4 raw = it < kXPre ? xl.raw[it < kXPre ? it : 0] : pq::buf_load16(xr, (uint32_t)t * 16u);
    float v[8];
    pq::bf16x8_to_f32(raw, v);
    const float s = pq::fp8_block_scale16(v, valid);
    if (valid) {
      const uint2 c = pq::fp8_codes8(v, s);
      reinterpret_cast<uint2*>(xq_s)[t] = c;
      const bool lead = (threadIdx.x & 15) == 0;
      if (lead) xs_s[(t * 8) / pq::kBlock] = s;
      if (dbg) {
        reinterpret_cast<uint2*>(a.xq_dbg)[t] = c;
        if (lead && a.xs_dbg) a.xs_dbg[(t * 8) / pq::kBlock] = s;
      }
    }
  }
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// ---------------------------------------------------------------------------
// Kernel.  NROW = 1 (plain rows) or 2 (gate row r and up row r + R, fused
// SiLU*up epilogue).  D = depth of the per-lane load ring in chunk-steps.
// MT = number of tokens (M), a compile-time constant so that the per-token
// loops unroll exactly.
// ---------------------------------------------------------------------------
template <int NROW, int D, int MT>
__global__ __launch_bounds__(kThreads) void gemv_fp8_kernel(GemvArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* xq_s = smem;
  float* xs_s = reinterpret_cast<float*>(smem + xs_offset(MT, a.K));
  float* part = reinterpret_cast<float*>(smem + part_offset(MT, a.K));   // [(row + wave)][MT][NROW]

  const int lane = pq::lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(pq::wave_id());
  const int r0 = pq::split_start(a.R, (int)gridDim.x, (int)blockIdx.x);
  const int nrows = pq::split_start(a.R, (int)gridDim.x, (int)blockIdx.x + 1) - r0;
  const int nunits = nrows * a.nch;
  const int u0 = pq::split_start(nunits, kWaves, wv);
  const int nsteps = pq::split_start(nunits, kWaves, wv + 1) - u0;
  const int nb = a.K / pq::kBlock;

  // --- activation loads first, then the weight ring, then quantise -------
  const pq::rsrc_t xr = pq::make_rsrc(a.x, (uint32_t)a.M * a.K * 2u);
  const pq::rsrc_t wr = pq::make_rsrc(a.w, (uint32_t)((size_t)a.N * a.K));
  const pq::rsrc_t sr = pq::make_rsrc(a.wsc, (uint32_t)((size_t)a.N * nb * 4));
  XLoad xl;
  xq_issue(a, xr, xl);

  uint4 wbuf[D][NROW];
  float sbuf[D][NROW];
  int ir = u0 / a.nch, ic = u0 - (u0 / a.nch) * a.nch, left = nsteps;   // issue cursor (local row, chunk)
  const uint32_t lane16 = 16u * (uint32_t)lane;
  const uint32_t lane_blk4 = 4u * ((uint32_t)lane >> 3);     // this lane's scale block within a chunk
  auto issue = [&](uint4 (&wb)[NROW], float (&sb)[NROW]) {
    const uint32_t off = (uint32_t)(ic * pq::kChunk) + lane16;
    const bool ok = left > 0 && off < (uint32_t)a.K;
#pragma unroll
    for (int j = 0; j < NROW; ++j) {
      const uint32_t row = (uint32_t)(r0 + ir + j * a.R);
      wb[j] = pq::buf_load16_nt(wr, ok ? row * (uint32_t)a.K + off : pq::kOOB);
      sb[j] = pq::buf_load_f32_nt(sr, ok ? (row * (uint32_t)nb + (uint32_t)ic * 8u) * 4u + lane_blk4 : pq::kOOB);
    }
    --left;
    if (++ic == a.nch) { ic = 0; ++ir; }
  };
#pragma unroll
  for (int j = 0; j < D; ++j) issue(wbuf[j], sbuf[j]);

  xq_finish(a, xr, xl, xq_s, xs_s);
  __syncthreads();

  float acc[NROW][MT];
#pragma unroll
  for (int j = 0; j < NROW; ++j)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[j][m] = 0.0f;

  int cr = u0 / a.nch, cc = u0 - (u0 / a.nch) * a.nch;    // consume cursor (local row, chunk)
  auto consume = [&](const uint4 (&wb)[NROW], const float (&sb)[NROW], bool last) {
    const uint32_t off = (uint32_t)(cc * pq::kChunk) + lane16;
    if (off < (uint32_t)a.K) {
      pq::Bf16x16 wv16[NROW];
#pragma unroll
      for (int j = 0; j < NROW; ++j) wv16[j] = pq::widen16(wb[j]);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint4 xc = *reinterpret_cast<const uint4*>(xq_s + (size_t)m * a.K + off);
        const float xs = xs_s[m * nb + off / pq::kBlock];
        const pq::Bf16x16 xv = pq::widen16(xc);
#pragma unroll
        for (int j = 0; j < NROW; ++j) acc[j][m] = fmaf(pq::dot16(wv16[j], xv), sb[j] * xs, acc[j][m]);
      }
    }
    if (cc == a.nch - 1 || last) {                     // this wave's part of row cr is done
      float v = 0.0f;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < NROW; ++j) {
          const float s = pq::wave_sum(acc[j][m]);
          acc[j][m] = 0.0f;
          if (lane == m * NROW + j) v = s;
        }
      if (lane < MT * NROW) part[(cr + wv) * MT * NROW + lane] = v;
    }
    if (++cc == a.nch) { cc = 0; ++cr; }
  };

  int base = 0;
  for (; base + D < nsteps; base += D) {               // steady state: every slot refills
#pragma unroll
    for (int q = 0; q < D; ++q) {
      consume(wbuf[q], sbuf[q], false);
      issue(wbuf[q], sbuf[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < D; ++q)                          // drain
    if (base + q < nsteps) consume(wbuf[q], sbuf[q], base + q == nsteps - 1);
  __syncthreads();

  // each row: the parts of the waves that covered it, in wave order
  for (int i = (int)threadIdx.x; i < nrows * MT; i += kThreads) {
    const int r = i / MT, m = i - (i / MT) * MT;
    float g = 0.0f, u = 0.0f;
    for (int w = 0; w < kWaves; ++w) {
      const int a0 = pq::split_start(nunits, kWaves, w), a1 = pq::split_start(nunits, kWaves, w + 1);
      if (a0 < a1 && a0 < (r + 1) * a.nch && a1 > r * a.nch) {
        g += part[((r + w) * MT + m) * NROW];
        if (NROW == 2) u += part[((r + w) * MT + m) * NROW + 1];
      }
    }
    a.y[(size_t)m * a.R + r0 + r] = pq::bf16_rne(NROW == 2 ? silu_mul(g, u) : g);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
int check_shape(int M, int K, int N, int epi) {
  if (M < 1 || M > kMaxM || K < pq::kBlock || K % pq::kBlock != 0 || K > 16384 || N < 1) return PQ_ERR_SHAPE;
  if (epi != PQ_EPI_NONE && epi != PQ_EPI_SILU_MUL) return PQ_ERR_SHAPE;
  if (epi == PQ_EPI_SILU_MUL && N % 2 != 0) return PQ_ERR_SHAPE;
  if ((size_t)N * K > pq::kMaxBufferBytes) return PQ_ERR_SHAPE;
  return PQ_OK;
}

// Blocks: PQ_BLOCKS_PER_CU per CU (default 1), at most one per row and at
// least enough for kRowsCap rows per block.  The grid depends on R and the
// device only, so where a row's K range is cut between waves, and with it
// every output bit, is the same for every M.
int grid_for(int R, int num_cus) {
  const char* env = getenv("PQ_BLOCKS_PER_CU");
  const int per_cu = env && atoi(env) > 0 ? atoi(env) : 1;
  long grid = (long)num_cus * per_cu;
  if (grid > R) grid = R;
  const long need = ((long)R + kRowsCap - 1) / kRowsCap;
  if (grid < need) grid = need;
  return (int)grid;
}

template <int NROW, int D, int MT>
hipError_t launch_m(const GemvArgs& a, int grid, hipStream_t stream) {
  auto kern = gemv_fp8_kernel<NROW, D, MT>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int rows = (a.R + grid - 1) / grid;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds_bytes(a.M, a.K, rows, NROW), stream, a);
  return hipGetLastError();
}

template <int NROW, int D>
hipError_t launch(const GemvArgs& a, int grid, hipStream_t stream) {
  switch (a.M) {
    case 1: return launch_m<NROW, D, 1>(a, grid, stream);
    case 2: return launch_m<NROW, D, 2>(a, grid, stream);
    case 3: return launch_m<NROW, D, 3>(a, grid, stream);
    case 4: return launch_m<NROW, D, 4>(a, grid, stream);
    case 5: return launch_m<NROW, D, 5>(a, grid, stream);
    case 6: return launch_m<NROW, D, 6>(a, grid, stream);
    case 7: return launch_m<NROW, D, 7>(a, grid, stream);
    default: return launch_m<NROW, D, 8>(a, grid, stream);
  }
}

}  // namespace

extern "C" {

size_t pq_gemv_fp8_workspace(int, int, int, int) { return 0; }

int pq_gemv_fp8(const uint16_t* x, int M, int K, const uint8_t* w, const float* w_scale, int N, int epi,
                uint16_t* y, uint8_t* xq_dbg, float* xs_dbg, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (!x || !w || !w_scale || !y) return PQ_ERR_NULL;
  int st = check_shape(M, K, N, epi);
  if (st != PQ_OK) return st;
  if (!pqhost::aligned16(x) || !pqhost::aligned16(w) || !pqhost::aligned16(w_scale) || !pqhost::aligned16(y) ||
      (xq_dbg && !pqhost::aligned16(xq_dbg)) || (xs_dbg && !pqhost::aligned16(xs_dbg)))
    return PQ_ERR_ALIGN;
  pqhost::DeviceInfo dev;
  st = pqhost::current_device_info(&dev);
  if (st != PQ_OK) return st;

  GemvArgs a;
  a.x = x; a.w = w; a.wsc = w_scale; a.y = y; a.xq_dbg = xq_dbg; a.xs_dbg = xs_dbg;
  a.M = M; a.K = K; a.N = N;
  a.R = epi == PQ_EPI_SILU_MUL ? N / 2 : N;
  a.nch = (K + pq::kChunk - 1) / pq::kChunk;
  const int grid = grid_for(a.R, dev.num_cus);
  if (lds_bytes(M, K, (a.R + grid - 1) / grid, epi == PQ_EPI_SILU_MUL ? 2 : 1) > 160 * 1024) return PQ_ERR_SHAPE;

  hipError_t e = epi == PQ_EPI_SILU_MUL ? launch<2, 8>(a, grid, (hipStream_t)stream)
                                        : launch<1, 16>(a, grid, (hipStream_t)stream);
  if (e != hipSuccess) {
    pqhost::set_last_hip_error((int)e);
    return PQ_ERR_HIP;
  }
  return PQ_OK;
}

}  // extern "C"
