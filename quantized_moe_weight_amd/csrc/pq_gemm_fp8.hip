// Prefill / large-M block-scaled FP8 GEMM on the matrix cores:
//   y[m, n] = epi( sum_b s_x[m,b] s_w[n,b] sum_{k in b} q_x[m,k] q_w[n,k] )
// with the activation quantised live (the rule of pq_quantize_fp8) and the
// weights in the layout of the GEMV (E4M3 [N,K], fp32 [N,K/128]).
//
// [M3]: prefill reuses each prepared weight for many tokens and wide loads
// with merged passes raised its share of the matmul limit; with hundreds of
// tokens per weight byte the product is bound by the matrix cores, not HBM.
//
// gfx950 design
//   * a 512-thread block (8 waves, 2 x 4) owns a 256-token x 256-weight-row
//     tile (64 KB of operands per K step for 16.8 MFLOP: large tiles keep the
//     L2 traffic within what eight L2s deliver; 128-token tiles where 256 would
//     leave CUs without a tile); each wave a 128 x 64 part =
//     8 x 4 v_mfma_f32_16x16x128_f8f6f4 per 128-wide K block (the scale
//     block), whose fp32 results take both block scales (acc += d * (s_x *
//     s_w)) in fp32 on the vector unit; two waves per SIMD, so one wave's
//     matrix work covers the other's waits;
//   * operands stream from memory straight into LDS (buffer loads with an
//     LDS destination: no registers) for K step k + 1 while step k computes;
//     one block barrier per K step, after each wave has waited for its own
//     loads of the step; the loads are issued from inline assembly, because
//     the compiler's wait insertion cannot tell the two stages apart and
//     otherwise waits for the next stage before reading the current one
//     (which took away the overlap on every other step);
//   * the block scales of sub-tile t - 1 are applied while the matrix core
//     works on sub-tile t (on this chip the vector and matrix work of a
//     SIMD do not overlap in time, measured with a register-only probe, so
//     the scaling's two fp32 operations per output and block cost what the
//     matrix instructions cost: the kernel is bound by their sum);
//   * a wave's load instruction covers 8 rows x 128 bytes (whole lines) and
//     lands as 1 KB of LDS; in LDS the 16-byte slot s of row r holds global
//     slot s ^ (r % 8), which spreads the operand reads over all banks;
//   * operand layout as in the matrix-core GEMV: lane l carries row l % 16 of
//     a 16-row sub-tile, lane group g = l / 16 the bytes [16g, 16g+16) and
//     [64+16g, 80+16g) of the block, alike in A (tokens) and B (weight rows);
//   * SiLU(gate)*up: a tile holds 128 output columns, its 256 B rows ordered
//     in runs of 32 as gate, up, gate, up, ..., so each wave's column tiles b
//     and b + 2 are the gate and the up of the same outputs, in the same
//     lanes;
//   * tiles are dealt to the 8 XCDs in contiguous runs of a grouped order
//     (8 token tiles by as many weight tiles as the run needs), so the blocks
//     that share an operand tile share an L2.
#include <stdlib.h>
#include <string.h>

#include "pq_common.h"

extern "C" int pq_quantize_fp8(const void* in, int in_is_f32, int rows, int K, uint8_t* codes, float* scales,
                               void* stream);

namespace {

typedef int int32x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / pq::kWave;
constexpr int BN = 256;                       // weight rows per tile (tokens per tile: BM, 256 or 128)
// one pipeline stage in LDS: A and B tiles (128-byte rows, swizzled slots)
// and their block scales (the token-scale area always holds 256, the waves
// 0-3 each loading 64 of them)
template <int BM>
struct Stage {
  uint8_t a[BM * pq::kBlock];
  uint8_t b[BN * pq::kBlock];
  float sa[256];
  float sb[BN];
};
constexpr int kXcds = 8;
constexpr int kGroupM = 8;                    // token tiles per group of the tile order
static_assert(2 * sizeof(Stage<256>) <= 160 * 1024, "stages must fit LDS");

struct GArgs {
  const uint8_t* xq;     // [M][K]
  const float* xs;       // [M][K/128]
  const uint8_t* w;      // [N][K]
  const float* ws;       // [N][K/128]
  uint16_t* y;           // [M][R]
  int M, K, N, R;        // R: output columns (N, or N/2 under SiLU*up)
  int silu;
  int tm, tn;            // tiles along the tokens and along the output columns
};

__device__ __forceinline__ floatx4 mfma_e4m3(int32x8 a, int32x8 b) {
  // block-scale operands 0: the plain (unscaled) matrix instruction
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
}

using pq::dma16;
using pq::dma4;
using pq::int32x4;
using pq::lds_addr;
using pq::rsrc_words;

__device__ __forceinline__ int32x8 join8(uint4 lo, uint4 hi) {
  return int32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Weight row of B-tile row r (-1 past the matrix).  Plain: n0 + r.  SiLU*up:
// the tile covers output columns c0 .. c0 + 127 in runs of 32: gate 0..31,
// up 0..31, gate 32..63, up 32..63, ...
__device__ __forceinline__ int b_row(const GArgs& a, int tile_n, int r) {
  if (!a.silu) {
    const int n = tile_n * BN + r;
    return n < a.N ? n : -1;
  }
  const int q = r >> 5, i = r & 31;
  const int c = tile_n * (BN / 2) + (q >> 1) * 32 + i;
  if (c >= a.R) return -1;
  return (q & 1) ? c + a.R : c;
}

// The kernel body for BM-token tiles; st0 and st1 are the kernel's two
// stages (separate LDS objects, sized for the larger tile).
template <int BM>
__device__ __forceinline__ void gemm_body(const GArgs& a, Stage<256>& st0, Stage<256>& st1) {
  constexpr int WM = BM / 2 / 16;             // row tiles per wave (waves: 2 along the tokens)
  const int lane = pq::lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(pq::wave_id());
  const int wm = wv >> 2, wn = wv & 3;        // this wave's part of the tile: rows 128 wm.., cols 64 wn..
  const int rl = lane & 15, lg = lane >> 4;

  // tile of this block: contiguous runs per XCD (block b runs on XCD b % 8)
  // in an order that visits groups of kGroupM token tiles, token tiles
  // fastest inside a group, so an XCD's run is a compact rectangle of tiles
  // (32 tiles: 8 token tiles x 4 weight tiles, 12 operand tiles per K step
  // from outside its L2 instead of 18 for a 16 x 2 strip)
  const int T = a.tm * a.tn;
  const int T8 = T / kXcds * kXcds;
  const int b = (int)blockIdx.x;
  const int t = b < T8 ? (b % kXcds) * (T8 / kXcds) + b / kXcds : b;
  const int grp = t / (kGroupM * a.tn);
  const int gsz = min(kGroupM, a.tm - grp * kGroupM);
  const int tg = t - grp * kGroupM * a.tn;
  const int tile_m = grp * kGroupM + tg % gsz, tile_n = tg / gsz;
  const int m0 = tile_m * BM;
  const int nb = a.K / pq::kBlock;

  const int32x4 xr = rsrc_words(a.xq, (uint32_t)((size_t)a.M * a.K));
  const int32x4 wr = rsrc_words(a.w, (uint32_t)((size_t)a.N * a.K));
  const int32x4 xsr = rsrc_words(a.xs, (uint32_t)((size_t)a.M * nb * 4));
  const int32x4 wsr = rsrc_words(a.ws, (uint32_t)((size_t)a.N * nb * 4));

  // this lane's loads: row 64 i + 8 wv + lane / 8 of A and of B (i < 4),
  // global slot (lane % 8) ^ (lane / 8) of the K block (it lands in LDS slot
  // lane % 8 of that row); one scale per lane (waves 0-3: tokens, 4-7:
  // weight rows)
  const int lrow = 8 * wv + (lane >> 3);
  const uint32_t gslot = 16u * (uint32_t)((lane & 7) ^ (lane >> 3));
  uint32_t aoff[BM / 64], boff[BN / 64];
#pragma unroll
  for (int i = 0; i < BM / 64; ++i) {
    const int r = 64 * i + lrow;
    aoff[i] = m0 + r < a.M ? (uint32_t)(m0 + r) * (uint32_t)a.K + gslot : pq::kOOB;
  }
#pragma unroll
  for (int i = 0; i < BN / 64; ++i) {
    const int n = b_row(a, tile_n, 64 * i + lrow);
    boff[i] = n >= 0 ? (uint32_t)n * (uint32_t)a.K + gslot : pq::kOOB;
  }
  uint32_t soff;
  const bool xscale = wv < 4;
  if (xscale) {
    const int m = m0 + 64 * wv + lane;
    soff = 64 * wv + lane < BM && m < a.M ? (uint32_t)m * (uint32_t)nb * 4u : pq::kOOB;
  } else {
    const int n = b_row(a, tile_n, 64 * (wv - 4) + lane);
    soff = n >= 0 ? (uint32_t)n * (uint32_t)nb * 4u : pq::kOOB;
  }

  // the loads of K block kb into stage st (none past the last block); the
  // block's offset rides in the scalar offset, so the per-lane offsets above
  // (out of range for rows past the matrix) need no work per step
  auto issue = [&](Stage<256>& st, int kb) {
    if (kb >= nb) return;
    const uint32_t kofs = (uint32_t)__builtin_amdgcn_readfirstlane(kb * pq::kBlock);
#pragma unroll
    for (int i = 0; i < BM / 64; ++i) dma16(xr, lds_addr(st.a + (64 * i + 8 * wv) * pq::kBlock), aoff[i], kofs);
#pragma unroll
    for (int i = 0; i < BN / 64; ++i) dma16(wr, lds_addr(st.b + (64 * i + 8 * wv) * pq::kBlock), boff[i], kofs);
    dma4(xscale ? xsr : wsr, lds_addr(xscale ? st.sa + 64 * wv : st.sb + 64 * (wv - 4)), soff,
         (uint32_t)__builtin_amdgcn_readfirstlane(kb * 4));
  };

  float acc[WM][4][4];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;

  // operand reads: slots lg and lg + 4 of a row, after the swizzle
  const uint32_t sw_lo = 16u * (uint32_t)(lg ^ (rl & 7)), sw_hi = 16u * (uint32_t)((lg + 4) ^ (rl & 7));

  auto compute = [&](const Stage<256>& st) {
    int32x8 bf[4];
    float swv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint8_t* p = st.b + (64 * wn + 16 * j + rl) * pq::kBlock;
      bf[j] = join8(*reinterpret_cast<const uint4*>(p + sw_lo), *reinterpret_cast<const uint4*>(p + sw_hi));
      swv[j] = st.sb[64 * wn + 16 * j + rl];
    }
    // software pipeline over the 4 WM sub-tiles: the block scales of sub-tile
    // t - 1 are applied while the matrix core works on sub-tile t
    int32x8 af;
    float sxv[4], sxp[4];
    floatx4 dp;
#pragma unroll
    for (int t = 0; t < 4 * WM; ++t) {
      const int i = t >> 2, j = t & 3;
      if (j == 0) {
        const uint8_t* p = st.a + ((BM / 2) * wm + 16 * i + rl) * pq::kBlock;
        af = join8(*reinterpret_cast<const uint4*>(p + sw_lo), *reinterpret_cast<const uint4*>(p + sw_hi));
#pragma unroll
        for (int r = 0; r < 4; ++r) sxp[r] = sxv[r];
        const float4 sx = *reinterpret_cast<const float4*>(st.sa + (BM / 2) * wm + 16 * i + 4 * lg);
        sxv[0] = sx.x; sxv[1] = sx.y; sxv[2] = sx.z; sxv[3] = sx.w;
      }
      const floatx4 d = mfma_e4m3(af, bf[j]);
      if (t > 0) {
        const int ip = (t - 1) >> 2, jp = (t - 1) & 3;
        const float* s = jp == 3 ? sxp : sxv;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[ip][jp][r] = fmaf(dp[r], s[r] * swv[jp], acc[ip][jp][r]);
      }
      dp = d;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[WM - 1][3][r] = fmaf(dp[r], sxv[r] * swv[3], acc[WM - 1][3][r]);
  };
  // every wave's loads of the next stage have landed, and every wave is done
  // with the stage about to be refilled (the memory clobber keeps the LDS
  // accesses on their side of the barrier)
  auto step_barrier = [&]() { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); };

  issue(st0, 0);
  for (int kb = 0; kb < nb; kb += 2) {
    step_barrier();
    issue(st1, kb + 1);
    compute(st0);
    if (kb + 1 >= nb) break;
    step_barrier();
    issue(st0, kb + 2);
    compute(st1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // epilogue: lane (g, j) of sub-tile (i, b) holds tokens 4g..4g+3 of row
  // tile i and column j of column tile b
#pragma unroll
  for (int i = 0; i < WM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + (BM / 2) * wm + 16 * i + 4 * lg + r;
      if (m >= a.M) continue;
      if (!a.silu) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = tile_n * BN + 64 * wn + 16 * j + rl;
          if (n < a.N) a.y[(size_t)m * a.R + n] = pq::bf16_rne(acc[i][j][r]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int c = tile_n * (BN / 2) + 32 * wn + 16 * j + rl;
          if (c < a.R) a.y[(size_t)m * a.R + c] = pq::bf16_rne(silu_mul(acc[i][j][r], acc[i][j + 2][r]));
        }
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void gemm_fp8_kernel_t256(GArgs a) {
  __shared__ __align__(16) Stage<256> st0;
  __shared__ __align__(16) Stage<256> st1;
  gemm_body<256>(a, st0, st1);
}

__global__ __launch_bounds__(kThreads) void gemm_fp8_kernel_t128(GArgs a) {
  __shared__ __align__(16) Stage<256> st0;
  __shared__ __align__(16) Stage<256> st1;
  gemm_body<128>(a, st0, st1);
}

}  // namespace

extern "C" {

// The quantised activation lives in the workspace's data region, so the same
// workspace can serve the other entry points (their counters and their
// zero-between-calls region are left alone).
size_t pq_gemm_fp8_workspace(int M, int K, int N, int epi) {
  if (M < 1 || K < pq::kBlock || K % pq::kBlock != 0 || N < 1) return 0;
  (void)N;
  (void)epi;
  return pq::kWsDataOff + pqhost::align_up((size_t)M * K, 256) + pqhost::align_up((size_t)M * (K / pq::kBlock) * 4, 256);
}

int pq_gemm_fp8_prequant(const uint8_t* xq, const float* xs, int M, int K, const uint8_t* w, const float* w_scale,
                         int N, int epi, uint16_t* y, void* stream) {
  if (!xq || !xs || !w || !w_scale || !y) return PQ_ERR_NULL;
  if (M < 1 || K < pq::kBlock || K % pq::kBlock != 0 || N < 1) return PQ_ERR_SHAPE;
  if (epi != PQ_EPI_NONE && epi != PQ_EPI_SILU_MUL) return PQ_ERR_SHAPE;
  if (epi == PQ_EPI_SILU_MUL && N % 2 != 0) return PQ_ERR_SHAPE;
  if ((size_t)N * K > pq::kMaxBufferBytes || (size_t)M * K > pq::kMaxBufferBytes) return PQ_ERR_SHAPE;
  if (!pqhost::aligned16(xq) || !pqhost::aligned16(xs) || !pqhost::aligned16(w) || !pqhost::aligned16(w_scale) ||
      !pqhost::aligned16(y))
    return PQ_ERR_ALIGN;
  pqhost::DeviceInfo dev;
  const int st = pqhost::current_device_info(&dev);
  if (st != PQ_OK) return st;
  GArgs a;
  a.xq = xq; a.xs = xs; a.w = w; a.ws = w_scale; a.y = y;
  a.M = M; a.K = K; a.N = N;
  a.silu = epi == PQ_EPI_SILU_MUL;
  a.R = a.silu ? N / 2 : N;
  a.tn = a.silu ? (a.R + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;
  // 256-token tiles where they still give every CU a tile, else 128
  const bool big = (long)((M + 255) / 256) * a.tn >= dev.num_cus;
  a.tm = big ? (M + 255) / 256 : (M + 127) / 128;
  if (big)
    hipLaunchKernelGGL(gemm_fp8_kernel_t256, dim3((unsigned)(a.tm * a.tn)), dim3(kThreads), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(gemm_fp8_kernel_t128, dim3((unsigned)(a.tm * a.tn)), dim3(kThreads), 0, (hipStream_t)stream, a);
  PQ_HIP_CHECK(hipGetLastError());
  return PQ_OK;
}

int pq_gemm_fp8(const uint16_t* x, int M, int K, const uint8_t* w, const float* w_scale, int N, int epi,
                uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !w || !w_scale || !y) return PQ_ERR_NULL;
  if (M < 1 || K < pq::kBlock || K % pq::kBlock != 0 || N < 1) return PQ_ERR_SHAPE;
  if (epi != PQ_EPI_NONE && epi != PQ_EPI_SILU_MUL) return PQ_ERR_SHAPE;
  if (epi == PQ_EPI_SILU_MUL && N % 2 != 0) return PQ_ERR_SHAPE;
  if ((size_t)N * K > pq::kMaxBufferBytes || (size_t)M * K > pq::kMaxBufferBytes) return PQ_ERR_SHAPE;
  if (!pqhost::aligned16(x) || !pqhost::aligned16(w) || !pqhost::aligned16(w_scale) || !pqhost::aligned16(y))
    return PQ_ERR_ALIGN;
  const size_t need = pq_gemm_fp8_workspace(M, K, N, epi);
  if (ws == nullptr || ws_bytes < need) return PQ_ERR_WORKSPACE;
  if (!pqhost::aligned16(ws)) return PQ_ERR_ALIGN;
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws) + pq::kWsDataOff;
  float* xs = reinterpret_cast<float*>(xq + pqhost::align_up((size_t)M * K, 256));
  const int st = pq_quantize_fp8(x, 0, M, K, xq, xs, stream);      // the live activation rule, one pass
  if (st != PQ_OK) return st;
  return pq_gemm_fp8_prequant(xq, xs, M, K, w, w_scale, N, epi, y, stream);
}

}  // extern "C"
