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
#include <string.h>

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
// Matrix-core path (verify shapes, 4 <= M <= 8).
//
// The dot product of one 128-wide K block of 16 weight rows with every token
// is one v_mfma_f32_16x16x128_f8f6f4 (E4M3 x E4M3, fp32 result):
//   * B (128 k x 16 columns) holds the weights: lane l carries row l % 16 of
//     the tile;
//   * A (16 rows x 128 k) holds the quantised activation: lane l carries token
//     l % 16 (zeros for tokens >= M);
//   * in both operands lane group g = l / 16 carries bytes [16g, 16g+16) and
//     [64+16g, 80+16g) of the block, so both operands label k alike.
// The weights are not loaded in that layout: a load instruction whose 64
// lanes cover 16 rows x 64 bytes (half lines) streams about a fifth slower
// than one covering 8 rows x 128 bytes (whole lines) on MI355X.  Each step
// therefore loads the 16 x 128-byte block with two whole-line instructions
// (lane l: row 8h + l / 8, bytes 16 (l % 8)), and the wave passes it through a
// private 2.3 KB LDS slot (16-byte padded rows, so the reads are free of bank
// conflicts) into the operand layout.
// Result lane l holds the block sums of weight row l % 16 for tokens
// 4g .. 4g+3; the two block scales apply per lane and the block is folded into
// an fp32 accumulator, acc += sum * (s_w * s_x), as in the vector kernel.  The
// matrix core adds the 128 exact products of a block with its own internal
// precision (within about 1e-4 of the block's sum of |products| on random
// codes); the sum over blocks is fp32.
//
// Work is split stream-K style: the (16-row tile, 128-k block) units of the
// matrix are dealt to all waves of the grid in order.  A tile covered by one
// wave is finished by it; the parts of a tile cut between waves meet in the
// workspace, and the last of its waves to arrive (one arrival counter per
// tile, reset by that wave) adds them in wave order.
// ---------------------------------------------------------------------------
typedef int int32x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kRB = 16;        // weight rows per tile
constexpr int kXPad = 16;      // LDS row stride of the activation codes: K + 16 bytes
constexpr int kZeroBytes = 128;

struct MArgs {
  const uint16_t* x;
  const uint8_t* w;
  const float* wsc;
  uint16_t* y;
  uint8_t* xq_dbg;
  float* xs_dbg;
  float* part;       // [waves][2][4 * NROW][64]
  uint32_t* cnt;     // [nrb]
  int M, K, N, R;
  int nrb, nb, U;    // row tiles, K blocks per row, units = nrb * nb
};

constexpr int kStRow = pq::kBlock + 16;          // staging row stride (bytes)
constexpr int kStBytes = kRB * kStRow;             // one 16 x 128-byte block

// LDS: [codes M x (K + 16)][zero run 128 B][scales nb x 16 fp32]
//      [staging: waves x NROW x 16 x 144 B]
__host__ __device__ inline size_t m_zero_offset(int M, int K) { return (size_t)M * (K + kXPad); }
__host__ __device__ inline size_t m_scale_offset(int M, int K) { return m_zero_offset(M, K) + kZeroBytes; }
__host__ __device__ inline size_t m_stage_offset(int M, int K) {
  return m_scale_offset(M, K) + (size_t)(K / pq::kBlock) * kRB * sizeof(float);
}
__host__ __device__ inline size_t m_lds_bytes(int M, int K, int nrow) {
  return m_stage_offset(M, K) + (size_t)kWaves * nrow * kStBytes;
}

__device__ __forceinline__ floatx4 mfma_e4m3(int32x8 a, int32x8 b) {
  // block-scale operands 0: the plain (unscaled) matrix instruction
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ int32x8 join8(uint4 lo, uint4 hi) {
  return int32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// wave whose unit range [split_start(U, T, w), split_start(U, T, w + 1)) holds u
__device__ __forceinline__ int wave_of(int u, int U, int T) {
  const int q = U / T, r = U - (U / T) * T;
  return u < r * (q + 1) ? u / (q + 1) : r + (u - r * (q + 1)) / q;
}

template <int NROW, int D, int MT>
__global__ __launch_bounds__(kThreads) void gemv_fp8_mfma_kernel(MArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int Kp = a.K + kXPad;
  float* xs_s = reinterpret_cast<float*>(smem + m_scale_offset(MT, a.K));   // [nb][16]
  uint8_t* stage = smem + m_stage_offset(MT, a.K) + (size_t)pq::wave_id() * NROW * kStBytes;

  const int tid = (int)threadIdx.x;
  const int lane = pq::lane_id();
  const int T = (int)gridDim.x * kWaves;
  const int gw = __builtin_amdgcn_readfirstlane((int)blockIdx.x * kWaves + pq::wave_id());
  const int u0 = pq::split_start(a.U, T, gw);
  const int nsteps = pq::split_start(a.U, T, gw + 1) - u0;
  const int rl = lane & 15, lg = lane >> 4;

  // --- activation loads first, then the weight ring, then quantise -------
  const pq::rsrc_t xr = pq::make_rsrc(a.x, (uint32_t)(MT * a.K * 2));
  const pq::rsrc_t wr = pq::make_rsrc(a.w, (uint32_t)((size_t)a.N * a.K));
  const pq::rsrc_t sr = pq::make_rsrc(a.wsc, (uint32_t)((size_t)a.N * a.nb * 4));
  GemvArgs ga;
  ga.M = MT;
  ga.K = a.K;
  XLoad xl;
  xq_issue(ga, xr, xl);

  uint4 wbuf[D][NROW][2];
  float sbuf[D][NROW];
  int irb = u0 / a.nb, ib = u0 - (u0 / a.nb) * a.nb, left = nsteps;   // issue cursor (tile, block)
  const int lr8 = lane >> 3, lc8 = lane & 7;     // whole-line load: row within 8, 16-byte slot
  auto issue = [&](uint4 (&wb)[NROW][2], float (&sb)[NROW]) {
    const int row = irb * kRB + rl;               // the operand row (scales)
    const bool ok = left > 0 && row < a.R;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int lrow = irb * kRB + 8 * h + lr8;   // the row this lane loads
      const bool lok = left > 0 && lrow < a.R;
#pragma unroll
      for (int j = 0; j < NROW; ++j) {
        const uint32_t off = (uint32_t)(lrow + j * a.R) * (uint32_t)a.K + (uint32_t)ib * pq::kBlock + 16u * (uint32_t)lc8;
        wb[j][h] = pq::buf_load16_nt(wr, lok ? off : pq::kOOB);
      }
    }
#pragma unroll
    for (int j = 0; j < NROW; ++j) {
      const uint32_t grow = (uint32_t)(row + j * a.R);
      sb[j] = pq::buf_load_f32(sr, ok ? (grow * (uint32_t)a.nb + (uint32_t)ib) * 4u : pq::kOOB);
    }
    --left;
    if (++ib == a.nb) { ib = 0; ++irb; }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) issue(wbuf[d], sbuf[d]);

  // quantise x into LDS rows of stride K + 16; scales as [block][token]
  {
    const int total8 = MT * a.K / 8;
    const int iters = (total8 + kThreads - 1) / kThreads;
    const bool dbg = blockIdx.x == 0 && a.xq_dbg != nullptr;
    for (int it = 0; it < iters; ++it) {
      const int t = it * kThreads + tid;
      const bool valid = t < total8;
      const uint4 raw = it < kXPre ? xl.raw[it < kXPre ? it : 0] : pq::buf_load16(xr, (uint32_t)t * 16u);
      float v[8];
      pq::bf16x8_to_f32(raw, v);
      const float s = pq::fp8_block_scale16(v, valid);
      if (valid) {
        const int m = (t * 8) / a.K, k = t * 8 - m * a.K;
        const uint2 c = pq::fp8_codes8(v, s);
        *reinterpret_cast<uint2*>(smem + (size_t)m * Kp + k) = c;
        const bool lead = (tid & 15) == 0;
        if (lead) xs_s[(k / pq::kBlock) * kRB + m] = s;
        if (dbg) {
          reinterpret_cast<uint2*>(a.xq_dbg)[t] = c;
          if (lead && a.xs_dbg) a.xs_dbg[(t * 8) / pq::kBlock] = s;
        }
      }
    }
    for (int i = tid; i < a.nb * (kRB - MT); i += kThreads)      // scales of the absent tokens
      xs_s[(i / (kRB - MT)) * kRB + MT + i % (kRB - MT)] = 0.0f;
    if (tid < kZeroBytes / 16)
      reinterpret_cast<uint4*>(smem + m_zero_offset(MT, a.K))[tid] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();

  // this lane's A row: token rl, or the zero run for absent tokens
  // (the block offset is masked in rather than multiplied: a 32-bit multiply-add
  // here has been emitted as a 64-bit one whose unused high operand aliases a
  // load in flight, which forces a full wait on the load ring)
  const uint32_t abase = rl < MT ? (uint32_t)(rl * Kp + 16 * lg) : (uint32_t)m_zero_offset(MT, a.K);
  const uint32_t amask = rl < MT ? 0xFFFFFFFFu : 0u;

  float acc[NROW][4], st0[NROW][4], st1[NROW][4];
#pragma unroll
  for (int j = 0; j < NROW; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[j][r] = st0[j][r] = st1[j][r] = 0.0f;
  bool has0 = false, has1 = false;
  const int rb_first = u0 / a.nb;
  const int rb_last = nsteps > 0 ? (u0 + nsteps - 1) / a.nb : rb_first;
  // a tile strictly inside this wave's range is this wave's alone; the first
  // and the last tile are when the range starts / ends on their boundaries
  const bool solo_first = u0 == rb_first * a.nb && u0 + nsteps >= (rb_first + 1) * a.nb;
  const bool solo_last = u0 + nsteps == (rb_last + 1) * a.nb && u0 <= rb_last * a.nb;

  auto output = [&](int rb, const float (&v)[NROW][4]) {
    const int row = rb * kRB + rl;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * lg + r;
      if (m < MT && row < a.R)
        a.y[(size_t)m * a.R + row] = pq::bf16_rne(NROW == 2 ? silu_mul(v[0][r], v[NROW - 1][r]) : v[0][r]);
    }
  };
  auto ncover = [&](int rb) { return wave_of((rb + 1) * a.nb - 1, a.U, T) - wave_of(rb * a.nb, a.U, T) + 1; };

  int crb = rb_first, cb = u0 - rb_first * a.nb;            // consume cursor
  auto consume = [&](const uint4 (&wb)[NROW][2], const float (&sb)[NROW], bool last) {
    const uint32_t xo = abase + (((uint32_t)cb << 7) & amask);
    const uint4 x0 = *reinterpret_cast<const uint4*>(smem + xo);
    const uint4 x1 = *reinterpret_cast<const uint4*>(smem + xo + 64);
    const float4 sx = *reinterpret_cast<const float4*>(xs_s + cb * kRB + 4 * lg);
    const int32x8 av = join8(x0, x1);
    const float sxv[4] = {sx.x, sx.y, sx.z, sx.w};
    // whole-line registers -> LDS slot -> operand layout (LDS operations of one
    // wave complete in order; the empty asm keeps the compiler from moving the
    // reads above the writes, which other lanes made)
    uint4 blo[NROW], bhi[NROW];
#pragma unroll
    for (int j = 0; j < NROW; ++j) {
      uint8_t* st = stage + j * kStBytes;
      *reinterpret_cast<uint4*>(st + lr8 * kStRow + 16 * lc8) = wb[j][0];
      *reinterpret_cast<uint4*>(st + (8 + lr8) * kStRow + 16 * lc8) = wb[j][1];
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < NROW; ++j) {
      const uint8_t* st = stage + j * kStBytes + rl * kStRow + 16 * lg;
      blo[j] = *reinterpret_cast<const uint4*>(st);
      bhi[j] = *reinterpret_cast<const uint4*>(st + 64);
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < NROW; ++j) {
      const floatx4 d = mfma_e4m3(av, join8(blo[j], bhi[j]));
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[j][r] = fmaf(d[r], sb[j] * sxv[r], acc[j][r]);
    }
    if (cb == a.nb - 1 || last) {                             // end of this wave's part of tile crb
      if (crb == rb_first ? solo_first : (crb == rb_last ? solo_last : true)) {
        output(crb, acc);
      } else if (crb == rb_first) {
#pragma unroll
        for (int j = 0; j < NROW; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) st0[j][r] = acc[j][r];
        has0 = true;
      } else {
#pragma unroll
        for (int j = 0; j < NROW; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) st1[j][r] = acc[j][r];
        has1 = true;
      }
#pragma unroll
      for (int j = 0; j < NROW; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][r] = 0.0f;
    }
    if (++cb == a.nb) { cb = 0; ++crb; }
  };

  int base = 0;
  for (; base + D < nsteps; base += D) {
#pragma unroll
    for (int q = 0; q < D; ++q) {
      consume(wbuf[q], sbuf[q], false);
      issue(wbuf[q], sbuf[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < D; ++q)
    if (base + q < nsteps) consume(wbuf[q], sbuf[q], base + q == nsteps - 1);

  // tiles cut between waves: publish this wave's parts, then the last covering
  // wave to arrive adds all parts in wave order
  constexpr int NS = 4 * NROW;
  if (has0 || has1) {
    uint32_t* p32 = reinterpret_cast<uint32_t*>(a.part);
#pragma unroll
    for (int j = 0; j < NROW; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int k = j * 4 + r;
        if (has0) pq::st_agent_u32(p32 + ((size_t)(gw * 2 + 0) * NS + k) * 64 + lane, __float_as_uint(st0[j][r]));
        if (has1) pq::st_agent_u32(p32 + ((size_t)(gw * 2 + 1) * NS + k) * 64 + lane, __float_as_uint(st1[j][r]));
      }
    pq::wait_vm();
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      if (which == 0 ? !has0 : !has1) continue;
      const int rb = which == 0 ? rb_first : rb_last;
      uint32_t old = 0;
      if (lane == 0) old = pq::atomic_add_relaxed(&a.cnt[rb], 1u);
      old = __shfl(old, 0, pq::kWave);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      const int w0 = wave_of(rb * a.nb, a.U, T);
      const int nc = ncover(rb);
      if (old == (uint32_t)(nc - 1)) {
        float v[NROW][4];
#pragma unroll
        for (int j = 0; j < NROW; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) v[j][r] = 0.0f;
        // the parts in wave order, loaded 8 waves at a time (one round trip
        // per 8 parts; indexes past the last part re-read the first one and
        // are not added)
        constexpr int kBatch = 8;
        for (int wb0 = w0; wb0 < w0 + nc; wb0 += kBatch) {
          float t[kBatch][NROW][4];
#pragma unroll
          for (int q = 0; q < kBatch; ++q) {
            const int wc = wb0 + q < w0 + nc ? wb0 + q : w0;
            const int slot = pq::split_start(a.U, T, wc) / a.nb == rb ? 0 : 1;
#pragma unroll
            for (int j = 0; j < NROW; ++j)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                t[q][j][r] = __uint_as_float(pq::ld_agent_u32(p32 + ((size_t)(wc * 2 + slot) * NS + j * 4 + r) * 64 + lane));
          }
#pragma unroll
          for (int q = 0; q < kBatch; ++q)
#pragma unroll
            for (int j = 0; j < NROW; ++j)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (wb0 + q < w0 + nc) v[j][r] += t[q][j][r];
        }
        output(rb, v);
        if (lane == 0) pq::atomic_store_relaxed(&a.cnt[rb], 0u);
      }
    }
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

// ---- matrix-core path ------------------------------------------------------
int blocks_per_cu() {
  const char* env = getenv("PQ_BLOCKS_PER_CU");
  return env && atoi(env) > 0 ? atoi(env) : 1;
}

// The matrix-core kernel needs one arrival counter per 16-row tile and its
// LDS layout must fit.  By default it serves M >= 3 on weight matrices of at
// least 128 MB: there the vector kernel is bound by its dot products (LM head
// 6144 x 151552: 209 / 245 / 411 us at M = 3 / 4 / 8 against 176 / 177 / 188),
// while the matrix kernel carries some 10 us more fixed cost per call, which
// loses on small matrices (one expert's gate_up, 26 MB: 24.1 against 27.0 us
// even at M = 8) and at M = 1 (LM head: 157 against 171 us).  PQ_FP8_PATH=valu
// or =mfma forces one kernel (mfma only where its conditions hold).
bool use_mfma(int M, int K, int R, int nrow) {
  if ((size_t)((R + kRB - 1) / kRB) > pq::kWsMaxCounters) return false;
  if (m_lds_bytes(M, K, nrow) > 160 * 1024) return false;
  const char* env = getenv("PQ_FP8_PATH");
  if (env && strcmp(env, "valu") == 0) return false;
  if (env && strcmp(env, "mfma") == 0) return true;
  return M >= 3 && (size_t)R * nrow * K >= ((size_t)128 << 20);
}

// grid (blocks) and workspace bytes of the matrix-core path
void mfma_plan(int nrow, int num_cus, int* grid, size_t* ws) {
  *grid = num_cus * blocks_per_cu();
  *ws = pq::kWsDataOff + (size_t)(*grid) * kWaves * 2 * 4 * nrow * 64 * sizeof(float);
}

template <int NROW, int D, int MT>
hipError_t launch_mfma_m(const MArgs& a, int grid, hipStream_t stream) {
  auto kern = gemv_fp8_mfma_kernel<NROW, D, MT>;
  static pqhost::KernelAttrOnce attr;
  {
    hipError_t e = pqhost::set_dynamic_lds_once(attr, (const void*)kern, 160 * 1024);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), m_lds_bytes(MT, a.K, NROW), stream, a);
  return hipGetLastError();
}

template <int NROW, int D>
hipError_t launch_mfma(const MArgs& a, int grid, hipStream_t s) {
  switch (a.M) {
    case 1: return launch_mfma_m<NROW, D, 1>(a, grid, s);
    case 2: return launch_mfma_m<NROW, D, 2>(a, grid, s);
    case 3: return launch_mfma_m<NROW, D, 3>(a, grid, s);
    case 4: return launch_mfma_m<NROW, D, 4>(a, grid, s);
    case 5: return launch_mfma_m<NROW, D, 5>(a, grid, s);
    case 6: return launch_mfma_m<NROW, D, 6>(a, grid, s);
    case 7: return launch_mfma_m<NROW, D, 7>(a, grid, s);
    default: return launch_mfma_m<NROW, D, 8>(a, grid, s);
  }
}

// ---- vector path -----------------------------------------------------------
template <int NROW, int D, int MT>
hipError_t launch_m(const GemvArgs& a, int grid, hipStream_t stream) {
  auto kern = gemv_fp8_kernel<NROW, D, MT>;
  static pqhost::KernelAttrOnce attr;
  {
    hipError_t e = pqhost::set_dynamic_lds_once(attr, (const void*)kern, 160 * 1024);
    if (e != hipSuccess) return e;
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

size_t pq_gemv_fp8_workspace(int M, int K, int N, int epi) {
  if (check_shape(M, K, N, epi) != PQ_OK) return 0;
  const int R = epi == PQ_EPI_SILU_MUL ? N / 2 : N;
  if (!use_mfma(M, K, R, epi == PQ_EPI_SILU_MUL ? 2 : 1)) return 0;
  pqhost::DeviceInfo dev;
  if (pqhost::current_device_info(&dev) != PQ_OK) return 0;
  int grid;
  size_t ws;
  mfma_plan(epi == PQ_EPI_SILU_MUL ? 2 : 1, dev.num_cus, &grid, &ws);
  return ws;
}

int pq_gemv_fp8(const uint16_t* x, int M, int K, const uint8_t* w, const float* w_scale, int N, int epi,
                uint16_t* y, uint8_t* xq_dbg, float* xs_dbg, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !w || !w_scale || !y) return PQ_ERR_NULL;
  int st = check_shape(M, K, N, epi);
  if (st != PQ_OK) return st;
  if (!pqhost::aligned16(x) || !pqhost::aligned16(w) || !pqhost::aligned16(w_scale) || !pqhost::aligned16(y) ||
      (xq_dbg && !pqhost::aligned16(xq_dbg)) || (xs_dbg && !pqhost::aligned16(xs_dbg)))
    return PQ_ERR_ALIGN;
  pqhost::DeviceInfo dev;
  st = pqhost::current_device_info(&dev);
  if (st != PQ_OK) return st;

  const int R = epi == PQ_EPI_SILU_MUL ? N / 2 : N;
  if (use_mfma(M, K, R, epi == PQ_EPI_SILU_MUL ? 2 : 1)) {
    int grid;
    size_t need;
    mfma_plan(epi == PQ_EPI_SILU_MUL ? 2 : 1, dev.num_cus, &grid, &need);
    if (ws == nullptr || ws_bytes < need) return PQ_ERR_WORKSPACE;
    if (!pqhost::aligned16(ws)) return PQ_ERR_ALIGN;
    MArgs b;
    b.x = x; b.w = w; b.wsc = w_scale; b.y = y; b.xq_dbg = xq_dbg; b.xs_dbg = xs_dbg;
    b.cnt = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(ws) + pq::kWsCounterOff);
    b.part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + pq::kWsDataOff);
    b.M = M; b.K = K; b.N = N; b.R = R;
    b.nrb = (R + kRB - 1) / kRB;
    b.nb = K / pq::kBlock;
    b.U = b.nrb * b.nb;
    hipError_t e = epi == PQ_EPI_SILU_MUL ? launch_mfma<2, 4>(b, grid, (hipStream_t)stream)
                                          : launch_mfma<1, 8>(b, grid, (hipStream_t)stream);
    if (e != hipSuccess) {
      pqhost::set_last_hip_error((int)e);
      return PQ_ERR_HIP;
    }
    return PQ_OK;
  }

  GemvArgs a;
  a.x = x; a.w = w; a.wsc = w_scale; a.y = y; a.xq_dbg = xq_dbg; a.xs_dbg = xs_dbg;
  a.M = M; a.K = K; a.N = N;
  a.R = R;
  a.nch = (K + pq::kChunk - 1) / pq::kChunk;
  const int grid = grid_for(a.R, dev.num_cus);
  if (lds_bytes(M, K, (a.R + grid - 1) / grid, epi == PQ_EPI_SILU_MUL ? 2 : 1) > 160 * 1024) return PQ_ERR_SHAPE;

  // ring depths (chunk steps in flight per wave): 3 either way; deeper rings
  // were slower on expert-sized matrices (gate_up 6144->2x2048 M=1: 7.4 us at
  // 3, 8.6 at 8; down 2048->6144 M=8: 12.4 vs 14.1 at 16) and equal on the
  // 931 MB LM head
  hipError_t e = epi == PQ_EPI_SILU_MUL ? launch<2, 3>(a, grid, (hipStream_t)stream)
                                        : launch<1, 3>(a, grid, (hipStream_t)stream);
  if (e != hipSuccess) {
    pqhost::set_last_hip_error((int)e);
    return PQ_ERR_HIP;
  }
  return PQ_OK;
}

}  // extern "C"
