// Block-scaled FP8 weight-streaming GEMV / skinny GEMM (M <= 8) with the live
// FP8 activation quantisation fused in, optional split-K with a deterministic
// last-arriver reduction, and an optional fused SiLU(gate)*up epilogue.
//
// [Sionic] §1: at batch 1 the weight-streaming GEMM must keep every compute
// unit issuing loads (split K when rows are too few) and the live FP8
// quantisation of the activation must overlap the first weight loads rather
// than run ahead of them.  [Sionic] §2: the per-K-block scale must not stall
// the load pipeline.  [Sionic] §4: quantisation lives inside the GEMM launch.
//
// gfx950 design
//   * one wave (64 lanes) owns whole weight rows: a row is streamed as 1 KB
//     chunks, lane l reading bytes [16l, 16l+16) of each chunk with one
//     global_load_dwordx4, so every load instruction covers 8 full 128-byte
//     lines;
//   * the lane's 16 bytes lie inside one 128-wide scale block, so the block
//     scale is folded into the lane's running sum with a single FMA per 16
//     weights: no barrier, no cross-lane work inside the K loop;
//   * the lane keeps a ring of D chunk-steps of loads in flight;
//   * the activation is quantised once per block (workgroup) into LDS while
//     the first weight loads are in flight;
//   * one cross-lane butterfly per output row at the end.
#include <stdlib.h>

#include "pq_quant_dev.h"

namespace {

constexpr int kThreads = 512;   // 8 waves; one block per CU
constexpr int kWaves = kThreads / pq::kWave;
constexpr int kMaxM = 8;
constexpr int kXPre = 2;        // activation loads issued ahead of the weight prefetch

struct GemvArgs {
  const uint16_t* x;
  const uint8_t* w;
  const float* wsc;
  uint16_t* y;
  uint8_t* xq_dbg;
  float* xs_dbg;
  float* part;      // [S][M][NROW][R] split-K partials
  uint32_t* cnt;    // [R] split-K arrival counters (zero between calls)
  int M, K, N;
  int R;            // output rows: N, or N/2 under the SiLU epilogue
  int S;            // K splits
  int Ks;           // bytes of K per split (multiple of 128)
  int nch;          // 1 KB chunks per split
  int units;        // R * S
};

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
  float* xs_s = reinterpret_cast<float*>(smem + pqhost::align_up((size_t)a.M * a.K, 16));

  const int lane = pq::lane_id();
  const int gw = __builtin_amdgcn_readfirstlane((int)blockIdx.x * kWaves + pq::wave_id());  // wave-uniform
  const long T = (long)gridDim.x * kWaves;
  const int u0 = (int)((long)gw * a.units / T);
  const int u1 = (int)((long)(gw + 1) * a.units / T);
  const int nsteps = (u1 - u0) * a.nch;
  const int nb = a.K / pq::kBlock;

  // --- activation loads first, then the weight ring, then quantise -------
  const pq::rsrc_t xr = pq::make_rsrc(a.x, (uint32_t)a.M * a.K * 2u);
  const pq::rsrc_t wr = pq::make_rsrc(a.w, (uint32_t)((size_t)a.N * a.K));
  const pq::rsrc_t sr = pq::make_rsrc(a.wsc, (uint32_t)((size_t)a.N * nb * 4));
  XLoad xl;
  xq_issue(a, xr, xl);

  uint4 wbuf[D][NROW];
  float sbuf[D][NROW];
  // issue cursor: (row, split, chunk) of the next chunk-step to load
  int ir = u0 / a.S, is = u0 - (u0 / a.S) * a.S, ic = 0;
  const uint32_t lane16 = 16u * (uint32_t)lane;
  const uint32_t lane_blk4 = 4u * ((uint32_t)lane >> 3);     // this lane's scale block within a chunk
  auto issue = [&](uint4 (&wb)[NROW], float (&sb)[NROW]) {
    const uint32_t kc = (uint32_t)(is * a.Ks + ic * pq::kChunk);            // uniform chunk start
    const bool in_range = ir * a.S + is < u1;                               // uniform
    const bool ok = in_range && (uint32_t)(ic * pq::kChunk) + lane16 < (uint32_t)a.Ks;
#pragma unroll
    for (int j = 0; j < NROW; ++j) {
      const uint32_t row = (uint32_t)(ir + j * a.R);
      const uint32_t wbase = row * (uint32_t)a.K + kc;                       // uniform
      const uint32_t sbase = (row * (uint32_t)nb + kc / pq::kBlock) * 4u;   // uniform
      wb[j] = pq::buf_load16_nt(wr, ok ? wbase + lane16 : pq::kOOB);
      sb[j] = pq::buf_load_f32_nt(sr, ok ? sbase + lane_blk4 : pq::kOOB);
    }
    if (++ic == a.nch) {
      ic = 0;
      if (++is == a.S) { is = 0; ++ir; }
    }
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

  // consume cursor
  int cr = u0 / a.S, cs = u0 - (u0 / a.S) * a.S, cc = 0;
  for (int base = 0; base < nsteps; base += D) {
#pragma unroll
    for (int q = 0; q < D; ++q) {
      const int step = base + q;
      if (step < nsteps) {
        const int off = cc * pq::kChunk + 16 * lane;
        if (off < a.Ks) {
          const int kb = cs * a.Ks + off;
          pq::Bf16x16 wv[NROW];
#pragma unroll
          for (int j = 0; j < NROW; ++j) wv[j] = pq::widen16(wbuf[q][j]);
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const uint4 xc = *reinterpret_cast<const uint4*>(xq_s + (size_t)m * a.K + kb);
            const float xs = xs_s[m * nb + kb / pq::kBlock];
            const pq::Bf16x16 xv = pq::widen16(xc);
#pragma unroll
            for (int j = 0; j < NROW; ++j)
              acc[j][m] = fmaf(pq::dot16(wv[j], xv), sbuf[q][j] * xs, acc[j][m]);
          }
        }

        if (cc == a.nch - 1) {  // unit (cr, cs) complete: reduce across the wave
          const int r = cr, s = cs;
          float v[NROW][MT];
#pragma unroll
          for (int j = 0; j < NROW; ++j)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              v[j][m] = pq::wave_sum(acc[j][m]);
              acc[j][m] = 0.0f;
            }
          if (a.S == 1) {
            if (lane < MT) {
              float g = 0.0f, u = 0.0f;
#pragma unroll
              for (int m = 0; m < MT; ++m)
                if (m == lane) { g = v[0][m]; u = v[NROW - 1][m]; }
              const float out = NROW == 2 ? silu_mul(g, u) : g;
              a.y[(size_t)lane * a.R + r] = pq::bf16_rne(out);
            }
          } else {
            if (lane < MT * NROW) {
              float pv = 0.0f;
#pragma unroll
              for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int j = 0; j < NROW; ++j)
                  if (m * NROW + j == lane) pv = v[j][m];
              a.part[((size_t)s * a.M * NROW + lane) * a.R + r] = pv;
            }
            pq::fence_release();
            uint32_t old = 0;
            if (lane == 0) old = pq::atomic_add_relaxed(&a.cnt[r], 1u);
            old = __shfl(old, 0, pq::kWave);
            if (old == (uint32_t)(a.S - 1)) {      // last split of row r: reduce in split order
              pq::fence_acquire();
              if (lane < a.M) {
                float g = 0.0f, u = 0.0f;
                for (int ss = 0; ss < a.S; ++ss) {
                  g += a.part[((size_t)ss * a.M * NROW + lane * NROW) * a.R + r];
                  if (NROW == 2) u += a.part[((size_t)ss * a.M * NROW + lane * NROW + 1) * a.R + r];
                }
                const float out = NROW == 2 ? silu_mul(g, u) : g;
                a.y[(size_t)lane * a.R + r] = pq::bf16_rne(out);
              }
              if (lane == 0) pq::atomic_store_relaxed(&a.cnt[r], 0u);
            }
          }
        }
        if (++cc == a.nch) {
          cc = 0;
          if (++cs == a.S) { cs = 0; ++cr; }
        }
      }
      issue(wbuf[q], sbuf[q]);   // step + D (zero-filled past the end)
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct Plan {
  int S, Ks, nch, R, units, grid;
  size_t lds;
  size_t ws_cnt, ws_part, ws_total;
};

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  return v && *v ? atoi(v) : dflt;
}

int make_plan(int M, int K, int N, int epi, int num_cus, Plan* p) {
  if (M < 1 || M > kMaxM || K < pq::kBlock || K % pq::kBlock != 0 || K > 16384 || N < 1) return PQ_ERR_SHAPE;
  if (epi != PQ_EPI_NONE && epi != PQ_EPI_SILU_MUL) return PQ_ERR_SHAPE;
  if (epi == PQ_EPI_SILU_MUL && N % 2 != 0) return PQ_ERR_SHAPE;
  const int nb = K / pq::kBlock;
  p->R = epi == PQ_EPI_SILU_MUL ? N / 2 : N;
  const long waves = (long)num_cus * kWaves;
  int S = 1;
  const int forced = env_int("PQ_SPLITK", 0);
  if (forced > 0) {
    S = forced;
    if (S > nb || nb % S != 0) return PQ_ERR_SHAPE;
  } else if ((long)p->R < waves) {
    // smallest divisor of the block count that gives every wave a unit
    for (S = 1; S < nb; ++S)
      if (nb % S == 0 && (long)p->R * S >= waves) break;
    if (nb % S != 0) S = nb;
  }
  p->S = S;
  p->Ks = K / S;
  p->nch = (p->Ks + pq::kChunk - 1) / pq::kChunk;
  p->units = p->R * S;
  const long want_blocks = ((long)p->units + kWaves - 1) / kWaves;
  p->grid = (int)(want_blocks < num_cus ? want_blocks : num_cus);
  if (p->grid < 1) p->grid = 1;
  p->lds = pqhost::align_up((size_t)M * K, 16) + (size_t)M * nb * sizeof(float);
  if (p->lds > 160 * 1024) return PQ_ERR_SHAPE;
  const int nrow = epi == PQ_EPI_SILU_MUL ? 2 : 1;
  if (S == 1) {
    p->ws_cnt = p->ws_part = p->ws_total = 0;
  } else {
    if ((size_t)p->R > pq::kWsMaxCounters) return PQ_ERR_SHAPE;   // split-K needs one counter per row
    p->ws_cnt = pq::kWsDataOff;
    p->ws_part = (size_t)S * M * nrow * p->R * sizeof(float);
    p->ws_total = p->ws_cnt + p->ws_part;
  }
  return PQ_OK;
}

template <int NROW, int D, int MT>
hipError_t launch_m(const Plan& pl, const GemvArgs& a, hipStream_t stream) {
  auto kern = gemv_fp8_kernel<NROW, D, MT>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(pl.grid), dim3(kThreads), pl.lds, stream, a);
  return hipGetLastError();
}

template <int NROW, int D>
hipError_t launch(const Plan& pl, const GemvArgs& a, hipStream_t stream) {
  switch (a.M) {
    case 1: return launch_m<NROW, D, 1>(pl, a, stream);
    case 2: return launch_m<NROW, D, 2>(pl, a, stream);
    case 3: return launch_m<NROW, D, 3>(pl, a, stream);
    case 4: return launch_m<NROW, D, 4>(pl, a, stream);
    case 5: return launch_m<NROW, D, 5>(pl, a, stream);
    case 6: return launch_m<NROW, D, 6>(pl, a, stream);
    case 7: return launch_m<NROW, D, 7>(pl, a, stream);
    default: return launch_m<NROW, D, 8>(pl, a, stream);
  }
}

}  // namespace

extern "C" {

size_t pq_gemv_fp8_workspace(int M, int K, int N, int epi) {
  pqhost::DeviceInfo dev;
  if (pqhost::current_device_info(&dev) != PQ_OK) return 0;
  Plan pl;
  if (make_plan(M, K, N, epi, dev.num_cus, &pl) != PQ_OK) return 0;
  return pl.ws_total;
}

int pq_gemv_fp8(const uint16_t* x, int M, int K, const uint8_t* w, const float* w_scale, int N, int epi,
                uint16_t* y, uint8_t* xq_dbg, float* xs_dbg, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !w || !w_scale || !y) return PQ_ERR_NULL;
  if (M < 1 || M > kMaxM || K < pq::kBlock || K % pq::kBlock != 0 || K > 16384 || N < 1) return PQ_ERR_SHAPE;
  if (epi != PQ_EPI_NONE && epi != PQ_EPI_SILU_MUL) return PQ_ERR_SHAPE;
  if (epi == PQ_EPI_SILU_MUL && N % 2 != 0) return PQ_ERR_SHAPE;
  if (!pqhost::aligned16(x) || !pqhost::aligned16(w) || !pqhost::aligned16(w_scale) || !pqhost::aligned16(y) ||
      (xq_dbg && !pqhost::aligned16(xq_dbg)) || (xs_dbg && !pqhost::aligned16(xs_dbg)) ||
      (ws && !pqhost::aligned16(ws)))
    return PQ_ERR_ALIGN;
  pqhost::DeviceInfo dev;
  int st = pqhost::current_device_info(&dev);
  if (st != PQ_OK) return st;
  Plan pl;
  st = make_plan(M, K, N, epi, dev.num_cus, &pl);
  if (st != PQ_OK) return st;
  if (pl.ws_total > 0 && (ws == nullptr || ws_bytes < pl.ws_total)) return PQ_ERR_WORKSPACE;

  GemvArgs a;
  a.x = x; a.w = w; a.wsc = w_scale; a.y = y; a.xq_dbg = xq_dbg; a.xs_dbg = xs_dbg;
  a.cnt = pl.S > 1 ? reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(ws) + pq::kWsCounterOff) : nullptr;
  a.part = pl.S > 1 ? reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + pl.ws_cnt) : nullptr;
  a.M = M; a.K = K; a.N = N; a.R = pl.R; a.S = pl.S; a.Ks = pl.Ks; a.nch = pl.nch; a.units = pl.units;

  hipError_t e = epi == PQ_EPI_SILU_MUL ? launch<2, 8>(pl, a, (hipStream_t)stream)
                                        : launch<1, 16>(pl, a, (hipStream_t)stream);
  if (e != hipSuccess) {
    pqhost::set_last_hip_error((int)e);
    return PQ_ERR_HIP;
  }
  return PQ_OK;
}

}  // extern "C"
