// Routed MoE decode layer in a single kernel launch: route (top-k + softmax),
// live FP8 activation quantisation, gate_up GEMV with fused SiLU*up, live
// re-quantisation of h, down GEMV and the weighted combine over the k slots.
//
// [Sionic] intro: a decode step streams each active expert's weights from HBM
// once; §1: split the stream so that every compute unit issues loads and keep
// the live activation quantisation off the load path; §2: apply the per-block
// scales without stalling loads; §4: few kernels, no activation round trips;
// §5-6: one weight read serves every token of a verify batch.  [M1]: with 256
// experts and one launch per op the GPU sits idle (dispatch bound); [M3]:
// merging small kernels into few dispatches raised decode from 59% to 81% of
// measured bandwidth.  Here the whole layer is one launch.
//
// Structure (one persistent block per CU, 8 waves, static work split)
//   A. every block routes the M tokens redundantly (a few hundred ALU ops) and
//      builds the union of routed experts in first-appearance order; block 0
//      writes the routing outputs.
//   B. every block live-quantises x into LDS while its first gate_up weight
//      loads are in flight.
//   C. gate_up units (union entry u, h-row i): each wave streams a contiguous
//      range of units (gate row + up row, 1 KB chunks per lane-step, a ring of
//      D steps in flight) and writes h = silu(g)*u as bf16 for every token
//      routed to u.  Each wave then counts its rows into per-(u, 128-row group)
//      counters; the wave completing a group re-quantises that group of h for
//      every token (deterministic: the quantisation depends on values only)
//      and bumps the phase counter.
//   D. down units (output row n, all union entries): a wave issues its first
//      down weight loads, the block waits for the phase counter, stages the
//      quantised h of all (token, slot) pairs in LDS and streams the rows; per
//      row every (token, slot) partial is reduced across the wave and the
//      tokens' outputs are combined in slot order.
//   E. the last block to finish resets every counter it used, so the
//      workspace is ready for the next call without a clearing launch.
//
// Every weight byte of the union is read once per call.  The arithmetic done
// for one token does not depend on the other tokens of the call (same lane
// split, same reduction order), so a row of an M-token verify call is bitwise
// equal to the same token decoded alone.
#include <stdlib.h>

#include "pq_quant_dev.h"

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / pq::kWave;
constexpr int kMaxM = 8;
constexpr int kMaxTopK = 8;
constexpr int kMaxPairs = kMaxM * kMaxTopK;   // 64 = one lane per (token, slot)
constexpr int kMaxUnion = kMaxPairs;
constexpr int kMaxE = 1024;
constexpr int kXPre = 2;
constexpr int DG = 8;     // gate_up ring depth (chunk-steps; 2 rows per step)
constexpr int DD = 16;    // down ring depth (chunk-steps; 1 row per step)
constexpr uint32_t kSpinLimit = 1u << 20;

struct MoeArgs {
  const uint16_t* x;
  const float* logits;
  int32_t* topk_ids;
  float* topk_w;
  const uint8_t* w13;
  const float* s13;
  const uint8_t* w2;
  const float* s2;
  uint16_t* out;
  uint16_t* h_dbg;
  uint8_t* hq_dbg;
  float* hs_dbg;
  uint8_t* ws;
  uint16_t* hbuf;   // [P][I] bf16
  uint8_t* hq;      // [P][I] E4M3
  float* hs;        // [P][I/128]
  int M, H, I, E, top_k;
  int routed;
  uint32_t spin_limit;
};

struct Route {
  int ids[kMaxPairs];
  float w[kMaxPairs];
  int uexp[kMaxUnion];            // expert id of union entry u
  int unp[kMaxUnion];             // number of (token, slot) pairs routed to u
  int upairs[kMaxUnion][kMaxM];   // their pair indices p = m * top_k + j, ascending
  int nU;
};

__device__ __forceinline__ int ufl(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f == 0.0f ? 0.0f : f);   // -0 and +0 compare equal
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const uint32_t lo = __shfl_xor((uint32_t)v, o, pq::kWave);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, pq::kWave);
  return ((uint64_t)hi << 32) | lo;
}

// Phase A, executed by one wave.  Top-k of each token's logits (descending,
// ties to the lower id), softmax over the selected logits, then the union.
__device__ void route_wave(const MoeArgs& a, Route& r, pq::WsHeader* hdr) {
  const int lane = pq::lane_id();
  const int P = a.M * a.top_k;
  if (a.routed) {
    constexpr int kPer = kMaxE / pq::kWave;   // 16 logits per lane
    for (int m = 0; m < a.M; ++m) {
      uint32_t keys[kPer];
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int e = q * pq::kWave + lane;
        keys[q] = e < a.E ? order_key(a.logits[(size_t)m * a.E + e]) : 0u;
      }
      uint32_t taken = 0;
      float sel = 0.0f;
      int sel_id = 0;
      for (int j = 0; j < a.top_k; ++j) {
        // lane-local best: highest key, then lowest id
        uint64_t best = 0;
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const int e = q * pq::kWave + lane;
          const bool live = e < a.E && !((taken >> q) & 1u);
          const uint64_t k = live ? (((uint64_t)keys[q] << 32) | (uint32_t)(~e)) : 0ull;
          best = k > best ? k : best;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
          const uint64_t other = shfl_xor_u64(best, o);
          best = other > best ? other : best;
        }
        const int id = (int)(~(uint32_t)best);
        if ((id & (pq::kWave - 1)) == lane) taken |= 1u << (id / pq::kWave);
        if (lane == j) {
          sel_id = id;
          sel = a.logits[(size_t)m * a.E + id];
        }
      }
      // softmax over the k selected logits (lanes 0..k-1), relative to the top one
      const float l0 = __shfl(sel, 0, pq::kWave);
      const float ex = lane < a.top_k ? expf(sel - l0) : 0.0f;
      const float den = pq::wave_sum(ex);
      if (lane < a.top_k) {
        r.ids[m * a.top_k + lane] = sel_id;
        r.w[m * a.top_k + lane] = ex / den;
        if (blockIdx.x == 0) {
          a.topk_ids[m * a.top_k + lane] = sel_id;
          a.topk_w[m * a.top_k + lane] = ex / den;
        }
      }
    }
  } else if (lane < P) {
    int id = a.topk_ids[lane];
    if (id < 0 || id >= a.E) {
      if (blockIdx.x == 0) pq::record_error(hdr, PQ_ERR_BAD_EXPERT);
      id = 0;
    }
    r.ids[lane] = id;
    r.w[lane] = a.topk_w[lane];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // union in first-appearance order over pairs p = m * top_k + j
  const int id = lane < P ? r.ids[lane] : -1 - lane;
  int first = lane, before = 0, total = 0;
  for (int q = 0; q < P; ++q) {
    const int v = __shfl(id, q, pq::kWave);
    if (v == id) {
      first = q < first ? q : first;
      before += q < lane ? 1 : 0;
      ++total;
    }
  }
  const bool is_first = lane < P && first == lane;
  const uint64_t firsts = __ballot(is_first);
  const int u = __popcll(firsts & ((1ull << first) - 1ull));
  if (lane < P) {
    if (is_first) {
      r.uexp[u] = id;
      r.unp[u] = total < kMaxM ? total : kMaxM;
    }
    if (before < kMaxM) r.upairs[u][before] = lane;
    else if (blockIdx.x == 0) pq::record_error(hdr, PQ_ERR_BAD_EXPERT);   // duplicate ids in one token
  }
  if (lane == 0) r.nU = __popcll(firsts);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

__global__ __launch_bounds__(kThreads) void moe_layer_kernel(MoeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ Route route;
  __shared__ int s_last;

  pq::WsHeader* hdr = reinterpret_cast<pq::WsHeader*>(a.ws);
  uint32_t* gcnt = reinterpret_cast<uint32_t*>(a.ws + pq::kWsCounterOff);

  const int lane = pq::lane_id();
  const int wv = pq::wave_id();
  const int gw = ufl((int)blockIdx.x * kWaves + wv);
  const long T = (long)gridDim.x * kWaves;
  const int H = a.H, I = a.I, K = a.top_k;
  const int P = a.M * K;
  const int nbH = H / pq::kBlock, nbI = I / pq::kBlock;
  const int nchH = (H + pq::kChunk - 1) / pq::kChunk;
  const int nchI = (I + pq::kChunk - 1) / pq::kChunk;
  const uint32_t lane16 = 16u * (uint32_t)lane;
  const uint32_t lane_blk4 = 4u * ((uint32_t)lane >> 3);

  size_t act_bytes = (size_t)a.M * H > (size_t)P * I ? (size_t)a.M * H : (size_t)P * I;
  uint8_t* act = smem;                                                  // codes
  float* acts = reinterpret_cast<float*>(smem + pqhost::align_up(act_bytes, 16));   // scales

  // ---- x loads first (independent of routing) ------------------------------
  const long totx8 = (long)a.M * H / 8;
  const pq::rsrc_t xr = pq::make_rsrc(a.x, (uint32_t)(a.M * H * 2));
  uint4 xraw[kXPre];
#pragma unroll
  for (int it = 0; it < kXPre; ++it) xraw[it] = pq::buf_load16(xr, (uint32_t)(it * kThreads + threadIdx.x) * 16u);

  // ---- A. routing -----------------------------------------------------------
  if (wv == 0) route_wave(a, route, hdr);
  __syncthreads();
  const int nU = ufl(route.nU);

  // ---- C(prefetch). gate_up ring ------------------------------------------
  const int gu_units = nU * I;
  const int g0 = (int)((long)gw * gu_units / T);
  const int g1 = (int)((long)(gw + 1) * gu_units / T);
  const int gsteps = (g1 - g0) * nchH;

  uint4 wb[DG][2];
  float sb[DG][2];
  int iu = g0 / I, ii = g0 - (g0 / I) * I, ic = 0;
  int ie = ufl(route.uexp[iu < nU ? iu : 0]);
  auto issue_gu = [&](uint4 (&w)[2], float (&s)[2]) {
    const bool in_range = iu * I + ii < g1;
    const uint32_t kc = (uint32_t)(ic * pq::kChunk);
    const bool ok = in_range && kc + lane16 < (uint32_t)H;
    const uint8_t* wbase = a.w13 + (size_t)ie * 2 * I * H;
    const float* sbase = a.s13 + (size_t)ie * 2 * I * nbH;
    const pq::rsrc_t wr = pq::make_rsrc(wbase, (uint32_t)(2 * I * H));
    const pq::rsrc_t sr = pq::make_rsrc(sbase, (uint32_t)(2 * I * nbH * 4));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t row = (uint32_t)(ii + j * I);
      w[j] = pq::buf_load16(wr, ok ? row * (uint32_t)H + kc + lane16 : pq::kOOB);
      s[j] = pq::buf_load_f32(sr, ok ? (row * (uint32_t)nbH + kc / pq::kBlock) * 4u + lane_blk4 : pq::kOOB);
    }
    if (++ic == nchH) {
      ic = 0;
      if (++ii == I) {
        ii = 0;
        ++iu;
        ie = ufl(route.uexp[iu < nU ? iu : 0]);
      }
    }
  };
#pragma unroll
  for (int q = 0; q < DG; ++q) issue_gu(wb[q], sb[q]);

  // ---- B. live activation quantisation into LDS ----------------------------
  {
    const int iters = (int)((totx8 + kThreads - 1) / kThreads);
    for (int it = 0; it < iters; ++it) {
      const long t = (long)it * kThreads + threadIdx.x;
      const bool valid = t < totx8;
      const uint4 raw = it < kXPre ? xraw[it < kXPre ? it : 0] : pq::buf_load16(xr, (uint32_t)t * 16u);
      float v[8];
      pq::bf16x8_to_f32(raw, v);
      const float s = pq::fp8_block_scale16(v, valid);
      if (valid) {
        reinterpret_cast<uint2*>(act)[t] = pq::fp8_codes8(v, s);
        if ((threadIdx.x & 15) == 0) acts[(t * 8) / pq::kBlock] = s;
      }
    }
  }
  __syncthreads();

  // ---- C. gate_up + SiLU*up -------------------------------------------------
  {
    float accg[kMaxM], accu[kMaxM];
#pragma unroll
    for (int t = 0; t < kMaxM; ++t) accg[t] = accu[t] = 0.0f;
    int cu = g0 / I, ci = g0 - (g0 / I) * I, cc = 0;
    int cnp = ufl(route.unp[cu < nU ? cu : 0]);
    for (int base = 0; base < gsteps; base += DG) {
#pragma unroll
      for (int q = 0; q < DG; ++q) {
        if (base + q < gsteps) {
          const uint32_t off = (uint32_t)(cc * pq::kChunk) + lane16;
          if (off < (uint32_t)H) {
            const pq::Bf16x16 wg = pq::widen16(wb[q][0]);
            const pq::Bf16x16 wu = pq::widen16(wb[q][1]);
#pragma unroll
            for (int t = 0; t < kMaxM; ++t) {
              if (t < cnp) {
                const int p = ufl(route.upairs[cu][t]);
                const int m = p / K;
                const pq::Bf16x16 xv = pq::widen16(*reinterpret_cast<const uint4*>(act + (size_t)m * H + off));
                const float xs = acts[m * nbH + off / pq::kBlock];
                accg[t] = fmaf(pq::dot16(wg, xv), sb[q][0] * xs, accg[t]);
                accu[t] = fmaf(pq::dot16(wu, xv), sb[q][1] * xs, accu[t]);
              }
            }
          }
          if (cc == nchH - 1) {            // unit (cu, ci) done: h for every routed token
#pragma unroll
            for (int t = 0; t < kMaxM; ++t) {
              if (t < cnp) {
                const float g = pq::wave_sum(accg[t]);
                const float u = pq::wave_sum(accu[t]);
                if (lane == 0) {
                  const int p = route.upairs[cu][t];
                  const uint16_t hb = pq::bf16_rne(silu_mul(g, u));
                  a.hbuf[(size_t)p * I + ci] = hb;
                  if (a.h_dbg) a.h_dbg[(size_t)p * I + ci] = hb;
                }
              }
              accg[t] = accu[t] = 0.0f;
            }
          }
          if (++cc == nchH) {
            cc = 0;
            if (++ci == I) {
              ci = 0;
              ++cu;
              cnp = ufl(route.unp[cu < nU ? cu : 0]);
            }
          }
        }
        issue_gu(wb[q], sb[q]);
      }
    }
  }

  // ---- count finished h rows per (u, 128-row group); the completing wave
  //      re-quantises that group for every token routed to u ---------------
  if (g1 > g0) {
    pq::fence_release();
    for (int G = g0 >> 7; G <= (g1 - 1) >> 7; ++G) {
      const int lo = g0 > (G << 7) ? g0 : (G << 7);
      const int hi = g1 < ((G + 1) << 7) ? g1 : ((G + 1) << 7);
      uint32_t old = 0;
      if (lane == 0) old = pq::atomic_add_relaxed(&gcnt[G], (uint32_t)(hi - lo));
      old = (uint32_t)ufl((int)__shfl(old, 0, pq::kWave));
      if (old + (uint32_t)(hi - lo) == 128u) {
        pq::fence_acquire();
        const int u = G / nbI, g = G - (G / nbI) * nbI;
        const int np = ufl(route.unp[u]);
        for (int t = 0; t < np; ++t) {
          const int p = ufl(route.upairs[u][t]);
          const size_t e0 = (size_t)p * I + (size_t)g * pq::kBlock + 2 * lane;
          const uint32_t two = *reinterpret_cast<const uint32_t*>(a.hbuf + e0);
          float v[2] = {pq::bf16_to_f32(two & 0xffffu), pq::bf16_to_f32(two >> 16)};
          float m = fmaxf(fabsf(v[0]), fabsf(v[1]));
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, pq::kWave));
          const float s = pq::block_scale(m);
          const double rcp = 1.0 / (double)s;
          const uint32_t c0 = pq::e4m3_encode(pq::quotient_f32(v[0], rcp));
          const uint32_t c1 = pq::e4m3_encode(pq::quotient_f32(v[1], rcp));
          const uint16_t cc2 = (uint16_t)(c0 | (c1 << 8));
          *reinterpret_cast<uint16_t*>(a.hq + e0) = cc2;
          if (a.hq_dbg) *reinterpret_cast<uint16_t*>(a.hq_dbg + e0) = cc2;
          if (lane == 0) {
            a.hs[(size_t)p * nbI + g] = s;
            if (a.hs_dbg) a.hs_dbg[(size_t)p * nbI + g] = s;
          }
        }
        pq::fence_release();
        if (lane == 0) pq::atomic_add_relaxed(&hdr->done, 1u);
      }
    }
  }

  // ---- D. down projection + weighted combine --------------------------------
  const int d0 = (int)((long)gw * H / T);
  const int d1 = (int)((long)(gw + 1) * H / T);
  const int dsteps = (d1 - d0) * nU * nchI;
  uint4 wd[DD];
  float sd[DD];
  int jn = d0, ju = 0, jc = 0;
  int je = ufl(route.uexp[0]);
  auto issue_dn = [&](uint4& w, float& s) {
    const bool in_range = jn < d1;
    const uint32_t kc = (uint32_t)(jc * pq::kChunk);
    const bool ok = in_range && kc + lane16 < (uint32_t)I;
    const pq::rsrc_t wr = pq::make_rsrc(a.w2 + (size_t)je * H * I, (uint32_t)(H * I));
    const pq::rsrc_t sr = pq::make_rsrc(a.s2 + (size_t)je * H * nbI, (uint32_t)(H * nbI * 4));
    w = pq::buf_load16(wr, ok ? (uint32_t)jn * (uint32_t)I + kc + lane16 : pq::kOOB);
    s = pq::buf_load_f32(sr, ok ? ((uint32_t)jn * (uint32_t)nbI + kc / pq::kBlock) * 4u + lane_blk4 : pq::kOOB);
    if (++jc == nchI) {
      jc = 0;
      if (++ju == nU) {
        ju = 0;
        ++jn;
      }
      je = ufl(route.uexp[ju]);
    }
  };
#pragma unroll
  for (int q = 0; q < DD; ++q) issue_dn(wd[q], sd[q]);

  // wait for every h group of the call, then stage the quantised h in LDS
  __syncthreads();
  if (threadIdx.x == 0) pq::spin_wait_geq(&hdr->done, (uint32_t)(nU * nbI), hdr, a.spin_limit);
  __syncthreads();
  pq::fence_acquire();
  {
    const long n16 = (long)P * I / 16;
    for (long t = threadIdx.x; t < n16; t += kThreads)
      reinterpret_cast<uint4*>(act)[t] = reinterpret_cast<const uint4*>(a.hq)[t];
    for (long t = threadIdx.x; t < (long)P * nbI; t += kThreads) acts[t] = a.hs[t];
  }
  __syncthreads();

  {
    float acc[kMaxM];
#pragma unroll
    for (int t = 0; t < kMaxM; ++t) acc[t] = 0.0f;
    float ycap = 0.0f;                 // lane p holds y of pair p for the current row
    int cn = d0, cu = 0, cc = 0;
    int cnp = ufl(route.unp[0]);
    for (int base = 0; base < dsteps; base += DD) {
#pragma unroll
      for (int q = 0; q < DD; ++q) {
        if (base + q < dsteps) {
          const uint32_t off = (uint32_t)(cc * pq::kChunk) + lane16;
          if (off < (uint32_t)I) {
            const pq::Bf16x16 wv = pq::widen16(wd[q]);
#pragma unroll
            for (int t = 0; t < kMaxM; ++t) {
              if (t < cnp) {
                const int p = ufl(route.upairs[cu][t]);
                const pq::Bf16x16 hv = pq::widen16(*reinterpret_cast<const uint4*>(act + (size_t)p * I + off));
                const float hsc = acts[p * nbI + off / pq::kBlock];
                acc[t] = fmaf(pq::dot16(wv, hv), sd[q] * hsc, acc[t]);
              }
            }
          }
          if (cc == nchI - 1) {           // (row cn, union entry cu) done
#pragma unroll
            for (int t = 0; t < kMaxM; ++t) {
              if (t < cnp) {
                const float y = pq::wave_sum(acc[t]);
                const int p = ufl(route.upairs[cu][t]);
                ycap = lane == p ? y : ycap;
              }
              acc[t] = 0.0f;
            }
            if (cu == nU - 1) {           // row cn done: combine each token's slots in order
              float o = 0.0f;
              const int mine = lane < a.M ? lane : 0;
              for (int j = 0; j < K; ++j) {
                const float y = __shfl(ycap, mine * K + j, pq::kWave);
                o = fmaf(route.w[mine * K + j], y, o);
              }
              if (lane < a.M) a.out[(size_t)lane * H + cn] = pq::bf16_rne(o);
            }
          }
          if (++cc == nchI) {
            cc = 0;
            if (++cu == nU) {
              cu = 0;
              ++cn;
            }
            cnp = ufl(route.unp[cu]);
          }
        }
        issue_dn(wd[q], sd[q]);
      }
    }
  }

  // ---- E. the last block resets the counters of this call -------------------
  __syncthreads();
  if (threadIdx.x == 0) {
    pq::fence_release();
    const uint32_t old = pq::atomic_add_relaxed(&hdr->exit_count, 1u);
    s_last = old == gridDim.x - 1;
  }
  __syncthreads();
  if (s_last) {
    pq::fence_acquire();
    for (int t = threadIdx.x; t < nU * nbI; t += kThreads) pq::atomic_store_relaxed(&gcnt[t], 0u);
    if (threadIdx.x == 0) {
      pq::atomic_store_relaxed(&hdr->done, 0u);
      pq::atomic_store_relaxed(&hdr->exit_count, 0u);
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct MoePlan {
  size_t lds;
  size_t off_h, off_hq, off_hs, ws_total;
};

int moe_plan(int M, int H, int I, int E, int top_k, MoePlan* p) {
  if (M < 1 || M > kMaxM || top_k < 1 || top_k > kMaxTopK || E < top_k || E > kMaxE) return PQ_ERR_SHAPE;
  if (H < pq::kBlock || H % pq::kBlock || H > 16384 || I < pq::kBlock || I % pq::kBlock || I > 16384)
    return PQ_ERR_SHAPE;
  const size_t P = (size_t)M * top_k;
  const size_t nbI = I / pq::kBlock;
  if (P * nbI > pq::kWsMaxCounters) return PQ_ERR_SHAPE;
  if ((size_t)2 * I * H > pq::kMaxBufferBytes) return PQ_ERR_SHAPE;
  const size_t act = (size_t)M * H > P * I ? (size_t)M * H : P * I;
  const size_t actsc = ((size_t)M * H / pq::kBlock > P * nbI ? (size_t)M * H / pq::kBlock : P * nbI) * 4;
  p->lds = pqhost::align_up(act, 16) + actsc;
  if (p->lds + sizeof(Route) + 64 > 160 * 1024) return PQ_ERR_SHAPE;
  p->off_h = pq::kWsDataOff;
  p->off_hq = pqhost::align_up(p->off_h + P * I * 2, 256);
  p->off_hs = pqhost::align_up(p->off_hq + P * I, 256);
  p->ws_total = pqhost::align_up(p->off_hs + P * nbI * 4, 256);
  return PQ_OK;
}

}  // namespace

extern "C" {

size_t moe_decode_layer_workspace(int M, int H, int I, int E, int top_k) {
  MoePlan pl;
  if (moe_plan(M, H, I, E, top_k, &pl) != PQ_OK) return 0;
  return pl.ws_total;
}

int moe_decode_layer(const uint16_t* x, int M, int H, const float* router_logits, int32_t* topk_ids,
                     float* topk_w, int E, int top_k, int I, const uint8_t* w13, const float* s13,
                     const uint8_t* w2, const float* s2, uint16_t* out, uint16_t* h_dbg, uint8_t* hq_dbg,
                     float* hs_dbg, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !topk_ids || !topk_w || !w13 || !s13 || !w2 || !s2 || !out || !ws) return PQ_ERR_NULL;
  MoePlan pl;
  int st = moe_plan(M, H, I, E, top_k, &pl);
  if (st != PQ_OK) return st;
  const void* ptrs[] = {x, router_logits, topk_ids, topk_w, w13, s13, w2, s2, out, h_dbg, hq_dbg, hs_dbg, ws};
  for (const void* q : ptrs)
    if (q && !pqhost::aligned16(q)) return PQ_ERR_ALIGN;
  if (ws_bytes < pl.ws_total) return PQ_ERR_WORKSPACE;
  pqhost::DeviceInfo dev;
  st = pqhost::current_device_info(&dev);
  if (st != PQ_OK) return st;

  auto kern = moe_layer_kernel;
  static bool attr_set = false;
  if (!attr_set) {
    PQ_HIP_CHECK(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)(160 * 1024 - sizeof(Route) - 64)));
    attr_set = true;
  }
  int per_cu = 0;
  PQ_HIP_CHECK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kern, kThreads, pl.lds));
  if (per_cu < 1) return PQ_ERR_SHAPE;
  int grid = dev.num_cus * per_cu;                  // every block resident: blocks wait on each other

  MoeArgs a;
  a.x = x; a.logits = router_logits; a.topk_ids = topk_ids; a.topk_w = topk_w;
  a.w13 = w13; a.s13 = s13; a.w2 = w2; a.s2 = s2; a.out = out;
  a.h_dbg = h_dbg; a.hq_dbg = hq_dbg; a.hs_dbg = hs_dbg;
  a.ws = reinterpret_cast<uint8_t*>(ws);
  a.hbuf = reinterpret_cast<uint16_t*>(a.ws + pl.off_h);
  a.hq = a.ws + pl.off_hq;
  a.hs = reinterpret_cast<float*>(a.ws + pl.off_hs);
  a.M = M; a.H = H; a.I = I; a.E = E; a.top_k = top_k;
  a.routed = router_logits != nullptr;
  a.spin_limit = kSpinLimit;
  const char* lim = getenv("PQ_SPIN_LIMIT");
  if (lim && *lim) a.spin_limit = (uint32_t)strtoul(lim, nullptr, 10);

  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), pl.lds, (hipStream_t)stream, a);
  PQ_HIP_CHECK(hipGetLastError());
  return PQ_OK;
}

}  // extern "C"
