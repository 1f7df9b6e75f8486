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
// Structure (persistent blocks, one per CU, 16 waves each, static work split)
//   A. routing: wave m ranks token m's logits (top-k, ties to the lower id,
//      softmax over the selected logits); wave 0 then builds the union of
//      routed experts in first-appearance order.  Every block does this
//      redundantly (a few hundred ALU ops); block 0 writes the routing outputs.
//   B. the block live-quantises x into LDS while its first gate_up weight
//      loads are in flight.
//   C. gate_up units (union entry u, h-row i): each wave streams a contiguous
//      range of units (gate row + up row, one 1 KB chunk per lane-step, a ring
//      of DG steps in flight) and stores h = silu(g)*u (bf16) for every token
//      routed to u, then adds its row count to the phase counter.
//   D. down units (output row n, all union entries): waves issue their first
//      down weight loads, the block waits for the phase counter to reach every
//      h row, quantises h of every (token, slot) pair into LDS (each block
//      derives the same codes from the same values) and streams its rows; per
//      row each (token, slot) partial is reduced across the wave and each
//      token's slots are combined in slot order.
//   E. the last block to finish resets the counters it used, so the workspace
//      is ready for the next call without a clearing launch.
//
// Cross-block data (h and the counters) travels through the
// agent-coherent (sc1) path: no L2 writeback or invalidate is needed.
// Every weight byte of the union is read once per call.  The arithmetic done
// for one token does not depend on the other tokens of the call (same lane
// split, same reduction order), so a token's output in an M-token verify call
// is bitwise equal to the same token decoded alone.
#include <stdlib.h>

#include "pq_quant_dev.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / pq::kWave;
constexpr int kMaxM = 8;
constexpr int kMaxTopK = 8;
constexpr int kMaxPairs = kMaxM * kMaxTopK;   // 64 = one lane per (token, slot)
constexpr int kMaxUnion = kMaxPairs;
constexpr int kMaxE = 1024;
constexpr int DG = 4;     // gate_up ring depth (chunk-steps; 2 rows per step)
constexpr int DD = 8;     // down ring depth (chunk-steps; 1 row per step)
constexpr uint32_t kSpinLimit = 1u << 20;
constexpr int kAuxSC1 = 0x10;            // buffer aux bit: agent-coherent (sc1) access
constexpr int kFlagStride = 32;          // uint32 per release flag: one 128-byte line each

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
  int M, H, I, E, top_k;
  int routed;
  uint32_t spin_limit;
  int ybuf_off;     // offset (in floats) of the per-block y buffer after the LDS scales
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

// total order on finite floats as unsigned keys (-0 and +0 are one key)
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Top-k of token m's logits by one wave.  Lane l owns experts l, l+64, ...;
// it first sorts its own candidates (key descending, id ascending), then each
// of the k rounds takes the wave-wide maximum of the lanes' current heads;
// among lanes holding the maximum key the lowest expert id wins, so equal
// logits go to the lower id.  KPER = candidates per lane (E <= 64 * KPER).
template <int KPER>
__device__ void route_token(const MoeArgs& a, Route& r, int m) {
  const int lane = pq::lane_id();
  // all logit loads issued before the first wait (past E: zero-filled, key 0)
  const pq::rsrc_t lr = pq::make_rsrc(a.logits + (size_t)m * a.E, (uint32_t)a.E * 4u);
  float lv[KPER];
#pragma unroll
  for (int q = 0; q < KPER; ++q) lv[q] = pq::buf_load_f32(lr, (uint32_t)(q * pq::kWave + lane) * 4u);
  uint32_t key[KPER];
  int eid[KPER];
#pragma unroll
  for (int q = 0; q < KPER; ++q) {
    eid[q] = q * pq::kWave + lane;
    key[q] = eid[q] < a.E ? order_key(lv[q]) : 0u;
  }
  // insertion sort of the lane's candidates: larger key first; ids start
  // ascending and only strictly larger keys move up, so ties stay id-ascending
#pragma unroll
  for (int i = 1; i < KPER; ++i) {
#pragma unroll
    for (int j = i; j > 0; --j) {
      const bool sw = key[j] > key[j - 1];
      const uint32_t k0 = key[j - 1], k1 = key[j];
      const int e0 = eid[j - 1], e1 = eid[j];
      key[j - 1] = sw ? k1 : k0; key[j] = sw ? k0 : k1;
      eid[j - 1] = sw ? e1 : e0; eid[j] = sw ? e0 : e1;
    }
  }
  uint32_t my_key = 0;
  int my_id = 0;
  for (int j = 0; j < a.top_k; ++j) {
    const uint32_t mk = pq::wave_max_u32(key[0]);
    uint64_t tied = __ballot(key[0] == mk);
    int win = (int)__builtin_ctzll(tied);
    int id = __builtin_amdgcn_readlane(eid[0], win);
    tied &= tied - 1;
    while (tied) {                                   // rare: equal keys on several lanes
      const int l2 = (int)__builtin_ctzll(tied);
      const int other = __builtin_amdgcn_readlane(eid[0], l2);
      if (other < id) { id = other; win = l2; }
      tied &= tied - 1;
    }
    if (lane == win) {                               // the winning lane pops its head
#pragma unroll
      for (int q = 0; q + 1 < KPER; ++q) { key[q] = key[q + 1]; eid[q] = eid[q + 1]; }
      key[KPER - 1] = 0u;
    }
    if (lane == j) {
      my_id = id;
      my_key = mk;
    }
  }
  const float sel = key_value(my_key);
  const float l0 = __shfl(sel, 0, pq::kWave);
  const float ex = lane < a.top_k ? expf(sel - l0) : 0.0f;
  const float den = pq::wave_sum(ex);
  if (lane < a.top_k) {
    const float wgt = ex / den;
    r.ids[m * a.top_k + lane] = my_id;
    r.w[m * a.top_k + lane] = wgt;
    if (blockIdx.x == 0) {
      a.topk_ids[m * a.top_k + lane] = my_id;
      a.topk_w[m * a.top_k + lane] = wgt;
    }
  }
}

// Union of the routed experts in ascending expert id (the order does not
// change any result: every h row and every y row is computed whole by one
// wave, and each token's slots are combined in slot order), built in parallel
// by one wave with one LDS bitmap per token: lane p = (m, j) sets bit ids[p]
// in token m's map; the union index of an expert is the number of experts
// below it set in any map, a pair's place among the pairs of its expert is the
// number of lower tokens whose map holds it.  An expert given twice to one
// token is an error.
__device__ void build_union(const MoeArgs& a, Route& r, pq::WsHeader* hdr, uint32_t (*tmask)[kMaxE / 32]) {
  const int lane = pq::lane_id();
  const int P = a.M * a.top_k;
  const bool act = lane < P;
  const int id = act ? r.ids[lane] : 0;
  const int m = act ? lane / a.top_k : 0;
  const int w = id >> 5;
  const uint32_t bit = 1u << (id & 31);
  bool dup = false;
  if (act) dup = (atomicOr(&tmask[m][w], bit) & bit) != 0u;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);       // LDS ops of one wave complete in order
  const int nw = (a.E + 31) >> 5;
  uint32_t word = 0u;                              // lane's word of the union bitmap
  int n = 0, slot = 0;
  for (int mm = 0; mm < a.M; ++mm) {
    if (lane < nw) word |= __hip_atomic_load(&tmask[mm][lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const int has = (__hip_atomic_load(&tmask[mm][w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) & bit) != 0u;
    n += has;
    slot += mm < m ? has : 0;
  }
  const int cnt = __popc(word);
  int incl = cnt;                                  // inclusive prefix over the bitmap words
#pragma unroll
  for (int d = 1; d < 32; d <<= 1) {
    const int v = __shfl_up(incl, d, pq::kWave);
    if (lane >= d) incl += v;
  }
  const int excl = incl - cnt;
  const int total = __shfl(incl, 31, pq::kWave);
  const int u = __shfl(excl, w, pq::kWave) + __popc((uint32_t)__shfl((int)word, w, pq::kWave) & (bit - 1u));
  if (act) {
    // n <= M and slot < M; a duplicate shares its slot with the first copy
    if (slot == 0 && !dup) {
      r.uexp[u] = id;
      r.unp[u] = n;
    }
    if (!dup) r.upairs[u][slot] = lane;
    if (dup && blockIdx.x == 0) pq::record_error(hdr, PQ_ERR_BAD_EXPERT);
  }
  if (lane == 0) r.nU = total;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// TP: compile-time bound on the (token, slot) pairs routed to one expert in a
// call (the smallest power of two >= M), so the per-pair loops unroll tightly.
template <int TP>
__global__ __launch_bounds__(kThreads) void moe_layer_kernel(MoeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ Route route;
  __shared__ int s_last;
  __shared__ uint32_t s_tmask[kMaxM][kMaxE / 32];   // routed-expert bitmap of each token
  __shared__ uint32_t s_next;     // next gate_up unit of this block
  __shared__ uint32_t s_arrive;   // waves of this block done with gate_up
  __shared__ uint32_t s_epoch;    // value the release flags take in this call

  pq::WsHeader* hdr = reinterpret_cast<pq::WsHeader*>(a.ws);
  uint32_t* flags = reinterpret_cast<uint32_t*>(a.ws + pq::kWsCounterOff);   // one line per block

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

  const size_t act_bytes = (size_t)a.M * H > (size_t)P * I ? (size_t)a.M * H : (size_t)P * I;
  uint8_t* act = smem;                                                              // codes
  float* acts = reinterpret_cast<float*>(smem + pqhost::align_up(act_bytes, 16));   // scales

  // ---- x loads first (independent of routing); the waves that do not route
  //      quantise x while waves 0..M-1 rank the logits ------------------------
  const int nrt = a.routed ? a.M : 1;               // routing waves
  const long totx8 = (long)a.M * H / 8;
  // when the other waves cannot cover x in one pass, every wave takes a share
  // (the routing waves after routing)
  const bool xq_all = totx8 > (long)(kThreads - nrt * pq::kWave);
  const int tq = xq_all ? (int)threadIdx.x : (int)threadIdx.x - nrt * pq::kWave;   // < 0: routing wave only
  const int nq = xq_all ? kThreads : kThreads - nrt * pq::kWave;
  const pq::rsrc_t xr = pq::make_rsrc(a.x, (uint32_t)(a.M * H * 2));
  // enough loads in flight for the whole of x at H = 6144 up to M = 4 (16 bytes each)
  constexpr int kXPre = TP == 1 ? 1 : TP == 2 ? 2 : TP == 4 ? 4 : 8;
  uint4 xraw[kXPre];
#pragma unroll
  for (int it = 0; it < kXPre; ++it) {
    const long t = (long)it * nq + tq;
    xraw[it] = pq::buf_load16(xr, tq >= 0 && t < totx8 ? (uint32_t)t * 16u : pq::kOOB);
  }

  if (threadIdx.x == 0) {       // block counters; first used after the barriers below
    s_next = 0u;
    s_arrive = 0u;
    s_epoch = pq::ld_agent_u32(&hdr->epoch) + 1u;   // this call's flag value
  }
  if (threadIdx.x < kMaxM * kMaxE / 32) (&s_tmask[0][0])[threadIdx.x] = 0u;

  // ---- A. routing (waves 0..M-1, one token each) -----------------------------
  if (a.routed) {
    if (wv < a.M) {
      if (a.E <= 256) route_token<4>(a, route, wv);
      else route_token<16>(a, route, wv);
    }
  } else if (wv == 0 && lane < P) {
    int id = a.topk_ids[lane];
    if (id < 0 || id >= a.E) {
      if (blockIdx.x == 0) pq::record_error(hdr, PQ_ERR_BAD_EXPERT);
      id = 0;
    }
    route.ids[lane] = id;
    route.w[lane] = a.topk_w[lane];
  }

  // ---- B. live activation quantisation into LDS ------------------------------
  if (tq >= 0) {
    const int iters = (int)((totx8 + nq - 1) / nq);
    // 16 lanes share a scale, so whole waves run each step; the preloaded
    // steps are unrolled so the raw values stay in registers
    auto quant = [&](const uint4& raw, long t) {
      const bool valid = t < totx8;
      float v[8];
      pq::bf16x8_to_f32(raw, v);
      const float s = pq::fp8_block_scale16(v, valid);
      if (valid) {
        reinterpret_cast<uint2*>(act)[t] = pq::fp8_codes8(v, s);
        if ((tq & 15) == 0) acts[(t * 8) / pq::kBlock] = s;
      }
    };
#pragma unroll
    for (int it = 0; it < kXPre; ++it)
      if (it < iters) quant(xraw[it], (long)it * nq + tq);
    for (int it = kXPre; it < iters; ++it) {
      const long t = (long)it * nq + tq;
      quant(pq::buf_load16(xr, t < totx8 ? (uint32_t)t * 16u : pq::kOOB), t);
    }
  }

  __syncthreads();                            // routes and the quantised x visible
  if (wv == 0) build_union(a, route, hdr, s_tmask);
  __syncthreads();
  const int nU = ufl(route.nU);

  // ---- C. gate_up + SiLU*up -------------------------------------------------
  // The block owns the units [bu0, bu1) (union entry u, h-row i: one gate row
  // and one up row); its waves take them one at a time from an LDS counter,
  // so a wave whose loads issue later (the scheduler favours older waves)
  // simply takes fewer.  Each wave keeps DG chunk-steps in flight; every ring
  // slot remembers its unit and chunk.
  const int gu_units = nU * I;
  const int bu0 = pq::split_start(gu_units, (int)gridDim.x, (int)blockIdx.x);
  const int bu1 = pq::split_start(gu_units, (int)gridDim.x, (int)blockIdx.x + 1);

  uint4 wb[DG][2];
  float sb[DG][2];
  int su[DG], sch[DG];              // unit (-1: none) and chunk of each slot
  int iunit = bu0 - 1, ic = nchH;   // issue cursor
  bool more = true;
  int cur_e = -1;
  pq::rsrc_t gwr = pq::make_rsrc(a.w13, 0u), gsr = pq::make_rsrc(a.s13, 0u);
  auto issue_gu = [&](uint4 (&w)[2], float (&s)[2], int& su_q, int& sch_q) {
    if (ic == nchH && more) {       // take the block's next unit
      int u = 0;
      if (lane == 0) u = bu0 + (int)atomicAdd(&s_next, 1u);
      iunit = ufl(u);
      ic = 0;
      more = iunit < bu1;
      if (more) {
        const int e = ufl(route.uexp[iunit / I]);
        if (e != cur_e) {
          cur_e = e;
          gwr = pq::make_rsrc(a.w13 + (size_t)e * 2 * I * H, (uint32_t)(2 * I * H));
          gsr = pq::make_rsrc(a.s13 + (size_t)e * 2 * I * nbH, (uint32_t)(2 * I * nbH * 4));
        }
      }
    }
    const uint32_t kc = (uint32_t)(ic * pq::kChunk);
    const bool ok = more && kc + lane16 < (uint32_t)H;
    const uint32_t ii = more ? (uint32_t)(iunit - (iunit / I) * I) : 0u;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t row = ii + (uint32_t)(j * I);
      w[j] = pq::buf_load16_nt(gwr, ok ? row * (uint32_t)H + kc + lane16 : pq::kOOB);
      s[j] = pq::buf_load_f32_nt(gsr, ok ? (row * (uint32_t)nbH + kc / pq::kBlock) * 4u + lane_blk4 : pq::kOOB);
    }
    su_q = more ? iunit : -1;
    sch_q = ic;
    if (more) ++ic;
  };
#pragma unroll
  for (int q = 0; q < DG; ++q) issue_gu(wb[q], sb[q], su[q], sch[q]);


  {
    float accg[TP], accu[TP];
    int pr[TP], pm[TP];
#pragma unroll
    for (int t = 0; t < TP; ++t) accg[t] = accu[t] = 0.0f;
    int pairs_u = -1, cnp = 0;
    auto load_pairs = [&](int uu) {
      pairs_u = uu;
      cnp = ufl(route.unp[uu]);
#pragma unroll
      for (int t = 0; t < TP; ++t) {
        pr[t] = ufl(route.upairs[uu][t]);
        pm[t] = pr[t] / K;
      }
    };
    for (;;) {
#pragma unroll
      for (int q = 0; q < DG; ++q) {
        if (su[q] >= 0) {
          const int unit = su[q], cc = sch[q];
          const int uu = unit / I, ci = unit - (unit / I) * I;
          if (uu != pairs_u) load_pairs(uu);
          const uint32_t off = (uint32_t)(cc * pq::kChunk) + lane16;
          if (off < (uint32_t)H) {
            const pq::Bf16x16 wg = pq::widen16(wb[q][0]);
            const pq::Bf16x16 wu = pq::widen16(wb[q][1]);
#pragma unroll
            for (int t = 0; t < TP; ++t) {
              if (t < cnp) {
                const pq::Bf16x16 xv = pq::widen16(*reinterpret_cast<const uint4*>(act + (size_t)pm[t] * H + off));
                const float xs = acts[pm[t] * nbH + off / pq::kBlock];
                accg[t] = fmaf(pq::dot16(wg, xv), sb[q][0] * xs, accg[t]);
                accu[t] = fmaf(pq::dot16(wu, xv), sb[q][1] * xs, accu[t]);
              }
            }
          }
          if (cc == nchH - 1) {            // unit done: h for every routed token
#pragma unroll
            for (int t = 0; t < TP; ++t) {
              if (t < cnp) {
                const float g = pq::wave_sum(accg[t]);
                const float u = pq::wave_sum(accu[t]);
                if (lane == 0) {
                  const uint16_t hb = pq::bf16_rne(silu_mul(g, u));
                  pq::st_agent_u16(a.hbuf + (size_t)pr[t] * I + ci, hb);
                  if (a.h_dbg) a.h_dbg[(size_t)pr[t] * I + ci] = hb;
                }
              }
              accg[t] = accu[t] = 0.0f;
            }
          }
        }
        issue_gu(wb[q], sb[q], su[q], sch[q]);
      }
      bool busy = false;
#pragma unroll
      for (int q = 0; q < DG; ++q) busy |= su[q] >= 0;
      if (!busy) break;
    }
  }

  // Count the finished h rows: each wave's stores complete (sc1) before it
  // arrives; the last wave of the block to arrive adds the block's rows to
  // the phase counter (one device atomic per block: they serialise on one
  // address).
  // The block that completes the count releases every block through its own
  // flag line (value = this call's epoch, so a flag left by an earlier call
  // never matches).
  pq::wait_vm();
  uint32_t last = 0;
  if (lane == 0) {
    const uint32_t before = atomicAdd(&s_arrive, 1u);
    if (before == (uint32_t)(kWaves - 1) && bu1 > bu0) {
      const uint32_t rows = (uint32_t)(bu1 - bu0);
      last = pq::atomic_add_relaxed(&hdr->done, rows) + rows == (uint32_t)gu_units;
    }
  }
  if (ufl((int)last)) {
    const uint32_t ep = s_epoch;
    for (int b = lane; b < (int)gridDim.x; b += pq::kWave) pq::st_agent_u32(flags + (size_t)b * kFlagStride, ep);
  }

  // ---- D. down projection + weighted combine --------------------------------
  // Output rows are dealt to blocks as evenly as possible; inside a block the
  // (union entry, row) units are taken expert by expert (consecutive rows of
  // one expert are contiguous in memory) and split evenly over the waves.
  // Each unit's y for every routed token goes to LDS; the block then combines
  // each token's slots in slot order.
  const int r0 = pq::split_start(H, (int)gridDim.x, (int)blockIdx.x);
  const int r1 = pq::split_start(H, (int)gridDim.x, (int)blockIdx.x + 1);
  const int nrows = r1 - r0;
  const int bunits = nrows * nU;
  const int v0 = ufl(pq::split_start(bunits, kWaves, wv));
  const int v1 = ufl(pq::split_start(bunits, kWaves, wv + 1));
  const int dsteps = (v1 - v0) * nchI;
  float* ybuf = acts + a.ybuf_off;                 // [row_local][P] fp32
  uint4 wd[DD];
  float sd[DD];
  int ju = nrows > 0 ? v0 / nrows : 0;
  int jr = v0 - ju * nrows, jc = 0, dleft = dsteps;
  pq::rsrc_t dwr, dsr;
  auto set_dn_expert = [&]() {
    const int e = ufl(route.uexp[ju < nU ? ju : 0]);
    dwr = pq::make_rsrc(a.w2 + (size_t)e * H * I, (uint32_t)(H * I));
    dsr = pq::make_rsrc(a.s2 + (size_t)e * H * nbI, (uint32_t)(H * nbI * 4));
  };
  set_dn_expert();
  auto issue_dn = [&](uint4& w, float& s) {
    const uint32_t kc = (uint32_t)(jc * pq::kChunk);
    const bool ok = dleft > 0 && kc + lane16 < (uint32_t)I;
    const uint32_t row = (uint32_t)(r0 + jr);
    w = pq::buf_load16_nt(dwr, ok ? row * (uint32_t)I + kc + lane16 : pq::kOOB);
    s = pq::buf_load_f32_nt(dsr, ok ? (row * (uint32_t)nbI + kc / pq::kBlock) * 4u + lane_blk4 : pq::kOOB);
    --dleft;
    if (++jc == nchI) {
      jc = 0;
      if (++jr == nrows) {
        jr = 0;
        ++ju;
        set_dn_expert();
      }
    }
  };
#pragma unroll
  for (int q = 0; q < DD; ++q) issue_dn(wd[q], sd[q]);

  // wait for every h row of the call, then quantise h into LDS: every block
  // derives the same codes and scales from the same values (block 0 also
  // writes them out when asked)
  if (threadIdx.x == 0) pq::spin_wait_eq(flags + (size_t)blockIdx.x * kFlagStride, s_epoch, hdr, a.spin_limit);
  __syncthreads();
  {
    // 8 values per lane, 16 lanes per 128-value block (the layout of the
    // activation quantiser); agent-coherent 16-byte loads, a batch in flight
    const int nvec = P * I / 8;
    const pq::rsrc_t hr = pq::make_rsrc(a.hbuf, (uint32_t)(P * I * 2));
    constexpr int kBatch = 2;
    for (int t0 = 0; t0 < nvec; t0 += kBatch * kThreads) {
      uint4 raw[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int t = t0 + i * kThreads + (int)threadIdx.x;
        raw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
            hr, (int)(t < nvec ? (uint32_t)t * 16u : pq::kOOB), 0, kAuxSC1));
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int t = t0 + i * kThreads + (int)threadIdx.x;
        const bool valid = t < nvec;
        float v[8];
        pq::bf16x8_to_f32(raw[i], v);
        const float sc = pq::fp8_block_scale16(v, valid);
        if (valid) {
          const uint2 c8 = pq::fp8_codes8(v, sc);
          reinterpret_cast<uint2*>(act)[t] = c8;
          if ((threadIdx.x & 15) == 0) acts[t / 16] = sc;
          if (blockIdx.x == 0) {
            if (a.hq_dbg) reinterpret_cast<uint2*>(a.hq_dbg)[t] = c8;
            if (a.hs_dbg && (threadIdx.x & 15) == 0) a.hs_dbg[t / 16] = sc;
          }
        }
      }
    }
  }
  __syncthreads();

  {
    float acc[TP];
    int pr[TP];
#pragma unroll
    for (int t = 0; t < TP; ++t) acc[t] = 0.0f;
    int cu = nrows > 0 ? v0 / nrows : 0;
    int cr = v0 - cu * nrows, cc = 0;
    int cnp = 0;
    auto load_pairs = [&]() {
      const int uu = cu < nU ? cu : 0;
      cnp = ufl(route.unp[uu]);
#pragma unroll
      for (int t = 0; t < TP; ++t) pr[t] = ufl(route.upairs[uu][t]);
    };
    load_pairs();
    auto consume_dn = [&](const uint4& w, float sw) {
      const uint32_t off = (uint32_t)(cc * pq::kChunk) + lane16;
      if (off < (uint32_t)I) {
        const pq::Bf16x16 wv2 = pq::widen16(w);
#pragma unroll
        for (int t = 0; t < TP; ++t) {
          if (t < cnp) {
            const pq::Bf16x16 hv = pq::widen16(*reinterpret_cast<const uint4*>(act + (size_t)pr[t] * I + off));
            const float hsc = acts[pr[t] * nbI + off / pq::kBlock];
            acc[t] = fmaf(pq::dot16(wv2, hv), sw * hsc, acc[t]);
          }
        }
      }
      if (cc == nchI - 1) {               // unit (union entry cu, row cr) done
#pragma unroll
        for (int t = 0; t < TP; ++t) {
          if (t < cnp) {
            const float y = pq::wave_sum(acc[t]);
            if (lane == 0) ybuf[cr * P + pr[t]] = y;
          }
          acc[t] = 0.0f;
        }
      }
      if (++cc == nchI) {
        cc = 0;
        if (++cr == nrows) {
          cr = 0;
          ++cu;
          load_pairs();
        }
      }
    };
    int base = 0;
    for (; base + DD < dsteps; base += DD) {     // steady state: every slot refills
#pragma unroll
      for (int q = 0; q < DD; ++q) {
        consume_dn(wd[q], sd[q]);
        issue_dn(wd[q], sd[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < DD; ++q)                 // drain
      if (base + q < dsteps) consume_dn(wd[q], sd[q]);
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < (r1 - r0) * a.M; idx += kThreads) {
    const int rl = idx / a.M, m = idx - (idx / a.M) * a.M;
    float o = 0.0f;
    for (int j = 0; j < K; ++j) o = fmaf(route.w[m * K + j], ybuf[rl * P + m * K + j], o);
    a.out[(size_t)m * H + r0 + rl] = pq::bf16_rne(o);
  }

  // ---- E. the last block resets the counters of this call -------------------
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = pq::atomic_add_relaxed(&hdr->exit_count, 1u);
    s_last = old == gridDim.x - 1;
  }
  __syncthreads();
  if (s_last) {
    if (threadIdx.x == 0) {
      pq::atomic_store_relaxed(&hdr->done, 0u);
      pq::atomic_store_relaxed(&hdr->exit_count, 0u);
      pq::atomic_store_relaxed(&hdr->epoch, s_epoch);
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
// LDS the kernel declares statically (routing tables, expert bitmap, block
// counters), reserved next to the dynamic area.
constexpr size_t kStaticLds = sizeof(Route) + kMaxM * kMaxE / 8 + 256;

struct MoePlan {
  size_t lds;
  int ybuf_off;
  size_t off_h, ws_total;
};

// num_cus bounds the rows a block can own (the grid has at least one block per
// CU); num_cus <= 0 checks the shape and sizes the workspace only.
int moe_plan(int M, int H, int I, int E, int top_k, int num_cus, MoePlan* p) {
  if (M < 1 || M > kMaxM || top_k < 1 || top_k > kMaxTopK || E < top_k || E > kMaxE) return PQ_ERR_SHAPE;
  if (H < pq::kBlock || H % pq::kBlock || H > 16384 || I < pq::kBlock || I % pq::kBlock || I > 16384)
    return PQ_ERR_SHAPE;
  const size_t P = (size_t)M * top_k;
  const size_t nbI = I / pq::kBlock;
  if ((size_t)2 * I * H > pq::kMaxBufferBytes) return PQ_ERR_SHAPE;
  const size_t act = (size_t)M * H > P * I ? (size_t)M * H : P * I;
  const size_t nsc = (size_t)M * H / pq::kBlock > P * nbI ? (size_t)M * H / pq::kBlock : P * nbI;
  p->ybuf_off = (int)nsc;
  p->lds = 0;
  if (num_cus > 0) {
    const size_t rows_max = ((size_t)H + num_cus - 1) / num_cus;
    p->lds = pqhost::align_up(act, 16) + (nsc + rows_max * P) * 4;
    if (p->lds + kStaticLds > 160 * 1024) return PQ_ERR_SHAPE;
  }
  p->off_h = pq::kWsDataOff;
  p->ws_total = pqhost::align_up(p->off_h + P * I * 2, 256);
  return PQ_OK;
}

template <int TP>
int launch_moe(const MoeArgs& a, const MoePlan& pl, const pqhost::DeviceInfo& dev, hipStream_t stream) {
  auto kern = moe_layer_kernel<TP>;
  static bool attr_set = false;
  if (!attr_set) {
    PQ_HIP_CHECK(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)(160 * 1024 - kStaticLds)));
    attr_set = true;
  }
  int per_cu = 0;
  PQ_HIP_CHECK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kern, kThreads, pl.lds));
  if (per_cu < 1) return PQ_ERR_SHAPE;
  // one block per CU (blocks wait on each other, so all must be resident; one
  // per CU also keeps the per-block staging of h to one copy per CU)
  const int grid = dev.num_cus;
  if ((size_t)grid * kFlagStride * 4 > pq::kWsDataOff - pq::kWsCounterOff) return PQ_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), pl.lds, stream, a);
  PQ_HIP_CHECK(hipGetLastError());
  return PQ_OK;
}

}  // namespace

extern "C" {

size_t moe_decode_layer_workspace(int M, int H, int I, int E, int top_k) {
  MoePlan pl;
  if (moe_plan(M, H, I, E, top_k, 0, &pl) != PQ_OK) return 0;
  return pl.ws_total;
}

int moe_decode_layer(const uint16_t* x, int M, int H, const float* router_logits, int32_t* topk_ids,
                     float* topk_w, int E, int top_k, int I, const uint8_t* w13, const float* s13,
                     const uint8_t* w2, const float* s2, uint16_t* out, uint16_t* h_dbg, uint8_t* hq_dbg,
                     float* hs_dbg, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !topk_ids || !topk_w || !w13 || !s13 || !w2 || !s2 || !out || !ws) return PQ_ERR_NULL;
  MoePlan pl;
  int st = moe_plan(M, H, I, E, top_k, 0, &pl);       // shape checks (device independent)
  if (st != PQ_OK) return st;
  const void* ptrs[] = {x, router_logits, topk_ids, topk_w, w13, s13, w2, s2, out, h_dbg, hq_dbg, hs_dbg, ws};
  for (const void* q : ptrs)
    if (q && !pqhost::aligned16(q)) return PQ_ERR_ALIGN;
  if (ws_bytes < pl.ws_total) return PQ_ERR_WORKSPACE;
  pqhost::DeviceInfo dev;
  st = pqhost::current_device_info(&dev);
  if (st != PQ_OK) return st;
  st = moe_plan(M, H, I, E, top_k, dev.num_cus, &pl);
  if (st != PQ_OK) return st;

  MoeArgs a;
  a.x = x; a.logits = router_logits; a.topk_ids = topk_ids; a.topk_w = topk_w;
  a.w13 = w13; a.s13 = s13; a.w2 = w2; a.s2 = s2; a.out = out;
  a.h_dbg = h_dbg; a.hq_dbg = hq_dbg; a.hs_dbg = hs_dbg;
  a.ws = reinterpret_cast<uint8_t*>(ws);
  a.hbuf = reinterpret_cast<uint16_t*>(a.ws + pl.off_h);
  a.M = M; a.H = H; a.I = I; a.E = E; a.top_k = top_k;
  a.routed = router_logits != nullptr;
  a.spin_limit = kSpinLimit;
  a.ybuf_off = pl.ybuf_off;
  const char* lim = getenv("PQ_SPIN_LIMIT");
  if (lim && *lim) a.spin_limit = (uint32_t)strtoul(lim, nullptr, 10);

  hipStream_t s = (hipStream_t)stream;
  if (M == 1) return launch_moe<1>(a, pl, dev, s);
  if (M == 2) return launch_moe<2>(a, pl, dev, s);
  if (M <= 4) return launch_moe<4>(a, pl, dev, s);
  return launch_moe<8>(a, pl, dev, s);
}

}  // extern "C"
