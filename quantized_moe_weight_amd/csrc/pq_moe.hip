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
//      of DG steps in flight) and stores h = silu(g)*u (bf16, bit-inverted into
//      a region that is zero between calls) for every token routed to u.
//   D. down units (output row n, all union entries): waves issue their first
//      down weight loads, then quantise h of every (token, slot) pair into LDS
//      as its values arrive (a zero word is a value not yet written; each
//      block derives the same codes from the same values) and stream their
//      rows; per row each (token, slot) partial is reduced across the wave and
//      each token's slots are combined in slot order.
//   E. the last block to finish clears h and resets the counter it used, so
//      the workspace is ready for the next call without a clearing launch.
//
// Cross-block data (h and the counters) travels through the
// agent-coherent (sc1) path: no L2 writeback or invalidate is needed.
// Every weight byte of the union is read once per call.  The arithmetic done
// for one token does not depend on the other tokens of the call (same lane
// split, same reduction order), so a token's output in an M-token verify call
// is bitwise equal to the same token decoded alone.
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "pq_quant_dev.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / pq::kWave;
constexpr int kMaxM = 8;
constexpr int kMaxTopK = 8;
constexpr int kMaxPairs = kMaxM * kMaxTopK;   // 64 = one lane per (token, slot)
constexpr int kMaxPairs2 = kMaxPairs + kMaxM;  // with the shared expert's pair of each token
constexpr int kMaxUnion = kMaxPairs + 1;       // with the shared expert's entry
constexpr int kMaxE = 1024;
// Ring depths in chunk-steps (gate_up: 1 KB of 2 rows per step; down: 1 KB of
// 1 row).  Measured on the routed layer, both kernels are fastest with 3 / 6
// (barrier kernel at M=1: 4 / 8 costs 0.7 µs, 8 / 8 4.5 µs; stream kernel at
// M=4 / M=8: 4 / 8 costs 2 µs, 6 / 10 4–5 µs).
constexpr int DG = 3, DD = 2;        // stream kernel (its down steps carry kDnRows rows)
constexpr int kDnRows = 2;           // stream kernel: rows of one union entry per down step
constexpr int kDnClaim = 2;          // stream kernel: down units (row groups) per claim
constexpr int BDG = 3, BDD = 6;      // barrier kernel
constexpr uint32_t kSpinLimit = 1u << 20;
// Polls of an LDS word before a wait inside a block gives up.  Every such word
// is set by waves of the same block that themselves only wait on bounded
// conditions, so in a correct run these waits end in microseconds; the bound
// turns a defect (a producer wave that never arrives) into PQ_ERR_TIMEOUT
// instead of a hung GPU.
constexpr uint32_t kLdsSpinLimit = 1u << 21;
constexpr int kAuxSC1 = 0x10;            // buffer aux bit: agent-coherent (sc1) access
// Scale windows of the barrier kernel's gate_up: each wave owns kScWins
// windows of kWinFloats fp32 block scales in LDS, filled by buffer-to-LDS
// loads (one load instruction per window) and read at each step instead of
// two per-step scale loads.  A unit takes two (its gate and up rows), so four
// units rotate, one more than the ring of BDG steps can hold.
constexpr int kWinFloats = 64;
constexpr int kScWins = 8;
constexpr size_t kScWaveBytes = (size_t)kScWins * kWinFloats * 4;
static_assert(2 * (BDG + 1) <= kScWins, "a window pair per unit in the ring, plus the unit being taken");

struct MoeArgs {
  const uint16_t* x;
  const float* logits;
  const uint16_t* wr;     // router weights bf16 [E][H] (null: logits or ids are given)
  float* logits_out;      // router logits computed here [M][E] (nullable)
  uint32_t* lx;           // logit exchange [M][E]: inverted bits, zero between calls
  const uint8_t* sw13;    // shared expert (null: none), layout of one bank entry
  const float* ss13;
  const uint8_t* sw2;
  const float* ss2;
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
  int32_t* status_out;   // nullable: the call's device-side status, written by the last block
  uint16_t* hbuf;   // [P2][I] bf16 (stream kernel: bits inverted, zero between calls)
  int M, H, I, E, top_k;
  int routed;       // routes from logits (given or computed), else from given ids
  int router;       // logits computed in the launch from wr
  int sh;           // 1 with a shared expert: union entry 0, pairs P .. P + M - 1
  int P2;           // M * top_k + sh * M
  uint32_t spin_limit;
  int xs_off, ha_off, hs_off, yb_off;   // byte offsets of the LDS regions
  int alias;        // h codes and scales reuse the x region
  // stream kernel: x codes at xa_off; h codes by staging slot (union order),
  // slot s at ha_off + s * I; with alias, the slots from hsplit on overlay the
  // x codes
  int xa_off, hsplit;
  int sc_off;       // barrier kernel: LDS byte offset of the per-wave scale windows, or -1
};

struct Route {
  int ids[kMaxPairs];
  float w[kMaxPairs];
  int uexp[kMaxUnion];            // expert id of union entry u
  int unp[kMaxUnion];             // number of (token, slot) pairs routed to u
  int upairs[kMaxUnion][kMaxM];   // their pair indices p = m * top_k + j, ascending
  int items[kMaxPairs2];          // (entry u, pair slot t) = u | t << 8, in union order
  int ustart[kMaxUnion];          // index in items of entry u's first pair slot
  int nU, nitems;
};

__device__ __forceinline__ int ufl(int v) { return __builtin_amdgcn_readfirstlane(v); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Claim the next index of a block counter in LDS.  Every lane of the (fully
// active) wave adds 1, so the counter advances by 64 per claim and the claim
// is the first lane's value before the add, divided by 64.  No lane-divergent
// branch surrounds the atomic: a "lane 0 only" branch inside a loop may be
// compiled into a divergent loop in which the lane that performed the add is
// no longer the first active lane.
__device__ __forceinline__ int wave_claim(uint32_t* p) {
  const uint32_t r = __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return __builtin_amdgcn_readfirstlane((int)(r >> 6));
}

// Wave-wide bounded wait on an LDS word that other waves of the block set:
// returns once done(value) holds, or after kLdsSpinLimit polls with
// PQ_ERR_TIMEOUT recorded.  After a timeout the wave goes on with whatever the
// block's tables hold; the route tables only ever hold in-range entries (see
// layer_prologue), so the results are wrong but every access stays in bounds.
template <class Done>
__device__ __forceinline__ void lds_wait(const uint32_t* p, Done done, pq::WsHeader* hdr) {
  for (uint32_t it = 0;; ++it) {
    const uint32_t v = (uint32_t)ufl((int)__hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
    if (done(v)) return;
    if (it >= kLdsSpinLimit) {
      if (pq::lane_id() == 0) pq::record_error(hdr, PQ_ERR_TIMEOUT);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Number of union entries of the call, read after the routes are released
// (acquire: the union tables written before it are visible).
__device__ __forceinline__ int routes_nU(const Route& r) {
  return ufl(__hip_atomic_load(&r.nU, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
}

// true when either 16-bit half of w is zero
__device__ __forceinline__ bool has_zero_half(uint32_t w) { return (w & 0xFFFFu) == 0u || (w >> 16) == 0u; }

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
// XCH: the logits come from the exchange buffer, where the blocks that
// computed them publish them inverted; wait until every one is there (bounded
// wait: on a timeout the error is recorded and the routing goes on).
template <int KPER, bool XCH>
__device__ void route_token(const MoeArgs& a, Route& r, int m) {
  const int lane = pq::lane_id();
  // all logit loads issued before the first wait (past E: zero-filled, key 0)
  float lv[KPER];
  if (XCH) {
    const pq::rsrc_t lr = pq::make_rsrc(a.lx + (size_t)m * a.E, (uint32_t)a.E * 4u);
    uint32_t raw[KPER];
    for (uint32_t it = 0;; ++it) {
      bool miss = false;
#pragma unroll
      for (int q = 0; q < KPER; ++q) {
        const int e = q * pq::kWave + lane;
        raw[q] = __builtin_amdgcn_raw_buffer_load_b32(lr, (int)((uint32_t)e * 4u), 0, kAuxSC1);
        miss |= e < a.E && raw[q] == 0u;
      }
      if (__ballot(miss) == 0ull) break;
      if (it >= a.spin_limit) {
        if (lane == 0) pq::record_error(reinterpret_cast<pq::WsHeader*>(a.ws), PQ_ERR_TIMEOUT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int q = 0; q < KPER; ++q) lv[q] = __uint_as_float(~raw[q]);
  } else {
    const pq::rsrc_t lr = pq::make_rsrc(a.logits + (size_t)m * a.E, (uint32_t)a.E * 4u);
#pragma unroll
    for (int q = 0; q < KPER; ++q) lv[q] = pq::buf_load_f32(lr, (uint32_t)(q * pq::kWave + lane) * 4u);
  }
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
__device__ void build_union(const MoeArgs& a, Route& r, pq::WsHeader* hdr, uint32_t (*tmask)[kMaxE / 32], int sh) {
  const int lane = pq::lane_id();
  const int P = a.M * a.top_k;
  const bool act = lane < P;
  // ids are in range whenever the routes are complete; the clamp keeps the
  // bitmaps in bounds should a bounded wait have ended early
  const int id = act ? min(max(r.ids[lane], 0), a.E - 1) : 0;
  const int m = act ? lane / a.top_k : 0;
  const int w = id >> 5;
  const uint32_t bit = 1u << (id & 31);
  bool dup = false;
  if (act) dup = (atomicOr(&tmask[m][w], bit) & bit) != 0u;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);       // LDS ops of one wave complete in order
  const int nw = (a.E + 31) >> 5;
  uint32_t word = 0u;                              // lane's word of the union bitmap
  int n = 0, slot = 0, below = 0, nitems = 0;      // below: pairs of lower experts
  for (int mm = 0; mm < a.M; ++mm) {
    const uint32_t wm = lane < nw ? __hip_atomic_load(&tmask[mm][lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) : 0u;
    word |= wm;
    const int has = (__hip_atomic_load(&tmask[mm][w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) & bit) != 0u;
    n += has;
    slot += mm < m ? has : 0;
    const int c = __popc(wm);
    int inc = c;                                   // prefix popcount over token mm's words
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) {
      const int v = __shfl_up(inc, d, pq::kWave);
      if (lane >= d) inc += v;
    }
    below += __shfl(inc - c, w, pq::kWave) + __popc((uint32_t)__shfl((int)wm, w, pq::kWave) & (bit - 1u));
    nitems += __shfl(inc, 31, pq::kWave);
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
    const int us = u + sh;                        // after the shared entry
    if (slot == 0 && !dup) {
      r.uexp[us] = id;
      r.unp[us] = n;
      r.ustart[us] = sh * a.M + below;
    }
    if (!dup) {
      r.upairs[us][slot] = lane;
      r.items[sh * a.M + below + slot] = us | slot << 8;
    }
    if (dup && blockIdx.x == 0) pq::record_error(hdr, PQ_ERR_BAD_EXPERT);
  }
  if (lane == 0) {
    r.nitems = nitems + sh * a.M;
    __hip_atomic_store(&r.nU, total + sh, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// h of pair slot t of union entry uu: wait until every value is stored (none
// reads as the zero word; a poll loads again only the vectors still missing),
// then quantise it into LDS with the layout of the activation quantiser (8
// values per lane, 16 lanes per 128-value block): the codes to hrow (the
// pair's I bytes), the scales to hsc by pair index.
__device__ __forceinline__ void stage_pair(const MoeArgs& a, const Route& r, pq::WsHeader* hdr, int uu, int t,
                                           uint8_t* hrow, float* hsc) {
  const int lane = pq::lane_id();
  const int I = a.I;
  const int p = ufl(r.upairs[uu][t]);
  const int nvec = I / 8;
  const pq::rsrc_t hr = pq::make_rsrc(a.hbuf, (uint32_t)(a.P2 * I * 2));
  constexpr int kSB = 4;
  for (int v0 = 0; v0 < nvec; v0 += kSB * pq::kWave) {
    uint4 raw[kSB];
    bool have[kSB];
#pragma unroll
    for (int j = 0; j < kSB; ++j) {
      have[j] = v0 + j * pq::kWave + lane >= nvec;
      raw[j] = make_uint4(0u, 0u, 0u, 0u);
    }
    for (uint32_t it = 0;; ++it) {
      bool miss = false;
#pragma unroll
      for (int j = 0; j < kSB; ++j) {
        const int idx = v0 + j * pq::kWave + lane;
        const uint4 r4 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
            hr, (int)(have[j] ? pq::kOOB : (uint32_t)(p * nvec + idx) * 16u), 0, kAuxSC1));
        if (!have[j]) {
          raw[j] = r4;
          have[j] = !(has_zero_half(r4.x) || has_zero_half(r4.y) || has_zero_half(r4.z) || has_zero_half(r4.w));
        }
        miss |= !have[j];
      }
      if (__ballot(miss) == 0ull) break;
      if (it >= a.spin_limit) {
        if (lane == 0) pq::record_error(hdr, PQ_ERR_TIMEOUT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int j = 0; j < kSB; ++j) {
      const int idx = v0 + j * pq::kWave + lane;
      const bool valid = idx < nvec;
      const uint4 hv = make_uint4(~raw[j].x, ~raw[j].y, ~raw[j].z, ~raw[j].w);
      float v[8];
      pq::bf16x8_to_f32(hv, v);
      const float sc = pq::fp8_block_scale16(v, valid);
      if (valid) {
        const int gi = p * nvec + idx;
        const uint2 c8 = pq::fp8_codes8(v, sc);
        reinterpret_cast<uint2*>(hrow)[idx] = c8;
        if ((lane & 15) == 0) hsc[gi / 16] = sc;
        if (blockIdx.x == 0) {
          if (a.hq_dbg) reinterpret_cast<uint2*>(a.hq_dbg)[gi] = c8;
          if (a.hs_dbg && (lane & 15) == 0) a.hs_dbg[gi / 16] = sc;
        }
      }
    }
  }
}

// One routed token: its top-k experts are distinct, so the union is its slots
// in slot order (the order of the union entries changes no result), written
// by the routing wave itself — no bitmap and no block barrier in between.
__device__ void single_token_union(const MoeArgs& a, Route& r, int sh) {
  const int lane = pq::lane_id();
  if (lane < a.top_k) {
    const int us = lane + sh;                    // after the shared entry
    r.uexp[us] = r.ids[lane];                    // written by this same lane
    r.unp[us] = 1;
    r.upairs[us][0] = lane;
    r.items[sh + lane] = us;
    r.ustart[us] = sh + lane;
  }
  if (lane == 0) {
    r.nitems = a.top_k + sh;
    __hip_atomic_store(&r.nU, a.top_k + sh, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// The shared expert as union entry 0 (expert id E stands for it): every token
// is routed to it once, as pair P + m; its items come first in union order.
// Independent of the routing, so every block sets it up at the start.
__device__ void shared_entry(const MoeArgs& a, Route& r) {
  const int lane = pq::lane_id();
  if (lane < a.M) {
    r.upairs[0][lane] = a.M * a.top_k + lane;
    r.items[lane] = lane << 8;
  }
  if (lane == 0) {
    r.uexp[0] = a.E;
    r.unp[0] = a.M;
    r.ustart[0] = 0;
  }
}

// Weights of union entry expert e (e == E with a shared expert: that one).
template <bool EXT>
__device__ __forceinline__ const uint8_t* gu_weights(const MoeArgs& a, int e) {
  return EXT && e == a.E ? a.sw13 : a.w13 + (size_t)e * 2 * a.I * a.H;
}
template <bool EXT>
__device__ __forceinline__ const float* gu_scales(const MoeArgs& a, int e) {
  return EXT && e == a.E ? a.ss13 : a.s13 + (size_t)e * 2 * a.I * (a.H / pq::kBlock);
}
template <bool EXT>
__device__ __forceinline__ const uint8_t* dn_weights(const MoeArgs& a, int e) {
  return EXT && e == a.E ? a.sw2 : a.w2 + (size_t)e * a.H * a.I;
}
template <bool EXT>
__device__ __forceinline__ const float* dn_scales(const MoeArgs& a, int e) {
  return EXT && e == a.E ? a.ss2 : a.s2 + (size_t)e * a.H * (a.I / pq::kBlock);
}

// Router rows [e0, e1) of this block for every token: l[m][e] = sum_k x[m][k]
// Wr[e][k] from the bf16 values, fp32 accumulation (each lane sums its 8-value
// slices of every 1 KB chunk in chunk order, then the wave adds the lanes in a
// fixed tree).  Published inverted (a zero word means "not yet written") with
// agent-coherent stores; the routing waves of every block wait for them.
template <int TP>
__device__ void router_rows(const MoeArgs& a, int e) {
  const int lane = pq::lane_id();
  const int H = a.H;
  const uint32_t rowb = (uint32_t)H * 2u;
  const int nck = (int)((rowb + pq::kChunk - 1) / pq::kChunk);
  const pq::rsrc_t wrr = pq::make_rsrc(a.wr + (size_t)e * H, rowb);
  const pq::rsrc_t xr = pq::make_rsrc(a.x, (uint32_t)a.M * rowb);
  float acc[TP];
#pragma unroll
  for (int m = 0; m < TP; ++m) acc[m] = 0.0f;
  constexpr int kB = TP <= 2 ? 4 : TP == 4 ? 2 : 1;   // chunks per batch of loads
  for (int c0 = 0; c0 < nck; c0 += kB) {
    uint4 wv[kB], xv[kB][TP];
#pragma unroll
    for (int q = 0; q < kB; ++q) {
      const uint32_t off = (uint32_t)((c0 + q) * pq::kChunk) + 16u * (uint32_t)lane;
      const bool ok = c0 + q < nck && off < rowb;
      wv[q] = pq::buf_load16(wrr, ok ? off : pq::kOOB);
#pragma unroll
      for (int m = 0; m < TP; ++m)
        xv[q][m] = pq::buf_load16(xr, ok && m < a.M ? (uint32_t)m * rowb + off : pq::kOOB);
    }
#pragma unroll
    for (int q = 0; q < kB; ++q) {
      const uint32_t w4[4] = {wv[q].x, wv[q].y, wv[q].z, wv[q].w};
#pragma unroll
      for (int m = 0; m < TP; ++m) {
        const uint32_t x4[4] = {xv[q][m].x, xv[q][m].y, xv[q][m].z, xv[q][m].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(pq::bf16x2, w4[i]),
                                                   __builtin_bit_cast(pq::bf16x2, x4[i]), acc[m], false);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < TP; ++m) {
    if (m < a.M) {
      const float l = pq::wave_sum(acc[m]);
      if (lane == 0) {
        uint32_t inv = ~__float_as_uint(l);
        if (inv == 0u) inv = ~0x7FC00000u;          // the all-ones NaN: keep the word non-zero
        pq::st_agent_u32(a.lx + (size_t)m * a.E + e, inv);
        if (a.logits_out) a.logits_out[(size_t)m * a.E + e] = l;
      }
    }
  }
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Phases A and B of both kernels: the router rows of this block (when the
// logits are computed in the launch), the routing, the live quantisation of
// x into LDS and the union of the routed experts (after the shared entry).
// On return the quantised x is visible to the whole block; the routes are
// visible once *ready is non-zero: at once when the logits or the ids are
// given, else when the routing waves have waited for every block's logits
// and ranked them (the other waves meanwhile stream the shared expert).
template <int TP, bool EXT>
__device__ __forceinline__ void layer_prologue(const MoeArgs& a, Route& route, uint32_t (*s_tmask)[kMaxE / 32],
                                               uint32_t* s_ready, uint32_t* s_rdone, uint8_t* xa, float* xsc,
                                               pq::WsHeader* hdr) {
  const int lane = pq::lane_id();
  const int wv = pq::wave_id();
  const int H = a.H;
  const int P = a.M * a.top_k;
  const int G = (int)gridDim.x;
  const bool router = EXT && a.router;
  const int sh = EXT ? a.sh : 0;

  // router rows of this block, by its top waves (before they quantise, so the
  // logits are published as early as possible)
  const int e0 = router ? pq::split_start(a.E, G, (int)blockIdx.x) : 0;
  const int e1 = router ? pq::split_start(a.E, G, (int)blockIdx.x + 1) : 0;
  const int nrw = e1 - e0 < kWaves / 2 ? e1 - e0 : kWaves / 2;
  // waves that route before quantising (given logits or ids)
  const int nrt = router ? 0 : (a.routed ? a.M : 1);
  const bool one_token = a.routed && a.M == 1;       // block-uniform
  // given logits of several tokens: the last wave builds the union of their
  // experts as soon as the routing waves are done, while the others quantise x
  const bool early_union = TP > 1 && !router && a.routed && !one_token;   // (TP = 1: one token)
  const int nub = early_union ? 1 : 0;
  const long totx8 = (long)a.M * H / 8;
  const int qthreads = kThreads - (nrt + nrw + nub) * pq::kWave;
  // when the other waves cannot cover x in one pass, every wave but the union
  // builder takes a share (the routing and router waves after their own work)
  const bool xq_all = totx8 > (long)qthreads;
  const bool qwave = wv >= nrt && wv < kWaves - nrw - nub;
  const int nq = xq_all ? kThreads - nub * pq::kWave : qthreads;
  const int tq = xq_all ? ((int)threadIdx.x < nq ? (int)threadIdx.x : -1)
                        : (qwave ? (int)threadIdx.x - nrt * pq::kWave : -1);
  const pq::rsrc_t xr = pq::make_rsrc(a.x, (uint32_t)(a.M * H * 2));
  // enough loads in flight for the whole of x at H = 6144 up to M = 4 (16 bytes each)
  constexpr int kXPre = TP == 1 ? 1 : TP == 2 ? 2 : TP == 4 ? 4 : 8;
  uint4 xraw[kXPre];
#pragma unroll
  for (int it = 0; it < kXPre; ++it) {
    const long t = (long)it * nq + tq;
    xraw[it] = pq::buf_load16(xr, tq >= 0 && t < totx8 ? (uint32_t)t * 16u : pq::kOOB);
  }
  if (threadIdx.x < kMaxM * kMaxE / 32) (&s_tmask[0][0])[threadIdx.x] = 0u;
  if (threadIdx.x == 0) {
    *s_ready = router ? 0u : 1u;
    *s_rdone = 0u;
    // until the union is built, only the shared entry (set up below) is known;
    // a wave whose wait for the routes timed out sees exactly that
    route.nitems = sh * a.M;
    route.nU = sh;
  }
  if (sh && wv == 0) shared_entry(a, route);
  if (early_union) __syncthreads();   // the words above set before any routing wave counts itself done

  // ---- A. routing from given logits (waves 0..M-1, one token each), or the
  //      router rows ---------------------------------------------------------
  if (router) {
    const int k = kWaves - 1 - wv;
    if (k < nrw)
      for (int e = e0 + k; e < e1; e += nrw) router_rows<TP>(a, e);
  } else if (a.routed) {
    if (wv < a.M) {
      if (a.E <= 256) route_token<4, false>(a, route, wv);
      else route_token<16, false>(a, route, wv);
      if (one_token) single_token_union(a, route, sh);
      else if (lane == 0) __hip_atomic_fetch_add(s_rdone, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (early_union && wv == kWaves - 1) {
      const uint32_t nm = (uint32_t)a.M;
      lds_wait(s_rdone, [nm](uint32_t v) { return v >= nm; }, hdr);
      // (after a timeout the routes stay the shared entry's alone)
      if ((uint32_t)ufl((int)__hip_atomic_load(s_rdone, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) >= nm)
        build_union(a, route, hdr, s_tmask, sh);
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
      const float sc = pq::fp8_block_scale16(v, valid);
      if (valid) {
        reinterpret_cast<uint2*>(xa)[t] = pq::fp8_codes8(v, sc);
        if ((tq & 15) == 0) xsc[(t * 8) / pq::kBlock] = sc;
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

  __syncthreads();                            // the quantised x (and given routes) visible
  if (router) {
    // routing waves: wait for every block's logits and rank them; wave 0 then
    // builds the union once all of them are done and releases the routes
    if (wv < a.M) {
      if (a.E <= 256) route_token<4, true>(a, route, wv);
      else route_token<16, true>(a, route, wv);
      if (one_token) {
        single_token_union(a, route, sh);
        if (lane == 0) __hip_atomic_store(s_ready, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else {
        if (lane == 0) __hip_atomic_fetch_add(s_rdone, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (wv == 0) {
          const uint32_t nm = (uint32_t)a.M;
          lds_wait(s_rdone, [nm](uint32_t v) { return v >= nm; }, hdr);
          build_union(a, route, hdr, s_tmask, sh);
          if (lane == 0) __hip_atomic_store(s_ready, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    }
  } else if (!one_token && !early_union) {
    if (wv == 0) build_union(a, route, hdr, s_tmask, sh);
    __syncthreads();
  }
}

// The last block hands the call's recorded status to the caller when asked
// (and clears the record, so every call reports its own).  Every block's waves
// made their memory operations complete before the block counted itself out,
// so every error of the call is recorded by now.
__device__ __forceinline__ void report_status(const MoeArgs& a, pq::WsHeader* hdr) {
  if (a.status_out)
    *a.status_out = (int32_t)__hip_atomic_exchange(&hdr->error, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait (wave-wide, bounded) until the routes of the call are visible.
__device__ __forceinline__ void wait_routes(const uint32_t* s_ready, pq::WsHeader* hdr) {
  lds_wait(s_ready, [](uint32_t v) { return v != 0u; }, hdr);
}

// The barrier kernel: all gate_up units of the call, then every block stages
// all of h (waiting for the rows of slower blocks value by value: a barrier on
// the data itself) and runs its down rows.  Fewer instructions per step than
// the stream kernel below, which pays off when the call streams few experts
// (one token).
// TP: compile-time bound on the (token, slot) pairs routed to one expert in a
// call (the smallest power of two >= M), so the per-pair loops unroll tightly.
template <int TP, bool EXT>
__global__ __launch_bounds__(kThreads) void moe_barrier_kernel(MoeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ Route route;
  __shared__ int s_last;
  __shared__ uint32_t s_tmask[kMaxM][kMaxE / 32];   // routed-expert bitmap of each token
  __shared__ uint32_t s_next;     // next gate_up unit of this block
  __shared__ uint32_t s_ready;    // routes visible (set by the routing waves)
  __shared__ uint32_t s_rdone;    // routing waves done

  pq::WsHeader* hdr = reinterpret_cast<pq::WsHeader*>(a.ws);

  const int lane = pq::lane_id();
  const int wv = pq::wave_id();
  const int gw = ufl((int)blockIdx.x * kWaves + wv);
  const long T = (long)gridDim.x * kWaves;
  const int H = a.H, I = a.I, K = a.top_k;
  const int P = a.M * K;
  const int sh = EXT ? a.sh : 0;              // shared expert: union entry 0, pairs P .. P + M - 1
  const int P2 = EXT ? a.P2 : P;
  const bool router = EXT && a.router;
  const int nbH = H / pq::kBlock, nbI = I / pq::kBlock;
  const int nchH = (H + pq::kChunk - 1) / pq::kChunk;
  const int nchI = (I + pq::kChunk - 1) / pq::kChunk;
  const uint32_t lane16 = 16u * (uint32_t)lane;
  const uint32_t lane_blk4 = 4u * ((uint32_t)lane >> 3);

  uint8_t* act = smem;                                           // x codes, later h codes
  float* acts = reinterpret_cast<float*>(smem + a.xs_off);       // their scales

  if (threadIdx.x == 0) {       // block counters; first used after the barriers below
    s_next = 0u;
  }
  layer_prologue<TP, EXT>(a, route, s_tmask, &s_ready, &s_rdone, act, acts, hdr);

  // ---- C. gate_up + SiLU*up -------------------------------------------------
  // Units (union entry u, h-row i: one gate row and one up row) are numbered
  // u * I + i.  The block owns its share [sh0, sh0 + nsh) of the shared
  // expert's units (entry 0; independent of the routing, so they go first)
  // and its share [bu0, bu1) of the routed units (known once the routes are);
  // its waves take them one at a time from an LDS counter, so a wave whose
  // loads issue later (the scheduler favours older waves) simply takes fewer.
  // Each wave keeps BDG chunk-steps in flight; every ring slot remembers its
  // unit and chunk.
  const int sh0 = pq::split_start(sh * I, (int)gridDim.x, (int)blockIdx.x);
  const int nsh = pq::split_start(sh * I, (int)gridDim.x, (int)blockIdx.x + 1) - sh0;
  int bu0 = 0, bu1 = 0, nU = sh;
  bool routes_known = false;
  auto know_routes = [&]() {
    if (!routes_known) {
      if (router) wait_routes(&s_ready, hdr);
      nU = routes_nU(route);
      const int nur = nU - sh;
      bu0 = pq::split_start(nur * I, (int)gridDim.x, (int)blockIdx.x);
      bu1 = pq::split_start(nur * I, (int)gridDim.x, (int)blockIdx.x + 1);
      routes_known = true;
    }
  };
  if (!router) know_routes();         // the routes are visible already

  // Block scales: with the LDS windows (sc_off >= 0) a unit's gate and up
  // rows' scales arrive by one buffer-to-LDS load each when the unit is
  // taken (before its weight loads, so they have landed once the step's
  // weights have) and each step reads its 8 from LDS; otherwise each step
  // loads them with its weights.
  const bool scw = a.sc_off >= 0;
  const uint32_t wbase = scw ? pq::lds_addr(smem + a.sc_off + (size_t)wv * kScWaveBytes) : 0u;
  uint4 wb[BDG][2];
  float sb[BDG][2];
  uint32_t sa[BDG];                   // LDS address of the step's gate-row scales (windows)
  int su[BDG], sch[BDG];              // unit (-1: none) and chunk of each slot
  int iunit = -1, ic = nchH;          // issue cursor
  bool more = true;
  int cur_e = -1, gseq = 0;
  pq::rsrc_t gwr = pq::make_rsrc(a.w13, 0u), gsr = pq::make_rsrc(a.s13, 0u);
  pq::int32x4 gsr4 = {0, 0, 0, 0};
  auto issue_gu = [&](uint4 (&w)[2], float (&s)[2], uint32_t& sa_q, int& su_q, int& sch_q) {
    if (ic == nchH && more) {       // take the block's next unit
      const int c = wave_claim(&s_next);
      if (c < nsh) {
        iunit = sh0 + c;
      } else {
        know_routes();
        const int r = bu0 + (c - nsh);
        more = r < bu1;
        iunit = sh * I + r;
      }
      ic = 0;
      if (more) {
        const int e = ufl(route.uexp[iunit / I]);
        if (e != cur_e) {
          cur_e = e;
          gwr = pq::make_rsrc(gu_weights<EXT>(a, e), (uint32_t)(2 * I * H));
          gsr = pq::make_rsrc(gu_scales<EXT>(a, e), (uint32_t)(2 * I * nbH * 4));
          if (scw) gsr4 = pq::rsrc_words(gu_scales<EXT>(a, e), (uint32_t)(2 * I * nbH * 4));
        }
        if (scw) {                     // the unit's two scale rows into windows 2g, 2g + 1
          gseq = (gseq + 1) & 3;
          const uint32_t ii0 = (uint32_t)(iunit - (iunit / I) * I);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            pq::dma4_keep_m0(gsr4, wbase + (uint32_t)((2 * gseq + j) * kWinFloats * 4),
                             lane < nbH ? ((ii0 + (uint32_t)(j * I)) * (uint32_t)nbH + (uint32_t)lane) * 4u : pq::kOOB,
                             0u);
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
      s[j] = scw ? 0.0f
                 : pq::buf_load_f32_nt(gsr, ok ? (row * (uint32_t)nbH + kc / pq::kBlock) * 4u + lane_blk4 : pq::kOOB);
    }
    sa_q = wbase + (uint32_t)((2 * gseq * kWinFloats + ic * (pq::kChunk / pq::kBlock)) * 4);
    su_q = more ? iunit : -1;
    sch_q = ic;
    if (more) ++ic;
  };
#pragma unroll
  for (int q = 0; q < BDG; ++q) issue_gu(wb[q], sb[q], sa[q], su[q], sch[q]);


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
        pm[t] = pr[t] < P ? pr[t] / K : pr[t] - P;   // the shared expert's pair P + m is token m
      }
    };
    for (;;) {
#pragma unroll
      for (int q = 0; q < BDG; ++q) {
        if (su[q] >= 0) {
          const int unit = su[q], cc = sch[q];
          const int uu = unit / I, ci = unit - (unit / I) * I;
          if (uu != pairs_u) load_pairs(uu);
          const uint32_t off = (uint32_t)(cc * pq::kChunk) + lane16;
          if (off < (uint32_t)H) {
            float sg = sb[q][0], sv = sb[q][1];
            if (scw)
              pq::lds_read2_after(sa[q] + lane_blk4, sa[q] + kWinFloats * 4 + lane_blk4, wb[q][0].x, sg, sv);
            const pq::Bf16x16 wg = pq::widen16(wb[q][0]);
            const pq::Bf16x16 wu = pq::widen16(wb[q][1]);
#pragma unroll
            for (int t = 0; t < TP; ++t) {
              if (t < cnp) {
                const pq::Bf16x16 xv = pq::widen16(*reinterpret_cast<const uint4*>(act + (size_t)pm[t] * H + off));
                const float xs = acts[pm[t] * nbH + off / pq::kBlock];
                accg[t] = fmaf(pq::dot16(wg, xv), sg * xs, accg[t]);
                accu[t] = fmaf(pq::dot16(wu, xv), sv * xs, accu[t]);
              }
            }
          }
          if (cc == nchH - 1) {            // unit done: h for every routed token
            float gs[TP], us[TP];
            pq::wave_sum_pairs<TP>(accg, accu, cnp, gs, us);
#pragma unroll
            for (int t = 0; t < TP; ++t) {
              if (t < cnp && lane == 0) {
                uint16_t hb = pq::bf16_rne(silu_mul(gs[t], us[t]));
                if (hb == 0xFFFFu) hb = 0xFFC0u;           // keep the inverted word non-zero
                pq::st_agent_u16(a.hbuf + (size_t)pr[t] * I + ci, (uint16_t)~hb);
                if (a.h_dbg) a.h_dbg[(size_t)pr[t] * I + ci] = hb;
              }
              accg[t] = accu[t] = 0.0f;
            }
          }
        }
        issue_gu(wb[q], sb[q], sa[q], su[q], sch[q]);
      }
      bool busy = false;
#pragma unroll
      for (int q = 0; q < BDG; ++q) busy |= su[q] >= 0;
      if (!busy) break;
    }
  }

  know_routes();                      // (every wave's last claim already waited)

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
  // Short rows (I = 128, 256 or 512: one chunk) are packed: a step carries
  // pr_rows = 64 / (I / 16) consecutive rows of one entry, lane segment k
  // holding row k, so the lanes of a step are not mostly idle; a row's sum is
  // reduced inside its segment by the first stages of the wave-wide sum, the
  // same additions in the same order as for a row alone in the wave.
  const int lpr = I / 16;                            // lanes per row
  const bool packed = nchI == 1 && (I == 128 || I == 256 || I == 512);
  float* ybuf = reinterpret_cast<float*>(smem + a.yb_off);   // [row_local][P] fp32
  // The two forms are separate instantiations, so the unpacked steps carry
  // none of the packed bookkeeping.
  // Unpacked, a step carries two consecutive rows of one entry (kR loads per
  // lane, the pair's h read and widened once for both), in a ring of half the
  // depth: the same bytes in flight.
  auto down_phase = [&](auto packed_c) {
    constexpr bool kP = decltype(packed_c)::value;
    constexpr int kR = kP ? 1 : 2;                 // row loads per lane and step
    constexpr int RD = kP ? BDD : BDD / 2;         // ring depth in steps
    const int pr_rows = kP ? pq::kWave / lpr : kR; // rows per step
    const int prr = kP ? lane / lpr : 0;           // this lane's row in a packed step
    const uint32_t plk16 = kP ? 16u * (uint32_t)(lane % lpr) : lane16;
    int dsteps = 0;                                // per entry: ceil(rows / pr_rows) row steps
    for (int u = v0; u < v1;) {
      const int e_end = (u / nrows + 1) * nrows;
      const int n = (v1 < e_end ? v1 : e_end) - u;
      dsteps += (n + pr_rows - 1) / pr_rows * (kP ? 1 : nchI);
      u += n;
    }
    // (the down steps keep their per-step scale loads: a down step does half
    // a gate_up step's work, and an LDS read in its dependency chain measured
    // slower than the load that arrives with the weights)
    uint4 wd[RD][kR];
    float sd[RD][kR];
    int ju = nrows > 0 ? v0 / nrows : 0;
    int jr = v0 - ju * nrows, jc = 0, dleft = dsteps, uleft = v1 - v0;
    pq::rsrc_t dwr, dsr;
    auto set_dn_expert = [&]() {
      const int e = ufl(route.uexp[ju < nU ? ju : 0]);
      dwr = pq::make_rsrc(dn_weights<EXT>(a, e), (uint32_t)(H * I));
      dsr = pq::make_rsrc(dn_scales<EXT>(a, e), (uint32_t)(H * nbI * 4));
    };
    set_dn_expert();
    auto issue_dn = [&](uint4 (&w)[kR], float (&s)[kR]) {
      const uint32_t kc = (uint32_t)(jc * pq::kChunk);
      int nr = nrows - jr < uleft ? nrows - jr : uleft;   // rows of this step
      nr = nr < pr_rows ? nr : pr_rows;
#pragma unroll
      for (int j = 0; j < kR; ++j) {
        const int rj = kP ? prr : j;                   // this lane's row of the step
        const bool ok = dleft > 0 && rj < nr && kc + plk16 < (uint32_t)I;
        const uint32_t row = (uint32_t)(r0 + jr + rj);
        w[j] = pq::buf_load16_nt(dwr, ok ? row * (uint32_t)I + kc + plk16 : pq::kOOB);
        const uint32_t soff = kP ? (row * (uint32_t)nbI + plk16 / pq::kBlock) * 4u
                                 : (row * (uint32_t)nbI + kc / pq::kBlock) * 4u + lane_blk4;
        s[j] = pq::buf_load_f32_nt(dsr, ok ? soff : pq::kOOB);
      }
      --dleft;
      if (kP || ++jc == nchI) {                      // (packed rows are one chunk)
        jc = 0;
        uleft -= nr;
        jr += nr;
        if (jr == nrows) {
          jr = 0;
          ++ju;
          set_dn_expert();
        }
      }
    };
#pragma unroll
    for (int q = 0; q < RD; ++q) issue_dn(wd[q], sd[q]);

    // Every h row of the call, quantised into LDS as soon as it is there: h
    // is stored bit-inverted into a region that is zero between calls, so a
    // zero word is a value not yet written.  The h codes overwrite the x codes,
    // so the block first waits for all its waves to be past gate_up; then each
    // wave polls its share (only the vectors still missing are loaded again)
    // while the last gate_up units of slower blocks finish.  Every block derives
    // the same codes and scales from the same values (block 0 also writes them
    // out when asked).
    __syncthreads();
    {
      // 8 values per lane, 16 lanes per 128-value block (the layout of the
      // activation quantiser); agent-coherent 16-byte loads, a batch in flight
      const int nvec = P2 * I / 8;
      const pq::rsrc_t hr = pq::make_rsrc(a.hbuf, (uint32_t)(P2 * I * 2));
      constexpr int kBatch = 2;
      for (int t0 = 0; t0 < nvec; t0 += kBatch * kThreads) {
        uint4 raw[kBatch];
        bool have[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          have[i] = t0 + i * kThreads + (int)threadIdx.x >= nvec;
          raw[i] = make_uint4(0u, 0u, 0u, 0u);
        }
        for (uint32_t it = 0;; ++it) {
          bool miss = false;
#pragma unroll
          for (int i = 0; i < kBatch; ++i) {
            const int t = t0 + i * kThreads + (int)threadIdx.x;
            const uint4 r = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                hr, (int)(have[i] ? pq::kOOB : (uint32_t)t * 16u), 0, kAuxSC1));
            if (!have[i]) {
              raw[i] = r;
              have[i] = !(has_zero_half(r.x) || has_zero_half(r.y) || has_zero_half(r.z) || has_zero_half(r.w));
            }
            miss |= !have[i];
          }
          if (__ballot(miss) == 0ull) break;
          if (it >= a.spin_limit) {
            if (lane == 0) pq::record_error(hdr, PQ_ERR_TIMEOUT);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const int t = t0 + i * kThreads + (int)threadIdx.x;
          const bool valid = t < nvec;
          raw[i] = make_uint4(~raw[i].x, ~raw[i].y, ~raw[i].z, ~raw[i].w);
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
      float acc[kR][TP];
      int pr[TP];
#pragma unroll
      for (int j = 0; j < kR; ++j)
#pragma unroll
        for (int t = 0; t < TP; ++t) acc[j][t] = 0.0f;
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
      int cleft = v1 - v0;
      auto consume_dn = [&](const uint4 (&w)[kR], const float (&sw)[kR]) {
        int nr = nrows - cr < cleft ? nrows - cr : cleft;
        nr = nr < pr_rows ? nr : pr_rows;
        const uint32_t off = (uint32_t)(cc * pq::kChunk) + plk16;
        if (prr < nr && off < (uint32_t)I) {
          pq::Bf16x16 wv[kR];
#pragma unroll
          for (int j = 0; j < kR; ++j) wv[j] = pq::widen16(w[j]);
#pragma unroll
          for (int t = 0; t < TP; ++t) {
            if (t < cnp) {
              const pq::Bf16x16 hv = pq::widen16(*reinterpret_cast<const uint4*>(act + (size_t)pr[t] * I + off));
              const float hsc = acts[pr[t] * nbI + off / pq::kBlock];
#pragma unroll
              for (int j = 0; j < kR; ++j) acc[j][t] = fmaf(pq::dot16(wv[j], hv), sw[j] * hsc, acc[j][t]);
            }
          }
        }
        if (kP || cc == nchI - 1) {         // unit(s) (union entry cu, rows cr ..) done
          if constexpr (kP) {
#pragma unroll
            for (int t = 0; t < TP; ++t) {
              if (t < cnp) {                          // every lane of a segment holds its row's sum
                const float y = pq::segment_sum_xor(acc[0][t], lpr);
                if (lane % lpr == lpr - 1 && prr < nr) ybuf[(cr + prr) * P2 + pr[t]] = y;
              }
              acc[0][t] = 0.0f;
            }
          } else {                                    // rows cr and cr + 1 of every pair in one butterfly
            float y0[TP], y1[TP];
            pq::wave_sum_pairs<TP>(acc[0], acc[kR - 1], cnp, y0, y1);
#pragma unroll
            for (int t = 0; t < TP; ++t) {
              if (t < cnp && lane == 0) {
                ybuf[cr * P2 + pr[t]] = y0[t];
                if (nr > 1) ybuf[(cr + 1) * P2 + pr[t]] = y1[t];
              }
#pragma unroll
              for (int j = 0; j < kR; ++j) acc[j][t] = 0.0f;
            }
          }
        }
        if (kP || ++cc == nchI) {
          cc = 0;
          cleft -= nr;
          cr += nr;
          if (cr == nrows) {
            cr = 0;
            ++cu;
            load_pairs();
          }
        }
      };
      int base = 0;
      for (; base + RD < dsteps; base += RD) {       // steady state: every slot refills
#pragma unroll
        for (int q = 0; q < RD; ++q) {
          consume_dn(wd[q], sd[q]);
          issue_dn(wd[q], sd[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < RD; ++q)                  // drain
        if (base + q < dsteps) consume_dn(wd[q], sd[q]);
    }
  };
  if (packed)
    down_phase(pq::BoolC<true>{});
  else
    down_phase(pq::BoolC<false>{});
  __syncthreads();
  for (int idx = threadIdx.x; idx < (r1 - r0) * a.M; idx += kThreads) {
    const int rl = idx / a.M, m = idx - (idx / a.M) * a.M;
    float o = 0.0f;
    for (int j = 0; j < K; ++j) o = fmaf(route.w[m * K + j], ybuf[rl * P2 + m * K + j], o);
    if (sh) o += ybuf[rl * P2 + P + m];              // the shared expert, weight 1, last
    a.out[(size_t)m * H + r0 + rl] = pq::bf16_rne(o);
  }

  // ---- E. the last block to finish clears h for the next call ----------------
  // A block counts itself out once it has read every h value (so every h
  // store of the call has landed) and its own stores are complete: the
  // clearing stores below are the last writes to h.
  pq::wait_vm();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = pq::atomic_add_relaxed(&hdr->exit_count, 1u);
    s_last = old == gridDim.x - 1;
  }
  __syncthreads();
  if (s_last) {
    const pq::rsrc_t hr = pq::make_rsrc(a.hbuf, (uint32_t)(P2 * I * 2));
    const int nz = P2 * I / 8;
    for (int t = threadIdx.x; t < nz; t += kThreads)
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, hr, t * 16, 0, kAuxSC1);
    if (router)
      for (int t = threadIdx.x; t < a.M * a.E; t += kThreads) pq::st_agent_u32(a.lx + t, 0u);
    if (threadIdx.x == 0) {
      pq::atomic_store_relaxed(&hdr->exit_count, 0u);
      report_status(a, hdr);
    }
  }
}

// The stream kernel: no grid-wide barrier; see section C.
// TP: compile-time bound on the (token, slot) pairs routed to one expert in a
// call (the smallest power of two >= M), so the per-pair loops unroll tightly.
template <int TP, bool EXT>
__global__ __launch_bounds__(kThreads) void moe_stream_kernel(MoeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ Route route;
  __shared__ int s_last;
  __shared__ uint32_t s_tmask[kMaxM][kMaxE / 32];   // routed-expert bitmap of each token
  __shared__ uint32_t s_iclaim;              // staging items of the block claimed
  __shared__ uint32_t s_staged[kMaxUnion];  // pairs of union entry u whose h codes are in LDS
  __shared__ uint32_t s_next;      // gate_up units of this block handed out
  __shared__ uint32_t s_dnext;     // down units of this block handed out
  __shared__ uint32_t s_gu_busy;   // waves still consuming gate_up steps
  __shared__ uint32_t s_ready;     // routes visible (set by the routing waves)
  __shared__ uint32_t s_rdone;     // routing waves done

  pq::WsHeader* hdr = reinterpret_cast<pq::WsHeader*>(a.ws);

  const int lane = pq::lane_id();
  const int wv = pq::wave_id();
  const int H = a.H, I = a.I, K = a.top_k;
  const int P = a.M * K;
  const int sh = EXT ? a.sh : 0;              // shared expert: union entry 0, pairs P .. P + M - 1
  const int P2 = EXT ? a.P2 : P;
  const bool router = EXT && a.router;
  const int nbH = H / pq::kBlock, nbI = I / pq::kBlock;
  const int nchH = (H + pq::kChunk - 1) / pq::kChunk;
  const uint32_t lane16 = 16u * (uint32_t)lane;
  const uint32_t lane_blk4 = 4u * ((uint32_t)lane >> 3);

  // Unit-end sums: with several pairs per unit the lanes that hold them store
  // them (the sums stay out of scalar registers; M=8 260.9 against 265.9 µs);
  // with the router and shared expert in the launch, whose registers are at
  // their limit, lane 0 reads them back (M=4 212.5 against 222 µs)
  constexpr bool kLaneStores = TP > 1 && !EXT;
  uint8_t* xa = smem + a.xa_off;                               // x codes   [M][H]
  float* xsc = reinterpret_cast<float*>(smem + a.xs_off);      // x scales  [M][H/128]
  uint8_t* ha = smem + a.ha_off;                               // h codes   [nitems][I] by staging slot
  float* hsc = reinterpret_cast<float*>(smem + a.hs_off);      // h scales  [P2][I/128]
  float* ybuf = reinterpret_cast<float*>(smem + a.yb_off);     // y partials [row][P2]

  if (threadIdx.x == 0) {       // block counters; first used after the barriers below
    s_next = 0u;
    s_dnext = 0u;
    s_iclaim = 0u;
    s_gu_busy = (uint32_t)kWaves;
  }
  if (threadIdx.x < kMaxUnion) s_staged[threadIdx.x] = 0u;
  layer_prologue<TP, EXT>(a, route, s_tmask, &s_ready, &s_rdone, xa, xsc, hdr);

  // ---- C. per wave: gate_up units, then down units, no block barrier -------
  // gate_up unit (union entry u, h-row i) = gate row i and up row i of expert
  // u.  Unit k of this block is entry blockIdx.x + k * gridDim.x of the
  // expert-major list, so every block works through the experts in union
  // order and the h of the first experts is complete early.  down unit (u,
  // output row n), n among this block's rows, taken expert by expert.  Waves
  // take units from LDS counters (a wave whose loads issue later simply takes
  // fewer); a wave out of gate_up units goes on with down units at once while
  // other waves and other blocks still finish gate_up.  The h a down unit
  // needs is quantised into LDS by the first wave that needs it (per pair),
  // once every block has stored it: the stager polls the values themselves,
  // which are stored bit-inverted so that a zero word means "not yet written".
  // The shared expert is entry 0, so its units are the first I of the list and
  // need no routes; a wave that reaches the routed units waits for them.
  const int G = (int)gridDim.x;
  int gu_total = sh * I;               // the whole list once the routes are known
  int nU = sh;
  bool routes_known = false;
  auto know_routes = [&]() {
    if (!routes_known) {
      if (router) wait_routes(&s_ready, hdr);
      nU = routes_nU(route);
      gu_total = nU * I;
      routes_known = true;
    }
  };
  if (!router) know_routes();         // the routes are visible already
  const int r0 = pq::split_start(H, G, (int)blockIdx.x);
  const int r1 = pq::split_start(H, G, (int)blockIdx.x + 1);
  const int nrows = r1 - r0;
  const int nchI = (I + pq::kChunk - 1) / pq::kChunk;

  // gate_up: a ring of DG steps (one 1 KB chunk of the gate row and of the up
  // row); a slot descriptor holds valid (bit 31) | step | union entry | row.
  {
    uint4 wb[DG][2];
    float sb[DG][2];
    uint32_t sd[DG];
    int ucur = 0, crow = 0, cstep = nchH, ce = -1;
    bool more = true;
    pq::rsrc_t wr = pq::make_rsrc(a.w13, 0u), sr = pq::make_rsrc(a.s13, 0u);
    auto issue_gu = [&](uint4 (&w)[2], float (&s)[2], uint32_t& d) {
      if (cstep == nchH && more) {            // take the block's next unit
        const int v = (int)blockIdx.x + wave_claim(&s_next) * G;
        if (v >= sh * I) know_routes();
        more = v < gu_total;
        if (more) {
          ucur = v / I;
          crow = v - ucur * I;
          cstep = 0;
          const int e = ufl(route.uexp[ucur]);
          if (e != ce) {
            ce = e;
            wr = pq::make_rsrc(gu_weights<EXT>(a, e), (uint32_t)(2 * I * H));
            sr = pq::make_rsrc(gu_scales<EXT>(a, e), (uint32_t)(2 * I * nbH * 4));
          }
        }
      }
      const uint32_t kc = (uint32_t)(cstep * pq::kChunk);
      const bool ok = more && kc + lane16 < (uint32_t)H;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t row = (uint32_t)(crow + j * I);
        w[j] = pq::buf_load16_nt(wr, ok ? row * (uint32_t)H + kc + lane16 : pq::kOOB);
        s[j] = pq::buf_load_f32_nt(sr, ok ? (row * (uint32_t)nbH + kc / pq::kBlock) * 4u + lane_blk4 : pq::kOOB);
      }
      d = more ? 0x80000000u | ((uint32_t)cstep << 23) | ((uint32_t)ucur << 16) | (uint32_t)crow : 0u;
      if (more) ++cstep;
    };

    float accg[TP], accu[TP];
    int pr[TP], pm[TP];
#pragma unroll
    for (int t = 0; t < TP; ++t) accg[t] = accu[t] = 0.0f;
    int pairs_u = -1, cnp = 0;
    auto consume_gu = [&](const uint4 (&w)[2], const float (&s)[2], uint32_t d) {
      if (!(d >> 31)) return;
      const int step = (int)((d >> 23) & 255u), uu = (int)((d >> 16) & 127u), row = (int)(d & 0xFFFFu);
      if (uu != pairs_u) {
        pairs_u = uu;
        cnp = ufl(route.unp[uu]);
#pragma unroll
        for (int t = 0; t < TP; ++t) {
          pr[t] = ufl(route.upairs[uu][t]);
          pm[t] = pr[t] < P ? pr[t] / K : pr[t] - P;   // the shared expert's pair P + m is token m
        }
      }
      const uint32_t off = (uint32_t)(step * pq::kChunk) + lane16;
      if (off < (uint32_t)H) {
        const pq::Bf16x16 wg = pq::widen16(w[0]);
        const pq::Bf16x16 wu = pq::widen16(w[1]);
#pragma unroll
        for (int t = 0; t < TP; ++t) {
          if (t < cnp) {
            const pq::Bf16x16 xv = pq::widen16(*reinterpret_cast<const uint4*>(xa + (size_t)pm[t] * H + off));
            const float xs = xsc[pm[t] * nbH + off / pq::kBlock];
            accg[t] = fmaf(pq::dot16(wg, xv), s[0] * xs, accg[t]);
            accu[t] = fmaf(pq::dot16(wu, xv), s[1] * xs, accu[t]);
          }
        }
      }
      if (step == nchH - 1) {            // unit done: h for every token routed to u
        if constexpr (kLaneStores) {
          // lane 2t: pair t's gate sum; its up sum comes from lane 2t + 1, its
          // pair index from the union table, and the lane stores its h itself
          const float gsum = pq::wave_sum_pairs_lanes<TP>(accg, accu, cnp);
          const float usum = pq::xor_lane<1>(gsum);
          const int tl = lane >> 1;
          if ((lane & 1) == 0 && tl < cnp) {
            const int p = route.upairs[uu][tl];
            uint16_t hb = pq::bf16_rne(silu_mul(gsum, usum));
            if (hb == 0xFFFFu) hb = 0xFFC0u;           // keep the inverted word non-zero
            pq::st_agent_u16(a.hbuf + (size_t)p * I + row, (uint16_t)~hb);
            if (a.h_dbg) a.h_dbg[(size_t)p * I + row] = hb;
          }
#pragma unroll
          for (int t = 0; t < TP; ++t) accg[t] = accu[t] = 0.0f;
        } else {
          float gs[TP], us[TP];
          pq::wave_sum_pairs<TP>(accg, accu, cnp, gs, us);
#pragma unroll
          for (int t = 0; t < TP; ++t) {
            if (t < cnp && lane == 0) {
              uint16_t hb = pq::bf16_rne(silu_mul(gs[t], us[t]));
              if (hb == 0xFFFFu) hb = 0xFFC0u;         // keep the inverted word non-zero
              pq::st_agent_u16(a.hbuf + (size_t)pr[t] * I + row, (uint16_t)~hb);
              if (a.h_dbg) a.h_dbg[(size_t)pr[t] * I + row] = hb;
            }
            accg[t] = accu[t] = 0.0f;
          }
        }
      }
    };

#pragma unroll
    for (int q = 0; q < DG; ++q) issue_gu(wb[q], sb[q], sd[q]);
    for (;;) {
#pragma unroll
      for (int q = 0; q < DG; ++q) {
        consume_gu(wb[q], sb[q], sd[q]);
        issue_gu(wb[q], sb[q], sd[q]);
      }
      uint32_t busy = 0u;
#pragma unroll
      for (int q = 0; q < DG; ++q) busy |= sd[q];
      if (busy == 0u) break;
    }
  }
  if (lane == 0) atomicSub(&s_gu_busy, 1u);   // this wave no longer reads x
  know_routes();                               // (its last claim already waited)
  const int nrp = (nrows + kDnRows - 1) / kDnRows;   // down units: kDnRows consecutive rows of one entry
  const int dn_total = nU * nrp;

  // h staging: the (entry, pair) items of the block are quantised into LDS in
  // union order, each by the wave that claims it; a wave out of gate_up units
  // claims items until none is left, then goes on with down units.
  {
    // (a routed union always has more entries than the shared one: nU == sh
    // only if the wait for the routes ended early, and then only the shared
    // entry's items are known)
    const int nitems = nU > sh ? ufl(route.nitems) : sh * a.M;
    for (;;) {
      const int jj = wave_claim(&s_iclaim);
      if (jj >= nitems) break;
      const int it = ufl(route.items[jj]);
      const int v = it & 255, t = it >> 8;
      if (a.alias && jj >= a.hsplit)   // these h codes overwrite x codes: the block must be past gate_up
        lds_wait(&s_gu_busy, [](uint32_t v) { return v == 0u; }, hdr);
      stage_pair(a, route, hdr, v, t, ha + (size_t)jj * I, hsc);
      if (lane == 0) __hip_atomic_fetch_add(&s_staged[v], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }

  // down: a ring of DD steps (one 1 KB chunk of a down row); a cycle's slots
  // are consumed once the h of their union entries is in LDS.
  {
    // A down step carries kDnRows consecutive rows of one union entry: every
    // lane loads the same 16 bytes of each and reads and widens each pair's
    // h once for all of them, which divides the LDS reads and h conversions
    // per weight byte where several tokens share an expert.  Each row's sums
    // are the same additions in the same order as for a row alone, so the
    // results equal the barrier kernel's bit for bit.
    uint4 wd[DD][kDnRows];
    float sw[DD][kDnRows];
    uint32_t sd[DD];
    int ucur = 0, crow = 0, cstep = nchI, ce = -1;
    bool more = true;
    pq::rsrc_t wr = pq::make_rsrc(a.w2, 0u), sr = pq::make_rsrc(a.s2, 0u);
    // a claim takes kDnClaim consecutive units (row groups of one entry,
    // mostly): one LDS round trip per few rows instead of per row
    int dk_left = 0, dk_base = 0;
    auto issue_dn = [&](uint4 (&w)[kDnRows], float (&s)[kDnRows], uint32_t& d) {
      if (cstep == nchI && more) {            // take the block's next unit
        if (dk_left == 0) {
          dk_base = kDnClaim * wave_claim(&s_dnext);
          dk_left = kDnClaim;
        }
        const int tt = dk_base + (kDnClaim - dk_left);
        --dk_left;
        more = tt < dn_total;
        if (more) {
          ucur = tt / nrp;
          crow = kDnRows * (tt - ucur * nrp);
          cstep = 0;
          const int e = ufl(route.uexp[ucur]);
          if (e != ce) {
            ce = e;
            wr = pq::make_rsrc(dn_weights<EXT>(a, e), (uint32_t)(H * I));
            sr = pq::make_rsrc(dn_scales<EXT>(a, e), (uint32_t)(H * nbI * 4));
          }
        }
      }
      const uint32_t kc = (uint32_t)(cstep * pq::kChunk);
      const bool ok = more && kc + lane16 < (uint32_t)I;
#pragma unroll
      for (int j = 0; j < kDnRows; ++j) {
        const bool okj = ok && crow + j < nrows;
        const uint32_t row = (uint32_t)(r0 + crow + j);
        w[j] = pq::buf_load16_nt(wr, okj ? row * (uint32_t)I + kc + lane16 : pq::kOOB);
        s[j] = pq::buf_load_f32_nt(sr, okj ? (row * (uint32_t)nbI + kc / pq::kBlock) * 4u + lane_blk4 : pq::kOOB);
      }
      d = more ? 0x80000000u | ((uint32_t)cstep << 23) | ((uint32_t)ucur << 16) | (uint32_t)crow : 0u;
      if (more) ++cstep;
    };

    float acc[kDnRows][TP];
    int pr[TP];
#pragma unroll
    for (int j = 0; j < kDnRows; ++j)
#pragma unroll
      for (int t = 0; t < TP; ++t) acc[j][t] = 0.0f;
    int pairs_u = -1, cnp = 0, s0 = 0, ready_next = 0;
    auto consume_dn = [&](const uint4 (&w)[kDnRows], const float (&s)[kDnRows], uint32_t d) {
      if (!(d >> 31)) return;
      const int step = (int)((d >> 23) & 255u), uu = (int)((d >> 16) & 127u), row = (int)(d & 0xFFFFu);
      if (uu != pairs_u) {
        pairs_u = uu;
        cnp = ufl(route.unp[uu]);
        s0 = ufl(route.ustart[uu]);            // the entry's staging slots s0 .. s0 + cnp - 1
#pragma unroll
        for (int t = 0; t < TP; ++t) pr[t] = ufl(route.upairs[uu][t]);
      }
      const uint32_t off = (uint32_t)(step * pq::kChunk) + lane16;
      if (off < (uint32_t)I) {
        pq::Bf16x16 wj[kDnRows];
#pragma unroll
        for (int j = 0; j < kDnRows; ++j) wj[j] = pq::widen16(w[j]);
#pragma unroll
        for (int t = 0; t < TP; ++t) {
          if (t < cnp) {
            const pq::Bf16x16 hv = pq::widen16(*reinterpret_cast<const uint4*>(ha + (size_t)(s0 + t) * I + off));
            const float hs = hsc[pr[t] * nbI + off / pq::kBlock];
#pragma unroll
            for (int j = 0; j < kDnRows; ++j) acc[j][t] = fmaf(pq::dot16(wj[j], hv), s[j] * hs, acc[j][t]);
          }
        }
      }
      if (step == nchI - 1) {             // unit (u, rows row, row + 1) done: all its sums in one butterfly
        static_assert(kDnRows == 2, "two rows per down step");
        if constexpr (kLaneStores) {    // lane 2t + j stores row + j of pair t
          const float y = pq::wave_sum_pairs_lanes<TP>(acc[0], acc[1], cnp);
          const int tl = lane >> 1, jl = lane & 1;
          if (tl < cnp && row + jl < nrows) ybuf[(row + jl) * P2 + route.upairs[uu][tl]] = y;
#pragma unroll
          for (int t = 0; t < TP; ++t)
#pragma unroll
            for (int j = 0; j < kDnRows; ++j) acc[j][t] = 0.0f;
        } else {
          float y0[TP], y1[TP];
          pq::wave_sum_pairs<TP>(acc[0], acc[1], cnp, y0, y1);
#pragma unroll
          for (int t = 0; t < TP; ++t) {
            if (t < cnp && lane == 0) {
              ybuf[row * P2 + pr[t]] = y0[t];
              if (row + 1 < nrows) ybuf[(row + 1) * P2 + pr[t]] = y1[t];
            }
#pragma unroll
            for (int j = 0; j < kDnRows; ++j) acc[j][t] = 0.0f;
          }
        }
      }
    };
    // wait until the h of union entry uu is in LDS (its stagers poll with a
    // bounded wait, and this wait is bounded too)
    auto wait_staged = [&](int uu) {
      const uint32_t n = (uint32_t)ufl(route.unp[uu]);
      lds_wait(&s_staged[uu], [n](uint32_t v) { return v >= n; }, hdr);
    };

#pragma unroll
    for (int q = 0; q < DD; ++q) issue_dn(wd[q], sw[q], sd[q]);
    for (;;) {
      int lo = nU, hi = -1;
#pragma unroll
      for (int q = 0; q < DD; ++q) {
        if (sd[q] >> 31) {
          const int uu = (int)((sd[q] >> 16) & 127u);
          lo = uu < lo ? uu : lo;
          hi = uu > hi ? uu : hi;
        }
      }
      for (int uu = lo > ready_next ? lo : ready_next; uu <= hi; ++uu) wait_staged(uu);
      ready_next = hi + 1 > ready_next ? hi + 1 : ready_next;
#pragma unroll
      for (int q = 0; q < DD; ++q) {
        consume_dn(wd[q], sw[q], sd[q]);
        issue_dn(wd[q], sw[q], sd[q]);
      }
      uint32_t busy = 0u;
#pragma unroll
      for (int q = 0; q < DD; ++q) busy |= sd[q];
      if (busy == 0u) break;
    }
  }

  // ---- D. weighted combine of each token's slots, in slot order --------------
  __syncthreads();
  for (int idx = threadIdx.x; idx < nrows * a.M; idx += kThreads) {
    const int rl = idx / a.M, m = idx - (idx / a.M) * a.M;
    float o = 0.0f;
    for (int j = 0; j < K; ++j) o = fmaf(route.w[m * K + j], ybuf[rl * P2 + m * K + j], o);
    if (sh) o += ybuf[rl * P2 + P + m];              // the shared expert, weight 1, last
    a.out[(size_t)m * H + r0 + rl] = pq::bf16_rne(o);
  }

  // ---- E. the last block to finish clears h for the next call ----------------
  // Every block is done reading h when it counts itself out; the waits make
  // its own h stores complete first.
  pq::wait_vm();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = pq::atomic_add_relaxed(&hdr->exit_count, 1u);
    s_last = old == gridDim.x - 1;
  }
  __syncthreads();
  if (s_last) {
    const pq::rsrc_t hr = pq::make_rsrc(a.hbuf, (uint32_t)(P2 * I * 2));
    const int nz = P2 * I / 8;
    for (int t = threadIdx.x; t < nz; t += kThreads)
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, hr, t * 16, 0, kAuxSC1);
    if (router)
      for (int t = threadIdx.x; t < a.M * a.E; t += kThreads) pq::st_agent_u32(a.lx + t, 0u);
    if (threadIdx.x == 0) {
      pq::atomic_store_relaxed(&hdr->exit_count, 0u);
      report_status(a, hdr);
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
// LDS the kernel declares statically (routing tables, expert bitmaps, block
// counters), reserved next to the dynamic area.
constexpr size_t kStaticLds = sizeof(Route) + kMaxM * kMaxE / 8 + kMaxUnion * 4 + 256;
constexpr size_t kLdsBytes = 160 * 1024;

struct MoePlan {
  size_t lds;
  int xs_off, ha_off, hs_off, yb_off, alias, sc_off, xa_off, hsplit;
  size_t off_h, ws_total;
};

// Which kernel runs a call: the barrier kernel for one token, the stream
// kernel from two on (H = 6144, I = 2048, 256 experts, top-8: M=1 56.9 against
// 60.0 µs, M=2 98.5-98.7 against 99.8-100.1, M=3 133.5 against 138.4);
// PQ_MOE_PATH=barrier|stream overrides.
enum { kPathBarrier = 0, kPathStream = 1 };
int moe_path(int M) {
  const char* e = getenv("PQ_MOE_PATH");
  if (e && strcmp(e, "barrier") == 0) return kPathBarrier;
  if (e && strcmp(e, "stream") == 0) return kPathStream;
  return M <= 1 ? kPathBarrier : kPathStream;
}

// num_cus bounds the rows a block can own (the grid has one block per CU);
// num_cus <= 0 checks the shape and sizes the workspace only.  The stream
// kernel gives x and h separate LDS regions when both fit (a wave may stage h
// while others still read x).  Otherwise it places as many h rows (staging
// slots, in union order) as fit before the x codes, followed by the x codes,
// the scales and y; the remaining slots continue over the x codes and wait
// for the block to be past gate_up, so the first experts' h is staged while
// the last gate_up units still stream.  Where even that does not fit (or PQ_MOE_ALIAS=full),
// and always in the barrier kernel, h and its scales reuse the x region once
// the block is past gate_up.  The workspace covers
// both kernels: the stream kernel's h in the zero-between-calls region, the
// barrier kernel's in the data region.
// The logit exchange sits at the end of the zero-between-calls region.
constexpr size_t kLxBytes = (size_t)kMaxM * kMaxE * 4;
constexpr size_t kWsLxOff = pq::kWsZeroOff + pq::kWsZeroBytes - kLxBytes;

int moe_plan(int M, int H, int I, int E, int top_k, int num_cus, int path, MoePlan* p, int sh = 1) {
  if (M < 1 || M > kMaxM || top_k < 1 || top_k > kMaxTopK || E < top_k || E > kMaxE) return PQ_ERR_SHAPE;
  if (H < pq::kBlock || H % pq::kBlock || H > 16384 || I < pq::kBlock || I % pq::kBlock || I > 16384)
    return PQ_ERR_SHAPE;
  // pairs: (token, slot) plus, with a shared expert, one per token; the
  // workspace is always sized for the shared expert
  const size_t P = (size_t)M * top_k + (size_t)sh * M;
  const size_t Pws = (size_t)M * top_k + M;
  if ((size_t)2 * I * H > pq::kMaxBufferBytes) return PQ_ERR_SHAPE;
  if (Pws * I * 2 > pq::kWsZeroBytes - kLxBytes) return PQ_ERR_SHAPE;
  const size_t xb = pqhost::align_up((size_t)M * H, 16), xsb = pqhost::align_up((size_t)M * (H / pq::kBlock) * 4, 16);
  const size_t hb = pqhost::align_up(P * I, 16), hsb = pqhost::align_up(P * (I / pq::kBlock) * 4, 16);
  p->lds = 0;
  p->xs_off = (int)xb;
  p->alias = 0;
  p->sc_off = -1;
  p->xa_off = 0;
  p->hsplit = (int)P;
  if (num_cus > 0) {
    const size_t yb = ((size_t)H + num_cus - 1) / num_cus * P * 4;
    const size_t sep = xb + xsb + hb + hsb + yb;
    const size_t apart = xb + xsb + hsb + yb;   // all but the h codes
    const char* fa = getenv("PQ_MOE_ALIAS");
    const bool full = fa && strcmp(fa, "full") == 0;
    const size_t room = apart + kStaticLds < kLdsBytes ? (kLdsBytes - kStaticLds - apart) / I : 0;
    if (path == kPathStream && sep + kStaticLds <= kLdsBytes) {
      p->ha_off = (int)(xb + xsb);
      p->hs_off = (int)(xb + xsb + hb);
      p->yb_off = (int)(xb + xsb + hb + hsb);
      p->lds = sep;
    } else if (path == kPathStream && !full && room < P && (P - room) * I <= xb) {
      p->alias = 1;
      p->hsplit = (int)room;
      p->ha_off = 0;
      p->xa_off = (int)(room * I);
      p->xs_off = (int)(room * I + xb);
      p->hs_off = (int)(room * I + xb + xsb);
      p->yb_off = (int)(room * I + xb + xsb + hsb);
      p->lds = room * I + apart;
    } else {
      const size_t cb = xb > hb ? xb : hb, sb = xsb > hsb ? xsb : hsb;
      p->alias = 1;
      p->hsplit = 0;
      p->xs_off = (int)cb;
      p->ha_off = 0;
      p->hs_off = (int)cb;
      p->yb_off = (int)(cb + sb);
      p->lds = cb + sb + yb;
      if (p->lds + kStaticLds > kLdsBytes) return PQ_ERR_SHAPE;
    }
    // the barrier kernel's scale windows, where they fit
    const size_t sco = pqhost::align_up(p->lds, 16);
    if (path != kPathStream && H / pq::kBlock <= kWinFloats &&
        sco + kScWaveBytes * kWaves + kStaticLds <= kLdsBytes) {
      p->sc_off = (int)sco;
      p->lds = sco + kScWaveBytes * kWaves;
    }
  }
  p->off_h = pq::kWsZeroOff;
  p->ws_total = pqhost::align_up(pq::kWsDataOff + Pws * I * 2, 256);
  return PQ_OK;
}

// PQ_MOE_LAUNCH=cooperative launches the layer kernels with
// hipLaunchCooperativeKernel, which makes the runtime guarantee that every
// block of the grid is resident at once (or refuse the launch); the default
// plain launch relies on the grid being one block per CU of an otherwise idle
// device, and a block that is kept waiting anyway ends its bounded waits with
// PQ_ERR_TIMEOUT.
bool cooperative_launch() {
  const char* e = getenv("PQ_MOE_LAUNCH");
  return e && strcmp(e, "cooperative") == 0;
}

template <int TP, bool STREAM, bool EXT>
int launch_moe(const MoeArgs& a, const MoePlan& pl, const pqhost::DeviceInfo& dev, hipStream_t stream) {
  auto kern = STREAM ? moe_stream_kernel<TP, EXT> : moe_barrier_kernel<TP, EXT>;
  static pqhost::KernelAttrOnce attr;
  PQ_HIP_CHECK(pqhost::set_dynamic_lds_once(attr, (const void*)kern, (int)(kLdsBytes - kStaticLds)));
  int per_cu = 0;
  PQ_HIP_CHECK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kern, kThreads, pl.lds));
  if (per_cu < 1) return PQ_ERR_SHAPE;
  // one block per CU (blocks wait on each other, so all must be resident; one
  // per CU also keeps the per-block staging of h to one copy per CU)
  const int grid = dev.num_cus;
  if (cooperative_launch()) {
    MoeArgs arg = a;
    void* params[] = {&arg};
    PQ_HIP_CHECK(hipLaunchCooperativeKernel((const void*)kern, dim3(grid), dim3(kThreads), params,
                                            (unsigned)pl.lds, stream));
    return PQ_OK;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), pl.lds, stream, a);
  PQ_HIP_CHECK(hipGetLastError());
  return PQ_OK;
}

// EXT: the router GEMV or a shared expert in the launch (the plain layer is
// compiled without their code, so its registers are as before)
template <int TP>
int launch_moe_path(int path, const MoeArgs& a, const MoePlan& pl, const pqhost::DeviceInfo& dev, hipStream_t s) {
  if (a.router || a.sh)
    return path == kPathStream ? launch_moe<TP, true, true>(a, pl, dev, s) : launch_moe<TP, false, true>(a, pl, dev, s);
  return path == kPathStream ? launch_moe<TP, true, false>(a, pl, dev, s) : launch_moe<TP, false, false>(a, pl, dev, s);
}

// ---------------------------------------------------------------------------
// Allocation-free entry point: the layer's workspace in a static device array
// ---------------------------------------------------------------------------
// moe_decode_layer_noalloc serves callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops).  Its workspace is this
// file-scope array: one copy per GPU the library runs on, held until the
// process ends.  The host only ever uses the device address that
// hipGetSymbolAddress returns for it (the array's name is a host-side stand-in
// in host code).  Every call on a GPU shares that GPU's copy, so calls that
// can overlap in time on one GPU race.  The layer kernels leave the counters
// and the exchange region at zero when they finish, as they do in a
// caller's workspace; the copy is zeroed once, when the device first uses it.
constexpr size_t kScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ __launch_bounds__(256) void scratch_clear_kernel(uint4* p, int n16) {
  for (int i = (int)(blockIdx.x * 256 + threadIdx.x); i < n16; i += (int)(gridDim.x * 256)) p[i] = make_uint4(0, 0, 0, 0);
}

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  int status = PQ_OK;
  int hip_error = 0;
};
DeviceScratch g_scratch[pqhost::kMaxDevices];

// The device address of this device's scratch copy, looked up (and the copy
// zeroed on `stream`) the first time the device uses it.
int device_scratch(int device, hipStream_t stream, void** out) {
  if (device < 0 || device >= pqhost::kMaxDevices) return PQ_ERR_UNSUPPORTED;
  DeviceScratch& d = g_scratch[device];
  std::call_once(d.once, [&] {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e == hipSuccess && p == nullptr) e = hipErrorInvalidSymbol;
    if (e == hipSuccess) {
      hipLaunchKernelGGL(scratch_clear_kernel, dim3(256), dim3(256), 0, stream, reinterpret_cast<uint4*>(p),
                         (int)(kScratchBytes / 16));
      e = hipGetLastError();
    }
    if (e != hipSuccess) {
      d.status = PQ_ERR_HIP;
      d.hip_error = (int)e;
      return;
    }
    d.ptr = p;
  });
  if (d.status != PQ_OK) {
    pqhost::set_last_hip_error(d.hip_error);
    return d.status;
  }
  *out = d.ptr;
  return PQ_OK;
}

// The layer call behind moe_decode_layer_ex (caller's workspace) and
// moe_decode_layer_noalloc (ws == NULL: the device's static scratch).
int layer_call(const uint16_t* x, int M, int H, const uint16_t* router_w, float* router_logits, int32_t* topk_ids,
               float* topk_w, int E, int top_k, int I, const uint8_t* w13, const float* s13, const uint8_t* w2,
               const float* s2, const uint8_t* sh_w13, const float* sh_s13, const uint8_t* sh_w2,
               const float* sh_s2, uint16_t* out, uint16_t* h_dbg, uint8_t* hq_dbg, float* hs_dbg, void* ws,
               size_t ws_bytes, int32_t* status_out, void* stream) {
  if (!x || !topk_ids || !topk_w || !w13 || !s13 || !w2 || !s2 || !out) return PQ_ERR_NULL;
  const int nsh = (sh_w13 != nullptr) + (sh_s13 != nullptr) + (sh_w2 != nullptr) + (sh_s2 != nullptr);
  if (nsh != 0 && nsh != 4) return PQ_ERR_NULL;      // all four shared-expert tensors or none
  const int sh = nsh == 4 ? 1 : 0;
  MoePlan pl;
  const int path = moe_path(M);
  int st = moe_plan(M, H, I, E, top_k, 0, path, &pl, sh);   // shape checks (device independent)
  if (st != PQ_OK) return st;
  const void* ptrs[] = {x, router_w, router_logits, topk_ids, topk_w, w13, s13, w2, s2,
                        sh_w13, sh_s13, sh_w2, sh_s2, out, h_dbg, hq_dbg, hs_dbg, ws};
  for (const void* q : ptrs)
    if (q && !pqhost::aligned16(q)) return PQ_ERR_ALIGN;
  if (router_w && (size_t)E * H * 2 > pq::kMaxBufferBytes) return PQ_ERR_SHAPE;
  if (ws == nullptr && pl.ws_total > kScratchBytes) return PQ_ERR_SCRATCH;
  if (ws != nullptr && ws_bytes < pl.ws_total) return PQ_ERR_WORKSPACE;
  pqhost::DeviceInfo dev;
  st = pqhost::current_device_info(&dev);
  if (st != PQ_OK) return st;
  if (ws == nullptr) {                 // allocation-free call: this device's static scratch
    st = device_scratch(dev.device, (hipStream_t)stream, &ws);
    if (st != PQ_OK) return st;
  }
  st = moe_plan(M, H, I, E, top_k, dev.num_cus, path, &pl, sh);
  if (st != PQ_OK) return st;

  MoeArgs a;
  a.x = x;
  a.wr = router_w;
  a.logits = router_w ? nullptr : router_logits;
  a.logits_out = router_w ? router_logits : nullptr;
  a.lx = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(ws) + kWsLxOff);
  a.sw13 = sh_w13; a.ss13 = sh_s13; a.sw2 = sh_w2; a.ss2 = sh_s2;
  a.topk_ids = topk_ids; a.topk_w = topk_w;
  a.w13 = w13; a.s13 = s13; a.w2 = w2; a.s2 = s2; a.out = out;
  a.h_dbg = h_dbg; a.hq_dbg = hq_dbg; a.hs_dbg = hs_dbg;
  a.ws = reinterpret_cast<uint8_t*>(ws);
  a.status_out = status_out;
  a.hbuf = reinterpret_cast<uint16_t*>(a.ws + pl.off_h);
  a.M = M; a.H = H; a.I = I; a.E = E; a.top_k = top_k;
  a.router = router_w != nullptr;
  a.routed = router_w != nullptr || router_logits != nullptr;
  a.sh = sh;
  a.P2 = M * top_k + sh * M;
  a.spin_limit = kSpinLimit;
  a.xs_off = pl.xs_off; a.ha_off = pl.ha_off; a.hs_off = pl.hs_off; a.yb_off = pl.yb_off;
  a.alias = pl.alias;
  a.xa_off = pl.xa_off;
  a.hsplit = pl.hsplit;
  a.sc_off = pl.sc_off;
  const char* sce = getenv("PQ_MOE_SCALES");          // "step": per-step scale loads (for tests)
  if (sce && strcmp(sce, "step") == 0) a.sc_off = -1;
  const char* lim = getenv("PQ_SPIN_LIMIT");
  if (lim && *lim) a.spin_limit = (uint32_t)strtoul(lim, nullptr, 10);

  hipStream_t s = (hipStream_t)stream;
  if (M == 1) return launch_moe_path<1>(path, a, pl, dev, s);
  if (M == 2) return launch_moe_path<2>(path, a, pl, dev, s);
  if (M <= 4) return launch_moe_path<4>(path, a, pl, dev, s);
  return launch_moe_path<8>(path, a, pl, dev, s);
}


}  // namespace

extern "C" {

size_t moe_decode_layer_workspace(int M, int H, int I, int E, int top_k) {
  MoePlan pl;
  if (moe_plan(M, H, I, E, top_k, 0, kPathStream, &pl) != PQ_OK) return 0;
  return pl.ws_total;
}

int moe_decode_layer_config(int M, int H, int I, int E, int top_k, int shared, int* kernel, int* alias,
                            size_t* lds_bytes) {
  if (!kernel || !alias || !lds_bytes) return PQ_ERR_NULL;
  MoePlan pl;
  const int path = moe_path(M);
  int st = moe_plan(M, H, I, E, top_k, 0, path, &pl, shared ? 1 : 0);
  if (st != PQ_OK) return st;
  pqhost::DeviceInfo dev;
  st = pqhost::current_device_info(&dev);
  if (st != PQ_OK) return st;
  st = moe_plan(M, H, I, E, top_k, dev.num_cus, path, &pl, shared ? 1 : 0);
  if (st != PQ_OK) return st;
  *kernel = path;
  *alias = pl.alias;
  *lds_bytes = pl.lds;
  return PQ_OK;
}

int moe_decode_layer_ex(const uint16_t* x, int M, int H, const uint16_t* router_w, float* router_logits,
                        int32_t* topk_ids, float* topk_w, int E, int top_k, int I, const uint8_t* w13,
                        const float* s13, const uint8_t* w2, const float* s2, const uint8_t* sh_w13,
                        const float* sh_s13, const uint8_t* sh_w2, const float* sh_s2, uint16_t* out,
                        uint16_t* h_dbg, uint8_t* hq_dbg, float* hs_dbg, void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return PQ_ERR_NULL;
  return layer_call(x, M, H, router_w, router_logits, topk_ids, topk_w, E, top_k, I, w13, s13, w2, s2, sh_w13,
                    sh_s13, sh_w2, sh_s2, out, h_dbg, hq_dbg, hs_dbg, ws, ws_bytes, nullptr, stream);
}

int moe_decode_layer_noalloc(const uint16_t* x, int M, int H, const uint16_t* router_w, float* router_logits,
                             int32_t* topk_ids, float* topk_w, int E, int top_k, int I, const uint8_t* w13,
                             const float* s13, const uint8_t* w2, const float* s2, const uint8_t* sh_w13,
                             const float* sh_s13, const uint8_t* sh_w2, const float* sh_s2, uint16_t* out,
                             uint16_t* h_dbg, uint8_t* hq_dbg, float* hs_dbg, int32_t* status, void* stream) {
  if (status && !pqhost::aligned16(status)) return PQ_ERR_ALIGN;
  return layer_call(x, M, H, router_w, router_logits, topk_ids, topk_w, E, top_k, I, w13, s13, w2, s2, sh_w13,
                    sh_s13, sh_w2, sh_s2, out, h_dbg, hq_dbg, hs_dbg, nullptr, 0, status, stream);
}

int moe_decode_layer(const uint16_t* x, int M, int H, const float* router_logits, int32_t* topk_ids,
                     float* topk_w, int E, int top_k, int I, const uint8_t* w13, const float* s13,
                     const uint8_t* w2, const float* s2, uint16_t* out, uint16_t* h_dbg, uint8_t* hq_dbg,
                     float* hs_dbg, void* ws, size_t ws_bytes, void* stream) {
  return moe_decode_layer_ex(x, M, H, nullptr, const_cast<float*>(router_logits), topk_ids, topk_w, E, top_k, I,
                             w13, s13, w2, s2, nullptr, nullptr, nullptr, nullptr, out, h_dbg, hq_dbg, hs_dbg, ws,
                             ws_bytes, stream);
}

}  // extern "C"
