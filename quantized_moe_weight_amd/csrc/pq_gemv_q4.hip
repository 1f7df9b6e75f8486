// int4 g32 weight-streaming GEMV (W4A16, M <= 8) with an optional fused
// SiLU(gate)*up epilogue.
//
// [M3]: Q4 weight-streaming decode kernels; [CMP]: routed experts held at 4
// bits.  Weights are symmetric int4 with one fp16 scale per 32 consecutive K
// values, stored as offset-binary nibbles (low nibble = even k).
//
// gfx950 design
//   * each block owns a contiguous range of output rows and streams them in
//     1 KB chunks (one 16-byte load per lane = 32 weights = exactly one scale
//     group); the (row, chunk) units of the block are dealt to its waves as
//     contiguous runs, so K is split inside the block wherever a row
//     straddles two waves, and the split is reduced through LDS after one
//     barrier: no global partials, atomics or store waits in the stream;
//   * each wave keeps D chunk steps in flight in a ring of raw buffer loads
//     issued without branches (out-of-range slots return zero without memory
//     traffic), and the last D steps drain the ring without issuing; shallow
//     rings (3-4 steps) stream faster here than deep ones;
//   * unpacking without a packed bf16 subtract: nibble n becomes the bf16
//     value 1 + n/16 (n shifted into the top mantissa bits under the exponent
//     of 1.0) with one shift and one and-or per pair, v_dot2 multiplies it with
//     bf16 x exactly, and the group's sum is corrected with the group's sum of
//     x:  sum (n-8) x = 16 * (sum (1 + n/16) x - 1.5 * sum x);
//   * x is staged once per block in LDS as bf16 with each run of 8 values
//     stored as the pairs (x0,x4)(x1,x5)(x2,x6)(x3,x7) that the unpack yields,
//     plus 1.5 times the per-group sums of x; the activation loads are issued
//     before the weight ring so staging does not wait for weights.
#include <stdlib.h>
#include <type_traits>
#include <string.h>


#include "pq_common.h"

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / pq::kWave;
constexpr int kMaxM = 8;
constexpr int kGroup = 32;                 // weights per fp16 scale
constexpr int kXGroups = 2;                // x groups per thread loaded before the weight ring
constexpr long kMaxMK = 69632;             // M*K bound: activation + sums + partials fit LDS
constexpr uint32_t kOne = 0x3F803F80u;     // bf16 pair (1.0, 1.0)
constexpr uint32_t kNibMask = 0x00780078u; // mantissa bits 3..6 of both halves

// The constant (1.0, 1.0) held in a VGPR the compiler cannot see through:
// with it in a register each pair below is one shift and one v_and_or_b32
// (the mask rides in an SGPR) instead of shift, and, or with two literals.
__device__ __forceinline__ uint32_t one_pair_reg() {
  uint32_t v = kOne;
  asm volatile("" : "+v"(v));
  return v;
}

// bf16 pair (1 + n_j/16, 1 + n_{j+4}/16) from the 8 nibbles of one dword
template <int J>
__device__ __forceinline__ uint32_t nib_pair(uint32_t d, uint32_t one) {
  if constexpr (J == 0) return ((d << 3) & kNibMask) | one;
  else return ((d >> (4 * J - 3)) & kNibMask) | one;
}

struct Pairs16 { uint32_t v[16]; };        // 32 weights as 16 bf16 pairs

__device__ __forceinline__ Pairs16 unpack32(uint4 w, uint32_t one) {
  Pairs16 r;
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    r.v[4 * t + 0] = nib_pair<0>(d[t], one);
    r.v[4 * t + 1] = nib_pair<1>(d[t], one);
    r.v[4 * t + 2] = nib_pair<2>(d[t], one);
    r.v[4 * t + 3] = nib_pair<3>(d[t], one);
  }
  return r;
}

__device__ __forceinline__ float dot32(const Pairs16& w, const uint4 (&x)[4]) {
  float p = 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t xs[4] = {x[t].x, x[t].y, x[t].z, x[t].w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(pq::bf16x2, w.v[4 * t + j]),
                                          __builtin_bit_cast(pq::bf16x2, xs[j]), p, false);
  }
  return p;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }


// 8 bf16 values x0..x7 -> the pairs (x0,x4)(x1,x5)(x2,x6)(x3,x7)
__device__ __forceinline__ uint4 pair_order(uint4 r) {
  uint4 o;
  o.x = __builtin_amdgcn_perm(r.z, r.x, 0x05040100u);
  o.y = __builtin_amdgcn_perm(r.z, r.x, 0x07060302u);
  o.z = __builtin_amdgcn_perm(r.w, r.y, 0x05040100u);
  o.w = __builtin_amdgcn_perm(r.w, r.y, 0x07060302u);
  return o;
}

// ---------------------------------------------------------------------------
// Vector path.  One launch runs a list of independent linears (one when
// called through pq_gemv_q4), each with its own x, weights, scales, output and
// epilogue, all with M tokens.
//
//   * Work unit: one pair of weight rows at one 1 KB chunk.  Every lane loads
//     the same 16 bytes of row A and of row B (2 KB per wave step) and reads
//     the activation once for both rows.  Under SiLU*up, A is gate row i and
//     B up row i; otherwise A and B are consecutive rows.
//   * Block b owns the same share of every linear's rows (the split of the
//     rows over the grid depends on the linear's shape and the CU count only),
//     and a linear's units of the block are dealt to the block's waves as
//     contiguous runs (wave w takes units [split(U, 16, w), split(U, 16,
//     w+1)), unit = pair * nch + chunk), linear by linear, exactly as if the
//     linear ran alone: a linear's output bits do not depend on the other
//     linears of the launch, nor on M.  A wave accumulates a row pair's
//     chunks of its run per lane and reduces them across the wave once, at the
//     run's last chunk of the pair (writing an exact zero for the run's other
//     chunks of it), instead of reducing every chunk: 2 * M wave reductions
//     per pair-run rather than per 2 KB step (dealt round-robin, so that the
//     block read one window of consecutive chunks, the stack was 13% slower
//     at M = 4 and 4% at M = 1).  Each wave streams its share of every linear back to back;
//     its ring of load steps runs across linear boundaries, so the start-up
//     and ring fill are paid once per launch.
//   * The activations of every linear of the launch are staged in LDS at
//     the start, pieces of 16 bytes stored piece-major ([token][t][group]):
//     the 64 lanes of a step read consecutive pieces, free of bank conflicts.
//   * Row pairs cut between waves are reduced through LDS after one barrier at
//     the end, in wave order.
// ---------------------------------------------------------------------------
constexpr int kMaxLin = 12;      // linears per launch (kernel arguments by value)
// 16 waves per CU: the loop is bound by vector instructions (unpacking and
// dot products, ~190 per 2 KB step at M = 1), and four waves per SIMD hide
// their load and LDS latencies better than two (10.57 GB dense stack at M = 1:
// 2.50 ms per pass against 2.66 with 512 threads)
constexpr int kVThreads = 1024;
constexpr int kVWaves = kVThreads / pq::kWave;
constexpr uint32_t kStepBytes = 1024;  // bytes of each row of the pair per wave step

struct Q4Lin {
  const uint16_t* x;
  const uint8_t* w;
  const uint16_t* wsc;
  uint16_t* y;
  int K, N, R;     // R: output rows (N, or N/2 under SiLU*up)
  int silu;        // rows [0,R) gate, [R,2R) up; one output per row pair
  int ng;          // 32-groups per row
  int nch;         // 512-byte chunks per row
  int xoff;        // LDS: x pieces of this linear (16 B each), [MT][4][ng]
  int soff;        // LDS: group offsets (floats), [MT][ng]
  int poff;        // LDS: partials (floats), [pairs + waves][MT][2]
};

struct Q4Group {
  Q4Lin lin[kMaxLin];
  int n;
  int dummy_piece;  // LDS piece written by threads without a group
  int dummy_float;  // LDS float written by threads without a group
};

// this block's rows of a linear, as row pairs
struct BlockRows {
  int rs, re, pairs;
};
__device__ __forceinline__ BlockRows block_rows(const Q4Lin& L, int G, int b) {
  BlockRows r;
  r.rs = pq::split_start(L.R, G, b);
  r.re = pq::split_start(L.R, G, b + 1);
  r.pairs = L.silu ? r.re - r.rs : (r.re - r.rs + 1) / 2;
  return r;
}

// Stage one 32-value group of x: its 4 pieces in the paired order, and c =
// the v_dot2 chain of dot32 with every weight pair (1.5, 1.5), in the same
// order, so that a group whose nibbles are all 8 (q = 0) contributes exactly
// zero.  piece0 / stride: where piece t goes (piece0 + t * stride).
__device__ __forceinline__ void stage_group(uint4* xs_l, float* cs, int piece0, int stride, int cslot,
                                            const uint4 (&raw)[4]) {
  uint4 xv[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    xv[t] = pair_order(raw[t]);
    xs_l[piece0 + t * stride] = xv[t];
  }
  Pairs16 th;
#pragma unroll
  for (int i = 0; i < 16; ++i) th.v[i] = 0x3FC03FC0u;
  cs[cslot] = dot32(th, xv);
}

// Walks one wave's steps through the linears of the launch: (linear, pair,
// chunk), linear by linear, skipping linears that give the wave no unit.  The
// per-linear starting points of every wave and the block's row ranges are
// computed once, into an LDS table, so moving to the next linear is one table
// read (an inlined search with divisions at every ring slot made the loop body
// several times larger).  The launch arguments are only ever indexed with the
// wave-uniform linear index (a per-lane index makes the compiler copy the
// whole argument block to scratch memory).
struct SegEntry {
  int p0, c0, left;         // this wave's first unit of a linear (pair, chunk) and its steps there
  int dp, dc;               // one step ahead: kVWaves units = dp pairs and dc chunks
  int rs, re, nch;          // this block's rows of the linear, chunks per row
};
struct StepCursor {
  int li, p, c, left, nch, rs, re, dp, dc;
};
__device__ __forceinline__ StepCursor cursor_at(const Q4Group& a, const SegEntry* seg, int li) {
  StepCursor s;
  for (; li < a.n; ++li)
    if (__builtin_amdgcn_readfirstlane(seg[li].left) > 0) break;
  s.li = li;
  s.p = s.c = s.left = s.rs = s.re = s.dp = s.dc = 0;
  s.nch = 1;
  if (li < a.n) {
    const SegEntry& e = seg[li];
    s.p = __builtin_amdgcn_readfirstlane(e.p0);
    s.c = __builtin_amdgcn_readfirstlane(e.c0);
    s.left = __builtin_amdgcn_readfirstlane(e.left);
    s.dp = __builtin_amdgcn_readfirstlane(e.dp);
    s.dc = __builtin_amdgcn_readfirstlane(e.dc);
    s.rs = __builtin_amdgcn_readfirstlane(e.rs);
    s.re = __builtin_amdgcn_readfirstlane(e.re);
    s.nch = __builtin_amdgcn_readfirstlane(e.nch);
  }
  return s;
}
__device__ __forceinline__ StepCursor cursor_next(const Q4Group& a, const SegEntry* seg, StepCursor s) {
  if (s.left == 1) return cursor_at(a, seg, s.li + 1);
  --s.left;
  s.p += s.dp;
  s.c += s.dc;
  if (s.c >= s.nch) {
    s.c -= s.nch;
    ++s.p;
  }
  return s;
}

// PAIR (every linear's groups per row even): each lane loads the aligned dword
// holding its group's scale and its neighbour's (lanes 2i and 2i + 1 share
// it) and keeps its half: 16-bit scale loads made the compiler pack the ring
// slots' scales pairwise, waiting for nearly every load in flight.
template <int D, int MT, bool PAIR>
__global__ __launch_bounds__(kVThreads) void gemv_q4_kernel(const Q4Group a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ SegEntry s_seg[kVWaves][kMaxLin];
  uint4* xs_l = reinterpret_cast<uint4*>(smem);
  float* fl = reinterpret_cast<float*>(smem);
  const int G = (int)gridDim.x;
  const int tid = (int)threadIdx.x;
  const int lane = pq::lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(pq::wave_id());

  // Activation loads of the first kXGroups groups per thread (counted over
  // the groups of all linears), then a plain barrier: every wave issues them
  // before any weight load, so staging waits for x only.
  uint4 xpre[kXGroups][4];
  int pre_li[kXGroups], pre_g[kXGroups];
#pragma unroll
  for (int i = 0; i < kXGroups; ++i) {
    pre_li[i] = a.n;
    pre_g[i] = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) xpre[i][t] = make_uint4(0u, 0u, 0u, 0u);
  }
  {
    int gbase = 0;
    for (int li = 0; li < a.n && gbase < kXGroups * kVThreads; ++li) {   // uniform: one linear at a time
      const Q4Lin& L = a.lin[li];
      const int ngr = MT * L.ng;
      const pq::rsrc_t xr = pq::make_rsrc(L.x, (uint32_t)(MT * L.K * 2));
#pragma unroll
      for (int i = 0; i < kXGroups; ++i) {
        const int g = tid + i * kVThreads - gbase;
        if (g >= 0 && g < ngr) {
          pre_li[i] = li;
          pre_g[i] = g;
#pragma unroll
          for (int t = 0; t < 4; ++t) xpre[i][t] = pq::buf_load16(xr, (uint32_t)g * 64u + 16u * t);
        }
      }
      gbase += ngr;
    }
  }
  __builtin_amdgcn_s_barrier();

  // This wave's units of every linear: the contiguous run [u0, u0 + left)
  // of units u = (pair u / nch, chunk u % nch) of the block's rows, walked
  // chunk by chunk.  Written and read by the wave itself (no barrier).
  int total = 0;
  for (int li = 0; li < a.n; ++li) {             // uniform
    const Q4Lin& L = a.lin[li];
    const BlockRows br = block_rows(L, G, (int)blockIdx.x);
    const int units = br.pairs * L.nch;
    const int u0 = pq::split_start(units, kVWaves, wv);
    const int left = pq::split_start(units, kVWaves, wv + 1) - u0;
    total += left;
    if (lane == 0)
      s_seg[wv][li] = SegEntry{u0 / L.nch, u0 - (u0 / L.nch) * L.nch, left, 0, 1, br.rs, br.re, L.nch};
  }
  const SegEntry* seg = s_seg[wv];

  // the weight ring: D steps in flight, issued without branches on validity
  StepCursor ic = cursor_at(a, seg, 0);
  int ili = -1;
  pq::rsrc_t wr = pq::make_rsrc(a.lin[0].w, 0u), sr = pq::make_rsrc(a.lin[0].wsc, 0u);
  uint32_t rowb = 0, ngs = 0;
  int rup = 0, silu = 0;
  auto issue = [&](uint4 (&wq)[2], uint32_t (&sq)[2]) {
    const bool ok = ic.li < a.n;
    if (ok && ic.li != ili) {                    // a new linear: its descriptors
      ili = ic.li;
      const Q4Lin& L = a.lin[ili];
      rowb = (uint32_t)(L.K / 2);
      ngs = (uint32_t)L.ng;
      wr = pq::make_rsrc(L.w, (uint32_t)((size_t)L.N * rowb));
      sr = pq::make_rsrc(L.wsc, (uint32_t)((size_t)L.N * L.ng * 2));
      silu = L.silu;
      rup = L.R;
    }
    // the pair's two rows, and this lane's 16 bytes of the chunk
    const int rowa = silu ? ic.rs + ic.p : ic.rs + 2 * ic.p;
    const int rowb2 = silu ? rowa + rup : rowa + 1;
    const uint32_t off = (uint32_t)ic.c * kStepBytes + 16u * (uint32_t)lane;
    const bool va = ok && off < rowb;
    const bool vb = va && (silu || rowb2 < ic.re);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool v = j == 0 ? va : vb;
      const uint32_t row = (uint32_t)(j == 0 ? rowa : rowb2);
      wq[j] = pq::buf_load16_nt(wr, v ? row * rowb + off : pq::kOOB);
      if constexpr (PAIR)
        sq[j] = __builtin_amdgcn_raw_buffer_load_b32(
            sr, (int)(v ? (row * ngs + ((off / 16u) & ~1u)) * 2u : pq::kOOB), 0, pq::kAuxNT);
      else
        sq[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
            sr, (int)(v ? (row * ngs + off / 16u) * 2u : pq::kOOB), 0, pq::kAuxNT);
    }
    if (ok) ic = cursor_next(a, seg, ic);
  };
  uint4 wbuf[D][2];
  uint32_t sbuf[D][2];
#pragma unroll
  for (int q = 0; q < D; ++q) issue(wbuf[q], sbuf[q]);
  __builtin_amdgcn_sched_barrier(0);               // keep the staging below the ring issue

  // stage x of every linear (preloaded groups first; a thread without a
  // group writes the dummy piece and float)
  {
    // preloaded groups (a thread without one writes the dummy piece and
    // float), then the remaining groups of every linear: global group numbers
    // run over the linears in order, a thread takes numbers tid + k * kVThreads
    bool staged[kXGroups];
#pragma unroll
    for (int i = 0; i < kXGroups; ++i) staged[i] = false;
    int gbase = 0;
    for (int li = 0; li < a.n; ++li) {                // uniform
      const Q4Lin& L = a.lin[li];
      const int ngr = MT * L.ng;
#pragma unroll
      for (int i = 0; i < kXGroups; ++i) {
        if (pre_li[i] == li) {
          const int m = pre_g[i] / L.ng, g = pre_g[i] - m * L.ng;
          stage_group(xs_l, fl, L.xoff + m * 4 * L.ng + g, L.ng, L.soff + m * L.ng + g, xpre[i]);
          staged[i] = true;
        }
      }
      const pq::rsrc_t xr = pq::make_rsrc(L.x, (uint32_t)(MT * L.K * 2));
      // first number >= max(gbase, kXGroups * kVThreads) that is tid modulo kVThreads
      const int lo = gbase > kXGroups * kVThreads ? gbase : kXGroups * kVThreads;
      const int first = lo + ((tid - lo) % kVThreads + kVThreads) % kVThreads;
      for (int gg = first; gg < gbase + ngr; gg += kVThreads) {
        const int g0 = gg - gbase;
        uint4 raw[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) raw[t] = pq::buf_load16(xr, (uint32_t)g0 * 64u + 16u * t);
        const int m = g0 / L.ng, g = g0 - m * L.ng;
        stage_group(xs_l, fl, L.xoff + m * 4 * L.ng + g, L.ng, L.soff + m * L.ng + g, raw);
      }
      gbase += ngr;
    }
#pragma unroll
    for (int i = 0; i < kXGroups; ++i)
      if (!staged[i]) stage_group(xs_l, fl, a.dummy_piece, 0, a.dummy_float, xpre[i]);
  }
  __syncthreads();

  const uint32_t one = one_pair_reg();
  float acc[2][MT];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[j][m] = 0.0f;

  StepCursor cc = cursor_at(a, seg, 0);
  int cli = -1;
  int c_ng = 0, c_nch = 0, c_xoff = 0, c_soff = 0, c_poff = 0;
  uint32_t c_rowb = 0;
  auto consume = [&](const uint4 (&wq)[2], const uint32_t (&sq)[2]) {
    if (cc.li != cli) {
      cli = cc.li;
      const Q4Lin& L = a.lin[cli];
      c_ng = L.ng;
      c_nch = L.nch;
      c_xoff = L.xoff;
      c_soff = L.soff;
      c_poff = L.poff;
      c_rowb = (uint32_t)(L.K / 2);
    }
    const uint32_t off = (uint32_t)cc.c * kStepBytes + 16u * (uint32_t)lane;
    if (off < c_rowb) {
      const int g = (int)(off / 16u);              // this lane's group in the row
      Pairs16 w[2];
      float sc[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        w[j] = unpack32(wq[j], one);
        if constexpr (PAIR)    // this lane's group is g; its parity is the lane's
          sc[j] = 16.0f * (float)__builtin_bit_cast(_Float16, (uint16_t)(sq[j] >> (16u * ((uint32_t)lane & 1u))));
        else
          sc[j] = 16.0f * (float)__builtin_bit_cast(_Float16, (uint16_t)sq[j]);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        uint4 xv[4];
        const int p0 = c_xoff + m * 4 * c_ng + g;
#pragma unroll
        for (int t = 0; t < 4; ++t) xv[t] = xs_l[p0 + t * c_ng];
        const float cv = fl[c_soff + m * c_ng + g];
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j][m] = fmaf(dot32(w[j], xv) - cv, sc[j], acc[j][m]);
      }
    }
    if (cc.c == c_nch - 1 || cc.left == 1) {      // the wave's last chunk of this pair: its partial sums
      constexpr int NV = 2 * MT <= 2 ? 2 : 2 * MT <= 4 ? 4 : 2 * MT <= 8 ? 8 : 16;
      float vals[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) vals[i] = i < 2 * MT ? acc[i & 1][i >> 1] : 0.0f;   // value 2m + j
      const float v = pq::wave_sum_many<NV, true>(vals);   // lane 2m + j: the sum of acc[j][m] (crossbar exchanges: fewer vector instructions)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j][m] = 0.0f;
      if (lane < 2 * MT) fl[c_poff + (size_t)(cc.p * c_nch + cc.c) * MT * 2 + lane] = v;
    } else if (lane < 2 * MT) {                    // an earlier chunk of the run: its slot adds nothing
      fl[c_poff + (size_t)(cc.p * c_nch + cc.c) * MT * 2 + lane] = 0.0f;
    }
    cc = cursor_next(a, seg, cc);
  };

  int base = 0;
  for (; base + D < total; base += D) {           // steady state: every slot refills
#pragma unroll
    for (int q = 0; q < D; ++q) {
      consume(wbuf[q], sbuf[q]);
      issue(wbuf[q], sbuf[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < D; ++q)                      // drain
    if (base + q < total) consume(wbuf[q], sbuf[q]);
  __syncthreads();

  // add each row pair's chunk partials in chunk order
  for (int li = 0; li < a.n; ++li) {
    const Q4Lin& L = a.lin[li];
    const BlockRows br = block_rows(L, G, (int)blockIdx.x);
    for (int i = tid; i < br.pairs * MT; i += kVThreads) {
      const int p = i / MT, m = i - (i / MT) * MT;
      float va = 0.0f, vb = 0.0f;
      for (int c = 0; c < L.nch; ++c) {
        const float* part = fl + L.poff + (size_t)(p * L.nch + c) * MT * 2;
        va += part[2 * m];
        vb += part[2 * m + 1];
      }
      if (L.silu) {
        L.y[(size_t)m * L.R + br.rs + p] = pq::bf16_rne(silu_mul(va, vb));
      } else {
        const int r = br.rs + 2 * p;
        L.y[(size_t)m * L.N + r] = pq::bf16_rne(va);
        if (r + 1 < br.re) L.y[(size_t)m * L.N + r + 1] = pq::bf16_rne(vb);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA path (K % 256 == 0).
//
// The dot products run on the matrix cores as D = A * B with
// v_mfma_f32_16x16x32_bf16, arranged "transposed":
//   * B (32 k x 16 columns) holds the weights of 16 rows: lane l feeds row
//     l % 16 with the 8 k of one nibble dword of the group picked by its lane
//     group q = l / 16, unpacked to (1 + n/16) pairs;
//   * A (16 rows x 32 k) holds x: A row i = 4 m' + q' is token m' and group
//     slot q'; its k entries are x where q' equals the lane group q that
//     carries them and zero elsewhere.
// Each output lane l then holds, for token l / 16 and weight row l % 16, the
// four per-group partial sums sum_k (1 + n/16) x of one 4-group window, so
// the fp16 group scales (the lane's own row) apply per lane with no cross-lane
// reduction.  The offset 1.5 * sum x is a second MFMA chain on the same A with
// every weight equal to 1.5: identical operand positions, so a group whose
// codes are all 8 gives exactly zero.
//
// Work is split stream-K style: the (16-row block, 256-k chunk) units of the
// whole matrix are dealt to all waves of the grid in order.  A row block
// covered by one wave is finished by it; one cut between waves is combined at
// the end of their streams (partials through the workspace, an arrival counter
// per block, the last arriver adds the parts in wave order), so the load ring
// never waits for a store.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kRB = 16;          // weight rows per tile
constexpr int kGroupsPerStep = 8;  // 256 k = 128 bytes of each row per step
constexpr int kKStep = kGroupsPerStep * kGroup;
constexpr int kMXPre = 4;        // 16-byte x pieces per thread loaded before the ring

struct Q4MArgs {
  const uint16_t* x;
  const uint8_t* w;
  const uint16_t* wsc;
  uint16_t* y;
  float* part;       // [waves][2][SETS * NROW][64]
  uint32_t* cnt;     // [nrb]
  int M, K, N, R;
  int nrb, nkc, U;   // row blocks, k steps per row block, units = nrb * nkc
};

__device__ __forceinline__ floatx4 mfma16(uint4 a, uint4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// the 4 bf16 pairs of one nibble dword, in the order of the x pieces
__device__ __forceinline__ uint4 unpack8(uint32_t d, uint32_t one) {
  uint4 r;
  r.x = nib_pair<0>(d, one);
  r.y = nib_pair<1>(d, one);
  r.z = nib_pair<2>(d, one);
  r.w = nib_pair<3>(d, one);
  return r;
}

// wave whose unit range [split_start(U, T, w), split_start(U, T, w + 1)) holds u
__device__ __forceinline__ int wave_of(int u, int U, int T) {
  const int q = U / T, r = U - (U / T) * T;
  return u < r * (q + 1) ? u / (q + 1) : r + (u - r * (q + 1)) / q;
}

template <int NROW, int D, int MT>
__global__ __launch_bounds__(kThreads) void gemv_q4_mfma_kernel(Q4MArgs a) {
  constexpr int SETS = (MT + 3) / 4;          // A tiles of 4 tokens
  constexpr int NS = SETS * NROW;             // partial values per lane per segment
  extern __shared__ __align__(16) uint8_t smem[];
  uint4* xs_l = reinterpret_cast<uint4*>(smem);   // [MT*K/8] pieces, a dummy piece, a zero piece
  const int nx = MT * a.K / 8;
  const int zero_piece = nx + 1;

  const int tid = (int)threadIdx.x;
  const int lane = pq::lane_id();
  const int T = (int)gridDim.x * kWaves;
  const int gw = __builtin_amdgcn_readfirstlane((int)blockIdx.x * kWaves + pq::wave_id());
  const int u0 = pq::split_start(a.U, T, gw);
  const int nsteps = pq::split_start(a.U, T, gw + 1) - u0;

  // activation loads first, then a plain barrier, then the weight ring
  const pq::rsrc_t xr = pq::make_rsrc(a.x, (uint32_t)(MT * a.K * 2));
  uint4 xpre[kMXPre];
#pragma unroll
  for (int i = 0; i < kMXPre; ++i) {
    const int p = tid + i * kThreads;
    xpre[i] = pq::buf_load16(xr, p < nx ? (uint32_t)p * 16u : pq::kOOB);
  }
  __builtin_amdgcn_s_barrier();

  const uint32_t rowb = (uint32_t)(a.K / 2);
  const int ng = a.K / kGroup;
  const pq::rsrc_t wr = pq::make_rsrc(a.w, (uint32_t)((size_t)a.N * rowb));
  const pq::rsrc_t sr = pq::make_rsrc(a.wsc, (uint32_t)((size_t)a.N * ng * 2));
  const int rl = lane & 15, lq = lane >> 4;

  uint4 wbuf[D][NROW][2];
  uint4 sbuf[D][NROW];
  int irb = u0 / a.nkc, ikc = u0 - (u0 / a.nkc) * a.nkc, left = nsteps;
  auto issue = [&](uint4 (&wb)[NROW][2], uint4 (&sb)[NROW]) {
    const int row = irb * kRB + rl;
    const bool ok = left > 0 && row < a.R;
#pragma unroll
    for (int j = 0; j < NROW; ++j) {
      const uint32_t grow = (uint32_t)(row + j * a.R);
      const uint32_t off = grow * rowb + (uint32_t)ikc * 128u + 16u * (uint32_t)lq;
      wb[j][0] = pq::buf_load16_nt(wr, ok ? off : pq::kOOB);
      wb[j][1] = pq::buf_load16_nt(wr, ok ? off + 64u : pq::kOOB);
      sb[j] = pq::buf_load16_nt(sr, ok ? (grow * (uint32_t)ng + (uint32_t)ikc * kGroupsPerStep) * 2u : pq::kOOB);
    }
    --left;
    if (++ikc == a.nkc) { ikc = 0; ++irb; }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) issue(wbuf[d], sbuf[d]);
  __builtin_amdgcn_sched_barrier(0);

  // stage x in the paired order (threads without a piece write the dummy)
#pragma unroll
  for (int i = 0; i < kMXPre; ++i) {
    const int p = tid + i * kThreads;
    xs_l[p < nx ? p : nx] = pair_order(xpre[i]);
  }
  for (int p = tid + kMXPre * kThreads; p < nx; p += kThreads) xs_l[p] = pair_order(pq::buf_load16(xr, (uint32_t)p * 16u));
  if (tid == 0) xs_l[zero_piece] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();

  // this lane's A row: token 4 s + (lane % 16) / 4, group slot lane % 4; it
  // carries x only where the slot equals its lane group
  int abase[SETS];
#pragma unroll
  for (int s = 0; s < SETS; ++s) {
    const int m = 4 * s + (rl >> 2);
    abase[s] = ((rl & 3) == lq && m < MT) ? m * (a.K / 8) + 4 * lq : -1;
  }
  const uint32_t one = one_pair_reg();
  const uint32_t th = one_pair_reg() + 0x00400040u;   // (1.5, 1.5)
  const uint4 b15 = make_uint4(th, th, th, th);

  float acc[SETS][NROW], st0[SETS][NROW], st1[SETS][NROW];
#pragma unroll
  for (int s = 0; s < SETS; ++s)
#pragma unroll
    for (int j = 0; j < NROW; ++j) acc[s][j] = st0[s][j] = st1[s][j] = 0.0f;
  bool has0 = false, has1 = false;
  const int rb_first = u0 / a.nkc;
  const int rb_last = nsteps > 0 ? (u0 + nsteps - 1) / a.nkc : rb_first;

  auto output = [&](int rb, const float (&v)[SETS][NROW]) {
    const int row = rb * kRB + rl;
#pragma unroll
    for (int s = 0; s < SETS; ++s) {
      const int m = 4 * s + lq;
      if (m < MT && row < a.R) {
        const float g = 16.0f * v[s][0];
        a.y[(size_t)m * a.R + row] = pq::bf16_rne(NROW == 2 ? silu_mul(g, 16.0f * v[s][NROW - 1]) : g);
      }
    }
  };
  auto ncover = [&](int rb) {
    return wave_of((rb + 1) * a.nkc - 1, a.U, T) - wave_of(rb * a.nkc, a.U, T) + 1;
  };

  int crb = rb_first, ckc = u0 - rb_first * a.nkc;
  auto consume = [&](const uint4 (&wb)[NROW][2], const uint4 (&sb)[NROW], bool last) {
    const int g0 = ckc * kGroupsPerStep;
    float sc[NROW][8];
#pragma unroll
    for (int j = 0; j < NROW; ++j) {
      const uint32_t h[4] = {sb[j].x, sb[j].y, sb[j].z, sb[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc[j][2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(h[e] & 0xffffu));
        sc[j][2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(h[e] >> 16));
      }
    }
#pragma unroll
    for (int s = 0; s < SETS; ++s) {
#pragma unroll
      for (int win = 0; win < 2; ++win) {
        uint4 af[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) af[t] = xs_l[abase[s] >= 0 ? abase[s] + 4 * (g0 + 4 * win) + t : zero_piece];
        floatx4 dc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < 4; ++t) dc = mfma16(af[t], b15, dc);
#pragma unroll
        for (int j = 0; j < NROW; ++j) {
          const uint32_t dw[4] = {wb[j][win].x, wb[j][win].y, wb[j][win].z, wb[j][win].w};
          floatx4 dd = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int t = 0; t < 4; ++t) dd = mfma16(af[t], unpack8(dw[t], one), dd);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[s][j] = fmaf(dd[e] - dc[e], sc[j][4 * win + e], acc[s][j]);
        }
      }
    }
    if (ckc == a.nkc - 1 || last) {            // end of this wave's part of row block crb
      if (ncover(crb) == 1) {
        output(crb, acc);
      } else if (crb == rb_first) {
#pragma unroll
        for (int s = 0; s < SETS; ++s)
#pragma unroll
          for (int j = 0; j < NROW; ++j) st0[s][j] = acc[s][j];
        has0 = true;
      } else {
#pragma unroll
        for (int s = 0; s < SETS; ++s)
#pragma unroll
          for (int j = 0; j < NROW; ++j) st1[s][j] = acc[s][j];
        has1 = true;
      }
#pragma unroll
      for (int s = 0; s < SETS; ++s)
#pragma unroll
        for (int j = 0; j < NROW; ++j) acc[s][j] = 0.0f;
    }
    if (++ckc == a.nkc) { ckc = 0; ++crb; }
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

  // row blocks cut between waves: publish this wave's parts, then the last
  // covering wave to arrive adds all parts in wave order
  if (has0 || has1) {
    uint32_t* p32 = reinterpret_cast<uint32_t*>(a.part);
#pragma unroll
    for (int s = 0; s < SETS; ++s)
#pragma unroll
      for (int j = 0; j < NROW; ++j) {
        const int k = s * NROW + j;
        if (has0) pq::st_agent_u32(p32 + ((size_t)(gw * 2 + 0) * NS + k) * 64 + lane, __float_as_uint(st0[s][j]));
        if (has1) pq::st_agent_u32(p32 + ((size_t)(gw * 2 + 1) * NS + k) * 64 + lane, __float_as_uint(st1[s][j]));
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
      const int w0 = wave_of(rb * a.nkc, a.U, T);
      const int nc = ncover(rb);
      if (old == (uint32_t)(nc - 1)) {
        float v[SETS][NROW];
#pragma unroll
        for (int s = 0; s < SETS; ++s)
#pragma unroll
          for (int j = 0; j < NROW; ++j) v[s][j] = 0.0f;
        for (int wc = w0; wc < w0 + nc; ++wc) {
          const int slot = pq::split_start(a.U, T, wc) / a.nkc == rb ? 0 : 1;
#pragma unroll
          for (int s = 0; s < SETS; ++s)
#pragma unroll
            for (int j = 0; j < NROW; ++j)
              v[s][j] += __uint_as_float(pq::ld_agent_u32(p32 + ((size_t)(wc * 2 + slot) * NS + s * NROW + j) * 64 + lane));
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
constexpr size_t kMaxLds = 160 * 1024;

int check_shape(int M, int K, int N, int epi) {
  if (M < 1 || M > kMaxM || K < kGroup || K % kGroup != 0 || N < 1) return PQ_ERR_SHAPE;
  if (epi != PQ_EPI_NONE && epi != PQ_EPI_SILU_MUL) return PQ_ERR_SHAPE;
  if (epi == PQ_EPI_SILU_MUL && N % 2 != 0) return PQ_ERR_SHAPE;
  if ((long)M * K > kMaxMK) return PQ_ERR_SHAPE;
  if ((size_t)N * (K / 2) > pq::kMaxBufferBytes) return PQ_ERR_SHAPE;
  return PQ_OK;
}

// ---- vector path: packing linears into launches ----------------------------
int blocks_per_cu();

// LDS bytes of one linear in a launch at M tokens with G blocks: x pieces,
// group offsets and the partials of the block with the most row pairs.
size_t lin_lds_bytes(int M, int K, int R, int silu, int G) {
  const size_t rows = ((size_t)R + G - 1) / G;
  const size_t pairs = silu ? rows : (rows + 1) / 2;
  const size_t nch = ((size_t)K / 2 + kStepBytes - 1) / kStepBytes;
  return (size_t)M * K * 2 + (size_t)M * (K / kGroup) * 4 + pairs * nch * M * 2 * 4;
}
constexpr size_t kLinSlack = 64 + 16;   // the dummy piece and float, alignment
// dynamic LDS of the vector kernel: what its static segment table leaves
constexpr size_t kGroupStaticLds = sizeof(SegEntry) * kVWaves * kMaxLin;
constexpr size_t kGroupMaxDyn = kMaxLds - (kGroupStaticLds + 255) / 256 * 256;

template <int D, int MT, bool PAIR>
hipError_t launch_group_m(const Q4Group& a, size_t lds, int grid, hipStream_t stream) {
  auto kern = gemv_q4_kernel<D, MT, PAIR>;
  static pqhost::KernelAttrOnce attr;
  {
    hipError_t e = pqhost::set_dynamic_lds_once(attr, (const void*)kern, (int)kGroupMaxDyn);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kVThreads), lds, stream, a);
  return hipGetLastError();
}

template <int D, bool PAIR>
hipError_t launch_group_p(const Q4Group& a, int M, size_t lds, int grid, hipStream_t s) {
  switch (M) {
    case 1: return launch_group_m<D, 1, PAIR>(a, lds, grid, s);
    case 2: return launch_group_m<D, 2, PAIR>(a, lds, grid, s);
    case 3: return launch_group_m<D, 3, PAIR>(a, lds, grid, s);
    case 4: return launch_group_m<D, 4, PAIR>(a, lds, grid, s);
    case 5: return launch_group_m<D, 5, PAIR>(a, lds, grid, s);
    case 6: return launch_group_m<D, 6, PAIR>(a, lds, grid, s);
    case 7: return launch_group_m<D, 7, PAIR>(a, lds, grid, s);
    default: return launch_group_m<D, 8, PAIR>(a, lds, grid, s);
  }
}

// Validated linears [0, n) with one M: packed in order into launches of at
// most kMaxLin linears whose LDS fits one CU and whose groups-per-row parity
// agrees (the scale-load form).  The grid (PQ_BLOCKS_PER_CU blocks per CU)
// depends on the device only, so each linear's output bits do not depend on
// how the list is packed, nor on M.
// Consecutive launches of one grouped call alternate between the caller's
// stream and a second stream of the device (forked from the caller's stream
// and joined back to it by events), so that a launch's blocks start on the
// CUs that the previous launch's blocks free while its last blocks still run;
// the linears are independent and no block waits for another.  Created on
// the first grouped call on a device; the mutex keeps one call's fork,
// launches and join together when host threads call at once.  Not used when
// two outputs of the call overlap (the later linear's values then win, as
// with one stream) or when PQ_Q4_STREAMS=1.
struct PackStreams {
  std::once_flag once;
  hipError_t status = hipSuccess;
  hipStream_t aux = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};
PackStreams g_pack[pqhost::kMaxDevices];

PackStreams* pack_streams(int dev) {
  if (dev < 0 || dev >= pqhost::kMaxDevices) return nullptr;
  PackStreams& p = g_pack[dev];
  std::call_once(p.once, [&] {
    p.status = hipStreamCreateWithFlags(&p.aux, hipStreamNonBlocking);
    if (p.status == hipSuccess) p.status = hipEventCreateWithFlags(&p.fork, hipEventDisableTiming);
    if (p.status == hipSuccess) p.status = hipEventCreateWithFlags(&p.join, hipEventDisableTiming);
  });
  return p.status == hipSuccess ? &p : nullptr;
}

// Whether two outputs of the call overlap (taken as true beyond 1024 linears,
// where the pairwise check would cost more than the second stream saves).
bool outputs_overlap(const pq_q4_linear* lin, int n, int M) {
  if (n > 1024) return true;
  auto range = [&](int i, uintptr_t& b, uintptr_t& e) {
    const size_t n_out = lin[i].epi == PQ_EPI_SILU_MUL ? (size_t)lin[i].N / 2 : (size_t)lin[i].N;
    b = reinterpret_cast<uintptr_t>(lin[i].y);
    e = b + (size_t)M * n_out * 2;
  };
  for (int i = 0; i < n; ++i) {
    uintptr_t bi, ei;
    range(i, bi, ei);
    for (int j = i + 1; j < n; ++j) {
      uintptr_t bj, ej;
      range(j, bj, ej);
      if (bi < ej && bj < ei) return true;
    }
  }
  return false;
}

// Packs the linears, in order, into launches whose LDS fits one CU and calls
// launch(group, lds bytes, pair, index) for each; returns the number of packs
// or the first error.
template <class Launch>
int for_each_pack(const pq_q4_linear* lin, int n, int M, int grid, Launch launch) {
  int made = 0;
  for (int i0 = 0; i0 < n;) {
    Q4Group g;
    memset(&g, 0, sizeof(g));
    const bool pair = (lin[i0].K / kGroup) % 2 == 0;
    size_t pieces = 0, floats = 0;      // x pieces (16 B) and floats, before the partials
    size_t xbytes = 0, cbytes = 0, pbytes = 0;
    int i1 = i0;
    for (; i1 < n && i1 - i0 < kMaxLin; ++i1) {
      const pq_q4_linear& L = lin[i1];
      if (((L.K / kGroup) % 2 == 0) != pair) break;
      const int silu = L.epi == PQ_EPI_SILU_MUL;
      const int R = silu ? L.N / 2 : L.N;
      const size_t x = (size_t)M * L.K * 2, c = (size_t)M * (L.K / kGroup) * 4;
      const size_t pb = lin_lds_bytes(M, L.K, R, silu, grid) - x - c;
      if (xbytes + x + cbytes + c + pbytes + pb + kLinSlack > kGroupMaxDyn) break;
      xbytes += x;
      cbytes += c;
      pbytes += pb;
    }
    if (i1 == i0) return PQ_ERR_SHAPE;   // one linear alone does not fit
    // layout: all x pieces, the dummy piece, then floats: group offsets, the dummy float, partials
    g.n = i1 - i0;
    for (int i = i0; i < i1; ++i) {
      const pq_q4_linear& L = lin[i];
      Q4Lin& q = g.lin[i - i0];
      q.x = L.x; q.w = L.w; q.wsc = L.w_scale; q.y = L.y;
      q.K = L.K; q.N = L.N;
      q.silu = L.epi == PQ_EPI_SILU_MUL;
      q.R = q.silu ? L.N / 2 : L.N;
      q.ng = L.K / kGroup;
      q.nch = (int)((L.K / 2 + kStepBytes - 1) / kStepBytes);
      q.xoff = (int)pieces;
      pieces += (size_t)M * L.K / 8;
    }
    g.dummy_piece = (int)pieces;
    floats = (pieces + 1) * 4;
    for (int i = 0; i < g.n; ++i) {
      Q4Lin& q = g.lin[i];
      q.soff = (int)floats;
      floats += (size_t)M * q.ng;
    }
    g.dummy_float = (int)floats++;
    for (int i = 0; i < g.n; ++i) {
      Q4Lin& q = g.lin[i];
      q.poff = (int)floats;
      floats += lin_lds_bytes(M, q.K, q.R, q.silu, grid) / 4 - (size_t)M * q.K / 2 - (size_t)M * q.ng;
    }
    const size_t lds = floats * 4;
    if (lds > kGroupMaxDyn) return PQ_ERR_SHAPE;
    const int st = launch(g, lds, pair, made);
    if (st != PQ_OK) return st;
    ++made;
    i0 = i1;
  }
  return made;
}

// The number of launches the packing makes (the same loop, nothing launched).
int count_packs(const pq_q4_linear* lin, int n, int M, int grid) {
  return for_each_pack(lin, n, M, grid, [](const Q4Group&, size_t, bool, int) { return (int)PQ_OK; });
}

int run_vector_group(const pq_q4_linear* lin, int n, int M, int num_cus, int device, hipStream_t stream,
                     int* launches) {
  const int grid = num_cus * blocks_per_cu();
  const int npacks = count_packs(lin, n, M, grid);
  if (npacks < 0) return npacks;                   // a linear that does not fit: nothing launched
  const char* ns = getenv("PQ_Q4_STREAMS");
  PackStreams* ps = nullptr;
  if (npacks >= 2 && !(ns && strcmp(ns, "1") == 0) && !outputs_overlap(lin, n, M)) ps = pack_streams(device);
  std::unique_lock<std::mutex> lock;
  if (ps) {
    lock = std::unique_lock<std::mutex>(ps->mu);
    PQ_HIP_CHECK(hipEventRecord(ps->fork, stream));
    PQ_HIP_CHECK(hipStreamWaitEvent(ps->aux, ps->fork, 0));
  }
  hipError_t err = hipSuccess;
  const int made = for_each_pack(lin, n, M, grid, [&](const Q4Group& g, size_t lds, bool pair, int k) {
    const hipStream_t s = ps && (k & 1) ? ps->aux : stream;
    // ring depth: 2 steps of two 1 KB row chunks in flight per wave (64 KB
    // per CU; 3 steps spill at 1024 threads)
    err = pair ? launch_group_p<2, true>(g, M, lds, grid, s) : launch_group_p<2, false>(g, M, lds, grid, s);
    return err == hipSuccess ? (int)PQ_OK : (int)PQ_ERR_HIP;
  });
  if (ps) {   // join even after a failed launch, so the caller's stream stays ordered after the aux work
    const hipError_t e1 = hipEventRecord(ps->join, ps->aux);
    const hipError_t e2 = e1 == hipSuccess ? hipStreamWaitEvent(stream, ps->join, 0) : e1;
    if (err == hipSuccess) err = e2;
  }
  if (err != hipSuccess) {
    pqhost::set_last_hip_error((int)err);
    return PQ_ERR_HIP;
  }
  if (made < 0) return made;
  if (launches) *launches = made;
  return PQ_OK;
}

// ---- MFMA path -----------------------------------------------------------
int blocks_per_cu() {
  const char* env = getenv("PQ_BLOCKS_PER_CU");
  return env && atoi(env) > 0 ? atoi(env) : 1;
}

// The matrix-core kernel needs K % 256 == 0 and one counter per 16-row tile.
// By default it serves M >= 5, where the vector kernel's dot products
// dominate; below that the vector kernel is faster on MI355X (measured on the
// 5120 / 2 x 17408 / 17408 dense-stack shapes).  PQ_Q4_PATH=valu or =mfma
// forces one of them (mfma only where its conditions hold).
bool use_mfma(int M, int K, int R) {
  if (K % kKStep != 0 || (size_t)((R + kRB - 1) / kRB) > pq::kWsMaxCounters) return false;
  const char* env = getenv("PQ_Q4_PATH");
  if (env && strcmp(env, "valu") == 0) return false;
  if (env && strcmp(env, "mfma") == 0) return true;
  // From five tokens the vector kernel is dot-product bound on every shape; at
  // four it still wins on small layers (5120x5120: 13.4 vs 16.5 us) and loses
  // on large ones (17408x2x5120 with SiLU*up: 44.1 vs 37.4 us), where the
  // matrix kernel's fixed stream-K cost is amortised.
  return M >= 5 || (M == 4 && (size_t)R * K >= ((size_t)48 << 20));
}

// grid (blocks) and workspace bytes of the MFMA path
void mfma_plan(int M, int R, int nrow, int num_cus, int* grid, size_t* ws) {
  *grid = num_cus * blocks_per_cu();
  const int sets = (M + 3) / 4;
  *ws = pq::kWsDataOff + (size_t)(*grid) * kWaves * 2 * sets * nrow * 64 * sizeof(float);
}

template <int NROW, int D, int MT>
hipError_t launch_mfma_m(const Q4MArgs& a, int grid, hipStream_t stream) {
  auto kern = gemv_q4_mfma_kernel<NROW, D, MT>;
  static pqhost::KernelAttrOnce attr;
  {
    hipError_t e = pqhost::set_dynamic_lds_once(attr, (const void*)kern, (int)kMaxLds);
    if (e != hipSuccess) return e;
  }
  const size_t lds = ((size_t)a.M * a.K / 8 + 2) * 16;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

template <int NROW, int D>
hipError_t launch_mfma(const Q4MArgs& a, int grid, hipStream_t s) {
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

}  // namespace

extern "C" {

size_t pq_gemv_q4_workspace(int M, int K, int N, int epi) {
  if (check_shape(M, K, N, epi) != PQ_OK) return 0;
  const int R = epi == PQ_EPI_SILU_MUL ? N / 2 : N;
  if (!use_mfma(M, K, R)) return 0;
  pqhost::DeviceInfo dev;
  if (pqhost::current_device_info(&dev) != PQ_OK) return 0;
  int grid;
  size_t ws;
  mfma_plan(M, R, epi == PQ_EPI_SILU_MUL ? 2 : 1, dev.num_cus, &grid, &ws);
  return ws;
}

int pq_gemv_q4(const uint16_t* x, int M, int K, const uint8_t* w, const uint16_t* w_scale, int N, int epi,
               uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !w || !w_scale || !y) return PQ_ERR_NULL;
  int st = check_shape(M, K, N, epi);
  if (st != PQ_OK) return st;
  if (!pqhost::aligned16(x) || !pqhost::aligned16(w) || !pqhost::aligned16(w_scale) || !pqhost::aligned16(y) ||
      (ws && !pqhost::aligned16(ws)))
    return PQ_ERR_ALIGN;
  pqhost::DeviceInfo dev;
  st = pqhost::current_device_info(&dev);
  if (st != PQ_OK) return st;
  const int R = epi == PQ_EPI_SILU_MUL ? N / 2 : N;
  hipError_t e;
  if (use_mfma(M, K, R)) {
    int grid;
    size_t need;
    mfma_plan(M, R, epi == PQ_EPI_SILU_MUL ? 2 : 1, dev.num_cus, &grid, &need);
    if (ws == nullptr || ws_bytes < need) return PQ_ERR_WORKSPACE;
    Q4MArgs a;
    a.x = x; a.w = w; a.wsc = w_scale; a.y = y;
    a.cnt = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(ws) + pq::kWsCounterOff);
    a.part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + pq::kWsDataOff);
    a.M = M; a.K = K; a.N = N; a.R = R;
    a.nrb = (R + kRB - 1) / kRB;
    a.nkc = K / kKStep;
    a.U = a.nrb * a.nkc;
    // ring depths (256-k steps in flight per wave): 2 with two rows per tile
    // step, 3 with one; deeper rings were slower (17408->5120 M=4: 24.8 us at
    // 3, 27.5 at 8; SiLU*up 5120->2x17408 M=8: 38.1 at 2, 39.5 at 4)
    e = epi == PQ_EPI_SILU_MUL ? launch_mfma<2, 2>(a, grid, (hipStream_t)stream)
                               : launch_mfma<1, 3>(a, grid, (hipStream_t)stream);
  } else {
    pq_q4_linear one;
    one.x = x; one.w = w; one.w_scale = w_scale; one.y = y;
    one.K = K; one.N = N; one.epi = epi;
    return run_vector_group(&one, 1, M, dev.num_cus, dev.device, (hipStream_t)stream, nullptr);
  }
  if (e != hipSuccess) {
    pqhost::set_last_hip_error((int)e);
    return PQ_ERR_HIP;
  }
  return PQ_OK;
}

int pq_gemv_q4_group(const pq_q4_linear* linears, int n, int M, int* launches, void* stream) {
  if (launches) *launches = 0;
  if (n < 0) return PQ_ERR_SHAPE;
  if (n > 0 && !linears) return PQ_ERR_NULL;
  for (int i = 0; i < n; ++i) {
    const pq_q4_linear& L = linears[i];
    if (!L.x || !L.w || !L.w_scale || !L.y) return PQ_ERR_NULL;
    const int st = check_shape(M, L.K, L.N, L.epi);
    if (st != PQ_OK) return st;
    if (!pqhost::aligned16(L.x) || !pqhost::aligned16(L.w) || !pqhost::aligned16(L.w_scale) ||
        !pqhost::aligned16(L.y))
      return PQ_ERR_ALIGN;
  }
  if (n == 0) return PQ_OK;
  pqhost::DeviceInfo dev;
  const int st = pqhost::current_device_info(&dev);
  if (st != PQ_OK) return st;
  return run_vector_group(linears, n, M, dev.num_cus, dev.device, (hipStream_t)stream, launches);
}

}  // extern "C"
