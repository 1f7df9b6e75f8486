// Shared device and host helpers of the gfx950 decode library.
//
// Device side: the FP8 E4M3FN encoder used by every live quantisation, the
// bf16 rounding of outputs, the FP8 x FP8 16-element block dot product on
// v_dot2 bf16 pairs, 64-lane wavefront reductions and the agent-scope
// release/acquire helpers used by the single-launch kernels.
// Host side: status codes, per-thread HIP error, device-property cache.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "../../include/pq.h"

namespace pq {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 128;        // FP8 scale block along K
constexpr int kChunk = 1024;       // bytes of one weight row covered by one wave load (64 lanes x 16 B)
constexpr float kE4M3Max = 448.0f;

// ---------------------------------------------------------------------------
// Live FP8 quantisation.
//
// The rule (scale s = fp32(amax/448), code = E4M3(fp32(v/s)), ties to even,
// saturating) is the reading taken of [Sionic] §1's live FP8 activation
// quantisation with one scale per 128-wide K block ([Sionic] §2).
// ---------------------------------------------------------------------------

// fp32 -> E4M3FN byte, round to nearest even, |v| >= 448 (and inf) saturate,
// NaN -> 0x7F.  Integer/rounding ops only; no fast-math.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7Fu;                  // NaN
  if (a >= 0x43e00000u) return sign | 0x7Eu;          // >= 448: satfinite
  uint32_t code;
  if (a < 0x3c800000u) {                              // < 2^-6: subnormal grid of 2^-9
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);   // exact scale, RNE
  } else {                                            // 3-bit mantissa, RNE
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);                   // exponent bias 127 -> 7
    code = code > 0x7Eu ? 0x7Eu : code;
  }
  return sign | code;
}

// Hardware form of the same encoding for two values at once: clamp to
// [-448, 448], then v_cvt_pk_fp8_f32 (round to nearest even).  Checked on
// MI355X against e4m3_encode for every non-NaN fp32 bit pattern (no
// mismatch); the quantisers only feed it finite quotients.  The two codes
// land in bytes [0,1] (HI = false) or [2,3] (HI = true) of `old`.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b, uint32_t old) {
  a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
  b = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// Correctly rounded fp32 quotient v / s for a shared divisor: with
// r = fp64(1/s), fp32(fp64(v * r)) equals the IEEE fp32 quotient for every
// fp32 v and positive fp32 s (the quotient of two 24-bit values is never an
// fp32 rounding midpoint and lies at least 2^-49 (relative) away from one,
// while the fp64 product is within 2^-52).  One fp64 divide per block
// instead of one fp32 divide per element.
__device__ __forceinline__ float quotient_f32(float v, double r) {
  return (float)((double)v * r);
}

__device__ __forceinline__ float block_scale(float amax) {
  return amax == 0.0f ? 1.0f : amax / kE4M3Max;       // IEEE fp32 division
}

// ---------------------------------------------------------------------------
// Output rounding
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((b >> 16) | 0x40u);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// ---------------------------------------------------------------------------
// FP8 x FP8 dot products.  Both operands are E4M3 codes; every E4M3 value is
// exact in bf16, so each pair of bytes is widened to a bf16 pair by the
// hardware converter and multiplied-accumulated by v_dot2 (exact products,
// fp32 accumulation).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x2 fp8x2_lo(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
}
__device__ __forceinline__ bf16x2 fp8x2_hi(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
}

struct Bf16x16 { bf16x2 v[8]; };

__device__ __forceinline__ Bf16x16 widen16(uint4 c) {
  Bf16x16 r;
  r.v[0] = fp8x2_lo(c.x); r.v[1] = fp8x2_hi(c.x);
  r.v[2] = fp8x2_lo(c.y); r.v[3] = fp8x2_hi(c.y);
  r.v[4] = fp8x2_lo(c.z); r.v[5] = fp8x2_hi(c.z);
  r.v[6] = fp8x2_lo(c.w); r.v[7] = fp8x2_hi(c.w);
  return r;
}

// sum of the 16 products of one lane's 16-byte slice
__device__ __forceinline__ float dot16(const Bf16x16& a, const Bf16x16& b) {
  float p = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) p = __builtin_amdgcn_fdot2_f32_bf16(a.v[j], b.v[j], p, false);
  return p;
}

// ---------------------------------------------------------------------------
// Raw buffer loads.  The descriptor lives in SGPRs (one per tensor), the
// per-lane offset is 32-bit, and an offset at or beyond the descriptor's size
// returns zeros without touching memory: masked lanes and drained pipeline
// slots issue loads unconditionally, which keeps the load stream free of
// branches so the compiler can count outstanding loads statically.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;            // any offset >= this is out of range
constexpr uint32_t kMaxBufferBytes = 0x7FFFFFF0u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
// Streaming (non-temporal) variants for weights and scales, read once per call:
// the nt policy keeps them from displacing reusable lines and measured ~13%
// more read bandwidth than the default policy on MI355X.
constexpr int kAuxNT = 2;
__device__ __forceinline__ uint4 buf_load16_nt(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kAuxNT));
}
__device__ __forceinline__ float buf_load_f32_nt(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kAuxNT));
}

// ---------------------------------------------------------------------------
// Buffer-to-LDS loads: lane l's bytes land at LDS byte address lds + l * size,
// read from byte offset voff + soff of the buffer (voff per lane, soff
// wave-uniform; a lane whose offset is past the buffer's size loads zeros).
// They are written as assembly on purpose: the compiler's wait insertion does
// not know which LDS reads depend on which of these loads and would wait for
// every one of them before any LDS read.  Callers order them themselves; all
// vector-memory loads of a wave complete in issue order, so once a load issued
// after one of these has returned (a wait the compiler inserts for its use),
// the LDS bytes are in place.
// ---------------------------------------------------------------------------
typedef int int32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

// A raw buffer resource (stride 0, num_records = bytes) as four scalar words.
__device__ __forceinline__ int32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  return int32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)p), __builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32)),
                 __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(size_t)(lds_ptr)p);
}
__device__ __forceinline__ void dma16(int32x4 r, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(r), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ void dma4(int32x4 r, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(r), "s"(soff) : "memory", "m0");
}
// dma4 that leaves M0 as it found it (the compiler does not track M0 across
// inline assembly, so kernels that may keep a value there use this one).  The
// scalar operands pass through readfirstlane (they are wave-uniform; this
// keeps them in scalar registers where the compiler cannot prove it).
__device__ __forceinline__ void dma4_keep_m0(int32x4 r, uint32_t lds, uint32_t voff, uint32_t soff) {
  uint32_t saved;
  const int32x4 rs = {__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
                      __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %2, %3, %4 offen lds\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved)
               : "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)lds)), "v"(voff), "s"(rs),
                 "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)soff))
               : "memory");
}
// Two LDS dwords read once `dep` (a register a vector-memory load wrote) is
// available: the dependency makes the compiler wait for that load first, so
// the read sees what earlier buffer-to-LDS loads wrote; the read waits for
// itself in the same block.
__device__ __forceinline__ void lds_read2_after(uint32_t a0, uint32_t a1, uint32_t dep, float& v0, float& v1) {
  asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(v0), "=&v"(v1) : "v"(a0), "v"(a1), "v"(dep));
}

// ---------------------------------------------------------------------------
// Wavefront reductions.  wave_sum / wave_max_u32 reduce with DPP row shifts
// and row broadcasts into lane 63 (a fixed association order, so the result
// is deterministic) and return lane 63's value to every lane.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ int dpp_i32(int v) {
  // lanes whose source is outside the row, or that are masked off, read 0
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, BANK_MASK, true);
}
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, dpp_i32<CTRL, ROW_MASK, BANK_MASK>(__builtin_bit_cast(int, v)));
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr3 = 0x113, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

__device__ __forceinline__ float wave_sum(float v) {
  float t = v + dpp_f32<kRowShr1>(v);          // lane i: v[i-1] + v[i]   (within a 16-lane row)
  t += dpp_f32<kRowShr2>(v);                   //        ... + v[i-2]
  t += dpp_f32<kRowShr3>(v);                   //        ... + v[i-3]
  t += dpp_f32<kRowShr4, 0xf, 0xe>(t);         // lanes 4..15 of a row: 8-lane sums
  t += dpp_f32<kRowShr8, 0xf, 0xc>(t);         // lanes 8..15: 16-lane sums; lane 15 = row total
  t += dpp_f32<kRowBcast15, 0xa>(t);           // rows 1, 3 add the previous row's total
  t += dpp_f32<kRowBcast31, 0xc>(t);           // rows 2, 3 add lane 31 (rows 0 + 1)
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, t), 63));
}

// The value of lane l ^ d (d = 1 ... 32).  Quad permutes for 1 and 2; then
// either (LDS = true) the LDS crossbar (swizzle in bit mode within 32 lanes,
// a permute across the halves), or, without it: for 4, the row rotation by 4
// (lane l reads l - 4 within its 16-lane row) where bit 2 of l is set, by 12
// (l + 4) where it is clear; for 8, the row rotation by 8; for 16 and 32, the
// permlane swaps of the value with itself, which give every lane the other
// row of its row pair (other half of the wave) in one of their two results.
// Both read the same lane, so sums built on either have the same bits; the
// crossbar takes fewer vector instructions, the other form less latency.
template <int D, bool LDS = false>
__device__ __forceinline__ float xor_lane(float v) {
  const int iv = __builtin_bit_cast(int, v);
  const int lane = (int)(threadIdx.x & (kWave - 1));
  if constexpr (D == 1) return dpp_f32<0xB1>(v);                 // quad_perm [1,0,3,2]
  else if constexpr (D == 2) return dpp_f32<0x4E>(v);            // quad_perm [2,3,0,1]
  else if constexpr (LDS && D < 32) return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(iv, (D << 10) | 0x1F));
  else if constexpr (LDS) return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, iv));
  else if constexpr (D == 4) {
    const float down = dpp_f32<0x124>(v), up = dpp_f32<0x12C>(v);   // row_ror:4, row_ror:12
    return (lane & 4) ? down : up;
  } else if constexpr (D == 8) return dpp_f32<0x128>(v);         // row_ror:8
  else if constexpr (D == 16) {
    const auto s = __builtin_amdgcn_permlane16_swap(iv, iv, false, false);   // rows (0,0,2,2), (1,1,3,3)
    return __builtin_bit_cast(float, (lane & 16) ? (int)s[0] : (int)s[1]);
  } else {
    static_assert(D == 32, "d = 1, 2, 4, 8, 16 or 32");
    const auto s = __builtin_amdgcn_permlane32_swap(iv, iv, false, false);   // halves (lo, lo), (hi, hi)
    return __builtin_bit_cast(float, (lane & 32) ? (int)s[0] : (int)s[1]);
  }
}

// Wave sums of N values per lane (N a power of two, at most 64), all in one
// butterfly: at the stage of distance d = 2^s a lane keeps the half of its
// values whose index bit s equals its lane bit s and adds its partner's
// (lane l ^ d) copy of them, so each stage halves the values a lane holds;
// once one is left, the remaining distances add it as a plain butterfly.
// Lane l ends with the sum of value l mod N.  Every value is summed over the
// same tree of lane pairs (distances 1, 2, 4, ..., 32 in that order), whatever
// its index and N (each pair's sum is the same in either lane: addition
// commutes), so a row's sum does not depend on how many values share the
// reduction.
template <int N, bool LDS = false>
__device__ __forceinline__ float wave_sum_many(const float (&v)[N]) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N: a power of two up to 64");
  const int lane = (int)(threadIdx.x & (kWave - 1));
  float c[N];
#pragma unroll
  for (int i = 0; i < N; ++i) c[i] = v[i];
  auto stage = [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    constexpr int S = __builtin_ctz(D);
    if constexpr ((N >> S) > 1) {                 // c[k]: value (lane bits below S) | k << S
      const bool hi = (lane >> S) & 1;
#pragma unroll
      for (int i = 0; i < (N >> S) / 2; ++i) {
        const float keep = hi ? c[2 * i + 1] : c[2 * i];
        const float send = hi ? c[2 * i] : c[2 * i + 1];
        c[i] = keep + xor_lane<D, LDS>(send);
      }
    } else {
      c[0] = c[0] + xor_lane<D, LDS>(c[0]);
    }
  };
  stage(std::integral_constant<int, 1>{});
  stage(std::integral_constant<int, 2>{});
  stage(std::integral_constant<int, 4>{});
  stage(std::integral_constant<int, 8>{});
  stage(std::integral_constant<int, 16>{});
  stage(std::integral_constant<int, 32>{});
  return c[0];
}

// Butterfly sum of each aligned segment of `lanes` lanes (2 ... 64): the first
// stages of wave_sum_many's tree, so every lane of a segment ends with the sum
// its row would have alone in the wave (the later stages only add zeros).
// After the quad stages every lane of a quad holds the same bits (each pair's
// sum is the same in both lanes), so the 8- and 16-lane stages may take their
// partner from the row's mirror images instead of lane l ^ 4 and l ^ 8: the
// same two group sums are added, without the LDS crossbar.
__device__ __forceinline__ float segment_sum_xor(float v, int lanes) {
  constexpr int kRowMirror = 0x140, kRowHalfMirror = 0x141;
  v += xor_lane<1>(v);
  if (lanes >= 4) v += xor_lane<2>(v);
  if (lanes >= 8) v += dpp_f32<kRowHalfMirror>(v);
  if (lanes >= 16) v += dpp_f32<kRowMirror>(v);
  if (lanes >= 32) v += xor_lane<16>(v);
  if (lanes >= 64) v += xor_lane<32>(v);
  return v;
}

// Wave sums of the value pairs (a[t], b[t]), t < n (n <= TP, wave-uniform):
// one wave_sum_many over the smallest power of two of values that holds the
// 2n (the tree, and so every sum, is the same for any width), read back into
// every lane.
template <int TP>
__device__ __forceinline__ void wave_sum_pairs(const float (&a)[TP], const float (&b)[TP], int n, float (&ra)[TP],
                                               float (&rb)[TP]) {
  auto run = [&](auto wc) {
    constexpr int W = decltype(wc)::value;        // pairs in the reduction
    static_assert(W <= TP, "at most TP pairs");
    float v[2 * W];
#pragma unroll
    for (int t = 0; t < W; ++t) {
      v[2 * t] = a[t];
      v[2 * t + 1] = b[t];
    }
    const float s = wave_sum_many<2 * W>(v);    // lane 2t: a's sum, lane 2t + 1: b's
#pragma unroll
    for (int t = 0; t < TP; ++t) {
      ra[t] = rb[t] = 0.0f;
      if (t < W) {
        ra[t] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 2 * t));
        rb[t] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 2 * t + 1));
      }
    }
  };
  if (n <= 1 || TP == 1) run(std::integral_constant<int, 1>{});
  else if (n <= 2 || TP == 2) run(std::integral_constant<int, (TP < 2 ? TP : 2)>{});
  else if (n <= 4 || TP <= 4) run(std::integral_constant<int, (TP < 4 ? TP : 4)>{});
  else run(std::integral_constant<int, (TP < 8 ? TP : 8)>{});
}

// The same sums left where the butterfly puts them: lane 2t ends with a[t]'s
// sum and lane 2t + 1 with b[t]'s, for t < n (for callers whose lanes store
// their own results instead of reading them all back into scalar registers).
template <int TP>
__device__ __forceinline__ float wave_sum_pairs_lanes(const float (&a)[TP], const float (&b)[TP], int n) {
  auto run = [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    static_assert(W <= TP, "at most TP pairs");
    float v[2 * W];
#pragma unroll
    for (int t = 0; t < W; ++t) {
      v[2 * t] = a[t];
      v[2 * t + 1] = b[t];
    }
    return wave_sum_many<2 * W>(v);
  };
  if (n <= 1 || TP == 1) return run(std::integral_constant<int, 1>{});
  if (n <= 2 || TP == 2) return run(std::integral_constant<int, (TP < 2 ? TP : 2)>{});
  if (n <= 4 || TP <= 4) return run(std::integral_constant<int, (TP < 4 ? TP : 4)>{});
  return run(std::integral_constant<int, (TP < 8 ? TP : 8)>{});
}

template <bool B>
struct BoolC {                                       // a compile-time flag passed to a generic lambda
  static constexpr bool value = B;
};

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  uint32_t t = umax(v, (uint32_t)dpp_i32<kRowShr1>((int)v));
  t = umax(t, (uint32_t)dpp_i32<kRowShr2>((int)v));
  t = umax(t, (uint32_t)dpp_i32<kRowShr3>((int)v));
  t = umax(t, (uint32_t)dpp_i32<kRowShr4, 0xf, 0xe>((int)t));
  t = umax(t, (uint32_t)dpp_i32<kRowShr8, 0xf, 0xc>((int)t));
  t = umax(t, (uint32_t)dpp_i32<kRowBcast15, 0xa>((int)t));
  t = umax(t, (uint32_t)dpp_i32<kRowBcast31, 0xc>((int)t));
  return (uint32_t)__builtin_amdgcn_readlane((int)t, 63);
}

// Maximum within aligned groups of `width` lanes (4, 8 or 16), in every lane
// of the group, by DPP lane swaps inside a 16-lane row (no LDS permute):
// swap neighbours, then pairs, then mirror the halves of 8 and of 16 lanes.
// A maximum is the same value in any order.  Every lane of the wave calls it.
__device__ __forceinline__ float group_max(float v, int width) {
  constexpr int kQuadSwap1 = 0xB1, kQuadSwap2 = 0x4E;   // quad_perm [1,0,3,2], [2,3,0,1]
  constexpr int kRowMirror = 0x140, kRowHalfMirror = 0x141;
  v = fmaxf(v, dpp_f32<kQuadSwap1>(v));
  v = fmaxf(v, dpp_f32<kQuadSwap2>(v));
  if (width >= 8) v = fmaxf(v, dpp_f32<kRowHalfMirror>(v));
  if (width >= 16) v = fmaxf(v, dpp_f32<kRowMirror>(v));
  return v;
}

// First index of part i when n items are dealt to p parts as evenly as
// possible (the first n % p parts get one more), without 64-bit division.
__device__ __forceinline__ int split_start(int n, int p, int i) {
  const int q = n / p, r = n - (n / p) * p;
  return i * q + (i < r ? i : r);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x >> 6); }

// ---------------------------------------------------------------------------
// Cross-block synchronisation at agent (device) scope.  Blocks of one launch
// run on all 8 XCDs, whose L2 caches are separate: a producer publishes with
// a release fence before its counter update, a consumer acquires after
// observing the counter.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

__device__ __forceinline__ uint32_t atomic_add_relaxed(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_load_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Agent-coherent data exchange between blocks.  Values one block produces and
// another consumes within the same launch are stored and loaded with the
// agent-scope (sc1) cache policy, which keeps them coherent across the eight
// XCD L2 caches without writing back or invalidating the whole L2.  A
// producer makes its stores complete (wait_vm) before it bumps the counter a
// consumer polls; the consumer issues its loads only after observing it.
__device__ __forceinline__ void st_agent_u16(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait for every outstanding memory operation of this wave (stores
// acknowledged); also a compiler barrier for the surrounding atomics.
__device__ __forceinline__ void wait_vm() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Workspace layout shared by every kernel that synchronises across blocks:
//   [0, 256)                   WsHeader
//   [256, kWsZeroOff)          arrival counters (uint32), zero between calls
//   [kWsZeroOff, kWsDataOff)   values exchanged between blocks whose zero
//                              word means "not yet written", zero between calls
//   [kWsDataOff, ...)          per-call scratch data (always written before read)
// The regions never move, whatever the shape of the call, so the
// zero-between-calls invariant holds across calls of different shapes and
// different kernels on one workspace.
constexpr size_t kWsCounterOff = 256;
constexpr size_t kWsZeroOff = 65536;
constexpr size_t kWsZeroBytes = (size_t)2 << 20;
constexpr size_t kWsDataOff = kWsZeroOff + kWsZeroBytes;
constexpr size_t kWsMaxCounters = (kWsZeroOff - kWsCounterOff) / 4;

// Workspace header shared by the kernels that synchronise across blocks.
struct WsHeader {
  uint32_t error;       // first pq_status recorded by a kernel (0 = none)
  uint32_t done;        // phase counter of the running call
  uint32_t exit_count;  // blocks that finished the running call
  uint32_t reserved;    // unused (zero)
  uint32_t pad[60];     // keep the header one 256-byte line
};
static_assert(sizeof(WsHeader) == 256, "workspace header is one 256-byte line");

__device__ __forceinline__ void record_error(WsHeader* h, int status) {
  uint32_t expected = 0u;
  __hip_atomic_compare_exchange_strong(&h->error, &expected, (uint32_t)status,
                                       __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Spin until *ctr >= target; gives up after `limit` polls, recording
// PQ_ERR_TIMEOUT, so that every wave always reaches the end of the kernel.
__device__ __forceinline__ bool spin_wait_geq(const uint32_t* ctr, uint32_t target, WsHeader* h,
                                              uint32_t limit) {
  for (uint32_t it = 0; it < limit; ++it) {
    if (atomic_load_relaxed(ctr) >= target) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  record_error(h, PQ_ERR_TIMEOUT);
  return false;
}

// Wait until *flag == value.  Each waiting block polls its own flag line, so
// the polls do not contend with the atomics of the phase counter.
__device__ __forceinline__ bool spin_wait_eq(const uint32_t* flag, uint32_t value, WsHeader* h, uint32_t limit) {
  for (uint32_t it = 0; it < limit; ++it) {
    if (atomic_load_relaxed(flag) == value) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  record_error(h, PQ_ERR_TIMEOUT);
  return false;
}

}  // namespace pq

// ---------------------------------------------------------------------------
// Host helpers
// ---------------------------------------------------------------------------
namespace pqhost {

struct DeviceInfo {
  int device = -1;
  int num_cus = 0;
  bool gfx950 = false;
};

// Properties of the current device (cached per device id).
int current_device_info(DeviceInfo* out);

void set_last_hip_error(int e);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The dynamic-LDS limit of one kernel, raised once per device.  Host threads
// that make their first call at the same time all wait for the one setter
// (std::call_once), and every later call returns the recorded status.
constexpr int kMaxDevices = 64;
struct KernelAttrOnce {
  std::once_flag once[kMaxDevices];
  hipError_t status[kMaxDevices] = {};
};
inline hipError_t set_dynamic_lds_once(KernelAttrOnce& o, const void* kern, int bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(o.once[dev], [&] {
    o.status[dev] = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  });
  return o.status[dev];
}

__host__ __device__ inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace pqhost

#define PQ_HIP_CHECK(expr)                                  \
  do {                                                      \
    hipError_t _e = (expr);                                 \
    if (_e != hipSuccess) {                                 \
      pqhost::set_last_hip_error((int)_e);                  \
      return PQ_ERR_HIP;                                    \
    }                                                       \
  } while (0)
