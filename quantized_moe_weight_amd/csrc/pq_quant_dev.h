// Device-side block quantisers shared by the standalone quantisers, the live
// activation prologue of the GEMV kernels and the h re-quantisation of the MoE
// layer.  Each thread owns 8 consecutive values of a row; 16 adjacent lanes
// therefore cover one 128-wide FP8 block (4 lanes one 32-wide int4 group).
#pragma once

#include "pq_common.h"

namespace pq {

// 8 bf16 values (one 16-byte load) -> fp32
__device__ __forceinline__ void bf16x8_to_f32(uint4 raw, float v[8]) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// FP8-quantise 8 values of one 128-block given the block scale s.
// Returns the 8 codes packed little-endian.
__device__ __forceinline__ uint2 fp8_codes8(const float v[8], float s) {
  const double r = 1.0 / (double)s;
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = quotient_f32(v[i], r);
  uint2 out;
  out.x = e4m3_pack2<true>(q[2], q[3], e4m3_pack2<false>(q[0], q[1], 0u));
  out.y = e4m3_pack2<true>(q[6], q[7], e4m3_pack2<false>(q[4], q[5], 0u));
  return out;
}

// Block amax over the 16 lanes that share a 128-block (lanes aligned to 16),
// then the block scale.  `valid` lanes contribute their |v|; all lanes must call.
__device__ __forceinline__ float fp8_block_scale16(const float v[8], bool valid) {
  float m = 0.0f;
  if (valid) {
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  m = group_max(m, 16);
  return block_scale(m);
}

}  // namespace pq
