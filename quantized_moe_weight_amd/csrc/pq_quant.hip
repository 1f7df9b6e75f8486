// Standalone block quantisers: FP8 E4M3 with one fp32 scale per 128 values of
// a row (weight encoding, and the live activation rule on its own), and
// symmetric int4 with one fp16 scale per 32 values.
#include "pq_quant_dev.h"

namespace {

constexpr int kThreads = 256;

// One thread per 8 consecutive values; 16 lanes per 128-block.
template <bool F32_IN>
__global__ __launch_bounds__(kThreads) void quantize_fp8_kernel(const void* in, long total8, int K,
                                                                 uint8_t* codes, float* scales) {
  const long t = (long)blockIdx.x * kThreads + threadIdx.x;
  const bool valid = t < total8;
  float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (valid) {
    if (F32_IN) {
      const float4* p = reinterpret_cast<const float4*>(in) + 2 * t;
      const float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      pq::bf16x8_to_f32(reinterpret_cast<const uint4*>(in)[t], v);
    }
  }
  const float s = pq::fp8_block_scale16(v, valid);       // all lanes take part in the shuffle
  if (!valid) return;
  reinterpret_cast<uint2*>(codes)[t] = pq::fp8_codes8(v, s);
  if ((threadIdx.x & 15) == 0) scales[(t * 8) / pq::kBlock] = s;
}

// One thread per 8 consecutive values; 4 lanes per 32-group.
__global__ __launch_bounds__(kThreads) void quantize_q4_kernel(const float* w, long total8,
                                                               uint8_t* packed, uint16_t* scales) {
  const long t = (long)blockIdx.x * kThreads + threadIdx.x;
  const bool valid = t < total8;
  float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (valid) {
    const float4* p = reinterpret_cast<const float4*>(w) + 2 * t;
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = pq::group_max(m, 4);
  if (!valid) return;
  const _Float16 s16 = (_Float16)(m / 7.0f);            // IEEE fp32 division, then RNE to fp16
  const float s = (float)s16;
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float q = 0.0f;
    if (s > 0.0f) {
      q = __builtin_rintf(v[i] / s);                     // IEEE fp32 division, RNE
      q = fminf(fmaxf(q, -8.0f), 7.0f);
      if (!(q == q)) q = 0.0f;
    }
    word |= ((uint32_t)((int)q + 8) & 0xFu) << (4 * i);  // element 2j in the low nibble of byte j
  }
  reinterpret_cast<uint32_t*>(packed)[t] = word;
  if ((threadIdx.x & 3) == 0) scales[(t * 8) / 32] = __builtin_bit_cast(uint16_t, s16);
}

}  // namespace

extern "C" {

int pq_quantize_fp8(const void* in, int in_is_f32, int rows, int K, uint8_t* codes, float* scales,
                    void* stream) {
  if (!in || !codes || !scales) return PQ_ERR_NULL;
  if (rows < 1 || K < pq::kBlock || K % pq::kBlock != 0) return PQ_ERR_SHAPE;
  if (!pqhost::aligned16(in) || !pqhost::aligned16(codes) || !pqhost::aligned16(scales)) return PQ_ERR_ALIGN;
  pqhost::DeviceInfo dev;
  int st = pqhost::current_device_info(&dev);
  if (st != PQ_OK) return st;
  const long total8 = (long)rows * K / 8;
  const long blocks = (total8 + kThreads - 1) / kThreads;
  if (in_is_f32)
    hipLaunchKernelGGL(quantize_fp8_kernel<true>, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                       in, total8, K, codes, scales);
  else
    hipLaunchKernelGGL(quantize_fp8_kernel<false>, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                       in, total8, K, codes, scales);
  PQ_HIP_CHECK(hipGetLastError());
  return PQ_OK;
}

int pq_quantize_q4(const float* w, int N, int K, uint8_t* packed, uint16_t* scales, void* stream) {
  if (!w || !packed || !scales) return PQ_ERR_NULL;
  if (N < 1 || K < 32 || K % 32 != 0) return PQ_ERR_SHAPE;
  if (!pqhost::aligned16(w) || !pqhost::aligned16(packed) || !pqhost::aligned16(scales)) return PQ_ERR_ALIGN;
  pqhost::DeviceInfo dev;
  int st = pqhost::current_device_info(&dev);
  if (st != PQ_OK) return st;
  const long total8 = (long)N * K / 8;
  const long blocks = (total8 + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(quantize_q4_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream, w, total8,
                     packed, scales);
  PQ_HIP_CHECK(hipGetLastError());
  return PQ_OK;
}

}  // extern "C"
