// Streaming-read probe: the HBM read bandwidth this library's weight streams
// can reach on the device, measured with their load path — 128-bit
// non-temporal buffer loads, lane l reading bytes [16l, 16l+16) of each 1 KB
// wave step, a ring of steps in flight per lane, one persistent block per CU
// reading a contiguous share.  Loaded words are folded into a checksum that
// is stored, so no load can be dropped.  The shape is the fastest of a sweep
// on MI355X (4 GiB, threads per block x loads in flight per lane): 512 x 3
// (24 KB in flight per CU) 7.25-7.29 TB/s; 256 x 8 7.21; 512 x 4 7.15;
// 1024 x 2 7.05; 1024 x 8 (128 KB per CU) 6.81; 1024 x 1 6.15 — more bytes in
// flight per CU than about 32 KB lower the rate.
#include "pq_common.h"

namespace {

constexpr int kThreads = 512;
constexpr int kRing = 3;                              // 16-byte loads in flight per lane
constexpr uint32_t kStep = kThreads * 16u;            // bytes per block-wide step

__global__ __launch_bounds__(kThreads) void stream_probe_kernel(const uint8_t* src, size_t bytes, uint32_t* sink) {
  const size_t nvec = bytes / 16;
  const size_t per = (nvec + gridDim.x - 1) / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < nvec ? lo + per : nvec;
  const uint32_t share = lo < hi ? (uint32_t)((hi - lo) * 16) : 0u;
  const pq::rsrc_t r = pq::make_rsrc(src + lo * 16, share);
  const uint32_t tid16 = 16u * threadIdx.x;
  uint4 v[kRing];
#pragma unroll
  for (int j = 0; j < kRing; ++j) v[j] = pq::buf_load16_nt(r, (uint32_t)j * kStep + tid16);
  uint32_t acc = 0;
  for (uint32_t base = 0; base < share; base += kRing * kStep) {
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
      acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
      const uint32_t off = base + (uint32_t)(kRing + j) * kStep + tid16;    // past the share: zeros, no traffic
      v[j] = pq::buf_load16_nt(r, off < share ? off : pq::kOOB);
    }
  }
#pragma unroll
  for (int d = 1; d < pq::kWave; d <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, d, pq::kWave);
  if (pq::lane_id() == 0) sink[blockIdx.x * (kThreads / pq::kWave) + pq::wave_id()] = acc;
}

}  // namespace

extern "C" {

int pq_stream_probe(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return PQ_ERR_NULL;
  if (!pqhost::aligned16(src) || !pqhost::aligned16(sink)) return PQ_ERR_ALIGN;
  if (bytes == 0 || bytes % 16) return PQ_ERR_SHAPE;
  pqhost::DeviceInfo dev;
  int st = pqhost::current_device_info(&dev);
  if (st != PQ_OK) return st;
  if (dev.num_cus * (kThreads / pq::kWave) * sizeof(uint32_t) > 65536) return PQ_ERR_UNSUPPORTED;
  const size_t per = (bytes / 16 + dev.num_cus - 1) / dev.num_cus * 16;
  if (per > 0x7FF00000u) return PQ_ERR_SHAPE;            // one block's share must fit 31-bit offsets
  hipLaunchKernelGGL(stream_probe_kernel, dim3(dev.num_cus), dim3(kThreads), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint8_t*>(src), bytes, sink);
  PQ_HIP_CHECK(hipGetLastError());
  return PQ_OK;
}

}  // extern "C"
