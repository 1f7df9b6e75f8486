// Runtime helpers of the C ABI: status strings, per-thread HIP error, the
// device-property cache, workspace initialisation and checking.
#include <mutex>
#include <string.h>

#include "pq_common.h"

namespace pqhost {

static thread_local int g_last_hip_error = 0;

void set_last_hip_error(int e) { g_last_hip_error = e; }

int current_device_info(DeviceInfo* out) {
  static std::mutex mu;
  static DeviceInfo cache[64];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_last_hip_error((int)e);
    return PQ_ERR_UNSUPPORTED;
  }
  if (dev < 0 || dev >= 64) return PQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev].device != dev) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      set_last_hip_error((int)e);
      return PQ_ERR_HIP;
    }
    DeviceInfo d;
    d.device = dev;
    d.num_cus = prop.multiProcessorCount;
    d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    cache[dev] = d;
  }
  *out = cache[dev];
  return out->gfx950 ? PQ_OK : PQ_ERR_UNSUPPORTED;
}

}  // namespace pqhost

extern "C" {

const char* pq_strerror(int status) {
  switch (status) {
    case PQ_OK: return "PQ_OK";
    case PQ_ERR_NULL: return "PQ_ERR_NULL: a required pointer is NULL";
    case PQ_ERR_SHAPE: return "PQ_ERR_SHAPE: a size is out of range or not a required multiple";
    case PQ_ERR_ALIGN: return "PQ_ERR_ALIGN: a pointer is not 16-byte aligned";
    case PQ_ERR_WORKSPACE: return "PQ_ERR_WORKSPACE: workspace missing or too small";
    case PQ_ERR_UNSUPPORTED: return "PQ_ERR_UNSUPPORTED: no gfx950 device is current";
    case PQ_ERR_HIP: return "PQ_ERR_HIP: a HIP runtime call failed";
    case PQ_ERR_TIMEOUT: return "PQ_ERR_TIMEOUT: a kernel's bounded spin-wait gave up";
    case PQ_ERR_BAD_EXPERT: return "PQ_ERR_BAD_EXPERT: a top-k expert id was out of range";
    case PQ_ERR_SCRATCH: return "PQ_ERR_SCRATCH: the call needs more than the library's static scratch holds";
    default: return "unknown pq_status";
  }
}

int pq_last_hip_error(void) { return pqhost::g_last_hip_error; }

int pq_launches_per_call(const char* entry_point) {
  if (entry_point == nullptr) return PQ_ERR_NULL;
  // pq_gemm_fp8 quantises the activation in a launch of its own before the
  // GEMM; every other compute entry point is one launch
  static const char* const kOne[] = {"pq_quantize_fp8", "pq_quantize_q4", "pq_gemv_fp8", "pq_gemm_fp8_prequant",
                                     "pq_gemv_q4", "moe_decode_layer", "moe_decode_layer_ex",
                                     "moe_decode_layer_noalloc", "pq_stream_probe"};
  if (strcmp(entry_point, "pq_gemm_fp8") == 0) return 2;
  for (const char* n : kOne)
    if (strcmp(entry_point, n) == 0) return 1;
  return PQ_ERR_UNSUPPORTED;
}

int pq_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (ws == nullptr) return ws_bytes == 0 ? PQ_OK : PQ_ERR_NULL;
  if (!pqhost::aligned16(ws)) return PQ_ERR_ALIGN;
  PQ_HIP_CHECK(hipMemsetAsync(ws, 0, ws_bytes, (hipStream_t)stream));
  return PQ_OK;
}

int pq_workspace_check(void* ws, void* stream) {
  if (ws == nullptr) return PQ_ERR_NULL;
  if (!pqhost::aligned16(ws)) return PQ_ERR_ALIGN;
  uint32_t err = 0;
  PQ_HIP_CHECK(hipMemcpyAsync(&err, ws, sizeof(err), hipMemcpyDeviceToHost, (hipStream_t)stream));
  PQ_HIP_CHECK(hipStreamSynchronize((hipStream_t)stream));
  if (err != 0) {
    const uint32_t zero = 0;
    PQ_HIP_CHECK(hipMemcpyAsync(ws, &zero, sizeof(zero), hipMemcpyHostToDevice, (hipStream_t)stream));
    PQ_HIP_CHECK(hipStreamSynchronize((hipStream_t)stream));
  }
  return (int)err;
}

}  // extern "C"
