// Temporary entry points for calls whose kernels are not built yet.
#include "pq_common.h"
extern "C" {
size_t pq_gemv_q4_workspace(int, int, int, int) { return 0; }
int pq_gemv_q4(const uint16_t*, int, int, const uint8_t*, const uint16_t*, int, int, uint16_t*, void*, size_t,
               void*) { return PQ_ERR_UNSUPPORTED; }
size_t moe_decode_layer_workspace(int, int, int, int, int) { return 0; }
int moe_decode_layer(const uint16_t*, int, int, const float*, int32_t*, float*, int, int, int, const uint8_t*,
                     const float*, const uint8_t*, const float*, uint16_t*, uint16_t*, uint8_t*, float*, void*,
                     size_t, void*) { return PQ_ERR_UNSUPPORTED; }
}
