// Temporary entry points for calls whose kernels are not built yet.
#include "pq_common.h"
extern "C" {
size_t pq_gemv_q4_workspace(int, int, int, int) { return 0; }
int pq_gemv_q4(const uint16_t*, int, int, const uint8_t*, const uint16_t*, int, int, uint16_t*, void*, size_t,
               void*) { return PQ_ERR_UNSUPPORTED; }
}
