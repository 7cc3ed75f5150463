// Gated multi-scale retention layer: placeholder until the GEMM lands.
#include "common.hpp"
#include "launch.hpp"
#include "retention.h"

extern "C" {

size_t msr_layer_fwd_workspace_bytes(int, int, int, int, int, int, int) { return 0; }

ret_status_t msr_layer_fwd(const void *, const void *, const void *, const void *, const void *,
                           const void *, void *, int, int, int, int, int, int, int, const float *,
                           const float *, long long, float, void *, size_t, void *) {
  return RET_ERR_UNSUPPORTED;
}

}  // extern "C"
