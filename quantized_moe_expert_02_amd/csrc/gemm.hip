// Prefill path (large batches): grouped GEMMs on the matrix cores.
#include "common.h"

namespace moe {

hipError_t launch_prefill_experts(const moe_dims_t& d, const Plan& p, const moe_weights_t& w,
                                  const uint16_t* x, const Route& r, void* ws, uint16_t* y, hipStream_t s,
                                  const StageEvents& se) {
  (void)d; (void)p; (void)w; (void)x; (void)r; (void)ws; (void)y; (void)s; (void)se;
  return hipErrorNotSupported;
}

}  // namespace moe
