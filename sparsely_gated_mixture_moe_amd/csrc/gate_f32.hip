// Gating kernels for x float / gate weights float storage.
#include "gate_impl.h"

namespace moe {

hipError_t gate_dispatch_f32(const GateLaunch& g, const gate_detail::GateParams& p, bool pass2,
                              hipStream_t s) {
  return gate_detail::gate_dispatch_d<float, float>(g, p, pass2, s);
}

}  // namespace moe
