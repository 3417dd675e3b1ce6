// Gating kernels for x bf16 / gate weights float storage.
#include "gate_impl.h"

namespace moe {

hipError_t gate_dispatch_bf16x_f32w(const GateLaunch& g, const gate_detail::GateParams& p, bool pass2,
                              hipStream_t s) {
  return gate_detail::gate_dispatch_d<bf16, float>(g, p, pass2, s);
}

}  // namespace moe
