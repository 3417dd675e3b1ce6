// Gating kernels for x bf16 / gate weights bf16 storage.
#include "gate32_impl.h"

namespace moe {

hipError_t gate_dispatch_bf16(const GateLaunch& g, const gate_detail::GateParams& p, bool pass2,
                              hipStream_t s) {
  using namespace gate_detail;
  if (gate_uses_g32(g)) {
    const dim3 grid = gate_grid(g, kG32Rows);
    const dim3 block(kG32Threads);
    const bool k4 = g.k <= 4;
#define MOE_G32(DD)                                                                        \
  if (g.d == DD) {                                                                         \
    if (!g.train) {                                                                        \
      if (p.scores)                                                                        \
        hipLaunchKernelGGL((gate32_kernel<DD, 5, false, false, true, true>), grid, block, 0, s, p); \
      else if (g.gate_order && k4)                                                         \
        hipLaunchKernelGGL((gate32_kernel<DD, 5, false, true, false, true>), grid, block, 0, s, p); \
      else if (g.gate_order)                                                               \
        hipLaunchKernelGGL((gate32_kernel<DD, 9, false, true, false, true>), grid, block, 0, s, p); \
      else if (k4)                                                                         \
        hipLaunchKernelGGL((gate32_kernel<DD, 5, false, false, false, true>), grid, block, 0, s, p); \
      else                                                                                 \
        hipLaunchKernelGGL((gate32_kernel<DD, 9, false, false, false, true>), grid, block, 0, s, p); \
    } else if (p.scores) {                                                                 \
      hipLaunchKernelGGL((gate32_kernel<DD, 5, false, false, true>), grid, block, 0, s, p);  \
    } else if (pass2 && p.dcu) {                                                           \
      hipLaunchKernelGGL((gate32_kernel<DD, 5, true, false, false, false, true>), grid, block, 0, s, p); \
    } else if (pass2) {                                                                    \
      if (k4) hipLaunchKernelGGL((gate32_kernel<DD, 5, true>), grid, block, 0, s, p);      \
      else hipLaunchKernelGGL((gate32_kernel<DD, 9, true>), grid, block, 0, s, p);         \
    } else if (g.gate_order) {                                                             \
      if (k4) hipLaunchKernelGGL((gate32_kernel<DD, 5, false, true>), grid, block, 0, s, p); \
      else hipLaunchKernelGGL((gate32_kernel<DD, 9, false, true>), grid, block, 0, s, p);    \
    } else {                                                                               \
      if (k4) hipLaunchKernelGGL((gate32_kernel<DD, 5, false>), grid, block, 0, s, p);     \
      else hipLaunchKernelGGL((gate32_kernel<DD, 9, false>), grid, block, 0, s, p);        \
    }                                                                                      \
    return hipGetLastError();                                                              \
  }
    MOE_G32(128)
    MOE_G32(256)
    MOE_G32(512)
#undef MOE_G32
  }
  return gate_detail::gate_dispatch_d<bf16, bf16>(g, p, pass2, s);
}

}  // namespace moe
