// The small glue kernels of the hierarchical layer (section "Hierarchical
// MoE": a primary gate picks groups, each picked group's own gate picks
// experts inside it, and a leaf's gate is the product of the two): the
// inverse of the primary route's slot map, the leaves of every token, and
// the leaf Load built from the two levels' Loads.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

// perm_slot[slot_pos[q]] = q: the (token, rank) slot of each routed row.
__global__ void invert_slots_kernel(const int32_t* __restrict__ slot_pos, int64_t npairs,
                                    int32_t* __restrict__ perm_slot) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= npairs) return;
  const int32_t p = slot_pos[q];
  if (p >= 0) perm_slot[p] = (int32_t)q;
}

// Leaves of token t in slot order (r, j): leaf sel1[t][r] * b + sel2[t*k1 + r][j]
// with gate gate1[t][r] * gate2[t*k1 + r][j]. One thread per leaf slot.
__global__ void hier_leaves_kernel(int64_t tokens, int k1, int k2, int b,
                                   const int32_t* __restrict__ sel1,
                                   const float* __restrict__ gate1,
                                   const int32_t* __restrict__ sel2,
                                   const float* __restrict__ gate2,
                                   int32_t* __restrict__ leaf_idx,
                                   float* __restrict__ leaf_gate) {
  const int K = k1 * k2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= tokens * K) return;
  const int64_t t = i / K;
  const int r = (int)(i % K) / k2;
  const int64_t s1 = t * k1 + r;  // primary slot = row of the secondary outputs
  leaf_idx[i] = sel1[s1] * b + sel2[i];
  leaf_gate[i] = gate1[s1] * gate2[i];
}

// load[i*b + j] = load1[i] * load2[i*b + j] / rows1[i], 0 for a group without rows.
__global__ void hier_leaf_load_kernel(int a, int b, const float* __restrict__ load1,
                                      const float* __restrict__ load2,
                                      const int32_t* __restrict__ rows1,
                                      float* __restrict__ load) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)a * b) return;
  const int i = (int)(e / b);
  const int r = rows1[i];
  load[e] = r > 0 ? load1[i] * load2[e] / (float)r : 0.f;
}

}  // namespace

hipError_t launch_invert_slots(const int32_t* slot_pos, int64_t npairs, int32_t* perm_slot,
                               hipStream_t s) {
  if (npairs > 0)
    hipLaunchKernelGGL(invert_slots_kernel, dim3((unsigned)((npairs + 255) / 256)), dim3(256), 0,
                       s, slot_pos, npairs, perm_slot);
  return hipGetLastError();
}

hipError_t launch_hier_leaves(int64_t tokens, int k1, int k2, int b, const int32_t* sel1,
                              const float* gate1, const int32_t* sel2, const float* gate2,
                              int32_t* leaf_idx, float* leaf_gate, hipStream_t s) {
  const int64_t total = tokens * k1 * k2;
  if (total > 0)
    hipLaunchKernelGGL(hier_leaves_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       s, tokens, k1, k2, b, sel1, gate1, sel2, gate2, leaf_idx, leaf_gate);
  return hipGetLastError();
}

hipError_t launch_hier_leaf_load(int a, int b, const float* load1, const float* load2,
                                 const int32_t* rows1, float* load, hipStream_t s) {
  const int64_t n = (int64_t)a * b;
  hipLaunchKernelGGL(hier_leaf_load_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     a, b, load1, load2, rows1, load);
  return hipGetLastError();
}

}  // namespace moe
