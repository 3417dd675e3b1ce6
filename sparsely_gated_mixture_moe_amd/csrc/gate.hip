// Host glue of the gating kernels (the kernel template is in gate_impl.h) and
// the block-order reduction of the Load partial sums.
#include "gate_impl.h"

namespace moe {
namespace {

using gate_detail::GateParams;

// load[e] = sum over gate blocks b of partial[b][e], in a fixed order: 32
// experts per workgroup, 8 threads per expert each summing a strided subset
// of the blocks, then the 8 partial sums in thread order.
__global__ __launch_bounds__(256) void load_reduce_kernel(const float* __restrict__ partial,
                                                          int nblocks, int n,
                                                          float* __restrict__ load) {
  __shared__ float red[8][32];
  const int col = threadIdx.x & 31;
  const int part = threadIdx.x >> 5;
  const int e = blockIdx.x * 32 + col;
  float s = 0.f;
  if (e < n)
    for (int b = part; b < nblocks; b += 8) s += partial[(int64_t)b * n + e];
  red[part][col] = s;
  __syncthreads();
  if (part == 0 && e < n) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) t += red[i][col];
    load[e] = t;
  }
}

hipError_t gate_dispatch(const GateLaunch& g, const GateParams& p, bool pass2, hipStream_t s) {
  if (g.x_dt == kBF16 && g.w_dt == kBF16) return gate_dispatch_bf16(g, p, pass2, s);
  if (g.x_dt == kBF16 && g.w_dt == kF32) return gate_dispatch_bf16x_f32w(g, p, pass2, s);
  if (g.x_dt == kF32 && g.w_dt == kF32) return gate_dispatch_f32(g, p, pass2, s);
  return hipErrorInvalidValue;
}

GateParams make_params(const GateLaunch& g) {
  GateParams p{};
  p.x = g.x;
  p.wg = g.w_gate;
  p.wn = g.w_noise;
  p.bias = g.bias;
  p.eps = g.eps;
  p.B = g.tokens;
  p.n = g.n;
  p.k = g.k;
  p.floor = g.noise_floor;
  return p;
}

}  // namespace

int gate_blocks(int64_t tokens) { return (int)((tokens + kGateRows - 1) / kGateRows); }

bool gate_supported(int d, Dt x_dt, Dt w_dt, int k) {
  if (!(d == 64 || d == 128 || d == 256 || d == 512)) return false;
  if (k < 1 || k > 8) return false;
  if (x_dt == kF32 && w_dt == kBF16) return false;
  return true;
}

hipError_t launch_gate(const GateLaunch& g, int32_t* topk_idx, float* topk_gate, float* thresh,
                       hipStream_t s) {
  if (g.tokens == 0) return hipSuccess;
  GateParams p = make_params(g);
  p.topk_idx = topk_idx;
  p.topk_gate = topk_gate;
  p.thresh = thresh;
  return gate_dispatch(g, p, false, s);
}

hipError_t launch_load(const GateLaunch& g, const int32_t* topk_idx, const float* thresh,
                       float* partial, float* load, hipStream_t s) {
  // partial has room for gate_blocks() rows: the 32x32 kernel's 256-row blocks need fewer
  const int rows = gate_uses_g32(g) ? 256 : kGateRows;
  const int nb = (int)((g.tokens + rows - 1) / rows);
  if (nb > 0) {
    GateParams p = make_params(g);
    p.sel_idx = topk_idx;
    p.sel_thr = thresh;
    p.partial = partial;
    hipError_t e = gate_dispatch(g, p, true, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(load_reduce_kernel, dim3((g.n + 31) / 32), dim3(256), 0, s, partial, nb,
                     g.n, load);
  return hipGetLastError();
}

}  // namespace moe
