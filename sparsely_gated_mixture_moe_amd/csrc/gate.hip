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

// Grouped Load: load[g * n + e] = sum over the units of group g (consecutive,
// unit_start[g] .. unit_start[g + 1] - 1) of partial[u][e], in the same fixed
// order as above; a group without rows gets 0.
__global__ __launch_bounds__(256) void load_reduce_grouped_kernel(
    const float* __restrict__ partial, const int32_t* __restrict__ unit_start, int n,
    float* __restrict__ load) {
  __shared__ float red[8][32];
  const int col = threadIdx.x & 31;
  const int part = threadIdx.x >> 5;
  const int e = blockIdx.x * 32 + col;
  const int grp = blockIdx.y;
  const int u0 = unit_start[grp], u1 = unit_start[grp + 1];
  float s = 0.f;
  if (e < n)
    for (int u = u0 + part; u < u1; u += 8) s += partial[(int64_t)u * n + e];
  red[part][col] = s;
  __syncthreads();
  if (part == 0 && e < n) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) t += red[i][col];
    load[(int64_t)grp * n + e] = t;
  }
}

// Lists the secondary-gating work units: group g gets ceil(rows_g / tile)
// units of `tile` consecutive routed rows, starting at unit unit_start[g]. One
// workgroup; thread t owns a contiguous span of groups.
__global__ __launch_bounds__(1024) void group_plan_kernel(const int32_t* __restrict__ offsets,
                                                          int groups, int tile,
                                                          int32_t* __restrict__ units,
                                                          int32_t* __restrict__ unit_start) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int per = (groups + 1023) / 1024;
  const int g0 = min(groups, t * per), g1 = min(groups, g0 + per);
  int s = 0;
  for (int g = g0; g < g1; ++g) s += (offsets[g + 1] - offsets[g] + tile - 1) / tile;
  part[t] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = (t >= o) ? part[t - o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int pos = part[t] - s;
  for (int g = g0; g < g1; ++g) {
    unit_start[g] = pos;
    const int cnt = offsets[g + 1] - offsets[g];
    for (int r = 0; r < cnt; r += tile) {
      units[1 + 2 * pos] = g;
      units[2 + 2 * pos] = r;
      ++pos;
    }
  }
  if (t == 1023) {
    units[0] = part[t];
    unit_start[groups] = part[t];
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
  p.units = g.units;
  p.seg_off = g.seg_off;
  p.row_token = g.row_token;
  p.row_slot = g.row_slot;
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

int gate_tile_rows(const GateLaunch& g) { return gate_uses_g32(g) ? kGate32Rows : kGateRows; }

int64_t gate_max_units(int64_t rows, int groups, int tile_rows) {
  return (rows + tile_rows - 1) / tile_rows + groups;
}

hipError_t launch_group_plan(const int32_t* offsets, int groups, int tile_rows, int32_t* units,
                             int32_t* unit_start, hipStream_t s) {
  hipLaunchKernelGGL(group_plan_kernel, dim3(1), dim3(1024), 0, s, offsets, groups, tile_rows,
                     units, unit_start);
  return hipGetLastError();
}

hipError_t launch_load_grouped(const GateLaunch& g, int groups, const int32_t* unit_start,
                               const int32_t* topk_idx, const float* thresh, float* partial,
                               float* load, hipStream_t s) {
  if (g.tokens > 0) {
    GateParams p = make_params(g);
    p.sel_idx = topk_idx;
    p.sel_thr = thresh;
    p.partial = partial;
    hipError_t e = gate_dispatch(g, p, true, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(load_reduce_grouped_kernel, dim3((g.n + 31) / 32, groups), dim3(256), 0, s,
                     partial, unit_start, g.n, load);
  return hipGetLastError();
}

hipError_t launch_load(const GateLaunch& g, const int32_t* topk_idx, const float* thresh,
                       float* partial, float* load, hipStream_t s) {
  // partial has room for gate_blocks() rows: the 32x32 kernel's 256-row blocks need fewer
  const int rows = gate_tile_rows(g);
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
