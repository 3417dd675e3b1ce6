// The gate-weighted sum of eq 1 (section "How a mixture-of-experts layer
// works") and the small reductions of the balancing losses (eqs 7 and 11,
// section "Why experts collapse, and the balancing losses").
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

// y[t] = sum_j gate[t, j] * expert_out[slot_pos[t*k + j]], fp32 accumulation
// in slot order. One thread per 16-byte unit of an output row: every read and
// write is a full 16-byte access and a row is read contiguously.
template <typename T, bool NT>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ eo,
                                                      const int32_t* __restrict__ slot_pos,
                                                      const float* __restrict__ gate,
                                                      int64_t tokens, int k, int d,
                                                      int64_t eo_rows, T* __restrict__ y) {
  constexpr int UE = Elem<T>::kPerUnit;
  const int units = d / UE;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t = gid / units;
  const int u = (int)(gid - t * units);
  if (t >= tokens) return;
  float acc[UE];
#pragma unroll
  for (int i = 0; i < UE; ++i) acc[i] = 0.f;
  // slots in groups of four: the group's positions, gates and rows are all
  // requested before the first is added, then added in slot order
  for (int j0 = 0; j0 < k; j0 += 4) {
    int sp[4];
    float g[4];
    U16 v[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const bool in = j0 + jj < k;
      sp[jj] = in ? slot_pos[t * k + j0 + jj] : -1;
      g[jj] = in ? gate[t * k + j0 + jj] : 0.f;
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      v[jj] = !(sp[jj] >= 0 && sp[jj] < eo_rows) ? zero_unit()
              : NT ? ld_unit_stream(eo + (int64_t)sp[jj] * d + u * UE)
                   : ld_unit(eo + (int64_t)sp[jj] * d + u * UE);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      if (sp[jj] < 0 || sp[jj] >= eo_rows) continue;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += g[jj] * __uint_as_float(v[jj].w[i] << 16);
          acc[2 * i + 1] += g[jj] * __uint_as_float(v[jj].w[i] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += g[jj] * __uint_as_float(v[jj].w[i]);
      }
    }
  }
  U16 o;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o.w[i] = f32_to_bf16_bits(acc[2 * i]) | (f32_to_bf16_bits(acc[2 * i + 1]) << 16);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) o.w[i] = __float_as_uint(acc[i]);
  }
  st_unit(y + t * d + u * UE, o);
}

__global__ void counts_to_load_kernel(const int32_t* __restrict__ counts, int n,
                                      float* __restrict__ load) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n) load[e] = (float)counts[e];
}

// The same from a route's offsets: load[e] = offsets[e + 1] - offsets[e].
__global__ void offsets_to_load_kernel(const int32_t* __restrict__ offsets, int n,
                                       float* __restrict__ load) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n) load[e] = (float)(offsets[e + 1] - offsets[e]);
}

// CV^2 = population variance / mean^2 of importance and of load, in fp64 with a
// fixed reduction order; losses = {CV2(imp), CV2(load), w_imp CV2(imp) + w_load CV2(load)}.
// One workgroup of T threads; thread t holds elements t, t + T, ... (PER of
// them, T * PER >= n) of both vectors in registers and sums them in that order;
// each wave adds its lanes' sums by a butterfly (lanes 32, 16, ..., 1 apart)
// and the waves' totals are added in wave order after one barrier. The squared
// deviations are formed from the same registers and reduced the same way.
constexpr int kCvMax = 32768;

__device__ __forceinline__ double cv_wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int T, int PER>
__global__ __launch_bounds__(T) void cv2_losses_kernel(const float* __restrict__ imp,
                                                       const float* __restrict__ load, int n,
                                                       float w_imp, float w_load,
                                                       float* __restrict__ losses) {
  constexpr int W = T / 64;
  __shared__ double red[2][2][W];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  float xi[PER], xl[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = t + j * T;
    xi[j] = i < n ? imp[i] : 0.f;
    xl[j] = i < n ? load[i] : 0.f;
  }
  // the two block totals; slot s has its own LDS cells, so one barrier each
  auto block_sum = [&](double a, double b, int s, double (&out)[2]) {
    a = cv_wave_sum(a);
    b = cv_wave_sum(b);
    if (lane == 0) {
      red[s][0][wave] = a;
      red[s][1][wave] = b;
    }
    __syncthreads();
    double u = 0.0, v = 0.0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      u += red[s][0][w];
      v += red[s][1][w];
    }
    out[0] = u;
    out[1] = v;
  };
  double si = 0.0, sl = 0.0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    si += (double)xi[j];
    sl += (double)xl[j];
  }
  double sum[2];
  block_sum(si, sl, 0, sum);
  const double mi = sum[0] / n, ml = sum[1] / n;
  double qi = 0.0, ql = 0.0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (t + j * T < n) {
      const double di = (double)xi[j] - mi, dl = (double)xl[j] - ml;
      qi += di * di;
      ql += dl * dl;
    }
  }
  double q[2];
  block_sum(qi, ql, 1, q);
  if (t == 0) {
    const double cvi = (n <= 1 || mi == 0.0) ? 0.0 : (q[0] / n) / (mi * mi);
    const double cvl = (n <= 1 || ml == 0.0) ? 0.0 : (q[1] / n) / (ml * ml);
    losses[0] = (float)cvi;
    losses[1] = (float)cvl;
    losses[2] = (float)((double)w_imp * cvi + (double)w_load * cvl);
  }
}

}  // namespace

hipError_t launch_combine(int64_t tokens, int k, int d, Dt dt, const void* expert_out,
                          const int32_t* slot_pos, const float* topk_gate, void* y,
                          hipStream_t s) {
  if (tokens == 0) return hipSuccess;
  const int ue = dt == kBF16 ? 8 : 4;
  const int64_t threads = tokens * (d / ue);
  const dim3 grid((unsigned)((threads + 255) / 256));
  const int64_t rows = tokens * k;
  // Expert outputs larger than the 256 MB Infinity Cache come from HBM and are
  // read with non-temporal loads (5.7 against 5.2 TB/s for 268 MB); smaller
  // ones, just written by the expert FFN, are still in that cache, which the
  // non-temporal loads would pass by (slower: 30 against 27 us for 134 MB).
  const bool nt = rows * d * (dt == kBF16 ? 2 : 4) > kStreamBytes;
#define MOE_COMBINE(TT, NTV)                                                                      \
  hipLaunchKernelGGL((combine_kernel<TT, NTV>), grid, dim3(256), 0, s,                           \
                     reinterpret_cast<const TT*>(expert_out), slot_pos, topk_gate, tokens, k, d, \
                     rows, reinterpret_cast<TT*>(y))
  if (dt == kBF16) {
    if (nt) MOE_COMBINE(bf16, true);
    else MOE_COMBINE(bf16, false);
  } else {
    if (nt) MOE_COMBINE(float, true);
    else MOE_COMBINE(float, false);
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

hipError_t launch_counts_to_load(const int32_t* counts, int n, float* load, hipStream_t s) {
  hipLaunchKernelGGL(counts_to_load_kernel, dim3((n + 255) / 256), dim3(256), 0, s, counts, n, load);
  return hipGetLastError();
}

hipError_t launch_offsets_to_load(const int32_t* offsets, int n, float* load, hipStream_t s) {
  hipLaunchKernelGGL(offsets_to_load_kernel, dim3((n + 255) / 256), dim3(256), 0, s, offsets, n,
                     load);
  return hipGetLastError();
}

hipError_t launch_cv2_losses(const float* importance, const float* load, int n, float w_imp,
                             float w_load, float* losses, hipStream_t s) {
  if (n > kCvMax) return hipErrorInvalidValue;
  // as few threads as keep every thread's share small: 256 x 16 up to 4096
  // experts, 512 x 32 up to 16384, 1024 x 32 beyond
  if (n <= 4096)
    hipLaunchKernelGGL((cv2_losses_kernel<256, 16>), dim3(1), dim3(256), 0, s, importance, load, n,
                       w_imp, w_load, losses);
  else if (n <= 16384)
    hipLaunchKernelGGL((cv2_losses_kernel<512, 32>), dim3(1), dim3(512), 0, s, importance, load, n,
                       w_imp, w_load, losses);
  else
    hipLaunchKernelGGL((cv2_losses_kernel<1024, 32>), dim3(1), dim3(1024), 0, s, importance, load,
                       n, w_imp, w_load, losses);
  return hipGetLastError();
}

}  // namespace moe
