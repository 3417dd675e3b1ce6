// Routing on gfx950: each expert's batch (the tokens whose gate for it is
// nonzero, the only ones eq 1 evaluates it on) laid out as one contiguous
// block per expert, which is how a single GPU keeps each expert's matrix
// products as large as the batch allows (section "Keeping each expert's batch
// large"). It is a stable counting sort of the B*k (token, slot) pairs by
// expert, plus Importance (eq 6) as a segmented sum.
//
//   1. count:   per block of 256 tokens, an LDS histogram over experts,
//               written expert-major as blockcnt[e][b].
//   2. scan_b:  per expert (one wave), exclusive prefix over blocks -> counts[e].
//   3. scan_e:  one workgroup: exclusive prefix of counts -> offsets.
//   4. scatter: per block, stable ranks. Each wave matches equal experts in its
//               64 pairs with 16 ballots; the waves of a block then claim
//               positions from LDS counters one wave at a time, in pair order,
//               which keeps tokens ascending inside every segment.
//   5. importance: one wave per expert sums its segment's gates in a fixed
//               order (no float atomics).
// All integer work is exact; the only float result (importance) is summed in
// a fixed order, so the output is deterministic.
#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__global__ __launch_bounds__(kThreads) void route_count(const int32_t* __restrict__ idx,
                                                        int64_t npairs, int pairs_per_block, int n,
                                                        int nblk, int32_t* __restrict__ blockcnt) {
  extern __shared__ int hist[];
  for (int e = threadIdx.x; e < n; e += kThreads) hist[e] = 0;
  __syncthreads();
  const int64_t p0 = (int64_t)blockIdx.x * pairs_per_block;
  const int64_t p1 = min(npairs, p0 + pairs_per_block);
  for (int64_t p = p0 + threadIdx.x; p < p1; p += kThreads) {
    const int e = idx[p];
    if (e >= 0 && e < n) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < n; e += kThreads) blockcnt[(int64_t)e * nblk + blockIdx.x] = hist[e];
}

// One wave per expert: lane b takes block b of each group of 64 blocks, an
// inclusive wave scan (shuffles) plus the running total of earlier groups
// gives the exclusive prefix.
__global__ __launch_bounds__(256) void route_scan_blocks(int32_t* __restrict__ blockcnt, int n,
                                                         int nblk, int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= n) return;
  int32_t* c = blockcnt + (int64_t)e * nblk;
  int carry = 0;
  for (int b0 = 0; b0 < nblk; b0 += 64) {
    const int b = b0 + lane;
    const int v = b < nblk ? c[b] : 0;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o);
      if (lane >= o) incl += u;
    }
    if (b < nblk) c[b] = carry + incl - v;
    carry += __shfl(incl, 63);
  }
  if (lane == 0) counts[e] = carry;
}

// Exclusive scan of n counts by one workgroup; thread t owns a contiguous span.
__global__ __launch_bounds__(kThreads) void route_scan_experts(const int32_t* __restrict__ counts,
                                                               int n, int32_t* __restrict__ offsets) {
  __shared__ int part[kThreads];
  const int t = threadIdx.x;
  const int per = (n + kThreads - 1) / kThreads;
  const int e0 = min(n, t * per), e1 = min(n, e0 + per);
  int s = 0;
  for (int e = e0; e < e1; ++e) s += counts[e];
  part[t] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan of the span sums.
  for (int o = 1; o < kThreads; o <<= 1) {
    const int v = (t >= o) ? part[t - o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - s;
  for (int e = e0; e < e1; ++e) {
    offsets[e] = run;
    run += counts[e];
  }
  if (t == kThreads - 1) offsets[n] = part[t];
}

__global__ __launch_bounds__(kThreads) void route_scatter(
    const int32_t* __restrict__ idx, const float* __restrict__ gate, int64_t npairs, int k,
    int pairs_per_block, int n, int nbits, int nblk, const int32_t* __restrict__ blockoff,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ perm_token,
    float* __restrict__ perm_gate, int32_t* __restrict__ slot_pos, int capacity) {
  extern __shared__ int ctr[];
  for (int e = threadIdx.x; e < n; e += kThreads)
    ctr[e] = offsets[e] + blockoff[(int64_t)e * nblk + blockIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t p0 = (int64_t)blockIdx.x * pairs_per_block;
  const int64_t p1 = min(npairs, p0 + pairs_per_block);
  for (int64_t base = p0; base < p1; base += kThreads) {
    const int64_t p = base + threadIdx.x;
    const bool valid = p < p1;
    const int e = valid ? idx[p] : -1;
    const bool live = valid && e >= 0 && e < n;
    // Lanes holding the same expert: AND over the bits of the key (e + 1; dead lanes 0).
    const uint32_t key = live ? (uint32_t)(e + 1) : 0u;
    uint64_t eq = ~0ull;
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1u;
      const uint64_t m = __ballot(bit);
      eq &= bit ? m : ~m;
    }
    const int rank = __popcll(eq & below);
    const int cnt = __popcll(eq);
    const int leader = __ffsll((unsigned long long)eq) - 1;
    int claim = 0;
    // Waves claim their segment positions in pair order.
    for (int w = 0; w < kWaves; ++w) {
      if (wave == w && live && rank == 0) {
        claim = ctr[e];
        ctr[e] = claim + cnt;
      }
      __syncthreads();
    }
    const int start = __shfl(claim, leader);
    if (live) {
      const int pos = start + rank;
      perm_token[pos] = (int32_t)(p / k);
      perm_gate[pos] = gate[p];
      // past the expert's capacity: routed, but not served
      slot_pos[p] = (capacity > 0 && pos - offsets[e] >= capacity) ? -1 : pos;
    } else if (valid) {
      slot_pos[p] = -1;
    }
  }
}

__global__ void route_importance(const float* __restrict__ perm_gate,
                                 const int32_t* __restrict__ offsets, int n,
                                 float* __restrict__ importance) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (e >= n) return;
  // lane l adds positions l, l + 64, ... of the segment in ascending order;
  // sixteen of them are loaded before any is added, so that a long segment
  // (a popular expert) is not one load latency per step
  const int end = offsets[e + 1];
  float s = 0.f;
  int i = offsets[e] + lane;
  for (; i + 64 * 15 < end; i += 64 * 16) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = perm_gate[i + 64 * j];
#pragma unroll
    for (int j = 0; j < 16; ++j) s += v[j];
  }
  for (; i < end; i += 64) s += perm_gate[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) importance[e] = s;
}

// Routing of a small batch in one workgroup and one launch instead of five:
// the same outputs as the multi-kernel path. Counts by LDS atomics (integers),
// offsets by the same span scan as route_scan_experts, each pair's position
// = its expert's offset + the pairs before it with the same expert (stable),
// and each Importance summed in the same order as route_importance (lane l
// takes positions l, l + 64, ... of the segment, then a butterfly), from an
// LDS copy of the permuted gates.
constexpr int kSmallPairs = 1024;
constexpr int kSmallExperts = 16384;
constexpr size_t kSmallLds = (2 * (size_t)kSmallExperts + 1 + 3 * kSmallPairs) * sizeof(int);
__global__ __launch_bounds__(kThreads) void route_small(
    const int32_t* __restrict__ idx, const float* __restrict__ gate, int npairs, int k, int n,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm_token,
    float* __restrict__ perm_gate, int32_t* __restrict__ slot_pos, float* __restrict__ importance,
    int capacity) {
  extern __shared__ int sm[];
  int* cnt = sm;                                    // [n]
  int* off = cnt + n;                               // [n + 1]
  int* se = off + n + 1;                            // [npairs] expert of each pair, -1 dropped
  int* lst = se + kSmallPairs;                      // experts with rows
  float* pg = reinterpret_cast<float*>(lst + kSmallPairs);  // gates in perm order
  __shared__ int part[kThreads];
  __shared__ int nlst;
  const int t = threadIdx.x;
  for (int e = t; e < n; e += kThreads) cnt[e] = 0;
  if (t == 0) nlst = 0;
  __syncthreads();
  if (t < npairs) {
    const int e = idx[t];
    const bool live = e >= 0 && e < n;
    se[t] = live ? e : -1;
    if (live) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  const int per = (n + kThreads - 1) / kThreads;
  const int e0 = min(n, t * per), e1 = min(n, e0 + per);
  int s = 0;
  for (int e = e0; e < e1; ++e) s += cnt[e];
  part[t] = s;
  __syncthreads();
  for (int o = 1; o < kThreads; o <<= 1) {
    const int v = (t >= o) ? part[t - o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - s;
  for (int e = e0; e < e1; ++e) {
    off[e] = run;
    offsets[e] = run;
    counts[e] = cnt[e];
    if (importance) importance[e] = 0.f;
    run += cnt[e];
  }
  if (t == kThreads - 1) {
    off[n] = part[t];
    offsets[n] = part[t];
  }
  __syncthreads();
  if (t < npairs) {
    const int e = se[t];
    if (e >= 0) {
      int rank = 0;
      for (int q = 0; q < t; ++q) rank += se[q] == e;
      const int pos = off[e] + rank;
      const float gv = gate[t];
      perm_token[pos] = t / k;
      perm_gate[pos] = gv;
      pg[pos] = gv;
      slot_pos[t] = (capacity > 0 && rank >= capacity) ? -1 : pos;
      if (rank == 0) lst[atomicAdd(&nlst, 1)] = e;
    } else {
      slot_pos[t] = -1;
    }
  }
  __syncthreads();
  if (importance) {
    const int lane = t & 63;
    for (int i = t >> 6; i < nlst; i += kWaves) {
      const int e = lst[i];
      float v = 0.f;
      for (int j = off[e] + lane; j < off[e + 1]; j += 64) v += pg[j];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
      if (lane == 0) importance[e] = v;
    }
  }
}

__global__ void fill_zero_i32(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

int route_blocks(int64_t tokens) { return (int)((tokens + kRouteTokens - 1) / kRouteTokens); }

hipError_t launch_route(int64_t tokens, int k, int n, const int32_t* topk_idx,
                        const float* topk_gate, int32_t* blockcnt, int32_t* counts,
                        int32_t* offsets, int32_t* perm_token, float* perm_gate, int32_t* slot_pos,
                        float* importance, hipStream_t s, int capacity) {
  const int nblk = route_blocks(tokens);
  const int64_t npairs = tokens * k;
  const int ppb = kRouteTokens * k;
  const size_t lds = (size_t)n * sizeof(int);
  int nbits = 1;
  while ((1u << nbits) <= (uint32_t)n) ++nbits;  // keys 0..n need nbits bits
  // Up to 32768 experts: 128 KB of LDS counters (set once per process).
  static const bool lds_attr_set = [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(route_count),
                        hipFuncAttributeMaxDynamicSharedMemorySize, 32768 * (int)sizeof(int));
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(route_scatter),
                        hipFuncAttributeMaxDynamicSharedMemorySize, 32768 * (int)sizeof(int));
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(route_small),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmallLds);
    return true;
  }();
  (void)lds_attr_set;
  if (npairs > 0 && npairs <= kSmallPairs && n <= kSmallExperts) {
    const size_t small_lds = (2 * (size_t)n + 1 + 3 * kSmallPairs) * sizeof(int);
    hipLaunchKernelGGL(route_small, dim3(1), dim3(kThreads), small_lds, s, topk_idx, topk_gate,
                       (int)npairs, k, n, counts, offsets, perm_token, perm_gate, slot_pos,
                       importance, capacity);
    return hipGetLastError();
  }
  if (nblk > 0) {
    hipLaunchKernelGGL(route_count, dim3(nblk), dim3(kThreads), lds, s, topk_idx, npairs, ppb, n,
                       nblk, blockcnt);
    hipLaunchKernelGGL(route_scan_blocks, dim3((n + 3) / 4), dim3(256), 0, s, blockcnt, n, nblk,
                       counts);
  } else {
    hipLaunchKernelGGL(fill_zero_i32, dim3((n + 255) / 256), dim3(256), 0, s, counts, n);
  }
  hipLaunchKernelGGL(route_scan_experts, dim3(1), dim3(kThreads), 0, s, counts, n, offsets);
  if (nblk > 0)
    hipLaunchKernelGGL(route_scatter, dim3(nblk), dim3(kThreads), lds, s, topk_idx, topk_gate,
                       npairs, k, ppb, n, nbits, nblk, blockcnt, offsets, perm_token, perm_gate,
                       slot_pos, capacity);
  if (importance)
    hipLaunchKernelGGL(route_importance, dim3((n + 3) / 4), dim3(256), 0, s, perm_gate, offsets, n,
                       importance);
  return hipGetLastError();
}

}  // namespace moe
