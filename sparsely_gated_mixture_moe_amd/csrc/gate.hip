// Host glue of the gating kernels (the kernel template is in gate_impl.h) and
// the block-order reduction of the Load partial sums.
#include <algorithm>

#include "gate_impl.h"

namespace moe {
namespace {

using gate_detail::GateParams;
using gate_detail::GateShape;
using gate_detail::insert_any;
using gate_detail::write_selection;
using gate_detail::ExpSum;
using gate_detail::expsum_merge;

// load[e] = sum over gate blocks b of partial[b][e], in a fixed order: 32
// experts per workgroup, 8 threads per expert each summing a strided subset
// of the blocks, then the 8 partial sums in thread order; plus the selected
// pairs' corrections of expert e's slices (slice_start[e] ..
// slice_start[e + 1] - 1), in slice order.
__global__ __launch_bounds__(256) void load_reduce_kernel(const float* __restrict__ partial,
                                                          int nblocks, int n,
                                                          const float* __restrict__ corr,
                                                          const int32_t* __restrict__ slice_start,
                                                          float* __restrict__ load) {
  __shared__ float red[8][32];
  const int col = threadIdx.x & 31;
  const int part = threadIdx.x >> 5;
  const int e = blockIdx.x * 32 + col;
  float s = 0.f;
  if (e < n) {
    // four loads in flight, added in block order
    int b = part;
    for (; b + 24 < nblocks; b += 32) {
      const float v0 = partial[(int64_t)b * n + e], v1 = partial[(int64_t)(b + 8) * n + e];
      const float v2 = partial[(int64_t)(b + 16) * n + e], v3 = partial[(int64_t)(b + 24) * n + e];
      s += v0;
      s += v1;
      s += v2;
      s += v3;
    }
    for (; b < nblocks; b += 8) s += partial[(int64_t)b * n + e];
  }
  red[part][col] = s;
  __syncthreads();
  if (part == 0 && e < n) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) t += red[i][col];
    float c = 0.f;
    for (int i = slice_start[e]; i < slice_start[e + 1]; ++i) c += corr[i];
    load[e] = t + c;
  }
}

// Grouped Load: load[g * n + e] = sum over the units of group g (consecutive,
// unit_start[g] .. unit_start[g + 1] - 1) of partial[u][e], in the same fixed
// order as above; a group without rows gets 0.
__global__ __launch_bounds__(256) void load_reduce_grouped_kernel(
    const float* __restrict__ partial, const int32_t* __restrict__ unit_start, int n,
    const float* __restrict__ corr, const int32_t* __restrict__ slice_start,
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
    const int64_t leaf = (int64_t)grp * n + e;
    float c = 0.f;
    for (int i = slice_start[leaf]; i < slice_start[leaf + 1]; ++i) c += corr[i];
    load[leaf] = t + c;
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

// Slices of the selected pairs' correction: expert e's routed rows (offsets[e]
// .. offsets[e + 1] - 1) in slices of kCorrSliceRows; slice_start[e] is the
// index of e's first slice and slice_start[n] the number of slices. One
// workgroup; thread t owns a contiguous span of experts.
__global__ __launch_bounds__(1024) void corr_slice_scan_kernel(const int32_t* __restrict__ offsets,
                                                               int n,
                                                               int32_t* __restrict__ slice_start,
                                                               int32_t* __restrict__ slice_e) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int e0 = min(n, t * per), e1 = min(n, e0 + per);
  int s = 0;
  for (int e = e0; e < e1; ++e)
    s += (offsets[e + 1] - offsets[e] + kCorrSliceRows - 1) / kCorrSliceRows;
  part[t] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = (t >= o) ? part[t - o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int pos = part[t] - s;
  for (int e = e0; e < e1; ++e) {
    slice_start[e] = pos;
    const int ns = (offsets[e + 1] - offsets[e] + kCorrSliceRows - 1) / kCorrSliceRows;
    for (int i = 0; i < ns; ++i) slice_e[pos + i] = e;  // each slice's expert
    pos += ns;
  }
  if (t == 1023) slice_start[n] = part[t];
}

// Eight consecutive elements (storage type T) widened to fp32; 16 bytes for
// bf16, 32 for fp32.
template <typename T>
__device__ __forceinline__ void load8(const void* base, int64_t off, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const U16 u = ld_unit(reinterpret_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u.w[i] << 16);
      v[2 * i + 1] = __uint_as_float(u.w[i] & 0xFFFF0000u);
    }
  } else {
    const float* f = reinterpret_cast<const float*>(base) + off;
    const U16 a = ld_unit(f), b = ld_unit(f + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(a.w[i]);
      v[4 + i] = __uint_as_float(b.w[i]);
    }
  }
}

// The selected pairs of eq 8: the Load pass evaluates every (token, expert)
// pair against the row's k-th largest logit v_k, while a selected expert's
// threshold is the (k+1)-th, v_{k+1}. For expert e this kernel takes the rows
// routed to it (positions offsets[e] .. offsets[e+1] - 1, tokens perm_token[p])
// and sums Phi((clean - v_{k+1}) / sigma) - Phi((clean - v_k) / sigma), with
// clean = x . W_g[e] (+ bias) and sigma = Softplus(x . W_noise[e]) + floor
// recomputed by a dot product over d in fp32. Workgroup i, four waves, takes
// slice i of the slices corr_slice_scan_kernel lists (its expert slice_e[i]):
// kCorrSliceRows consecutive routed rows of e (fewer in e's last slice); lane
// l holds elements 8 l .. 8 l + 7 of both weight rows (d <= 512); wave w
// takes the slice's groups of eight rows with index w mod 4, all eight in
// flight at once. A group's 16 partial dots per lane (clean and noise, eight
// rows) are summed over the wave by a transposing reduction (each step
// exchanges half of the values a lane holds with its partner, keeping the
// other half), after which lane l holds the total of row (l / 4) % 8, clean
// for l < 32 and noise otherwise; eight lanes then evaluate the eight rows'
// Phi terms at once. The four waves' sums are added in wave order into
// corr[i], and the reductions add an expert's slices in order. Workgroups past
// the number of slices (the grid covers the largest possible count) exit at
// once.
// Secondary gates of a hierarchical layer: expert e is leaf (g, j) = (e / b,
// e % b), its weights are row e of the [a * b, d] secondary weights, and token
// t's thresholds are row t * k1 + r, where r is g's rank in sel1[t].
template <typename XS, typename WS>
__global__ __launch_bounds__(256) void load_correction_kernel(
    const void* __restrict__ x, const void* __restrict__ wg, const void* __restrict__ wn,
    const float* __restrict__ bias, int d, int n, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm_token, const float* __restrict__ thresh, float noise_floor,
    const int32_t* __restrict__ sel1, int k1, int b, const int32_t* __restrict__ slice_start,
    const int32_t* __restrict__ slice_e, float* __restrict__ corr) {
  constexpr int R = 8;
  static_assert(kCorrSliceRows % (4 * R) == 0, "slices are whole passes of the 4 x R rows");
  __shared__ float part[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slice = blockIdx.x;
  if (slice >= slice_start[n]) return;  // uniform: past the number of slices
  const int e = slice_e[slice];
  const int p0 = offsets[e] + (slice - slice_start[e]) * kCorrSliceRows;
  const int p1 = min(offsets[e + 1], p0 + kCorrSliceRows);
  const bool active = lane * 8 < d;
  float wgv[8], wnv[8];
  if (active) {
    load8<WS>(wg, (int64_t)e * d + lane * 8, wgv);
    load8<WS>(wn, (int64_t)e * d + lane * 8, wnv);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) wgv[i] = wnv[i] = 0.f;
  }
  const float be = bias ? bias[e] : 0.f;
  const int grp = e / b;
  // after the reduction: this lane's row of the group, and whether it holds
  // the noise dot (lanes 32-63) or the clean one
  const bool hi5 = lane >= 32, b4 = (lane & 16) != 0, b3 = (lane & 8) != 0, b2 = (lane & 4) != 0;
  const int myr = (lane >> 2) & 7;
  const bool evaluates = !hi5 && (lane & 3) == 0;  // 8 lanes, one row each
  float acc = 0.f;
  for (int p = p0 + wave * R; p < p1; p += 4 * R) {
    int64_t t[R];
#pragma unroll
    for (int r = 0; r < R; ++r) t[r] = perm_token[min(p + r, p1 - 1)];
    float c[R], u[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      c[r] = u[r] = 0.f;
      if (active) {
        float xv[8];
        load8<XS>(x, t[r] * d + lane * 8, xv);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          c[r] = fmaf(xv[i], wgv[i], c[r]);
          u[r] = fmaf(xv[i], wnv[i], u[r]);
        }
      }
    }
    // transposing reduction over the wave: lanes l, l ^ 32 (clean / noise),
    // l ^ 16 (rows 0-3 / 4-7), l ^ 8, l ^ 4, then the quad
    float v8[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float keep = hi5 ? u[i] : c[i], send = hi5 ? c[i] : u[i];
      v8[i] = keep + __shfl_xor(send, 32);
    }
    float v4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float keep = b4 ? v8[4 + i] : v8[i], send = b4 ? v8[i] : v8[4 + i];
      v4[i] = keep + __shfl_xor(send, 16);
    }
    float v2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float keep = b3 ? v4[2 + i] : v4[i], send = b3 ? v4[i] : v4[2 + i];
      v2[i] = keep + __shfl_xor(send, 8);
    }
    float v1 = (b2 ? v2[1] : v2[0]) + __shfl_xor(b2 ? v2[0] : v2[1], 4);
    v1 += __shfl_xor(v1, 2);
    v1 += __shfl_xor(v1, 1);
    const float un = __shfl_xor(v1, 32);  // the row's noise dot, for the clean lanes
    const int pr = p + myr;
    if (evaluates && pr < p1) {
      const int64_t tok = perm_token[pr];
      int64_t row = tok;
      if (sel1) {
        // the row of the secondary gate: the token's rank of the group
        int rank = 0;
        for (int j = 0; j < k1; ++j)
          if (sel1[tok * k1 + j] == grp) rank = j;
        row = tok * k1 + rank;
      }
      const float th0 = thresh[row * 2], th1 = thresh[row * 2 + 1];
      const float inv = rcp_f(softplus_f(un) + noise_floor);
      const float cl = v1 + be;
      acc += phi_f((cl - th1) * inv) - phi_f((cl - th0) * inv);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) part[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) corr[slice] = ((part[0] + part[1]) + part[2]) + part[3];
}

// Merges the candidate lists of a split selection: row t's `ranges` lists of
// L (value, expert) into its best L under the same order (value descending,
// ties to the lower expert), then the row's outputs. One wave per row: lane j
// takes candidates j, j + 64, ... (eight loads at a time), then the lanes'
// lists merge pairwise over six shuffle steps (the result does not depend on
// the merge order: the order is total and every expert appears in one range
// only).
template <int L>
__global__ __launch_bounds__(256) void gate_merge_kernel(GateParams p, int ranges) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= p.B) return;  // wave-uniform
  float lv[L];
  int li[L];
#pragma unroll
  for (int j = 0; j < L; ++j) {
    lv[j] = -INFINITY;
    li[j] = 0x7FFFFFFF;
  }
  const int total = ranges * L;
  const int64_t o = row * total;
  // eight candidates per lane loaded at once, then inserted
  for (int base = 0; base < total; base += 64 * 8) {
    float cv[8];
    int ci[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int c = base + lane + 64 * m;
      cv[m] = c < total ? p.cand_v[o + c] : -INFINITY;
      ci[m] = c < total ? p.cand_i[o + c] : 0x7FFFFFFF;
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) insert_any<L>(lv, li, cv[m], ci[m]);
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    float ov[L];
    int oi[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
      ov[j] = __shfl_xor(lv[j], s);
      oi[j] = __shfl_xor(li[j], s);
    }
#pragma unroll
    for (int j = 0; j < L; ++j) insert_any<L>(lv, li, ov[j], oi[j]);
  }
  // gate_order 1: the ranges' (max, sum) pairs, strided over the lanes, then
  // the same pairwise merge
  ExpSum es{-INFINITY, 0.f};
  if (p.cand_ms) {
    for (int r = lane; r < ranges; r += 64)
      es = expsum_merge(es, ExpSum{p.cand_ms[(row * ranges + r) * 2],
                                   p.cand_ms[(row * ranges + r) * 2 + 1]});
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1)
      es = expsum_merge(es, ExpSum{__shfl_xor(es.m, s), __shfl_xor(es.s, s)});
  }
  if (lane == 0) {
    GateParams q = p;
    q.cand_v = nullptr;
    q.cand_i = nullptr;
    q.cand_ms = nullptr;
    write_selection<L>(q, row, lv, li, es);
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

int gate_ranges(const GateLaunch& g) {
  if (g.units || g.tokens <= 0) return 1;
  const int rows = gate_tile_rows(g);
  const int64_t tiles = (g.tokens + rows - 1) / rows;
  constexpr int kTarget = 256;  // workgroups to aim for
  if (2 * tiles > kTarget) return 1;
  const int w = gate_uses_g32(g) ? (g.train ? kGate32Chunk : 2 * kGate32Chunk)
                                 : (g.x_dt == kBF16 && g.w_dt == kBF16 ? GateShape<bf16>::kChunk
                                                                        : GateShape<float>::kChunk);
  const int nch = (g.n + w - 1) / w;
  // ranges of two chunks or more; the 16x16 kernel also splits a sweep of two
  // or three chunks (a few dozen experts) into single chunks
  const int cap = gate_uses_g32(g) ? nch / 2 : std::max(nch / 2, std::min(nch, 2));
  const int64_t want = std::min<int64_t>((kTarget + tiles - 1) / tiles, cap);
  if (want <= 1) return 1;
  // equal ranges of `per` chunks, none empty
  const int per = (int)((nch + want - 1) / want);
  return (nch + per - 1) / per;
}

size_t gate_cand_bytes(const GateLaunch& g) {
  const int r = gate_ranges(g);
  if (r <= 1) return 0;
  // (value, expert) candidates, then a (max, sum) pair per row and range
  return (size_t)g.tokens * r * ((g.k <= 4 ? 5 : 9) * 8 + 8);
}

hipError_t launch_gate(const GateLaunch& g0, int32_t* topk_idx, float* topk_gate, float* thresh,
                       hipStream_t s, void* cand) {
  if (g0.tokens == 0) return hipSuccess;
  GateLaunch g = g0;
  g.ranges = cand ? gate_ranges(g) : 1;
  GateParams p = make_params(g);
  p.topk_idx = topk_idx;
  p.topk_gate = topk_gate;
  p.thresh = thresh;
  if (g.ranges <= 1) return gate_dispatch(g, p, false, s);
  // split sweep: each range's candidates, then one thread per row merges them
  const int L = g.k <= 4 ? 5 : 9;
  p.cand_v = static_cast<float*>(cand);
  p.cand_i = reinterpret_cast<int32_t*>(static_cast<char*>(cand) +
                                        (size_t)g.tokens * g.ranges * L * sizeof(float));
  if (g.gate_order)
    p.cand_ms = reinterpret_cast<float*>(static_cast<char*>(cand) +
                                         (size_t)g.tokens * g.ranges * L * 8);
  hipError_t e = gate_dispatch(g, p, false, s);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((g.tokens + 3) / 4));
  if (L == 5) hipLaunchKernelGGL((gate_merge_kernel<5>), grid, dim3(256), 0, s, p, g.ranges);
  else hipLaunchKernelGGL((gate_merge_kernel<9>), grid, dim3(256), 0, s, p, g.ranges);
  return hipGetLastError();
}

hipError_t launch_scores(const GateLaunch& g0, float* scores, int64_t sld, hipStream_t s) {
  if (g0.tokens == 0) return hipSuccess;
  GateLaunch g = g0;
  g.ranges = gate_ranges(g);  // each range writes its own experts' rows: no merge
  GateParams p = make_params(g);
  p.scores = scores;
  p.sld = sld;
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

int64_t corr_slices_max(int64_t pairs, int n) {
  // each expert has at most one partly filled slice
  return (int64_t)n + (pairs + kCorrSliceRows - 1) / kCorrSliceRows;
}

size_t corr_bytes(int64_t pairs, int n) {
  const size_t f = ((size_t)corr_slices_max(pairs, n) * sizeof(float) + 255) / 256 * 256;
  const size_t st = ((size_t)(n + 1) * sizeof(int32_t) + 255) / 256 * 256;
  const size_t se = ((size_t)corr_slices_max(pairs, n) * sizeof(int32_t) + 255) / 256 * 256;
  return f + st + se;
}

// The slice list of the corr region: after the slice sums.
int32_t* corr_slice_start(float* corr, int64_t pairs, int n) {
  const size_t f = ((size_t)corr_slices_max(pairs, n) * sizeof(float) + 255) / 256 * 256;
  return reinterpret_cast<int32_t*>(reinterpret_cast<char*>(corr) + f);
}

hipError_t launch_load_correction(const GateLaunch& g, int n, int64_t pairs,
                                  const int32_t* offsets, const int32_t* perm_token,
                                  const float* thresh, const int32_t* sel1, int k1, int b,
                                  float* corr, hipStream_t s) {
  int32_t* slice_start = corr_slice_start(corr, pairs, n);
  int32_t* slice_e = slice_start + ((size_t)(n + 1) * sizeof(int32_t) + 255) / 256 * 256 / sizeof(int32_t);
  hipLaunchKernelGGL(corr_slice_scan_kernel, dim3(1), dim3(1024), 0, s, offsets, n, slice_start,
                     slice_e);
  const dim3 grid((unsigned)corr_slices_max(pairs, n)), block(256);
  const void* bias = g.units ? nullptr : g.bias;
  const float* bp = reinterpret_cast<const float*>(bias);
#define MOE_CORR(XS, WS)                                                                      \
  hipLaunchKernelGGL((load_correction_kernel<XS, WS>), grid, block, 0, s, g.x, g.w_gate,      \
                     g.w_noise, bp, g.d, n, offsets, perm_token, thresh, g.noise_floor, sel1, \
                     k1, b, slice_start, slice_e, corr)
  if (g.x_dt == kBF16 && g.w_dt == kBF16) MOE_CORR(bf16, bf16);
  else if (g.x_dt == kBF16) MOE_CORR(bf16, float);
  else MOE_CORR(float, float);
#undef MOE_CORR
  return hipGetLastError();
}

hipError_t launch_load_grouped(const GateLaunch& g, int groups, const int32_t* unit_start,
                               const float* thresh, const int32_t* leaf_offsets,
                               const int32_t* leaf_perm_token, const int32_t* sel1, int k1,
                               float* partial, float* corr, float* load, hipStream_t s) {
  if (g.tokens > 0) {
    GateParams p = make_params(g);
    p.sel_thr = thresh;
    p.partial = partial;
    hipError_t e = gate_dispatch(g, p, true, s);
    if (e != hipSuccess) return e;
  }
  const int nleaves = groups * g.n;
  const int64_t pairs = g.tokens * g.k;
  hipError_t e = launch_load_correction(g, nleaves, pairs, leaf_offsets, leaf_perm_token, thresh,
                                        sel1, k1, g.n, corr, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(load_reduce_grouped_kernel, dim3((g.n + 31) / 32, groups), dim3(256), 0, s,
                     partial, unit_start, g.n, corr, corr_slice_start(corr, pairs, nleaves), load);
  return hipGetLastError();
}

bool gate_pair_grads_supported(const GateLaunch& g) {
  return g.train && !g.units && gate_uses_g32(g);
}

hipError_t launch_gate_pair_grads(const GateLaunch& g, const float* thresh, const float* dload,
                                  float* dcu, hipStream_t s) {
  if (g.tokens == 0) return hipSuccess;
  if (!gate_pair_grads_supported(g)) return hipErrorInvalidValue;
  GateLaunch gs = g;
  gs.ranges = gate_ranges(g);
  GateParams p = make_params(gs);
  p.sel_thr = thresh;
  p.dload = dload;
  p.dcu = dcu;
  return gate_dispatch(gs, p, true, s);
}

hipError_t launch_load(const GateLaunch& g, const float* thresh, const int32_t* offsets,
                       const int32_t* perm_token, float* partial, float* corr, float* load,
                       hipStream_t s) {
  // partial has room for gate_blocks() rows: the 32x32 kernel's 256-row blocks need fewer
  const int rows = gate_tile_rows(g);
  const int nb = (int)((g.tokens + rows - 1) / rows);
  if (nb > 0) {
    // a small batch splits each tile's sweep over the experts as the
    // selection does; every (tile, expert) column sum is still written once
    GateLaunch gs = g;
    gs.ranges = gate_ranges(g);
    GateParams p = make_params(gs);
    p.sel_thr = thresh;
    p.partial = partial;
    hipError_t e = gate_dispatch(gs, p, true, s);
    if (e != hipSuccess) return e;
  }
  const int64_t pairs = g.tokens * g.k;
  hipError_t e = launch_load_correction(g, g.n, pairs, offsets, perm_token, thresh, nullptr, 1, 1,
                                        corr, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(load_reduce_kernel, dim3((g.n + 31) / 32), dim3(256), 0, s, partial, nb,
                     g.n, corr, corr_slice_start(corr, pairs, g.n), load);
  return hipGetLastError();
}

}  // namespace moe
