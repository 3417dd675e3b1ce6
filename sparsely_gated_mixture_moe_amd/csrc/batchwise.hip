// Batchwise gating (section "What the paper measured" of the MoE explainer:
// the gate of the single-pair translation models, the paper's Appendix F).
// Instead of every token choosing its k best experts, every expert chooses
// rows of the batch: in training the m rows with the largest score H (m =
// k B / n gives every expert the same batch size); at inference the rows whose
// score exceeds the expert's threshold, here at most m of them (the largest).
// A token's gates are the softmax of the scores of the experts that took it
// (the softmax that eq 3 applies to the kept logits); y is eq 1.
//
//   1. scores     H of every (token, expert), written expert-major by the gate
//                 kernels (launch_scores): scores[e][t].
//   2. select     one workgroup per expert; its scores are read as
//                 order-preserving integer keys with 16-byte loads. The m-th
//                 largest of the threads' maxima is a lower bound of the cut (m
//                 distinct keys reach it); the few rows at or above it (about
//                 m) are gathered into LDS by a second pass, which mostly hits
//                 the caches, and ranked there: the cut, the ties (to the lower
//                 token) and each taken row's slot in token order. Expert e's
//                 rows go to slots [e m, e m + count_e). (When every row above
//                 the threshold is taken, or the candidates do not fit, a scan
//                 over all rows compacts.)
//   3. token lists  each token's slots: integer-atomic counts, a prefix sum,
//                 an atomic fill, then each list put in slot order by ranks
//                 (slot order is expert order, so every later sum over a
//                 token's experts has a fixed order).
//   4. expert FFNs  the grouped FFN kernel over the fixed-stride segments.
//   5. gates + combine  one wave per token: the softmax of its scores, then
//                 y = sum of gate * expert output, both in slot order.
//   6. importance per expert, the sum of its rows' gates in slot order; the
//                 load is the count (no noise estimate: the counts are fixed).
#include <climits>

#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kTileRows = 4 * kSelThreads;  // rows per pass step: 4 per thread
constexpr int kMaxTiles = 65536 / kTileRows;
constexpr int kCandCap = 2048;  // rows at or above the lower bound kept in LDS

// Order-preserving map of floats to unsigned keys (-0 is read as +0, so that
// equal numbers get equal keys); key_value is its inverse.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v == 0.f ? 0.f : v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Workgroup-wide sums of up to three per-thread integers. The LDS array is used by parity, so one barrier per call
// suffices: a wave writes slot p again only after every wave has passed the
// next call's barrier, i.e. has read slot p.
struct BlockSum {
  int (*red)[3][kSelWaves];
  int parity = 0;
  template <int N>
  __device__ __forceinline__ void finish(int (&v)[N]) {
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
      for (int i = 0; i < N; ++i) red[parity][i][wave] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int t = 0;
#pragma unroll
      for (int w = 0; w < kSelWaves; ++w) t += red[parity][i][w];
      v[i] = t;
    }
    parity ^= 1;
  }
  template <int N>
  __device__ __forceinline__ void sum(int (&v)[N]) {
    static_assert(N <= 3, "three sums per call");
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = wave_sum_i(v[i]);
    finish(v);
  }
};

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

// One workgroup per expert e: chooses its rows among scores[e * ld + 0 .. B)
// and writes them in token order to sel_token / sel_score [e m ...], their
// number to counts[e]. B <= 65536, ld a multiple of 4. Thread tid reads rows
// j * 2048 + 4 tid + (0..3) with one 16-byte load per step j; the first pass
// reads the column from HBM, later passes mostly hit the caches.
__global__ __launch_bounds__(kSelThreads) void batch_select_kernel(
    const float* __restrict__ scores, int B, int64_t ld, int m, const float* __restrict__ thr,
    int32_t* __restrict__ counts, int32_t* __restrict__ sel_token, float* __restrict__ sel_score) {
  __shared__ int red[2][3][kSelWaves];
  __shared__ uint32_t cand_k[kCandCap];
  __shared__ int32_t cand_r[kCandCap];
  __shared__ uint8_t cand_sel[kCandCap];
  __shared__ int cell_g[kMaxTiles * kSelWaves], cell_e[kMaxTiles * kSelWaves];
  __shared__ int wtot[2][kSelWaves];
  __shared__ uint32_t mxs[kSelThreads];
  __shared__ int ncand;
  __shared__ uint32_t tsh;
  BlockSum bs{red};
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tiles = (B + kTileRows - 1) / kTileRows;
  const float* col = scores + (int64_t)e * ld;
  // every step's keys, eight steps' loads issued before any is used
  auto each_step = [&](auto&& fn) {
    constexpr int kB = 8;
    for (int j0 = 0; j0 < tiles; j0 += kB) {
      f32x4 raw[kB];
#pragma unroll
      for (int q = 0; q < kB; ++q) {
        const int r0 = (j0 + q) * kTileRows + 4 * tid;
        raw[q] = r0 < B ? *reinterpret_cast<const f32x4*>(col + r0) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int q = 0; q < kB; ++q) {
        const int j = j0 + q;
        if (j >= tiles) break;
        const int r0 = j * kTileRows + 4 * tid;
        uint32_t k[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) k[i] = r0 + i < B ? order_key(raw[q][i]) : 0u;
        fn(j, k);
      }
    }
  };
  const float tv = thr ? thr[e] : -INFINITY;
  // a NaN threshold passes nothing (no number exceeds it)
  const uint32_t tkey = tv != tv ? 0xFFFFFFFFu : order_key(tv);
  const int64_t base = (int64_t)e * m;

  // First pass: the rows above the threshold and this thread's largest key.
  uint32_t mx = 0;
  int above = 0;
  each_step([&](int, const uint32_t (&k)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      above += k[i] > tkey;
      mx = max(mx, k[i]);
    }
  });
  int cv[1] = {above};
  bs.sum(cv);
  const int c = cv[0];  // rows above the threshold
  if (tid == 0) counts[e] = c < m ? c : m;

  // Rows with key > t are taken, and of those with key == t the first need_eq
  // in token order (with at most m rows above the threshold: all of them).
  // Compaction over every row: each (step, wave) cell's counts of rows above
  // t and of tied rows, an exclusive scan over the cells, then every taken
  // row's slot.
  auto compact_rows = [&](uint32_t t, int need_eq) {
    each_step([&](int j, const uint32_t (&k)[4]) {
      int g = 0, q = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g += k[i] > t;
        q += need_eq > 0 && k[i] == t;
      }
      g = wave_incl_scan(g, lane);
      q = wave_incl_scan(q, lane);
      if (lane == 63) {
        cell_g[j * kSelWaves + wave] = g;
        cell_e[j * kSelWaves + wave] = q;
      }
    });
    __syncthreads();
    {
      const int nc = tiles * kSelWaves;
      int vg = tid < nc ? cell_g[tid] : 0;
      int ve = tid < nc ? cell_e[tid] : 0;
      const int og = vg, oe = ve;
      vg = wave_incl_scan(vg, lane);
      ve = wave_incl_scan(ve, lane);
      if (lane == 63) {
        wtot[0][wave] = vg;
        wtot[1][wave] = ve;
      }
      __syncthreads();
      for (int w = 0; w < wave; ++w) {
        vg += wtot[0][w];
        ve += wtot[1][w];
      }
      if (tid < nc) {
        cell_g[tid] = vg - og;
        cell_e[tid] = ve - oe;
      }
    }
    __syncthreads();
    each_step([&](int j, const uint32_t (&k)[4]) {
      int g = 0, q = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g += k[i] > t;
        q += need_eq > 0 && k[i] == t;
      }
      int gb = cell_g[j * kSelWaves + wave] + wave_incl_scan(g, lane) - g;
      int eb = cell_e[j * kSelWaves + wave] + wave_incl_scan(q, lane) - q;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool gt = k[i] > t;
        const bool eq = need_eq > 0 && k[i] == t;
        const int pos = gb + min(eb, need_eq);
        if ((gt || (eq && eb < need_eq)) && pos < m) {
          sel_token[base + pos] = j * kTileRows + 4 * tid + i;
          sel_score[base + pos] = key_value(k[i]);
        }
        gb += gt;
        eb += eq;
      }
    });
  };

  if (c <= m) {
    compact_rows(tkey, 0);
    return;
  }
  if (m <= kSelThreads) {
    // lower bound lb <= t: the m-th largest of the threads' maxima (m
    // distinct keys are >= it), by a bitwise search that one wave runs alone
    // over the maxima in LDS (no workgroup barrier per step)
    mxs[tid] = mx;
    __syncthreads();
    if (wave == 0) {
      constexpr int PER = kSelThreads / 64;
      uint32_t v[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) v[i] = mxs[lane * PER + i];
      uint32_t l = 0;
      for (int b = 31; b >= 0; --b) {
        const uint32_t cb = l | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) cnt += v[i] >= cb;
        if (wave_sum_i(cnt) >= m) l = cb;
      }
      if (lane == 0) tsh = l;
    }
    __syncthreads();
    const uint32_t lb = tsh;
    // the rows with keys >= lb (at least m of them, and every row with a key
    // >= t) to LDS, in any order, from a second pass over the column (it
    // mostly hits the caches)
    if (tid == 0) ncand = 0;
    __syncthreads();
    each_step([&](int j, const uint32_t (&k)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (k[i] >= lb) {
          const int at = atomicAdd(&ncand, 1);
          if (at < kCandCap) {
            cand_k[at] = k[i];
            cand_r[at] = j * kTileRows + 4 * tid + i;
          }
        }
      }
    });
    __syncthreads();
    const int nc = ncand;
    if (nc <= kCandCap) {
      // t: the candidate with fewer than m candidates above it and at least m
      // at or above it (all such candidates hold the same key)
      for (int q = tid; q < nc; q += kSelThreads) {
        const uint32_t v = cand_k[q];
        int gt = 0, ge = 0;
        for (int r = 0; r < nc; ++r) {
          const uint32_t w = cand_k[r];
          gt += w > v;
          ge += w >= v;
        }
        if (gt < m && ge >= m) tsh = v;
      }
      __syncthreads();
      const uint32_t t = tsh;
      int gtc[1] = {0};
      for (int q = tid; q < nc; q += kSelThreads) gtc[0] += cand_k[q] > t;
      bs.sum(gtc);
      const int need_eq = m - gtc[0];
      // taken: above t, or tied and among the first need_eq tied rows
      for (int q = tid; q < nc; q += kSelThreads) {
        const uint32_t v = cand_k[q];
        bool sel = v > t;
        if (v == t) {
          const int r = cand_r[q];
          int er = 0;
          for (int p = 0; p < nc; ++p) er += cand_k[p] == t && cand_r[p] < r;
          sel = er < need_eq;
        }
        cand_sel[q] = sel;
      }
      __syncthreads();
      // slot: the taken candidates on lower rows
      for (int q = tid; q < nc; q += kSelThreads) {
        if (!cand_sel[q]) continue;
        const int r = cand_r[q];
        int pos = 0;
        for (int p = 0; p < nc; ++p) pos += cand_sel[p] && cand_r[p] < r;
        if (pos < m) {
          sel_token[base + pos] = r;
          sel_score[base + pos] = key_value(cand_k[q]);
        }
      }
      return;
    }
  }
  // general case: a bitwise search for the largest t with at least m keys >= t
  uint32_t t = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cb = t | (1u << b);
    int cnt[1] = {0};
    each_step([&](int, const uint32_t (&k)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) cnt[0] += k[i] >= cb;
    });
    bs.sum(cnt);
    if (cnt[0] >= m) t = cb;
  }
  int gt[1] = {0};
  each_step([&](int, const uint32_t (&k)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) gt[0] += k[i] > t;
  });
  bs.sum(gt);
  compact_rows(t, m - gt[0]);
}

// Exclusive prefix sum of n counts into offsets [n + 1], one workgroup of
// 1024 threads: steps of 4096 counts, 4 consecutive per thread, a wave scan
// and the waves' totals, plus the running total of earlier steps.
__global__ __launch_bounds__(1024) void batch_scan_kernel(const int32_t* __restrict__ in, int n,
                                                          int32_t* __restrict__ out) {
  __shared__ int wsum[2][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  for (int s0 = 0, it = 0; s0 < n; s0 += 4096, ++it) {
    const int i0 = s0 + 4 * tid;
    int v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = i0 + i < n ? in[i0 + i] : 0;
    const int own = v[0] + v[1] + v[2] + v[3];
    const int incl = wave_incl_scan(own, lane);
    if (lane == 63) wsum[it & 1][wave] = incl;
    __syncthreads();
    int before = carry + incl - own, total = carry;
    for (int w = 0; w < 16; ++w) {
      const int x = wsum[it & 1][w];
      if (w < wave) before += x;
      total += x;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i0 + i < n) out[i0 + i] = before;
      before += v[i];
    }
    carry = total;
  }
  if (tid == 0) out[n] = carry;
}

__global__ void batch_zero_kernel(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Rows each token was taken for (integer atomics: the counts do not depend on
// the order of the additions).
__global__ void batch_tok_count_kernel(const int32_t* __restrict__ counts,
                                       const int32_t* __restrict__ sel_token, int64_t slots, int m,
                                       int B, int32_t* __restrict__ tok_cnt) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= slots) return;
  const int e = (int)(q / m);
  if (q - (int64_t)e * m >= counts[e]) return;
  const int tok = sel_token[q];
  if (tok >= 0 && tok < B) atomicAdd(&tok_cnt[tok], 1);
}

// Each taken slot into its token's list (in any order; counted down from the
// token's count, which ends at 0).
__global__ void batch_tok_fill_kernel(const int32_t* __restrict__ counts,
                                      const int32_t* __restrict__ sel_token, int64_t slots, int m,
                                      int B,
                                      const int32_t* __restrict__ tok_off,
                                      int32_t* __restrict__ tok_cnt,
                                      int32_t* __restrict__ tok_list) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= slots) return;
  const int e = (int)(q / m);
  if (q - (int64_t)e * m >= counts[e]) return;
  const int tok = sel_token[q];
  if (tok < 0 || tok >= B) return;
  const int pos = atomicSub(&tok_cnt[tok], 1) - 1;
  if (pos >= 0) tok_list[tok_off[tok] + pos] = (int32_t)q;
}

// One wave per token: its list in slot order (ranks; the slots are distinct).
__global__ __launch_bounds__(256) void batch_tok_sort_kernel(const int32_t* __restrict__ tok_off,
                                                             const int32_t* __restrict__ tok_list,
                                                             int B, int32_t* __restrict__ tok_sorted) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= B) return;
  const int o = tok_off[tok];
  const int c = tok_off[tok + 1] - o;
  for (int a0 = 0; a0 < c; a0 += 64) {
    const int a = a0 + lane;
    const int va = a < c ? tok_list[o + a] : INT_MAX;
    int rank = 0;
    for (int b0 = 0; b0 < c; b0 += 64) {
      const int vb = b0 + lane < c ? tok_list[o + b0 + lane] : INT_MAX;
      const int nb = min(64, c - b0);
      for (int s = 0; s < nb; ++s) rank += __shfl(vb, s) < va;
    }
    if (a < c) tok_sorted[o + rank] = va;
  }
}

// One wave per token: its gates (softmax of its scores, slot order) to
// sel_gate, and y[tok] = sum over its slots, in slot order, of gate * expert
// output (fp32 accumulation), one 16-byte unit of the row per lane and step.
template <typename T, bool NT>
__global__ __launch_bounds__(256) void batch_combine_kernel(
    const T* __restrict__ eo, const int32_t* __restrict__ tok_off,
    const int32_t* __restrict__ tok_sorted, const float* __restrict__ sel_score,
    float* __restrict__ sel_gate, int B, int d, T* __restrict__ y) {
  constexpr int UE = Elem<T>::kPerUnit;
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= B) return;
  const int o = tok_off[tok];
  const int c = tok_off[tok + 1] - o;
  float mx = -INFINITY;
  for (int a = lane; a < c; a += 64) mx = fmaxf(mx, sel_score[tok_sorted[o + a]]);
  mx = wave_max_f(mx);
  float den = 0.f;
  for (int a = lane; a < c; a += 64) den += expf(sel_score[tok_sorted[o + a]] - mx);
  den = wave_sum_f(den);
  for (int a = lane; a < c; a += 64) {
    const int q = tok_sorted[o + a];
    sel_gate[q] = expf(sel_score[q] - mx) / den;
  }
  const int units = d / UE;
  for (int u = lane; u < units; u += 64) {
    float acc[UE];
#pragma unroll
    for (int i = 0; i < UE; ++i) acc[i] = 0.f;
    // slots in groups of four: positions, gates and rows requested first,
    // then added in slot order
    for (int a0 = 0; a0 < c; a0 += 4) {
      int q[4];
      float g[4];
      U16 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = a0 + i < c ? tok_sorted[o + a0 + i] : -1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g[i] = q[i] >= 0 ? expf(sel_score[q[i]] - mx) / den : 0.f;
        v[i] = q[i] < 0 ? zero_unit()
               : NT ? ld_unit_stream(eo + (int64_t)q[i] * d + u * UE)
                    : ld_unit(eo + (int64_t)q[i] * d + u * UE);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (q[i] < 0) continue;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            acc[2 * w] += g[i] * __uint_as_float(v[i].w[w] << 16);
            acc[2 * w + 1] += g[i] * __uint_as_float(v[i].w[w] & 0xFFFF0000u);
          }
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) acc[w] += g[i] * __uint_as_float(v[i].w[w]);
        }
      }
    }
    U16 out;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w)
        out.w[w] = f32_to_bf16_bits(acc[2 * w]) | (f32_to_bf16_bits(acc[2 * w + 1]) << 16);
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) out.w[w] = __float_as_uint(acc[w]);
    }
    st_unit(y + (int64_t)tok * d + u * UE, out);
  }
}

// One wave per expert: Importance (eq 6) = the sum of its rows' gates,
// lane-strided in slot order, then a fixed butterfly.
__global__ __launch_bounds__(256) void batch_importance_kernel(const int32_t* __restrict__ counts,
                                                               const float* __restrict__ sel_gate,
                                                               int n, int m,
                                                               float* __restrict__ importance) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= n) return;
  const int c = counts[e];
  const float* g = sel_gate + (int64_t)e * m;
  float s = 0.f;
  for (int r = lane; r < c; r += 64) s += g[r];
  s = wave_sum_f(s);
  if (lane == 0) importance[e] = s;
}

// Row stride of the score matrix: B rounded up to 4 floats, so that every
// row starts 16-byte aligned.
int64_t score_ld(int64_t B) { return (B + 3) / 4 * 4; }

}  // namespace

size_t batchwise_ws_bytes(int64_t tokens, int n, int m, int d, int h, Dt act_dt) {
  const int64_t slots = (int64_t)n * m;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  return al((size_t)score_ld(tokens) * n * sizeof(float)) +  // scores
         al((size_t)tokens * sizeof(int32_t)) +            // tok_cnt
         al((size_t)(tokens + 1) * sizeof(int32_t)) +      // tok_off
         2 * al((size_t)slots * sizeof(int32_t)) +         // tok_list, tok_sorted
         al(ffn_plan_bytes(slots, n, d, h, act_dt)) +      // FFN work units
         al((size_t)slots * d * (act_dt == kBF16 ? 2 : 4)); // expert outputs
}

void batchwise_carve(BatchwiseLaunch& b, void* ws, int d, int h, Dt act_dt) {
  const int64_t B = b.gate.tokens;
  const int n = b.gate.n;
  const int64_t slots = (int64_t)n * b.m;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  char* p = static_cast<char*>(ws);
  b.scores = reinterpret_cast<float*>(p);
  p += al((size_t)score_ld(B) * n * sizeof(float));
  b.tok_cnt = reinterpret_cast<int32_t*>(p);
  p += al((size_t)B * sizeof(int32_t));
  b.tok_off = reinterpret_cast<int32_t*>(p);
  p += al((size_t)(B + 1) * sizeof(int32_t));
  b.tok_list = reinterpret_cast<int32_t*>(p);
  p += al((size_t)slots * sizeof(int32_t));
  b.tok_sorted = reinterpret_cast<int32_t*>(p);
  p += al((size_t)slots * sizeof(int32_t));
  b.ffn_blocks = reinterpret_cast<int32_t*>(p);
  p += al(ffn_plan_bytes(slots, n, d, h, act_dt));
  b.expert_out = p;
}

hipError_t launch_batchwise(const BatchwiseLaunch& b, hipStream_t s, hipEvent_t ev0,
                            hipEvent_t ev1) {
  const int64_t B = b.gate.tokens;
  const int n = b.gate.n;
  const int m = b.m;
  const int64_t slots = (int64_t)n * m;
  if (B > 65536 || m < 1 || slots >= INT_MAX) return hipErrorInvalidValue;
  const int64_t ld = score_ld(B);
  hipError_t e = launch_scores(b.gate, b.scores, ld, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(batch_select_kernel, dim3((unsigned)n), dim3(kSelThreads), 0, s, b.scores,
                     (int)B, ld, m, b.threshold, b.counts, b.sel_token, b.sel_score);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const unsigned slot_blocks = (unsigned)((slots + 255) / 256);
  if (B > 0) {
    hipLaunchKernelGGL(batch_zero_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s,
                       b.tok_cnt, (int)B);
    hipLaunchKernelGGL(batch_tok_count_kernel, dim3(slot_blocks), dim3(256), 0, s, b.counts,
                       b.sel_token, slots, m, (int)B, b.tok_cnt);
  }
  hipLaunchKernelGGL(batch_scan_kernel, dim3(1), dim3(1024), 0, s, b.tok_cnt, (int)B, b.tok_off);
  if (B > 0) {
    hipLaunchKernelGGL(batch_tok_fill_kernel, dim3(slot_blocks), dim3(256), 0, s, b.counts,
                       b.sel_token, slots, m, (int)B, b.tok_off, b.tok_cnt, b.tok_list);
    hipLaunchKernelGGL(batch_tok_sort_kernel, dim3((unsigned)((B + 3) / 4)), dim3(256), 0, s,
                       b.tok_off, b.tok_list, (int)B, b.tok_sorted);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = launch_ffn(slots, 1, b.gate.d, b.h, n, b.act_dt, b.gate.x, nullptr, b.sel_token, b.w1, b.b1,
                 b.w2, b.b2, b.expert_out, b.ffn_blocks, s, ev0, ev1, 0, b.counts, m, b.packed);
  if (e != hipSuccess) return e;
  if (B > 0) {
    const dim3 grid((unsigned)((B + 3) / 4));
    // expert outputs past the Infinity Cache's size: non-temporal loads (as in the combine)
    const bool nt = (int64_t)slots * b.gate.d * (b.act_dt == kBF16 ? 2 : 4) > kStreamBytes;
#define MOE_BCOMBINE(TT, NTV)                                                                    \
  hipLaunchKernelGGL((batch_combine_kernel<TT, NTV>), grid, dim3(256), 0, s,                    \
                     reinterpret_cast<const TT*>(b.expert_out), b.tok_off, b.tok_sorted,         \
                     b.sel_score, b.sel_gate, (int)B, b.gate.d, reinterpret_cast<TT*>(b.y))
    if (b.act_dt == kBF16) {
      if (nt) MOE_BCOMBINE(bf16, true);
      else MOE_BCOMBINE(bf16, false);
    } else {
      if (nt) MOE_BCOMBINE(float, true);
      else MOE_BCOMBINE(float, false);
    }
#undef MOE_BCOMBINE
  }
  hipLaunchKernelGGL(batch_importance_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s,
                     b.counts, b.sel_gate, n, m, b.importance);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_counts_to_load(b.counts, n, b.load, s)) != hipSuccess) return e;
  return launch_cv2_losses(b.importance, b.load, n, b.w_importance, b.w_load, b.losses, s);
}

}  // namespace moe
