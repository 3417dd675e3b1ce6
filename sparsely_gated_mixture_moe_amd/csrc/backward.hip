// Backward pass of the MoE layer on gfx950. Which parameters receive gradients
// follows the explainer's paragraph after its forward-pass code ("Implementation
// notes"): each expert only from the rows routed to it, scaled by their gates;
// W_g through the softmax over the kept logits (task and Importance losses) and
// through the numerator of eq 9 (Load loss, also for experts that were not
// kept); W_noise through the noise term of the kept logits and through the
// denominator of eq 9. The selection and eq 9's thresholds pass no gradient.
// The experts' hidden activations are recomputed here, not stored by the
// forward pass (the memory saving the same section describes).
//
// The matrix products run on the fp32 matrix cores (v_mfma_f32_16x16x4f32,
// bf16 operands widened exactly), in two grouped forms over the contiguous
// per-expert segments that routing produces:
//   * row products: out[p] = f(a[p] . W_e) for the rows p of expert e's
//     segment (a's rows optionally gathered through the token list and scaled
//     by the row's gate), 64 x 64 output tiles, K in steps of 16 through LDS;
//   * weight-gradient products: dW_e = sum over e's rows of a[p]^T b[p], one
//     64 x 64 tile of dW_e per workgroup, the segment's rows in steps of 16,
//     with the column sums of a (the bias gradients) on the side.
// Every sum runs in a fixed order, so the results are deterministic.
#include <cmath>

#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kT = 64;   // output tile edge of both product kernels
constexpr int kKS = 16;  // K (or rows) per LDS step

template <typename T>
__device__ __forceinline__ float ld_f(const void* p, int64_t i) {
  if constexpr (sizeof(T) == 2) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  } else {
    return reinterpret_cast<const float*>(p)[i];
  }
}

template <typename T>
__device__ __forceinline__ void st_f(void* p, int64_t i, float v) {
  if constexpr (sizeof(T) == 2) {
    reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16_bits(v);
  } else {
    reinterpret_cast<float*>(p)[i] = v;
  }
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Row products
// ---------------------------------------------------------------------------

struct RowGemm {
  // rows: with `units` (null: one segment of `rows` rows), unit u covers rows
  // seg_off[g] + r0 .. of segment g, (g, r0) = (units[1 + 2u], units[2 + 2u]),
  // up to the segment's end; units[0] is the number of units.
  const int32_t* units;
  const int32_t* seg_off;
  int64_t rows;
  // a: [rows][K] (row p at a + row(p) * lda, row(p) = gather ? gather[p] : p),
  // optionally times scale[p]
  const void* a;
  int64_t lda;
  const int32_t* gather;
  const float* scale;
  // W of segment g at w + g * w_stride: wt = 1: [N][K] row-major (out = a W^T);
  // wt = 0: [K][N] row-major (out = a W)
  const void* w;
  int64_t w_stride;
  int wt;
  int K, N;
  // epilogue: + bias[g * N + c] (storage type of W; fp32 with bias_f32), ReLU,
  // times (mask[p][c] > 0) (mask fp32, or bf16 with mask_bf16), accumulate into out
  const void* bias;
  int bias_f32;
  int relu;
  const void* mask;  // row stride ldm
  int mask_bf16;
  int64_t ldm;
  int accumulate;
  void* out;
  int64_t ldo;
};

template <typename TA, typename TW, typename TO>
__global__ __launch_bounds__(256) void row_gemm_kernel(RowGemm p) {
  __shared__ float as[kT][kKS + 1];
  __shared__ float bs[kKS][kT + 1];
  int g = 0;
  int64_t r0, rend;
  if (p.units) {
    const int u = blockIdx.x;
    if (u >= p.units[0]) return;
    g = p.units[1 + 2 * u];
    r0 = (int64_t)p.seg_off[g] + p.units[2 + 2 * u];
    rend = p.seg_off[g + 1];
  } else {
    r0 = (int64_t)blockIdx.x * kT;
    rend = p.rows;
    if (r0 >= rend) return;
  }
  const int c0 = blockIdx.y * kT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, q = lane >> 4;
  const char* wseg = reinterpret_cast<const char*>(p.w) + (int64_t)g * p.w_stride * sizeof(TW);
  f32x4 acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the four A elements of this thread: row tid / 4, K (tid % 4) * 4 + 0..3
  const int ar = tid >> 2, ak = (tid & 3) * 4;
  const int64_t arow_p = r0 + ar;
  const bool arow_ok = arow_p < rend;
  int64_t arow = 0;
  float ascale = 1.f;
  if (arow_ok) {
    arow = p.gather ? (int64_t)p.gather[arow_p] : arow_p;
    if (p.scale) ascale = p.scale[arow_p];
  }
  for (int k0 = 0; k0 < p.K; k0 += kKS) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = k0 + ak + i;
      as[ar][ak + i] = (arow_ok && kk < p.K) ? ascale * ld_f<TA>(p.a, arow * p.lda + kk) : 0.f;
    }
    if (p.wt) {  // W [N][K]: thread reads 4 consecutive K of one column n
      const int n = tid >> 2, kq = (tid & 3) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = k0 + kq + i, nn = c0 + n;
        bs[kq + i][n] = (kk < p.K && nn < p.N) ? ld_f<TW>(wseg, (int64_t)nn * p.K + kk) : 0.f;
      }
    } else {  // W [K][N]: thread reads 4 consecutive N of one K row
      const int kq = tid >> 4, n4 = (tid & 15) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = k0 + kq, nn = c0 + n4 + i;
        bs[kq][n4 + i] = (kk < p.K && nn < p.N) ? ld_f<TW>(wseg, (int64_t)kk * p.N + nn) : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kKS / 4; ++ks) {
      const float a = as[16 * wave + lr][ks * 4 + q];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[ct] = mfma4(a, bs[ks * 4 + q][16 * ct + lr], acc[ct]);
    }
    __syncthreads();
  }
  // C layout: lane holds rows 4q + i of its wave's 16, column lr of each tile
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int c = c0 + 16 * ct + lr;
    if (c >= p.N) continue;
    float b = 0.f;
    if (p.bias)
      b = p.bias_f32 ? ld_f<float>(p.bias, (int64_t)g * p.N + c) : ld_f<TW>(p.bias, (int64_t)g * p.N + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t rp = r0 + 16 * wave + 4 * q + i;
      if (rp >= rend) continue;
      float v = acc[ct][i] + b;
      if (p.relu) v = v > 0.f ? v : 0.f;
      if (p.mask) {
        const float mv = p.mask_bf16 ? ld_f<bf16>(p.mask, rp * p.ldm + c)
                                     : ld_f<float>(p.mask, rp * p.ldm + c);
        v = mv > 0.f ? v : 0.f;
      }
      const int64_t o = rp * p.ldo + c;
      if (p.accumulate) v += ld_f<TO>(p.out, o);
      st_f<TO>(p.out, o, v);
    }
  }
}

// ---------------------------------------------------------------------------
// Weight-gradient products
// ---------------------------------------------------------------------------

struct Wgrad {
  // segment g: rows seg_off[g] .. seg_off[g + 1] - 1 (null: one segment of
  // `rows` rows)
  const int32_t* seg_off;
  int64_t rows;
  // a: [rows][M], b: [rows][N], each row optionally gathered and scaled
  const void* a;
  int64_t lda;
  const int32_t* a_gather;
  const float* a_scale;
  const void* b;
  int64_t ldb;
  const int32_t* b_gather;
  const float* b_scale;
  int M, N;
  // out_g [M][N] fp32 at out + g * out_stride (row stride N)
  float* out;
  int64_t out_stride;
  // optional: colsum[g * M + m] = sum over g's rows of a[p][m], in row order
  float* colsum;
};

template <typename TA, typename TB>
__global__ __launch_bounds__(256) void wgrad_kernel(Wgrad p) {
  __shared__ float at[kKS][kT + 1];
  __shared__ float bt[kKS][kT + 1];
  const int mtiles = (p.M + kT - 1) / kT;
  const int m0 = (blockIdx.x % mtiles) * kT, n0 = (blockIdx.x / mtiles) * kT;
  const int g = blockIdx.y;
  const int64_t s0 = p.seg_off ? p.seg_off[g] : 0;
  const int64_t s1 = p.seg_off ? p.seg_off[g + 1] : p.rows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, q = lane >> 4;
  const bool do_colsum = p.colsum != nullptr && n0 == 0;
  f32x4 acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float cs = 0.f;
  // the four elements of each operand this thread loads: row tid / 16, column (tid % 16) * 4 + 0..3
  const int lrow = tid >> 4, lc = (tid & 15) * 4;
  for (int64_t r = s0; r < s1; r += kKS) {
    const int64_t rp = r + lrow;
    const bool ok = rp < s1;
    int64_t ra = 0, rb = 0;
    float sa = 1.f, sb = 1.f;
    if (ok) {
      ra = p.a_gather ? (int64_t)p.a_gather[rp] : rp;
      rb = p.b_gather ? (int64_t)p.b_gather[rp] : rp;
      if (p.a_scale) sa = p.a_scale[rp];
      if (p.b_scale) sb = p.b_scale[rp];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + lc + i, n = n0 + lc + i;
      at[lrow][lc + i] = (ok && m < p.M) ? sa * ld_f<TA>(p.a, ra * p.lda + m) : 0.f;
      bt[lrow][lc + i] = (ok && n < p.N) ? sb * ld_f<TB>(p.b, rb * p.ldb + n) : 0.f;
    }
    __syncthreads();
    if (do_colsum && tid < kT) {
#pragma unroll
      for (int i = 0; i < kKS; ++i) cs += at[i][tid];
    }
#pragma unroll
    for (int ks = 0; ks < kKS / 4; ++ks) {
      const float a = at[ks * 4 + q][16 * wave + lr];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[ct] = mfma4(a, bt[ks * 4 + q][16 * ct + lr], acc[ct]);
    }
    __syncthreads();
  }
  float* og = p.out + (int64_t)g * p.out_stride;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int n = n0 + 16 * ct + lr;
    if (n >= p.N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 16 * wave + 4 * q + i;
      if (m < p.M) og[(int64_t)m * p.N + n] = acc[ct][i];
    }
  }
  if (do_colsum && tid < kT && m0 + tid < p.M) p.colsum[(int64_t)g * p.M + m0 + tid] = cs;
}

// ---------------------------------------------------------------------------
// The same products on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16), for
// bf16 storage. Operands in bf16 storage are exact; an fp32 operand (the
// recomputed hidden layer, the hidden and logit gradients) is split into
// hi = bf16(v) and lo = bf16(v - hi), exact to about 2^-17 of v, and its
// products take the hi and lo parts against the other operand (hi x lo'
// cross terms of two split operands are kept, lo x lo' dropped). Row scales
// (the gates) are applied where they keep an exact operand exact: in the row
// products' epilogue, in the weight-gradient products to the split operand.
// ---------------------------------------------------------------------------

constexpr int kK16 = 32;  // K (or rows) per LDS step of the bf16 products
constexpr int kP16 = 8;   // bf16 elements of padding per LDS row

__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  const uint32_t h = f32_to_bf16_bits(v);
  hi = (uint16_t)h;
  lo = (uint16_t)f32_to_bf16_bits(v - bf16_bits_to_f32(h));
}

__device__ __forceinline__ f32x4 mfma16(const U16& a, const U16& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_short8(a), as_short8(b), c, 0, 0, 0);
}

// Eight consecutive elements of row `row` from column `col` (zero past `lim`).
template <typename T>
__device__ __forceinline__ void load8_row(const void* base, int64_t row, int64_t ld, int col,
                                          int lim, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (col + i < lim) ? ld_f<T>(base, row * ld + col + i) : 0.f;
}

template <typename TA, typename TW, typename TO, bool SA, bool SW>
__global__ __launch_bounds__(256) void row_gemm16_kernel(RowGemm p) {
  __shared__ __attribute__((aligned(16))) uint16_t ash[kT][kK16 + kP16];
  __shared__ __attribute__((aligned(16))) uint16_t asl[SA ? kT : 1][kK16 + kP16];
  __shared__ __attribute__((aligned(16))) uint16_t bsh[kT][kK16 + kP16];
  __shared__ __attribute__((aligned(16))) uint16_t bsl[SW ? kT : 1][kK16 + kP16];
  int g = 0;
  int64_t r0, rend;
  if (p.units) {
    const int u = blockIdx.x;
    if (u >= p.units[0]) return;
    g = p.units[1 + 2 * u];
    r0 = (int64_t)p.seg_off[g] + p.units[2 + 2 * u];
    rend = p.seg_off[g + 1];
  } else {
    r0 = (int64_t)blockIdx.x * kT;
    rend = p.rows;
    if (r0 >= rend) return;
  }
  const int c0 = blockIdx.y * kT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, q = lane >> 4;
  const char* wseg = reinterpret_cast<const char*>(p.w) + (int64_t)g * p.w_stride * sizeof(TW);
  f32x4 acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  // A: row tid / 4, K run (tid % 4) * 8 .. + 7
  const int ar = tid >> 2, ak = (tid & 3) * 8;
  const int64_t arow_p = r0 + ar;
  const bool arow_ok = arow_p < rend;
  const int64_t arow = arow_ok ? (p.gather ? (int64_t)p.gather[arow_p] : arow_p) : 0;
  for (int k0 = 0; k0 < p.K; k0 += kK16) {
    {
      float v[8];
      load8_row<TA>(p.a, arow, p.lda, k0 + ak, arow_ok ? p.K : 0, v);
      uint16_t h[8], l[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) split_bf16(v[i], h[i], l[i]);
#pragma unroll
      for (int i = 0; i < 8; ++i) ash[ar][ak + i] = h[i];
      if constexpr (SA) {
#pragma unroll
        for (int i = 0; i < 8; ++i) asl[ar][ak + i] = l[i];
      }
    }
    if (p.wt) {  // W [N][K]: 8 consecutive K of column n
      const int n = tid >> 2, kq = (tid & 3) * 8;
      float v[8];
      load8_row<TW>(wseg, c0 + n, p.K, k0 + kq, (c0 + n < p.N) ? p.K : 0, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint16_t h, l;
        split_bf16(v[i], h, l);
        bsh[n][kq + i] = h;
        if constexpr (SW) bsl[n][kq + i] = l;
      }
    } else {  // W [K][N]: 8 consecutive N of K row k
      const int kr = tid >> 3, n8 = (tid & 7) * 8;
      float v[8];
      load8_row<TW>(wseg, k0 + kr, p.N, c0 + n8, (k0 + kr < p.K) ? p.N : 0, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint16_t h, l;
        split_bf16(v[i], h, l);
        bsh[n8 + i][kr] = h;
        if constexpr (SW) bsl[n8 + i][kr] = l;
      }
    }
    __syncthreads();
    const U16 a = *reinterpret_cast<const U16*>(&ash[16 * wave + lr][8 * q]);
    U16 al;
    if constexpr (SA) al = *reinterpret_cast<const U16*>(&asl[16 * wave + lr][8 * q]);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const U16 b = *reinterpret_cast<const U16*>(&bsh[16 * ct + lr][8 * q]);
      acc[ct] = mfma16(a, b, acc[ct]);
      if constexpr (SA) acc[ct] = mfma16(al, b, acc[ct]);
      if constexpr (SW) {
        const U16 bl = *reinterpret_cast<const U16*>(&bsl[16 * ct + lr][8 * q]);
        acc[ct] = mfma16(a, bl, acc[ct]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int c = c0 + 16 * ct + lr;
    if (c >= p.N) continue;
    float b = 0.f;
    if (p.bias)
      b = p.bias_f32 ? ld_f<float>(p.bias, (int64_t)g * p.N + c) : ld_f<TW>(p.bias, (int64_t)g * p.N + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t rp = r0 + 16 * wave + 4 * q + i;
      if (rp >= rend) continue;
      float v = acc[ct][i];
      if (p.scale) v *= p.scale[rp];
      v += b;
      if (p.relu) v = v > 0.f ? v : 0.f;
      if (p.mask) {
        const float mv = p.mask_bf16 ? ld_f<bf16>(p.mask, rp * p.ldm + c)
                                     : ld_f<float>(p.mask, rp * p.ldm + c);
        v = mv > 0.f ? v : 0.f;
      }
      const int64_t o = rp * p.ldo + c;
      if (p.accumulate) v += ld_f<TO>(p.out, o);
      st_f<TO>(p.out, o, v);
    }
  }
}

template <typename TA, typename TB, bool SA, bool SB>
__global__ __launch_bounds__(256) void wgrad16_kernel(Wgrad p) {
  static_assert(SA || SB, "a row scale needs a split operand");
  __shared__ __attribute__((aligned(16))) uint16_t ath[kT][kK16 + kP16];  // [m][row]
  __shared__ __attribute__((aligned(16))) uint16_t atl[SA ? kT : 1][kK16 + kP16];
  __shared__ __attribute__((aligned(16))) uint16_t bth[kT][kK16 + kP16];  // [n][row]
  __shared__ __attribute__((aligned(16))) uint16_t btl[SB ? kT : 1][kK16 + kP16];
  __shared__ float cst[kK16][kT + 1];  // the colsum's scaled A values, fp32
  const int mtiles = (p.M + kT - 1) / kT;
  const int m0 = (blockIdx.x % mtiles) * kT, n0 = (blockIdx.x / mtiles) * kT;
  const int g = blockIdx.y;
  const int64_t s0 = p.seg_off ? p.seg_off[g] : 0;
  const int64_t s1 = p.seg_off ? p.seg_off[g + 1] : p.rows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, q = lane >> 4;
  const bool do_colsum = p.colsum != nullptr && n0 == 0;
  f32x4 acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float cs = 0.f;
  // loads: row tid / 8 of the step, 8 consecutive columns from (tid % 8) * 8
  const int lrow = tid >> 3, lc = (tid & 7) * 8;
  for (int64_t r = s0; r < s1; r += kK16) {
    const int64_t rp = r + lrow;
    const bool ok = rp < s1;
    int64_t ra = 0, rb = 0;
    float sa = 1.f, sb = 1.f;
    if (ok) {
      ra = p.a_gather ? (int64_t)p.a_gather[rp] : rp;
      rb = p.b_gather ? (int64_t)p.b_gather[rp] : rp;
      if (p.a_scale) sa = p.a_scale[rp];
      if (p.b_scale) sb = p.b_scale[rp];
    }
    // the row's scale goes to a split operand, so that an exact one stays exact
    const float s_a = SB ? 1.f : sa * sb, s_b = SB ? sa * sb : 1.f;
    float va[8], vb[8];
    load8_row<TA>(p.a, ra, p.lda, m0 + lc, ok ? p.M : 0, va);
    load8_row<TB>(p.b, rb, p.ldb, n0 + lc, ok ? p.N : 0, vb);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t h, l;
      split_bf16(s_a * va[i], h, l);
      ath[lc + i][lrow] = h;
      if constexpr (SA) atl[lc + i][lrow] = l;
      split_bf16(s_b * vb[i], h, l);
      bth[lc + i][lrow] = h;
      if constexpr (SB) btl[lc + i][lrow] = l;
      if (do_colsum) cst[lrow][lc + i] = sa * va[i];
    }
    __syncthreads();
    if (do_colsum && tid < kT) {
#pragma unroll
      for (int i = 0; i < kK16; ++i) cs += cst[i][tid];
    }
    const U16 a = *reinterpret_cast<const U16*>(&ath[16 * wave + lr][8 * q]);
    U16 al;
    if constexpr (SA) al = *reinterpret_cast<const U16*>(&atl[16 * wave + lr][8 * q]);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const U16 b = *reinterpret_cast<const U16*>(&bth[16 * ct + lr][8 * q]);
      acc[ct] = mfma16(a, b, acc[ct]);
      if constexpr (SA) acc[ct] = mfma16(al, b, acc[ct]);
      if constexpr (SB) {
        const U16 bl = *reinterpret_cast<const U16*>(&btl[16 * ct + lr][8 * q]);
        acc[ct] = mfma16(a, bl, acc[ct]);
      }
    }
    __syncthreads();
  }
  float* og = p.out + (int64_t)g * p.out_stride;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int n = n0 + 16 * ct + lr;
    if (n >= p.N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 16 * wave + 4 * q + i;
      if (m < p.M) og[(int64_t)m * p.N + n] = acc[ct][i];
    }
  }
  if (do_colsum && tid < kT && m0 + tid < p.M) p.colsum[(int64_t)g * p.M + m0 + tid] = cs;
}

// ---------------------------------------------------------------------------
// Elementwise parts
// ---------------------------------------------------------------------------

// d CV^2 / d v for Importance and Load, times their weights and aux_scale:
// (2 / (n m^2)) ((v_i - m) - V / m), 0 when n == 1 or m == 0. Means and
// variances in fp64 over a fixed-order tree. One workgroup.
__global__ __launch_bounds__(1024) void cv2_grad_kernel(const float* __restrict__ imp,
                                                        const float* __restrict__ load, int n,
                                                        float s_imp, float s_load, int train,
                                                        float* __restrict__ dimp,
                                                        float* __restrict__ dload) {
  __shared__ double red[2][1024];
  const int t = threadIdx.x;
  double stat[2][2];  // [vector][mean, variance]
  for (int v = 0; v < 2; ++v) {
    const float* x = v ? load : imp;
    double s = 0.0;
    for (int i = t; i < n; i += 1024) s += x[i];
    red[v][t] = s;
  }
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (t < o) {
      red[0][t] += red[0][t + o];
      red[1][t] += red[1][t + o];
    }
    __syncthreads();
  }
  stat[0][0] = red[0][0] / n;
  stat[1][0] = red[1][0] / n;
  __syncthreads();
  for (int v = 0; v < 2; ++v) {
    const float* x = v ? load : imp;
    double s = 0.0;
    for (int i = t; i < n; i += 1024) s += (x[i] - stat[v][0]) * (x[i] - stat[v][0]);
    red[v][t] = s;
  }
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if (t < o) {
      red[0][t] += red[0][t + o];
      red[1][t] += red[1][t + o];
    }
    __syncthreads();
  }
  stat[0][1] = red[0][0] / n;
  stat[1][1] = red[1][0] / n;
  for (int v = 0; v < 2; ++v) {
    const float* x = v ? load : imp;
    float* out = v ? dload : dimp;
    const double m = stat[v][0], V = stat[v][1];
    const double sc = v ? (train ? s_load : 0.0) : s_imp;
    for (int i = t; i < n; i += 1024) {
      double g = 0.0;
      if (n > 1 && m != 0.0) g = 2.0 / ((double)n * m * m) * ((x[i] - m) - V / m);
      out[i] = (float)(sc * g);
    }
  }
}

// Per token, one wave: the gradient of each kept gate, dy_t . E(x_t) of its
// expert (recomputed rows, fp32, at slot_pos) plus the Importance loss's
// d/dImportance of the expert, then the kept softmax's backward, g_j (dg_j -
// sum_l g_l dg_l), into dHk [B][k].
template <typename TY>
__global__ __launch_bounds__(256) void slot_grad_kernel(int64_t B, int k, int d,
                                                        const void* __restrict__ dy,
                                                        const float* __restrict__ eo,
                                                        const int32_t* __restrict__ slot_pos,
                                                        const int32_t* __restrict__ topk_idx,
                                                        const float* __restrict__ topk_gate,
                                                        const float* __restrict__ dimp,
                                                        float* __restrict__ dHk) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= B) return;
  float dg[8], gv[8];
  float sgd = 0.f;
  for (int j = 0; j < k; ++j) {
    const int64_t row = slot_pos[t * k + j];  // -1: a slot the route dropped (no expert)
    float s = 0.f;
    if (row >= 0)
      for (int c = lane; c < d; c += 64) s += ld_f<TY>(dy, t * d + c) * eo[row * d + c];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    dg[j] = s + dimp[topk_idx[t * k + j]];
    gv[j] = topk_gate[t * k + j];
    sgd += gv[j] * dg[j];
  }
  if (lane < k) {
    float v = 0.f;
    for (int j = 0; j < k; ++j)
      if (j == lane) v = gv[j] * (dg[j] - sgd);
    dHk[t * k + lane] = v;
  }
}

// Per (token, expert): from the recomputed clean logit c (bias included) and
// noise pre-activation u in cu [B][2n] (c at column i, u at n + i), the
// gradients that replace them: dc = [kept] dH + dLoad_i dP/dc and du =
// ([kept] dH eps + dLoad_i dP/dsigma) Softplus'(u), with dP/dc = phi(z) /
// sigma, dP/dsigma = -phi(z) z / sigma, z = (c - thr) / sigma, thr = v_{k+1}
// for a kept expert, v_k otherwise (no threshold: 0). Without noise only dc
// = [kept] dH.
__global__ __launch_bounds__(256) void pair_grad_kernel(int64_t B, int n, int k, int train,
                                                        float floor_,
                                                        const float* __restrict__ eps,
                                                        const float* __restrict__ thresh,
                                                        const int32_t* __restrict__ topk_idx,
                                                        const float* __restrict__ dHk,
                                                        const float* __restrict__ dload,
                                                        float* __restrict__ cu) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= B * n) return;
  const int64_t t = idx / n;
  const int i = (int)(idx - t * n);
  float dh = 0.f;
  bool kept = false;
  for (int j = 0; j < k; ++j)
    if (topk_idx[t * k + j] == i) {
      kept = true;
      dh = dHk[t * k + j];
    }
  float* row = cu + t * 2 * (int64_t)n;
  if (!train) {
    row[i] = dh;
    return;
  }
  const float c = row[i], u = row[n + i];
  const float sigma = fmaxf(u, 0.f) + log1pf(expf(-fabsf(u))) + floor_;
  const float thr = kept ? thresh[t * 2 + 1] : thresh[t * 2];
  float pc = 0.f, ps = 0.f;
  if (!isinf(thr)) {
    const float z = (c - thr) / sigma;
    const float ph = expf(-0.5f * z * z) * 0.3989422804014327f;
    pc = ph / sigma;
    ps = -ph * z / sigma;
  }
  const float dl = dload[i];
  const float dc = dh + dl * pc;
  const float dsig = dh * eps[t * n + i] + dl * ps;
  const float sg = u >= 0.f ? 1.f / (1.f + expf(-u)) : expf(u) / (1.f + expf(u));
  row[i] = dc;
  row[n + i] = dsig * sg;
}

// dx[t] = dxg[t] + sum over the token's slots of dxe[slot_pos[t][j]] (fp32, slot order).
__global__ __launch_bounds__(256) void dx_sum_kernel(int64_t B, int k, int d,
                                                     const float* __restrict__ dxg,
                                                     const float* __restrict__ dxe,
                                                     const int32_t* __restrict__ slot_pos,
                                                     float* __restrict__ dx) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= B * d) return;
  const int64_t t = idx / d;
  const int c = (int)(idx - t * d);
  float v = dxg[idx];
  for (int j = 0; j < k; ++j) {
    const int64_t row = slot_pos[t * k + j];
    if (row >= 0) v += dxe[row * d + c];
  }
  dx[idx] = v;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------

unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

// bf16 storage: the products on the bf16 matrix cores (fp32 operands split);
// fp32 storage: on the fp32 matrix cores.
hipError_t run_row_gemm(const RowGemm& p, Dt ta, Dt tw, Dt to, int64_t grid_x, hipStream_t s,
                        bool bf16_cores = false) {
  if (grid_x <= 0) return hipSuccess;
  const dim3 grid((unsigned)grid_x, (unsigned)((p.N + kT - 1) / kT)), block(256);
  if (bf16_cores && to == kF32) {
#define MOE_RG16(A, W, SA, SW) \
  hipLaunchKernelGGL((row_gemm16_kernel<A, W, float, SA, SW>), grid, block, 0, s, p)
    if (ta == kBF16 && tw == kBF16) MOE_RG16(bf16, bf16, false, false);
    else if (ta == kF32 && tw == kBF16) MOE_RG16(float, bf16, true, false);
    else if (ta == kBF16 && tw == kF32) MOE_RG16(bf16, float, false, true);
    else MOE_RG16(float, float, true, true);
#undef MOE_RG16
    return hipGetLastError();
  }
#define MOE_RG(A, W, O) hipLaunchKernelGGL((row_gemm_kernel<A, W, O>), grid, block, 0, s, p)
  if (ta == kBF16 && tw == kBF16 && to == kBF16) MOE_RG(bf16, bf16, bf16);
  else if (ta == kBF16 && tw == kBF16 && to == kF32) MOE_RG(bf16, bf16, float);
  else if (ta == kBF16 && tw == kF32 && to == kF32) MOE_RG(bf16, float, float);
  else if (ta == kF32 && tw == kBF16 && to == kF32) MOE_RG(float, bf16, float);
  else if (ta == kF32 && tw == kF32 && to == kF32) MOE_RG(float, float, float);
  else return hipErrorInvalidValue;
#undef MOE_RG
  return hipGetLastError();
}

hipError_t run_wgrad(const Wgrad& p, Dt ta, Dt tb, int nseg, hipStream_t s,
                     bool bf16_cores = false) {
  if (nseg <= 0) return hipSuccess;
  const dim3 grid((unsigned)(((p.M + kT - 1) / kT) * ((p.N + kT - 1) / kT)), (unsigned)nseg);
  if (bf16_cores) {
    if (ta == kBF16 && tb == kF32)
      hipLaunchKernelGGL((wgrad16_kernel<bf16, float, false, true>), grid, dim3(256), 0, s, p);
    else if (ta == kF32 && tb == kBF16)
      hipLaunchKernelGGL((wgrad16_kernel<float, bf16, true, false>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((wgrad16_kernel<float, float, true, true>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
  }
#define MOE_WG(A, B_) hipLaunchKernelGGL((wgrad_kernel<A, B_>), grid, dim3(256), 0, s, p)
  if (ta == kBF16 && tb == kBF16) MOE_WG(bf16, bf16);
  else if (ta == kF32 && tb == kBF16) MOE_WG(float, bf16);
  else if (ta == kBF16 && tb == kF32) MOE_WG(bf16, float);
  else if (ta == kF32 && tb == kF32) MOE_WG(float, float);
  else return hipErrorInvalidValue;
#undef MOE_WG
  return hipGetLastError();
}

}  // namespace

size_t backward_ws_bytes(int64_t B, int n, int k, int d, int h, Dt act_dt) {
  const int64_t P = B * k;
  const size_t a = act_dt == kBF16 ? 2 : 4;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  const int64_t max_units = gate_max_units(P, n, kT);
  return al((size_t)n * 4) + al((size_t)(n + 1) * 4) + 3 * al((size_t)P * 4)  // route
         + al((size_t)n * route_blocks(B) * 4)                                  // blockcnt
         + al((size_t)(1 + 2 * max_units) * 4) + al((size_t)(n + 1) * 4)        // units
         + 2 * al((size_t)n * 4)                                                // dimp, dload
         + al((size_t)P * h * 4)                                                // hidden (fp32)
         + al((size_t)P * d * 4)                                                // expert out
         + al((size_t)B * k * 4)                                                // dHk
         + al((size_t)P * h * 4)                                                // dA
         + al((size_t)P * d * 4)                                                // dx per pair
         + al((size_t)B * 2 * n * 4)                                            // c|u grads
         + al((size_t)B * d * 4);                                               // dx via gate
}

hipError_t launch_backward(const BackwardLaunch& b, void* ws, hipStream_t s) {
  const int64_t B = b.tokens, P = B * b.k;
  const int n = b.n, k = b.k, d = b.d, h = b.h;
  const size_t a = b.act_dt == kBF16 ? 2 : 4;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  char* w = static_cast<char*>(ws);
  auto take = [&](size_t bytes) {
    char* r = w;
    w += al(bytes);
    return r;
  };
  int32_t* counts = reinterpret_cast<int32_t*>(take((size_t)n * 4));
  int32_t* offsets = reinterpret_cast<int32_t*>(take((size_t)(n + 1) * 4));
  int32_t* perm_token = reinterpret_cast<int32_t*>(take((size_t)P * 4));
  float* perm_gate = reinterpret_cast<float*>(take((size_t)P * 4));
  int32_t* slot_pos = reinterpret_cast<int32_t*>(take((size_t)P * 4));
  int32_t* blockcnt = reinterpret_cast<int32_t*>(take((size_t)n * route_blocks(B) * 4));
  const int64_t max_units = gate_max_units(P, n, kT);
  int32_t* units = reinterpret_cast<int32_t*>(take((size_t)(1 + 2 * max_units) * 4));
  int32_t* unit_start = reinterpret_cast<int32_t*>(take((size_t)(n + 1) * 4));
  float* dimp = reinterpret_cast<float*>(take((size_t)n * 4));
  float* dload = reinterpret_cast<float*>(take((size_t)n * 4));
  float* hid = reinterpret_cast<float*>(take((size_t)P * h * 4));
  float* eo = reinterpret_cast<float*>(take((size_t)P * d * 4));
  float* dHk = reinterpret_cast<float*>(take((size_t)B * k * 4));
  float* dA = reinterpret_cast<float*>(take((size_t)P * h * 4));
  float* dxe = reinterpret_cast<float*>(take((size_t)P * d * 4));
  float* cu = reinterpret_cast<float*>(take((size_t)B * 2 * n * 4));
  float* dxg = reinterpret_cast<float*>(take((size_t)B * d * 4));
  hipError_t e;

  // routing of the forward's selection, and the 64-row units of its segments
  e = launch_route(B, k, n, b.topk_idx, b.topk_gate, blockcnt, counts, offsets, perm_token,
                   perm_gate, slot_pos, nullptr, s);
  if (e != hipSuccess) return e;
  e = launch_group_plan(offsets, n, kT, units, unit_start, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cv2_grad_kernel, dim3(1), dim3(1024), 0, s, b.importance, b.load, n,
                     b.aux_scale * b.w_importance, b.aux_scale * b.w_load, b.train, dimp, dload);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // experts: hidden = ReLU(x W1^T + b1) and out = hidden W2^T + b2, both kept in fp32 (the
  // forward pass rounds them to the storage type; the gradients here are those of the
  // layer's unrounded function)
  RowGemm r{};
  r.units = units;
  r.seg_off = offsets;
  r.rows = P;
  r.a = b.x;
  r.lda = d;
  r.gather = perm_token;
  r.w = b.w1;
  r.w_stride = (int64_t)h * d;
  r.wt = 1;
  r.K = d;
  r.N = h;
  r.bias = b.b1;
  r.relu = 1;
  r.out = hid;
  r.ldo = h;
  if ((e = run_row_gemm(r, b.act_dt, b.act_dt, kF32, max_units, s, b.act_dt == kBF16)) != hipSuccess) return e;
  r = RowGemm{};
  r.units = units;
  r.seg_off = offsets;
  r.rows = P;
  r.a = hid;
  r.lda = h;
  r.w = b.w2;
  r.w_stride = (int64_t)d * h;
  r.wt = 1;
  r.K = h;
  r.N = d;
  r.bias = b.b2;
  r.out = eo;
  r.ldo = d;
  if ((e = run_row_gemm(r, kF32, b.act_dt, kF32, max_units, s, b.act_dt == kBF16)) != hipSuccess) return e;
  // kept gates: task + Importance gradients through the kept softmax
  if (B > 0) {
    if (b.act_dt == kBF16)
      hipLaunchKernelGGL(slot_grad_kernel<bf16>, dim3((unsigned)((B + 3) / 4)), dim3(256), 0, s,
                         B, k, d, b.dy, eo, slot_pos, b.topk_idx, b.topk_gate, dimp, dHk);
    else
      hipLaunchKernelGGL(slot_grad_kernel<float>, dim3((unsigned)((B + 3) / 4)), dim3(256), 0, s,
                         B, k, d, b.dy, eo, slot_pos, b.topk_idx, b.topk_gate, dimp, dHk);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // dA = (gate * dy[token]) W2 masked by hidden > 0
  r = RowGemm{};
  r.units = units;
  r.seg_off = offsets;
  r.rows = P;
  r.a = b.dy;
  r.lda = d;
  r.gather = perm_token;
  r.scale = perm_gate;
  r.w = b.w2;
  r.w_stride = (int64_t)d * h;
  r.wt = 0;
  r.K = d;
  r.N = h;
  r.out = dA;
  r.ldo = h;
  r.mask = hid;
  r.ldm = h;
  if ((e = run_row_gemm(r, b.act_dt, b.act_dt, kF32, max_units, s, b.act_dt == kBF16)) != hipSuccess) return e;
  // dW2_e = sum (gate dy[token])^T hidden, db2_e = sum gate dy[token]
  Wgrad wg{};
  wg.seg_off = offsets;
  wg.rows = P;
  wg.a = b.dy;
  wg.lda = d;
  wg.a_gather = perm_token;
  wg.a_scale = perm_gate;
  wg.b = hid;
  wg.ldb = h;
  wg.M = d;
  wg.N = h;
  wg.out = b.dw2;
  wg.out_stride = (int64_t)d * h;
  wg.colsum = b.db2;
  if ((e = run_wgrad(wg, b.act_dt, kF32, n, s, b.act_dt == kBF16)) != hipSuccess) return e;
  // dW1_e = sum dA^T x[token], db1_e = sum dA
  wg = Wgrad{};
  wg.seg_off = offsets;
  wg.rows = P;
  wg.a = dA;
  wg.lda = h;
  wg.b = b.x;
  wg.ldb = d;
  wg.b_gather = perm_token;
  wg.M = h;
  wg.N = d;
  wg.out = b.dw1;
  wg.out_stride = (int64_t)h * d;
  wg.colsum = b.db1;
  if ((e = run_wgrad(wg, kF32, b.act_dt, n, s, b.act_dt == kBF16)) != hipSuccess) return e;
  // dx per routed row: dA W1
  r = RowGemm{};
  r.units = units;
  r.seg_off = offsets;
  r.rows = P;
  r.a = dA;
  r.lda = h;
  r.w = b.w1;
  r.w_stride = (int64_t)h * d;
  r.wt = 0;
  r.K = h;
  r.N = d;
  r.out = dxe;
  r.ldo = d;
  if ((e = run_row_gemm(r, kF32, b.act_dt, kF32, max_units, s, b.act_dt == kBF16)) != hipSuccess) return e;

  // gate: c = x W_g^T + b, u = x W_noise^T into cu, then their gradients in place
  const int64_t rt = (B + kT - 1) / kT;
  r = RowGemm{};
  r.rows = B;
  r.a = b.x;
  r.lda = d;
  r.w = b.w_gate;
  r.wt = 1;
  r.K = d;
  r.N = n;
  r.bias = b.gate_bias;  // fp32 whatever the weights' type
  r.bias_f32 = 1;
  r.out = cu;
  r.ldo = 2 * (int64_t)n;
  if ((e = run_row_gemm(r, b.act_dt, b.gate_dt, kF32, rt, s, b.act_dt == kBF16)) != hipSuccess) return e;
  if (b.train) {
    r.w = b.w_noise;
    r.bias = nullptr;
    r.out = cu + n;
    if ((e = run_row_gemm(r, b.act_dt, b.gate_dt, kF32, rt, s, b.act_dt == kBF16)) != hipSuccess) return e;
  }
  if (B > 0) {
    hipLaunchKernelGGL(pair_grad_kernel, dim3(blocks_for(B * n)), dim3(256), 0, s, B, n, k,
                       b.train, b.noise_floor, b.eps, b.thresh, b.topk_idx, dHk, dload, cu);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // dW_g = dc^T x, db_g = sum dc; dW_noise = du^T x
  wg = Wgrad{};
  wg.rows = B;
  wg.a = cu;
  wg.lda = 2 * (int64_t)n;
  wg.b = b.x;
  wg.ldb = d;
  wg.M = n;
  wg.N = d;
  wg.out = b.dw_gate;
  wg.colsum = b.dgate_bias;
  if ((e = run_wgrad(wg, kF32, b.act_dt, 1, s, b.act_dt == kBF16)) != hipSuccess) return e;
  if (b.train) {
    wg.a = cu + n;
    wg.out = b.dw_noise;
    wg.colsum = nullptr;
    if ((e = run_wgrad(wg, kF32, b.act_dt, 1, s, b.act_dt == kBF16)) != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks_for((int64_t)n * d)), dim3(256), 0, s,
                       b.dw_noise, (int64_t)n * d);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // dx through the gate: dc W_g + du W_noise
  r = RowGemm{};
  r.rows = B;
  r.a = cu;
  r.lda = 2 * (int64_t)n;
  r.w = b.w_gate;
  r.wt = 0;
  r.K = n;
  r.N = d;
  r.out = dxg;
  r.ldo = d;
  if ((e = run_row_gemm(r, kF32, b.gate_dt, kF32, rt, s, b.act_dt == kBF16)) != hipSuccess) return e;
  if (b.train) {
    r.a = cu + n;
    r.w = b.w_noise;
    r.accumulate = 1;
    if ((e = run_row_gemm(r, kF32, b.gate_dt, kF32, rt, s, b.act_dt == kBF16)) != hipSuccess) return e;
  }
  if (B > 0) {
    hipLaunchKernelGGL(dx_sum_kernel, dim3(blocks_for(B * d)), dim3(256), 0, s, B, k, d, dxg, dxe,
                       slot_pos, b.dx);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
