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
// The matrix products come in two grouped forms over the contiguous
// per-expert segments that routing produces:
//   * row products: out[p] = f(a[p] . W_e) for the rows p of expert e's
//     segment (a's rows optionally gathered through the token list, the
//     row's gate applied in the epilogue), in 64-row units of a segment;
//   * weight-gradient products: dW_e = sum over e's rows of a[p]^T b[p], with
//     the column sums of a (the bias gradients) on the side; long segments
//     run in row chunks whose partial sums are added in chunk order.
// For fp32 storage they run on the fp32 matrix cores (v_mfma_f32_16x16x4f32,
// 64 x 64 tiles); for bf16 storage on the bf16 matrix cores (the tiled
// kernels below). The expert outputs are never recomputed: the kept gates'
// gradient needs only dy . E = (dy W2) . hidden + dy . b2, whose first term
// the dA product forms in its epilogue.
// Every sum runs in a fixed order, so the results are deterministic.
#include <algorithm>
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
  // a_blk > 0 (tiled bf16-core products only): a is in blocks of 16 K
  // columns, a_blk rows each, 32 floats a row: element (p, k) at
  // a + ((k / 16) * a_blk + row(p)) * 32 + k % 16 (lda unused)
  int64_t a_blk;
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
  // optional (with mask): rowdot[p * rd_n + blockIdx.y] = sum over the tile's
  // columns c of acc[p][c] * mask[p][c], the product before scale, bias and mask
  float* rowdot;
  int rd_n;
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
  if (arow_ok) arow = p.gather ? (int64_t)p.gather[arow_p] : arow_p;
  for (int k0 = 0; k0 < p.K; k0 += kKS) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = k0 + ak + i;
      as[ar][ak + i] = (arow_ok && kk < p.K) ? ld_f<TA>(p.a, arow * p.lda + kk) : 0.f;
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
  // C layout: lane holds rows 4q + i of its wave's 16, column lr of each tile.
  // A tile's mask and accumulate values are loaded together (rows past the
  // unit read its first row, columns past N column 0; neither is stored).
  float rs[4] = {0.f, 0.f, 0.f, 0.f}, sc[4];
  int64_t rr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t rp = r0 + 16 * wave + 4 * q + i;
    rr[i] = rp < rend ? rp : r0;
    sc[i] = p.scale ? p.scale[rr[i]] : 1.f;
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int c = c0 + 16 * ct + lr;
    const bool cok = c < p.N;
    const int cc = cok ? c : 0;
    float b = 0.f;
    if (p.bias)
      b = p.bias_f32 ? ld_f<float>(p.bias, (int64_t)g * p.N + cc) : ld_f<TW>(p.bias, (int64_t)g * p.N + cc);
    float mv[4], pv[4];
    if (p.mask) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        mv[i] = p.mask_bf16 ? ld_f<bf16>(p.mask, rr[i] * p.ldm + cc) : ld_f<float>(p.mask, rr[i] * p.ldm + cc);
    }
    if (p.accumulate) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = ld_f<TO>(p.out, rr[i] * p.ldo + cc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = acc[ct][i] * sc[i] + b;
      if (p.relu) v = v > 0.f ? v : 0.f;
      if (p.mask) {
        v = mv[i] > 0.f ? v : 0.f;
        if (cok) rs[i] += acc[ct][i] * mv[i];
      }
      if (p.accumulate) v += pv[i];
      const int64_t rp = r0 + 16 * wave + 4 * q + i;
      if (cok && rp < rend) st_f<TO>(p.out, rp * p.ldo + c, v);
    }
  }
  if (p.rowdot) {  // over the 16 columns of each tile (lanes lr), then the 4 tiles were summed
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) rs[i] += __shfl_xor(rs[i], o);
    if (lr == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t rp = r0 + 16 * wave + 4 * q + i;
        if (rp < rend) p.rowdot[rp * p.rd_n + blockIdx.y] = rs[i];
      }
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
  // a: [rows][M], b: [rows][N], each row optionally gathered and scaled;
  // a_blk > 0 (tiled kernel only): a is in blocks of 32 M columns, a_blk rows
  // each: element (row, m) at a + ((m / 32) * a_blk + row) * 32 + m % 32
  const void* a;
  int64_t lda;
  int64_t a_blk;
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
  // optional: colsum[g * M + m] = sum over g's rows of a[p][m], in a fixed order
  float* colsum;
  // optional row chunks (wg_chunk_plan_kernel): blockIdx.y is chunk c = (g,
  // first row, end row, slot) of chunks[1 + 4c ..], chunks[0] the count; a
  // chunk with slot >= 0 writes its partial sums to part + slot * M * N (and
  // its column sums to pcol + slot * M) instead of out_g and colsum
  const int32_t* chunks;
  float* part;
  float* pcol;
};

// The rows, output and column-sum destination of a weight-gradient workgroup.
struct WgSeg {
  bool valid;
  int g;
  int64_t s0, s1;
  float* out;
  float* colsum;
};
__device__ __forceinline__ WgSeg wg_segment(const Wgrad& p, int gy) {
  WgSeg r;
  if (p.chunks) {
    const int c = gy;
    r.valid = c < p.chunks[0];
    if (!r.valid) return r;
    const int32_t* e = p.chunks + 1 + 4 * c;
    r.g = e[0];
    r.s0 = e[1];
    r.s1 = e[2];
    const int slot = e[3];
    r.out = slot < 0 ? p.out + (int64_t)r.g * p.out_stride : p.part + (int64_t)slot * p.M * p.N;
    r.colsum = !p.colsum ? nullptr
               : slot < 0 ? p.colsum + (int64_t)r.g * p.M
                          : p.pcol + (int64_t)slot * p.M;
    return r;
  }
  r.valid = true;
  r.g = gy;
  r.s0 = p.seg_off ? p.seg_off[r.g] : 0;
  r.s1 = p.seg_off ? p.seg_off[r.g + 1] : p.rows;
  r.out = p.out + (int64_t)r.g * p.out_stride;
  r.colsum = p.colsum ? p.colsum + (int64_t)r.g * p.M : nullptr;
  return r;
}

template <typename TA, typename TB>
__global__ __launch_bounds__(256) void wgrad_kernel(Wgrad p) {
  __shared__ float at[kKS][kT + 1];
  __shared__ float bt[kKS][kT + 1];
  const int mtiles = (p.M + kT - 1) / kT;
  const int m0 = (blockIdx.x % mtiles) * kT, n0 = (blockIdx.x / mtiles) * kT;
  const WgSeg sg = wg_segment(p, blockIdx.y);
  if (!sg.valid) return;
  const int64_t s0 = sg.s0, s1 = sg.s1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, q = lane >> 4;
  const bool do_colsum = sg.colsum != nullptr && n0 == 0;
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
  float* og = sg.out;
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
  if (do_colsum && tid < kT && m0 + tid < p.M) sg.colsum[m0 + tid] = cs;
}

// ---------------------------------------------------------------------------
// The same products on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16), for
// bf16 storage. Operands in bf16 storage are exact; an fp32 operand (the
// recomputed hidden layer, the hidden and logit gradients, fp32 gate weights)
// is split into hi = bf16(v) and lo = bf16(v - hi), exact to about 2^-17 of v,
// and its products take the hi and lo parts against the other operand (hi x
// lo' cross terms of two split operands are kept, lo x lo' dropped). Row
// scales (the gates) are applied where they keep an exact operand exact: in
// the row products' epilogue, in the weight-gradient products to the split
// operand.
//
// Row products: four waves (2 x 2), 64 rows x 256 columns (a 64-row unit of a
// segment); weight gradients: 128 x 128 tiles (four waves) or 256 x 256 (eight
// waves, where segments are short). K runs in steps of 32 through two LDS
// buffers; the next step's operands are loaded into registers (16-byte loads,
// fp32 split on the way) while the current step is multiplied. Every operand
// tile is K-major in LDS, [R][32] bf16, 64 bytes a row, 16-byte unit u of row
// r at position u ^ (((r >> 1) ^ (r >> 3)) & 3), so that the 16-byte operand
// reads of 8 (or 16) consecutive rows hit distinct banks; a fragment is one
// such read. A K-contiguous source (x, dy, hidden, dA and logit-gradient rows,
// the rows of an [N][K] weight) is stored as loaded; a source whose rows are
// K-indexed (a [K][N] weight, the routed rows of a weight gradient) is
// transposed in registers on its way in, 4 K rows x 8 columns per thread.
// ---------------------------------------------------------------------------

constexpr int kBK = 32;  // K per step of the tiled bf16 products
// rows per workgroup (and per unit) of the tiled row products: 64, two
// workgroups per compute unit (128-row workgroups, one per compute unit, read
// each weight tile half as often but hide less latency: slower)
constexpr int kTR = 64;

__device__ __forceinline__ uint32_t split_pair(float a, float b, uint32_t& lo) {
  const uint32_t ha = f32_to_bf16_bits(a), hb = f32_to_bf16_bits(b);
  const uint32_t la = f32_to_bf16_bits(a - bf16_bits_to_f32(ha));
  const uint32_t lb = f32_to_bf16_bits(b - bf16_bits_to_f32(hb));
  lo = la | (lb << 16);
  return ha | (hb << 16);
}

// 8 consecutive elements from p: `valid` of them (0..8) are read, the rest are
// 0; vec: the 8 are in range and 16-byte aligned (one or two vector loads).
__device__ __forceinline__ void load8(const bf16* p, int valid, bool vec, uint32_t (&w)[4]) {
  if (vec && valid == 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
    return;
  }
  const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t a = 2 * j < valid ? q[2 * j] : 0u, b = 2 * j + 1 < valid ? q[2 * j + 1] : 0u;
    w[j] = a | (b << 16);
  }
}
__device__ __forceinline__ void load8(const float* p, int valid, bool vec, float (&f)[8]) {
  if (vec && valid == 8) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    f[0] = a.x;
    f[1] = a.y;
    f[2] = a.z;
    f[3] = a.w;
    f[4] = b.x;
    f[5] = b.y;
    f[6] = b.z;
    f[7] = b.w;
    return;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = j < valid ? p[j] : 0.f;
}


// One operand unit in registers between its load and its LDS store: raw bf16
// bits, or fp32 values (split, times a scale, at the store).
template <typename T>
struct Stage8;
template <>
struct Stage8<bf16> {
  uint32_t w[4];
  __device__ __forceinline__ void load(const void* base, int64_t off, int valid, bool vec) {
    load8(reinterpret_cast<const bf16*>(base) + off, valid, vec, w);
  }
  // hi (and no lo: bf16 operands are exact; a scale never lands here)
  __device__ __forceinline__ void store(uint8_t* hi, uint8_t* lo, float scale) const {
    (void)lo;
    (void)scale;
    *reinterpret_cast<uint4*>(hi) = uint4{w[0], w[1], w[2], w[3]};
  }
};
template <>
struct Stage8<float> {
  float f[8];
  __device__ __forceinline__ void load(const void* base, int64_t off, int valid, bool vec) {
    load8(reinterpret_cast<const float*>(base) + off, valid, vec, f);
  }
  __device__ __forceinline__ void store(uint8_t* hi, uint8_t* lo, float scale) const {
    uint4 h, l;
    h.x = split_pair(scale * f[0], scale * f[1], l.x);
    h.y = split_pair(scale * f[2], scale * f[3], l.y);
    h.z = split_pair(scale * f[4], scale * f[5], l.z);
    h.w = split_pair(scale * f[6], scale * f[7], l.w);
    *reinterpret_cast<uint4*>(hi) = h;
    *reinterpret_cast<uint4*>(lo) = l;
  }
};

// LDS placement of a K-major tile ([R][32] bf16) and of a tile with K-indexed
// rows ([32][R] bf16): byte offset of 16-byte unit u of row r (resp. k).
__device__ __forceinline__ int kmaj_pos(int r, int u) {
  return r * 64 + ((u ^ (((r >> 1) ^ (r >> 3)) & 3)) << 4);
}
// The A (or B) operand of one 32x32x16 product at k16 step s: lane l supplies
// row (column) r0 + l % 32 and K 16 s + 8 (l / 32) .. + 7.
__device__ __forceinline__ U16 frag_kmaj(const uint8_t* t, int r0, int s, int lane) {
  return *reinterpret_cast<const U16*>(t + kmaj_pos(r0 + (lane & 31), 2 * s + (lane >> 5)));
}
// Four K rows x 8 consecutive columns of a [K][N] operand, held between their
// loads and their transposed LDS store: each column's 4 K values become 8
// bytes of a K-major tile row (fp32 split into hi and lo on the way).
template <typename T>
struct StageT;
template <>
struct StageT<bf16> {
  uint32_t w[4][4];
  __device__ __forceinline__ void load(const void* base, int64_t off, int64_t ld, int krows,
                                       int valid, bool vec) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      load8(reinterpret_cast<const bf16*>(base) + off + j * ld, j < krows ? valid : 0, vec, w[j]);
  }
  // column e (0..7) of the block: 4 bf16 K values
  __device__ __forceinline__ void store(uint8_t* hi, uint8_t* lo, int e, int pos) const {
    (void)lo;
    const int sh = 16 * (e & 1), q = e >> 1;
    const uint32_t v0 = (w[0][q] >> sh) & 0xFFFFu, v1 = (w[1][q] >> sh) & 0xFFFFu;
    const uint32_t v2 = (w[2][q] >> sh) & 0xFFFFu, v3 = (w[3][q] >> sh) & 0xFFFFu;
    *reinterpret_cast<uint2*>(hi + pos) = uint2{v0 | (v1 << 16), v2 | (v3 << 16)};
  }
};
template <>
struct StageT<float> {
  float f[4][8];
  __device__ __forceinline__ void load(const void* base, int64_t off, int64_t ld, int krows,
                                       int valid, bool vec) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      load8(reinterpret_cast<const float*>(base) + off + j * ld, j < krows ? valid : 0, vec, f[j]);
  }
  __device__ __forceinline__ void store(uint8_t* hi, uint8_t* lo, int e, int pos) const {
    uint32_t l0, l1;
    const uint32_t h0 = split_pair(f[0][e], f[1][e], l0), h1 = split_pair(f[2][e], f[3][e], l1);
    *reinterpret_cast<uint2*>(hi + pos) = uint2{h0, h1};
    *reinterpret_cast<uint2*>(lo + pos) = uint2{l0, l1};
  }
};

// Row products on bf16 cores: TM = 32 MR rows x 256 columns a workgroup, 2 MR
// waves in an MR x 2 grid (32 rows x 128 columns each). The first 256 threads
// stage the weights, all threads the rows.
//
// Work item w = (unit or row block) * ncb + column block, nwork items. The
// workgroups of one XCD (workgroup b runs on XCD b % 8) take runs of 2 ncb
// consecutive items, the XCDs taking turns, so that two consecutive units
// (an expert's rows, its weights) and all their column blocks (the same rows)
// meet in one L2.
template <typename TA, typename TW, bool WT, int MR>
__global__ __launch_bounds__(128 * MR) __attribute__((amdgpu_waves_per_eu(2)))
void row_tgemm_kernel(RowGemm p, int vec, int64_t nwork, int ncb) {
  constexpr bool SA = sizeof(TA) == 4, SW = sizeof(TW) == 4;
  constexpr int TM = 32 * MR, TN = 256;
  constexpr int ABYTES = TM * 64, BBYTES = TN * 64;  // one bf16 tile of each operand
  __shared__ __attribute__((aligned(16))) uint8_t ah[2][ABYTES];
  __shared__ __attribute__((aligned(16))) uint8_t al[SA ? 2 : 1][SA ? ABYTES : 16];
  __shared__ __attribute__((aligned(16))) uint8_t bh[2][BBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t bl[SW ? 2 : 1][SW ? BBYTES : 16];
  const int64_t run = 2 * (int64_t)ncb, slot = blockIdx.x / 8;
  const int64_t w = ((slot / run) * 8 + blockIdx.x % 8) * run + slot % run;
  if (w >= nwork) return;
  const int cb = (int)(w % ncb);
  const int64_t ub = w / ncb;
  int g = 0;
  int64_t r0, rend;
  if (p.units) {
    if (ub >= p.units[0]) return;
    const int u = (int)ub;
    g = p.units[1 + 2 * u];
    r0 = (int64_t)p.seg_off[g] + p.units[2 + 2 * u];
    rend = p.seg_off[g + 1];
  } else {
    r0 = ub * TM;
    rend = p.rows;
    if (r0 >= rend) return;
  }
  const int n0 = cb * TN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const bool wstage = wave < 4;  // whole waves: the first 256 threads stage the weights
  const bool vv = vec != 0;
  const char* wseg = reinterpret_cast<const char*>(p.w) + (int64_t)g * p.w_stride * sizeof(TW);
  // A: row tid / 4 of the unit, K unit tid % 4
  const int ar = tid >> 2, au = tid & 3;
  const bool arow_ok = r0 + ar < rend;
  const int64_t arow = arow_ok ? (p.gather ? (int64_t)p.gather[r0 + ar] : r0 + ar) : 0;
  Stage8<TA> sa;
  Stage8<TW> sb[4];  // [N][K] weights: 4 units of K-contiguous rows
  StageT<TW> st;     // [K][N] weights: K rows k0 + 4 (tid / 32) .. + 3, columns 8 (tid % 32) .. + 7
  auto load = [&](int k0) __attribute__((always_inline)) {
    const int ka = k0 + 8 * au;
    const int64_t aoff = p.a_blk > 0 ? ((int64_t)(ka >> 4) * p.a_blk + arow) * 32 + (ka & 15)
                                     : arow * p.lda + ka;
    sa.load(p.a, aoff, arow_ok ? std::min(8, std::max(0, p.K - ka)) : 0, vv);
    if (wstage) {
      if constexpr (WT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // row n0 + tid / 4 + 64 i, K unit tid % 4
          const int n = n0 + (tid >> 2) + 64 * i, kb = k0 + 8 * (tid & 3);
          sb[i].load(wseg, (int64_t)n * p.K + kb, n < p.N ? std::min(8, std::max(0, p.K - kb)) : 0, vv);
        }
      } else {
        const int kr = k0 + 4 * (tid >> 5), nb = n0 + 8 * (tid & 31);
        st.load(wseg, (int64_t)kr * p.N + nb, p.N, std::max(0, std::min(4, p.K - kr)),
                std::min(8, std::max(0, p.N - nb)), vv);
      }
    }
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
    const int pa = kmaj_pos(ar, au);
    sa.store(ah[buf] + pa, al[SA ? buf : 0] + (SA ? pa : 0), 1.f);
    if (wstage) {
      if constexpr (WT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pb = kmaj_pos((tid >> 2) + 64 * i, tid & 3);
          sb[i].store(bh[buf] + pb, bl[SW ? buf : 0] + (SW ? pb : 0), 1.f);
        }
      } else {
        const int kq = tid >> 5, nu = tid & 31;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int pb = kmaj_pos(8 * nu + e, kq >> 1) + 8 * (kq & 1);
          st.store(bh[buf], bl[SW ? buf : 0], e, pb);
        }
      }
    }
  };
  f32x16 acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[nb][j] = 0.f;
  const int nk = (p.K + kBK - 1) / kBK;
  load(0);
  store(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) load((ks + 1) * kBK);
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const U16 a = frag_kmaj(ah[buf], wm * 32, s, lane);
      U16 a2;
      if constexpr (SA) a2 = frag_kmaj(al[buf], wm * 32, s, lane);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int c0 = wn * 128 + nb * 32;
        const U16 b = frag_kmaj(bh[buf], c0, s, lane);
        Mfma<bf16>::k32(acc[nb], a, b);
        if constexpr (SA) Mfma<bf16>::k32(acc[nb], a2, b);
        if constexpr (SW) {
          const U16 b2 = frag_kmaj(bl[buf], c0, s, lane);
          Mfma<bf16>::k32(acc[nb], a, b2);
        }
      }
    }
    if (ks + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }
  // C layout: lane holds column l % 32 of each 32-column block, rows
  // 8 (j / 4) + 4 (l / 32) + j % 4 of its wave's 32. Each block's mask and
  // accumulate values are loaded together (rows past the unit read its first
  // row, columns past N column 0; neither is stored), so their latencies overlap.
  float rs[16], sc[16];
  int32_t rr[16];  // routed rows are int32 indices
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    rs[j] = 0.f;
    const int64_t rp = r0 + wm * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
    rr[j] = (int32_t)(rp < rend ? rp : r0);
    sc[j] = p.scale ? p.scale[rr[j]] : 1.f;
  }
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int c = n0 + wn * 128 + nb * 32 + (lane & 31);
    const bool cok = c < p.N;
    const int cc = cok ? c : 0;
    float b = 0.f;
    if (p.bias)
      b = p.bias_f32 ? ld_f<float>(p.bias, (int64_t)g * p.N + cc) : ld_f<TW>(p.bias, (int64_t)g * p.N + cc);
    float mv[16], pv[16];
    if (p.mask) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        mv[j] = p.mask_bf16 ? ld_f<bf16>(p.mask, (int64_t)rr[j] * p.ldm + cc)
                            : ld_f<float>(p.mask, (int64_t)rr[j] * p.ldm + cc);
    }
    if (p.accumulate) {
#pragma unroll
      for (int j = 0; j < 16; ++j) pv[j] = ld_f<float>(p.out, (int64_t)rr[j] * p.ldo + cc);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float v = acc[nb][j] * sc[j] + b;
      if (p.relu) v = v > 0.f ? v : 0.f;
      if (p.mask) {
        v = mv[j] > 0.f ? v : 0.f;
        if (cok) rs[j] += acc[nb][j] * mv[j];
      }
      if (p.accumulate) v += pv[j];
      const int64_t rp = r0 + wm * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
      if (cok && rp < rend) st_f<float>(p.out, rp * p.ldo + c, v);
    }
    // one block's loads at a time: keeps the next block's loads (and their
    // registers) below this block's stores
    asm volatile("" ::: "memory");
  }
  if (p.rowdot) {  // over the wave's 128 columns (lanes l % 32), then the two column waves
    __shared__ float rdsum[2][TM];
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) rs[j] += __shfl_xor(rs[j], o);
    if ((lane & 31) == 0) {
#pragma unroll
      for (int j = 0; j < 16; ++j) rdsum[wn][wm * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3)] = rs[j];
    }
    __syncthreads();
    if (tid < TM && r0 + tid < rend) p.rowdot[(r0 + tid) * p.rd_n + cb] = rdsum[0][tid] + rdsum[1][tid];
  }
}

// Weight gradients: TM x TM output tiles, NW waves in a 2 x (NW / 2) grid;
// the first half of the threads loads A, the second half B, each thread 4
// rows x 8 columns per step, transposed into K-major tiles.
//
// PERSIST false: one tile per workgroup, tile blockIdx.x of segment blockIdx.y.
// PERSIST true: the grid (a multiple of 8) walks the nseg segments' tiles in
// order, tile T = v + i * gridDim.x, where v numbers the workgroups so that
// consecutive v run on one XCD (workgroup b runs on XCD b % 8) and a segment's
// tiles share that die's L2. A workgroup loads its next tile's first K step
// before it writes the current tile out, so that the loads' latency hides
// behind the stores.
// Stand-ins read for a missing row scale or gather index.
__device__ const float kOneF = 1.f;
__device__ const int32_t kZeroI = 0;

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* v) {
  return reinterpret_cast<P*>(uniform64((int64_t)reinterpret_cast<uintptr_t>(v)));
}

template <typename TA, typename TB, int TM, int NW, bool PERSIST>
__global__ __launch_bounds__(NW * 64) void wgrad_tgemm_kernel(Wgrad p, int vec, int nseg) {
  constexpr bool SA = sizeof(TA) == 4, SB = sizeof(TB) == 4;
  static_assert(SA || SB, "a row scale needs a split operand");
  static_assert(TM * 2 == NW * 64, "one 4 x 8 block of A or B per thread");
  constexpr int TN = TM, BYTES = TM * 64;
  constexpr int WM = TM / 2, WN = TN / (NW / 2), MB = WM / 32, NB = WN / 32;
  __shared__ __attribute__((aligned(16))) uint8_t ah[2][BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t al[SA ? 2 : 1][SA ? BYTES : 16];
  __shared__ __attribute__((aligned(16))) uint8_t bh[2][BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t bl[SB ? 2 : 1][SB ? BYTES : 16];
  __shared__ float csr[8][TM];  // the colsum's per-thread partials
  const int mtiles = (p.M + TM - 1) / TM;
  const int tps = mtiles * ((p.N + TN - 1) / TN);  // tiles per segment
  const int64_t tend = PERSIST ? (int64_t)tps * nseg : 0;
  int64_t T = PERSIST ? (int64_t)(blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8
                      : (int64_t)blockIdx.y * tps + blockIdx.x;
  if (PERSIST && T >= tend) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int wm = wave / (NW / 2), wn = wave % (NW / 2);
  const bool vv = vec != 0;
  // this thread's block: operand B for the second half of the threads (whole waves)
  const bool isb = wave >= NW / 2;
  const int bt = isb ? tid - TM : tid;
  const int kq = bt / (TM / 8), mu = bt % (TM / 8);  // rows 4 kq .. + 3, columns 8 mu .. + 7
  const int clim = isb ? p.N : p.M;
  // the current tile (uniform over the workgroup): output corner, rows, destinations
  int m0 = 0, n0 = 0;
  int64_t s0 = 0, s1 = 0;
  float* out = nullptr;
  float* colsum = nullptr;
  auto tile_at = [&](int64_t t) __attribute__((always_inline)) {
    const int g = (int)(t / tps), tt = (int)(t - (int64_t)g * tps);
    m0 = (tt % mtiles) * TM;
    n0 = (tt / mtiles) * TN;
    const WgSeg sg = wg_segment(p, g);
    if (!sg.valid) return false;
    s0 = uniform64(sg.s0);
    s1 = uniform64(sg.s1);
    out = uniform_ptr(sg.out);
    colsum = n0 == 0 ? uniform_ptr(sg.colsum) : nullptr;
    return true;
  };
  if (!tile_at(T)) return;
  // a thread stages either an A block or a B block
  union Staged {
    StageT<TA> a;
    StageT<TB> b;
  } stg;
  StageT<TA>& sa = stg.a;
  StageT<TB>& sb = stg.b;
  float cs[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) cs[i] = 0.f;
  // Per staged row: the A and B row scales and whether it holds data (bit j
  // of `on`). They are applied when the step is stored to LDS, after the
  // products that hide the loads' latency: a step's index and scale loads
  // issue together, then its data loads, and nothing waits on them before
  // the store. A wave stages A or B only, so every branch here is uniform.
  float rfa[4], rfb[4];
  int on = 0;
  auto load_rows = [&](const auto* src, int64_t ld, int64_t blk, const int32_t* gat, int64_t r,
                       auto& st) __attribute__((always_inline)) {
    const int64_t rb = r + 4 * kq;
    const int krows = (int)std::max<int64_t>(0, std::min<int64_t>(4, s1 - rb));
    const int c0 = (isb ? n0 : m0) + 8 * mu;
    const int nvalid = std::min(8, std::max(0, clim - c0));
    // rows past the segment's end read its first row (s0 < s1 whenever a
    // step is loaded) and stage zeros; a missing scale or gather reads a
    // constant, so that every load here is unconditional and unused until
    // the data loads (or the store)
    int32_t ri[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t rp = j < krows ? rb + j : s0;
      rfa[j] = *(p.a_scale ? p.a_scale + rp : &kOneF);
      rfb[j] = *(p.b_scale ? p.b_scale + rp : &kOneF);
      ri[j] = *(gat ? gat + rp : &kZeroI);
    }
    int64_t row[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) row[j] = gat ? (int64_t)ri[j] : (j < krows ? rb + j : s0);
    on = 0;
    if (vv) {
      // nvalid is 0 or 8; a row without data reads element 0 of its operand
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = j < krows && nvalid == 8;
        on |= ok ? (1 << j) : 0;
        const int64_t off = !ok ? 0 : blk > 0 ? ((int64_t)(c0 >> 5) * blk + row[j]) * 32 + (c0 & 31)
                                             : row[j] * ld + c0;
        if constexpr (sizeof(*src) == 4) {
          const float4* q = reinterpret_cast<const float4*>(src + off);
          const float4 x0 = q[0], x1 = q[1];
          st.f[j][0] = x0.x; st.f[j][1] = x0.y; st.f[j][2] = x0.z; st.f[j][3] = x0.w;
          st.f[j][4] = x1.x; st.f[j][5] = x1.y; st.f[j][6] = x1.z; st.f[j][7] = x1.w;
        } else {
          const uint4 v = *reinterpret_cast<const uint4*>(src + off);
          st.w[j][0] = v.x; st.w[j][1] = v.y; st.w[j][2] = v.z; st.w[j][3] = v.w;
        }
      }
    } else {
      on = 0xF;  // load8 zero-fills what it does not read
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int valid = j < krows ? nvalid : 0;
        const int64_t off = blk > 0 ? ((int64_t)(c0 >> 5) * blk + row[j]) * 32 + (c0 & 31)
                                    : row[j] * ld + c0;
        if constexpr (sizeof(*src) == 4) load8(src + off, valid, false, st.f[j]);
        else load8(src + off, valid, false, st.w[j]);
      }
    }
  };
  auto load = [&](int64_t r) __attribute__((always_inline)) {
    if (!isb) load_rows(reinterpret_cast<const TA*>(p.a), p.lda, p.a_blk, p.a_gather, r, sa);
    else load_rows(reinterpret_cast<const TB*>(p.b), p.ldb, (int64_t)0, p.b_gather, r, sb);
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
    // rows without data become zeros (a select: whatever they read stays out)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = (on >> j) & 1;
      if (!isb) {
        if constexpr (SA) {
#pragma unroll
          for (int e = 0; e < 8; ++e) sa.f[j][e] = ok ? sa.f[j][e] : 0.f;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) sa.w[j][e] = ok ? sa.w[j][e] : 0u;
        }
      } else {
        if constexpr (SB) {
#pragma unroll
          for (int e = 0; e < 8; ++e) sb.f[j][e] = ok ? sb.f[j][e] : 0.f;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) sb.w[j][e] = ok ? sb.w[j][e] : 0u;
        }
      }
    }
    // the column sums take A's rows times their scale; the row's two scales
    // go to the split operand, so that an exact one stays exact
    if (!isb) {
      if (colsum != nullptr) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if constexpr (SA) cs[e] += rfa[j] * sa.f[j][e];
            else cs[e] += rfa[j] * bf16_bits_to_f32((sa.w[j][e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
          }
      }
      if constexpr (!SB) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) sa.f[j][e] *= rfa[j] * rfb[j];
      }
    } else {
      if constexpr (SB) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) sb.f[j][e] *= rfa[j] * rfb[j];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int pos = kmaj_pos(8 * mu + e, kq >> 1) + 8 * (kq & 1);
      if (!isb) sa.store(ah[buf], al[SA ? buf : 0], e, pos);
      else sb.store(bh[buf], bl[SB ? buf : 0], e, pos);
    }
  };
  int64_t nk = (s1 - s0 + kBK - 1) / kBK;
  if (nk > 0) load(s0);
  for (;;) {
    if (nk > 0) store(0);
    __syncthreads();
    f32x16 acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[mb][nb][j] = 0.f;
    for (int64_t ks = 0; ks < nk; ++ks) {
      const int buf = (int)(ks & 1);
      if (ks + 1 < nk) load(s0 + (ks + 1) * kBK);
#pragma unroll
      for (int s = 0; s < kBK / 16; ++s) {
        U16 a[MB], a2[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          a[mb] = frag_kmaj(ah[buf], wm * WM + mb * 32, s, lane);
          if constexpr (SA) a2[mb] = frag_kmaj(al[buf], wm * WM + mb * 32, s, lane);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const U16 b = frag_kmaj(bh[buf], wn * WN + nb * 32, s, lane);
          U16 b2;
          if constexpr (SB) b2 = frag_kmaj(bl[buf], wn * WN + nb * 32, s, lane);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            Mfma<bf16>::k32(acc[mb][nb], a[mb], b);
            if constexpr (SA) Mfma<bf16>::k32(acc[mb][nb], a2[mb], b);
            if constexpr (SB) Mfma<bf16>::k32(acc[mb][nb], a[mb], b2);
          }
        }
      }
      if (ks + 1 < nk) store(buf ^ 1);
      __syncthreads();
    }
    // This tile's destinations; its column sums go to LDS (every wave is past
    // the tile's last LDS read) before the next tile's first step, loaded here
    // ahead of the stores, starts adding to cs.
    const int om0 = m0, on0 = n0;
    float* const og = out;
    float* const ocs = colsum;
    if (ocs && !isb) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        csr[kq][8 * mu + e] = cs[e];
        cs[e] = 0.f;
      }
    }
    bool more = false;
    if constexpr (PERSIST) {
      T += gridDim.x;
      if (T < tend && tile_at(T)) {
        more = true;
        nk = (s1 - s0 + kBK - 1) / kBK;
        if (nk > 0) load(s0);
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = on0 + wn * WN + nb * 32 + (lane & 31);
      if (n >= p.N) continue;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int m = om0 + wm * WM + mb * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
          if (m < p.M) {
            // persistent tiles (short segments) write gradients that no later
            // kernel reads: non-temporal stores; the other tiles' chunk
            // partials, summed by the next kernel, stay cached
            if constexpr (PERSIST) __builtin_nontemporal_store(acc[mb][nb][j], &og[(int64_t)m * p.N + n]);
            else og[(int64_t)m * p.N + n] = acc[mb][nb][j];
          }
        }
    }
    if (ocs) {  // the 8 threads of a column unit hold rows 4 kq .. : add in kq order
      __syncthreads();
      if (tid < TM && om0 + tid < p.M) {
        float v = 0.f;
        for (int i = 0; i < 8; ++i) v += csr[i][tid];
        ocs[om0 + tid] = v;
      }
    }
    if (!more) break;
  }
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
// expert, plus the Importance loss's d/dImportance of the expert, then the
// kept softmax's backward, g_j (dg_j - sum_l g_l dg_l), into dHk [B][k]. With
// E = hidden W2^T + b2, dy . E = (dy W2) . hidden + dy . b2: the first term is
// the dA product's row dot (rowdot, rd_n partial sums per routed row, added in
// order), the second is formed here.
template <typename TY>
__global__ __launch_bounds__(256) void slot_grad_kernel(int64_t B, int k, int d,
                                                        const void* __restrict__ dy,
                                                        const float* __restrict__ rowdot,
                                                        int rd_n,
                                                        const void* __restrict__ b2,
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
    const int e = topk_idx[t * k + j];
    float s = 0.f;
    if (row >= 0 && b2)
      for (int c = lane; c < d; c += 64) s += ld_f<TY>(dy, t * d + c) * ld_f<TY>(b2, (int64_t)e * d + c);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (row >= 0)
      for (int q = 0; q < rd_n; ++q) s += rowdot[row * rd_n + q];
    dg[j] = s + dimp[e];
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
__device__ __forceinline__ void pair_grad_one(float c, float u, float e, bool kept, float dh,
                                              const float* thr2, float dl, float floor_,
                                              float& dc, float& du) {
  const float sigma = softplus_f(u) + floor_;
  const float rs = rcp_f(sigma);
  const float thr = kept ? thr2[1] : thr2[0];
  float pc = 0.f, ps = 0.f;
  if (!isinf(thr)) {
    const float z = (c - thr) * rs;
    const float ph = exp_native(-0.5f * z * z) * 0.3989422804014327f;  // phi(z)
    pc = ph * rs;
    ps = -ph * z * rs;
  }
  dc = dh + dl * pc;
  const float dsig = dh * e + dl * ps;
  const float eu = exp_native(-fabsf(u));  // Softplus'(u) = sigmoid(u)
  du = dsig * (u >= 0.f ? 1.f : eu) * rcp_f(1.f + eu);
}

// One token per blockIdx.x, 4 consecutive experts per thread (1024 per
// blockIdx.y); vec: n % 4 == 0, so the 4 values of c, u and eps are 16-byte loads.
__global__ __launch_bounds__(256) void pair_grad_kernel(int64_t B, int n, int k, int train,
                                                        float floor_, int vec,
                                                        const float* __restrict__ eps,
                                                        const float* __restrict__ thresh,
                                                        const int32_t* __restrict__ topk_idx,
                                                        const float* __restrict__ dHk,
                                                        const float* __restrict__ dload,
                                                        float* __restrict__ cu) {
  const int64_t t = blockIdx.x;
  const int i0 = 4 * (blockIdx.y * 256 + threadIdx.x);
  if (i0 >= n) return;
  float dh[4] = {0.f, 0.f, 0.f, 0.f};
  bool kept[4] = {false, false, false, false};
  for (int j = 0; j < k; ++j) {
    const int e = topk_idx[t * k + j] - i0;
    if (e >= 0 && e < 4) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q == e) {
          kept[q] = true;
          dh[q] = dHk[t * k + j];
        }
    }
  }
  float* row = cu + t * 2 * (int64_t)n;
  const int cnt = min(4, n - i0);
  if (!train) {
    for (int q = 0; q < cnt; ++q) row[i0 + q] = dh[q];
    return;
  }
  const float* thr2 = thresh + t * 2;
  if (vec && cnt == 4) {
    const float4 c = *reinterpret_cast<const float4*>(row + i0);
    const float4 u = *reinterpret_cast<const float4*>(row + n + i0);
    const float4 e = *reinterpret_cast<const float4*>(eps + t * n + i0);
    const float4 dl = *reinterpret_cast<const float4*>(dload + i0);
    float4 dc, du;
    pair_grad_one(c.x, u.x, e.x, kept[0], dh[0], thr2, dl.x, floor_, dc.x, du.x);
    pair_grad_one(c.y, u.y, e.y, kept[1], dh[1], thr2, dl.y, floor_, dc.y, du.y);
    pair_grad_one(c.z, u.z, e.z, kept[2], dh[2], thr2, dl.z, floor_, dc.z, du.z);
    pair_grad_one(c.w, u.w, e.w, kept[3], dh[3], thr2, dl.w, floor_, dc.w, du.w);
    *reinterpret_cast<float4*>(row + i0) = dc;
    *reinterpret_cast<float4*>(row + n + i0) = du;
    return;
  }
  for (int q = 0; q < cnt; ++q) {
    float dc, du;
    pair_grad_one(row[i0 + q], row[n + i0 + q], eps[t * n + i0 + q], kept[q], dh[q], thr2,
                  dload[i0 + q], floor_, dc, du);
    row[i0 + q] = dc;
    row[n + i0 + q] = du;
  }
}

// The selected pairs of each token (one wave per token), for a gradient pass
// that took every pair as unselected: c and u from fp32 dot products of the
// bf16 x row with the expert's gate weight rows (bias added to c), then
// pair_grad_one with the (k+1)-th threshold and the pair's dH, over cu in the
// gradient pass's blocked layout (row t of expert block q = e / 16 at
// cu + (q B + t) 32: the 16 clean-logit gradients, then the 16 noise ones).
__global__ __launch_bounds__(256) void kept_pair_grad_kernel(
    int64_t B, int n, int k, int d, const bf16* __restrict__ x, const bf16* __restrict__ wg,
    const bf16* __restrict__ wn, const float* __restrict__ bias, const float* __restrict__ eps,
    const float* __restrict__ thresh, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ dHk, const float* __restrict__ dload, float floor_,
    float* __restrict__ cu) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= B) return;
  // lane l holds elements 8 l .. 8 l + 7 of the row (d <= 512, a multiple of 8)
  const int c0 = 8 * lane;
  const bool act = c0 < d;
  float xv[8];
  {
    uint4 v = act ? *reinterpret_cast<const uint4*>(x + t * d + c0) : uint4{0u, 0u, 0u, 0u};
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) xv[i] = bf16_bits_to_f32((w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
  }
  for (int j = 0; j < k; ++j) {
    const int e = topk_idx[t * k + j];
    if (e < 0 || e >= n) continue;  // uniform over the wave
    float c = 0.f, u = 0.f;
    if (act) {
      const uint4 a = *reinterpret_cast<const uint4*>(wg + (int64_t)e * d + c0);
      const uint4 q = *reinterpret_cast<const uint4*>(wn + (int64_t)e * d + c0);
      const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        c = fmaf(xv[i], bf16_bits_to_f32((wa[i >> 1] >> (16 * (i & 1))) & 0xFFFFu), c);
        u = fmaf(xv[i], bf16_bits_to_f32((wq[i >> 1] >> (16 * (i & 1))) & 0xFFFFu), u);
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      c += __shfl_xor(c, o);
      u += __shfl_xor(u, o);
    }
    if (lane == 0) {
      if (bias) c += bias[e];
      float dc, du;
      pair_grad_one(c, u, eps[t * n + e], true, dHk[t * k + j], thresh + t * 2, dload[e], floor_,
                    dc, du);
      float* blk = cu + ((int64_t)(e >> 4) * B + t) * 32 + (e & 15);
      blk[0] = dc;
      blk[16] = du;
    }
  }
}

// dx[t] = dxg[t] + sum over the token's slots of dxe[slot_pos[t][j]] (fp32, slot order).
template <bool NT>
__global__ __launch_bounds__(256) void dx_sum_kernel(int64_t B, int k, int d,
                                                     const float* __restrict__ dxg,
                                                     const float* __restrict__ dxe,
                                                     const int32_t* __restrict__ slot_pos,
                                                     float* __restrict__ dx) {
  // four consecutive columns of one token per thread (d is a multiple of 4 and
  // every buffer 16-byte aligned): 16-byte loads and stores, the token's slot
  // positions read once; each element is still the gate path's value plus the
  // k rows in slot order
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int du = d >> 2;
  if (q >= B * du) return;
  const int64_t t = q / du;
  const int c = (int)(q - t * du) * 4;
  f32x4 v = *reinterpret_cast<const f32x4*>(dxg + t * d + c);
  for (int j = 0; j < k; ++j) {
    const int64_t row = slot_pos[t * k + j];
    if (row >= 0) {
      f32x4 e;
      if constexpr (NT) {
        const U16 u = ld_unit_stream(dxe + row * d + c);
        __builtin_memcpy(&e, &u, 16);
      } else {
        e = *reinterpret_cast<const f32x4*>(dxe + row * d + c);
      }
      v[0] += e[0];
      v[1] += e[1];
      v[2] += e[2];
      v[3] += e[3];
    }
  }
  *reinterpret_cast<f32x4*>(dx + t * d + c) = v;
}

// Row chunks of a weight gradient over all B tokens (the gate's): chunk i is
// rows [i B / S, (i + 1) B / S).
__global__ __launch_bounds__(64) void chunk_offsets_kernel(int32_t* __restrict__ off, int S,
                                                           int64_t B) {
  for (int i = threadIdx.x; i <= S; i += 64) off[i] = (int32_t)((int64_t)i * B / S);
}

// dW_g (rows < n of the [M][d] partials) and dW_noise (rows n .. 2n - 1), and
// the gate bias's gradient from the partial column sums: the S chunks' partial
// sums added in chunk order.
// blk: the product's rows are in the blocked order of the gradient pass
// (row 32 q + i: the clean logit of expert 16 q + i for i < 16, the noise
// pre-activation of expert 16 q + i - 16 otherwise); else rows 0 .. n - 1 are
// the clean logits and n .. M - 1 the noise pre-activations.
__global__ __launch_bounds__(256) void gate_wgrad_reduce_kernel(
    const float* __restrict__ part, const float* __restrict__ pcol, int S, int n, int M, int d,
    int blk, float* __restrict__ dwg, float* __restrict__ dwn, float* __restrict__ dgb) {
  const int64_t md = (int64_t)M * d;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < md) {
    float v = 0.f;
    for (int c = 0; c < S; ++c) v += part[c * md + i];
    const int m = (int)(i / d), col = (int)(i - (int64_t)m * d);
    const bool noise = blk ? (m & 31) >= 16 : m >= n;
    const int e = blk ? 16 * (m >> 5) + (m & 15) : (noise ? m - n : m);
    (noise ? dwn : dwg)[(int64_t)e * d + col] = v;
  } else if (i < md + n && dgb) {
    const int e = (int)(i - md);
    const int m = blk ? 32 * (e >> 4) + (e & 15) : e;
    float v = 0.f;
    for (int c = 0; c < S; ++c) v += pcol[(int64_t)c * M + m];
    dgb[e] = v;
  }
}

// Row chunks of the per-expert weight gradients: segment g (offsets[g] ..
// offsets[g + 1]) in ceil(rows / ch) chunks of at most ch rows (one chunk when
// empty). A segment of one chunk writes its gradient directly (slot -1); the
// chunks of a longer one get consecutive partial-sum slots, and multi lists
// it as (g, first slot, slots) for wg_chunk_reduce_kernel. One workgroup;
// thread t owns a contiguous span of segments.
__global__ __launch_bounds__(1024) void wg_chunk_plan_kernel(const int32_t* __restrict__ offsets,
                                                             int n, int ch,
                                                             int32_t* __restrict__ chunks,
                                                             int32_t* __restrict__ multi) {
  __shared__ int sc[1024], ss[1024], sm[1024];
  const int t = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int g0 = min(n, t * per), g1 = min(n, g0 + per);
  int c = 0, sl = 0, mu = 0;
  for (int g = g0; g < g1; ++g) {
    const int rows = offsets[g + 1] - offsets[g];
    const int k = rows > ch ? (rows + ch - 1) / ch : 1;
    c += k;
    if (k > 1) {
      sl += k;
      ++mu;
    }
  }
  sc[t] = c;
  ss[t] = sl;
  sm[t] = mu;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int vc = t >= o ? sc[t - o] : 0, vs = t >= o ? ss[t - o] : 0, vm = t >= o ? sm[t - o] : 0;
    __syncthreads();
    sc[t] += vc;
    ss[t] += vs;
    sm[t] += vm;
    __syncthreads();
  }
  int pc = sc[t] - c, ps = ss[t] - sl, pm = sm[t] - mu;
  for (int g = g0; g < g1; ++g) {
    const int a = offsets[g], rows = offsets[g + 1] - a;
    const int k = rows > ch ? (rows + ch - 1) / ch : 1;
    if (k > 1) {
      multi[1 + 3 * pm] = g;
      multi[2 + 3 * pm] = ps;
      multi[3 + 3 * pm] = k;
      ++pm;
    }
    for (int j = 0; j < k; ++j) {
      int32_t* e = chunks + 1 + 4 * pc;
      e[0] = g;
      e[1] = a + j * ch;
      e[2] = min(a + rows, a + (j + 1) * ch);
      e[3] = k > 1 ? ps + j : -1;
      ++pc;
    }
    if (k > 1) ps += k;
  }
  if (t == 1023) {
    chunks[0] = sc[t];
    multi[0] = sm[t];
  }
}

// out_g (and colsum_g) of each multi-chunk segment: its chunks' partial sums
// added in chunk order. blockIdx.y: entry of the multi list.
__global__ __launch_bounds__(256) void wg_chunk_reduce_kernel(const int32_t* __restrict__ multi,
                                                              const float* __restrict__ part,
                                                              const float* __restrict__ pcol,
                                                              int M, int N,
                                                              float* __restrict__ out,
                                                              int64_t out_stride,
                                                              float* __restrict__ colsum) {
  if ((int)blockIdx.y >= multi[0]) return;
  const int32_t* e = multi + 1 + 3 * blockIdx.y;
  const int g = e[0], s0 = e[1], ns = e[2];
  const int64_t mn = (int64_t)M * N;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < mn) {
    float v = 0.f;
    for (int j = 0; j < ns; ++j) v += part[(int64_t)(s0 + j) * mn + i];
    out[(int64_t)g * out_stride + i] = v;
  }
  if (colsum && i < M) {
    float v = 0.f;
    for (int j = 0; j < ns; ++j) v += pcol[(int64_t)(s0 + j) * M + i];
    colsum[(int64_t)g * M + i] = v;
  }
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
bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; }

hipError_t run_row_gemm(const RowGemm& p0, Dt ta, Dt tw, Dt to, int64_t grid_x, hipStream_t s,
                        bool bf16_cores = false) {
  if (grid_x <= 0) return hipSuccess;
  RowGemm p = p0;
  const bool tiled = bf16_cores && to == kF32;
  if (p.a_blk > 0 && (!tiled || p.gather || p.K % 16 != 0)) return hipErrorInvalidValue;
  p.rd_n = tiled ? (p.N + 255) / 256 : (p.N + kT - 1) / kT;  // column tiles: the row dots' stride
  if (tiled) {
    // 16-byte operand loads when every unit of 8 is in range and aligned
    const size_t wsz = tw == kBF16 ? 2 : 4;
    const int vec = aligned16(p.a) && aligned16(p.w) && p.lda % 8 == 0 && p.K % 8 == 0 &&
                    p.N % 8 == 0 && (p.w_stride * wsz) % 16 == 0;
    // kTR rows a workgroup; without units the grid follows from the rows. The
    // grid covers whole rounds of 8 runs of 2 ncb items (see the kernel).
    if (!p.units) grid_x = (p.rows + kTR - 1) / kTR;
    const int ncb = (p.N + 255) / 256;
    const int64_t nwork = grid_x * ncb, round = 16 * (int64_t)ncb;
    const dim3 grid((unsigned)((nwork + round - 1) / round * round)), block(4 * kTR);
#define MOE_RT(A, W, WT) \
  hipLaunchKernelGGL((row_tgemm_kernel<A, W, WT, kTR / 32>), grid, block, 0, s, p, vec, nwork, ncb)
    const bool a32 = ta == kF32, w32 = tw == kF32;
    if (p.wt) {
      if (!a32 && !w32) MOE_RT(bf16, bf16, true);
      else if (a32 && !w32) MOE_RT(float, bf16, true);
      else if (!a32 && w32) MOE_RT(bf16, float, true);
      else MOE_RT(float, float, true);
    } else {
      if (!a32 && !w32) MOE_RT(bf16, bf16, false);
      else if (a32 && !w32) MOE_RT(float, bf16, false);
      else if (!a32 && w32) MOE_RT(bf16, float, false);
      else MOE_RT(float, float, false);
    }
#undef MOE_RT
    return hipGetLastError();
  }
  const dim3 grid((unsigned)grid_x, (unsigned)((p.N + kT - 1) / kT)), block(256);
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

// big_ok: 256 x 256 tiles allowed (segments short enough that their number,
// not one segment's length, sets the work per tile); persist_ok: those tiles
// walked by one persistent workgroup per compute unit (many short tiles)
hipError_t run_wgrad(const Wgrad& p, Dt ta, Dt tb, int nseg, hipStream_t s,
                     bool bf16_cores = false, bool big_ok = true, bool persist_ok = false) {
  if (nseg <= 0) return hipSuccess;
  if (p.a_blk > 0 && (!bf16_cores || p.a_gather || p.M % 32 != 0)) return hipErrorInvalidValue;
  if (bf16_cores) {
    const int vec = aligned16(p.a) && aligned16(p.b) && p.lda % 8 == 0 && p.ldb % 8 == 0 &&
                    p.M % 8 == 0 && p.N % 8 == 0;
    // 256 x 256 tiles (eight waves) once both dimensions fill them, else 128 x 128
    const bool big = big_ok && p.M >= 256 && p.N >= 256;
    const int tm = big ? 256 : 128;
    const int64_t tps = (int64_t)((p.M + tm - 1) / tm) * ((p.N + tm - 1) / tm);
    dim3 grid((unsigned)tps, (unsigned)nseg);
    int pseg = 0;
    if (big && persist_ok) {
      // one workgroup per compute unit (its LDS allows one), a multiple of 8
      int cus = 0;
      const hipError_t e = device_cus(&cus);
      if (e != hipSuccess) return e;
      const int64_t want = (tps * nseg + 7) / 8 * 8;
      grid = dim3((unsigned)std::min<int64_t>(want, std::max(8, cus / 8 * 8)), 1u);
      pseg = nseg;
    }
#define MOE_WT(A, B_)                                                                          \
  if (big && pseg > 0)                                                                         \
    hipLaunchKernelGGL((wgrad_tgemm_kernel<A, B_, 256, 8, true>), grid, dim3(512), 0, s, p,    \
                       vec, pseg);                                                             \
  else if (big)                                                                                \
    hipLaunchKernelGGL((wgrad_tgemm_kernel<A, B_, 256, 8, false>), grid, dim3(512), 0, s, p,   \
                       vec, 0);                                                                \
  else                                                                                         \
    hipLaunchKernelGGL((wgrad_tgemm_kernel<A, B_, 128, 4, false>), grid, dim3(256), 0, s, p,   \
                       vec, 0)
    // (the products that run on bf16 cores have one fp32 and one bf16 operand)
    if (ta == kBF16 && tb == kF32) {
      MOE_WT(bf16, float);
    } else if (ta == kF32 && tb == kBF16) {
      MOE_WT(float, bf16);
    } else {
      return hipErrorInvalidValue;
    }
#undef MOE_WT
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(((p.M + kT - 1) / kT) * ((p.N + kT - 1) / kT)), (unsigned)nseg);
#define MOE_WG(A, B_) hipLaunchKernelGGL((wgrad_kernel<A, B_>), grid, dim3(256), 0, s, p)
  if (ta == kBF16 && tb == kBF16) MOE_WG(bf16, bf16);
  else if (ta == kF32 && tb == kBF16) MOE_WG(float, bf16);
  else if (ta == kBF16 && tb == kF32) MOE_WG(bf16, float);
  else if (ta == kF32 && tb == kF32) MOE_WG(float, float);
  else return hipErrorInvalidValue;
#undef MOE_WG
  return hipGetLastError();
}

// Chunks of the gate's weight gradient: enough workgroups for the chip
// (about 2048 of the 128 x 128 tiles over the [2n][d] output), at least 512
// rows a chunk, at most 32 chunks.
int gate_wgrad_chunks(int64_t B, int n, int d) {
  const int64_t tiles = ((2 * (int64_t)n + 127) / 128) * (((int64_t)d + 127) / 128);
  int64_t c = std::max<int64_t>(1, 2048 / std::max<int64_t>(1, tiles));
  c = std::min<int64_t>(c, 32);
  c = std::min<int64_t>(c, std::max<int64_t>(1, B / 512));
  return (int)c;
}

}  // namespace

// Row chunks of the per-expert weight gradients: at most ch rows, ch at least
// 2048 and large enough that the partial sums of the longest segments fit in
// 256 MiB (a multi-chunk segment has more than ch rows, so its chunks number
// under 2 rows / ch and all of them under 2 P / ch).
static int wg_chunk_rows(int64_t P, int h, int d) {
  const double need = 2.0 * (double)P * h * d * 4.0 / (256.0 * 1024 * 1024);
  int64_t ch = std::max<int64_t>(2048, (int64_t)std::ceil(need));
  return (int)((ch + 31) / 32 * 32);
}
static int64_t wg_max_chunks(int64_t P, int n, int ch) { return n + P / ch + 1; }
static int64_t wg_max_slots(int64_t P, int ch) { return 2 * P / ch + 1; }
static int64_t wg_max_multi(int64_t P, int n, int ch) { return std::min<int64_t>(n, P / ch) + 1; }
static size_t wg_chunk_bytes(int64_t P, int n, int d, int h) {
  const int ch = wg_chunk_rows(P, h, d);
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  return al((size_t)(1 + 4 * wg_max_chunks(P, n, ch)) * 4) +
         al((size_t)(1 + 3 * wg_max_multi(P, n, ch)) * 4) +
         al((size_t)wg_max_slots(P, ch) * h * d * 4) +
         al((size_t)wg_max_slots(P, ch) * std::max(h, d) * 4);
}

static size_t gate_chunk_bytes(int64_t B, int n, int d) {
  const size_t S = (size_t)gate_wgrad_chunks(B, n, d);
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  return al(S * 2 * n * d * 4) + al(S * 2 * n * 4) + al((S + 1) * 4);
}

size_t backward_ws_bytes(int64_t B, int n, int k, int d, int h, Dt act_dt) {
  const int64_t P = B * k;
  (void)act_dt;  // every staging buffer is fp32
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  const int64_t max_units = gate_max_units(P, n, kT);
  return al((size_t)n * 4) + al((size_t)(n + 1) * 4) + 3 * al((size_t)P * 4)  // route
         + al((size_t)n * route_blocks(B) * 4)                                  // blockcnt
         + al((size_t)(1 + 2 * max_units) * 4) + al((size_t)(n + 1) * 4)        // units
         + 2 * al((size_t)n * 4)                                                // dimp, dload
         + al((size_t)P * h * 4)                                                // hidden (fp32)
         + al((size_t)P * ((h + kT - 1) / kT) * 4)                              // row dots
         + al((size_t)B * k * 4)                                                // dHk
         + al((size_t)P * h * 4)                                                // dA
         + al((size_t)P * d * 4)                                                // dx per pair
         + al((size_t)B * 2 * n * 4)                                            // c|u grads
         + al((size_t)B * d * 4)                                                // dx via gate
         + gate_chunk_bytes(B, n, d)                                            // dW_g chunks
         + wg_chunk_bytes(P, n, d, h);                                          // dW_e chunks
}

hipError_t launch_backward(const BackwardLaunch& b, void* ws, hipStream_t s) {
  const int64_t B = b.tokens, P = B * b.k;
  const int n = b.n, k = b.k, d = b.d, h = b.h;
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
  // units of the row products: kTR rows on bf16 cores, kT otherwise (the
  // workspace holds the larger count, kT's)
  const int urows = b.act_dt == kBF16 ? kTR : kT;
  const int64_t max_units = gate_max_units(P, n, urows);
  int32_t* units = reinterpret_cast<int32_t*>(take((size_t)(1 + 2 * gate_max_units(P, n, kT)) * 4));
  int32_t* unit_start = reinterpret_cast<int32_t*>(take((size_t)(n + 1) * 4));
  float* dimp = reinterpret_cast<float*>(take((size_t)n * 4));
  float* dload = reinterpret_cast<float*>(take((size_t)n * 4));
  float* hid = reinterpret_cast<float*>(take((size_t)P * h * 4));
  float* rowdot = reinterpret_cast<float*>(take((size_t)P * ((h + kT - 1) / kT) * 4));
  float* dHk = reinterpret_cast<float*>(take((size_t)B * k * 4));
  float* dA = reinterpret_cast<float*>(take((size_t)P * h * 4));
  float* dxe = reinterpret_cast<float*>(take((size_t)P * d * 4));
  float* cu = reinterpret_cast<float*>(take((size_t)B * 2 * n * 4));
  float* dxg = reinterpret_cast<float*>(take((size_t)B * d * 4));
  const int S = gate_wgrad_chunks(B, n, d);
  float* gpart = reinterpret_cast<float*>(take((size_t)S * 2 * n * d * 4));
  float* gcol = reinterpret_cast<float*>(take((size_t)S * 2 * n * 4));
  int32_t* gchunk = reinterpret_cast<int32_t*>(take((size_t)(S + 1) * 4));
  const int wch = wg_chunk_rows(P, h, d);
  const int64_t wmax_chunks = wg_max_chunks(P, n, wch), wmax_multi = wg_max_multi(P, n, wch);
  int32_t* wchunks = reinterpret_cast<int32_t*>(take((size_t)(1 + 4 * wmax_chunks) * 4));
  int32_t* wmulti = reinterpret_cast<int32_t*>(take((size_t)(1 + 3 * wmax_multi) * 4));
  float* wpart = reinterpret_cast<float*>(take((size_t)wg_max_slots(P, wch) * h * d * 4));
  float* wpcol = reinterpret_cast<float*>(take((size_t)wg_max_slots(P, wch) * std::max(h, d) * 4));
  hipError_t e;

  // routing of the forward's selection, and the units of its segments
  e = launch_route(B, k, n, b.topk_idx, b.topk_gate, blockcnt, counts, offsets, perm_token,
                   perm_gate, slot_pos, nullptr, s);
  if (e != hipSuccess) return e;
  e = launch_group_plan(offsets, n, urows, units, unit_start, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cv2_grad_kernel, dim3(1), dim3(1024), 0, s, b.importance, b.load, n,
                     b.aux_scale * b.w_importance, b.aux_scale * b.w_load, b.train, dimp, dload);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // experts: hidden = ReLU(x W1^T + b1), kept in fp32 (the forward pass rounds it to the
  // storage type; the gradients here are those of the layer's unrounded function)
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
  // dA = (gate * dy[token]) W2 masked by hidden > 0, and per routed row the dot of
  // dy[token] W2 with hidden (for the kept gates' gradient dy . E)
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
  r.rowdot = rowdot;
  if ((e = run_row_gemm(r, b.act_dt, b.act_dt, kF32, max_units, s, b.act_dt == kBF16)) != hipSuccess) return e;
  // kept gates: task + Importance gradients through the kept softmax
  if (B > 0) {
    const int rd_n = b.act_dt == kBF16 ? (h + 255) / 256 : (h + kT - 1) / kT;  // as run_row_gemm
    if (b.act_dt == kBF16)
      hipLaunchKernelGGL(slot_grad_kernel<bf16>, dim3((unsigned)((B + 3) / 4)), dim3(256), 0, s,
                         B, k, d, b.dy, rowdot, rd_n, b.b2, slot_pos, b.topk_idx, b.topk_gate,
                         dimp, dHk);
    else
      hipLaunchKernelGGL(slot_grad_kernel<float>, dim3((unsigned)((B + 3) / 4)), dim3(256), 0, s,
                         B, k, d, b.dy, rowdot, rd_n, b.b2, slot_pos, b.topk_idx, b.topk_gate,
                         dimp, dHk);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // the per-expert weight gradients run over row chunks of at most wch rows (a long
  // segment's chunks write partial sums, added in chunk order afterwards)
  hipLaunchKernelGGL(wg_chunk_plan_kernel, dim3(1), dim3(1024), 0, s, offsets, n, wch, wchunks,
                     wmulti);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  auto chunk_reduce = [&](const Wgrad& w) {
    hipLaunchKernelGGL(wg_chunk_reduce_kernel,
                       dim3(blocks_for((int64_t)w.M * w.N), (unsigned)wmax_multi), dim3(256), 0,
                       s, wmulti, wpart, wpcol, w.M, w.N, w.out, w.out_stride, w.colsum);
    return hipGetLastError();
  };
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
  wg.chunks = wchunks;
  wg.part = wpart;
  wg.pcol = wpcol;
  // long segments (over 256 rows per expert on average) keep 128 x 128 tiles, so that
  // one popular expert's rows are spread over more workgroups
  const bool short_segs = P < 256 * (int64_t)n;
  if ((e = run_wgrad(wg, b.act_dt, kF32, (int)wmax_chunks, s, b.act_dt == kBF16, short_segs,
                       short_segs)) != hipSuccess)
    return e;
  if ((e = chunk_reduce(wg)) != hipSuccess) return e;
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
  wg.chunks = wchunks;
  wg.part = wpart;
  wg.pcol = wpcol;
  if ((e = run_wgrad(wg, kF32, b.act_dt, (int)wmax_chunks, s, b.act_dt == kBF16, short_segs,
                       short_segs)) != hipSuccess)
    return e;
  if ((e = chunk_reduce(wg)) != hipSuccess) return e;
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

  // gate: the gradients of every (token, expert) pair's clean logit and noise
  // pre-activation into cu [B][2n]
  const int64_t rt = (B + kT - 1) / kT;
  GateLaunch gl{};
  gl.x = b.x;
  gl.w_gate = b.w_gate;
  gl.w_noise = b.w_noise;
  gl.bias = b.gate_bias;
  gl.eps = b.eps;
  gl.tokens = B;
  gl.d = d;
  gl.n = n;
  gl.k = k;
  gl.x_dt = b.act_dt;
  gl.w_dt = b.gate_dt;
  gl.train = b.train;
  gl.noise_floor = b.noise_floor;
  // fused: cu holds the gradient pass's blocked layout instead of [B][2n]
  const bool fused = B > 0 && gate_pair_grads_supported(gl);
  if (fused) {
    // the gate's matrix-core pass takes every pair as unselected, then the
    // selected pairs are rewritten from their own dot products
    if ((e = launch_gate_pair_grads(gl, b.thresh, dload, cu, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(kept_pair_grad_kernel, dim3((unsigned)((B + 3) / 4)), dim3(256), 0, s, B, n,
                       k, d, static_cast<const bf16*>(b.x), static_cast<const bf16*>(b.w_gate),
                       static_cast<const bf16*>(b.w_noise), b.gate_bias, b.eps, b.thresh,
                       b.topk_idx, dHk, dload, b.noise_floor, cu);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
    // c = x W_g^T + b, u = x W_noise^T into cu, then their gradients in place
    // (without noise only the selected pairs' dH, which needs neither)
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
    if (b.train) {
      if ((e = run_row_gemm(r, b.act_dt, b.gate_dt, kF32, rt, s, b.act_dt == kBF16)) != hipSuccess) return e;
      r.w = b.w_noise;
      r.bias = nullptr;
      r.out = cu + n;
      if ((e = run_row_gemm(r, b.act_dt, b.gate_dt, kF32, rt, s, b.act_dt == kBF16)) != hipSuccess) return e;
    }
    if (B > 0) {
      const int vec = n % 4 == 0 && (reinterpret_cast<uintptr_t>(b.eps) & 15) == 0;
      hipLaunchKernelGGL(pair_grad_kernel, dim3((unsigned)B, (unsigned)((n + 1023) / 1024)),
                         dim3(256), 0, s, B, n, k, b.train, b.noise_floor, vec, b.eps, b.thresh,
                         b.topk_idx, dHk, dload, cu);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  // dW_g = dc^T x, db_g = sum dc; dW_noise = du^T x: one product over the [B][2n]
  // logit gradients (n columns without noise), the B rows in S chunks whose
  // partial sums are added in chunk order
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(64), 0, s, gchunk, S, B);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int gm = b.train ? 2 * n : n;
  wg = Wgrad{};
  wg.seg_off = gchunk;
  wg.rows = B;
  wg.a = cu;
  wg.lda = 2 * (int64_t)n;
  wg.a_blk = fused ? B : 0;
  wg.b = b.x;
  wg.ldb = d;
  wg.M = gm;
  wg.N = d;
  wg.out = gpart;
  wg.out_stride = (int64_t)gm * d;
  wg.colsum = gcol;
  // 256 x 256 tiles while they still give 512 workgroups with the chunks
  const bool gate_big = ((gm + 255) / 256) * (int64_t)((d + 255) / 256) * S >= 512;
  if ((e = run_wgrad(wg, kF32, b.act_dt, S, s, b.act_dt == kBF16, gate_big)) != hipSuccess) return e;
  hipLaunchKernelGGL(gate_wgrad_reduce_kernel, dim3(blocks_for((int64_t)gm * d + n)), dim3(256),
                     0, s, gpart, gcol, S, n, gm, d, fused ? 1 : 0, b.dw_gate, b.dw_noise,
                     b.dgate_bias);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (!b.train) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks_for((int64_t)n * d)), dim3(256), 0, s,
                       b.dw_noise, (int64_t)n * d);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // dx through the gate: dc W_g + du W_noise
  r = RowGemm{};
  r.rows = B;
  r.a = cu;
  r.lda = 2 * (int64_t)n;
  r.a_blk = fused ? B : 0;
  r.w = b.w_gate;
  r.wt = 0;
  r.K = n;
  r.N = d;
  r.out = dxg;
  r.ldo = d;
  if ((e = run_row_gemm(r, kF32, b.gate_dt, kF32, rt, s, b.act_dt == kBF16)) != hipSuccess) return e;
  if (b.train) {
    r.a = fused ? cu + 16 : cu + n;
    r.w = b.w_noise;
    r.accumulate = 1;
    if ((e = run_row_gemm(r, kF32, b.gate_dt, kF32, rt, s, b.act_dt == kBF16)) != hipSuccess) return e;
  }
  if (B > 0) {
    // the routed rows' dx (P x d fp32) is read once: non-temporal past the Infinity Cache
    if ((int64_t)P * d * 4 > kStreamBytes)
      hipLaunchKernelGGL((dx_sum_kernel<true>), dim3(blocks_for(B * (d / 4))), dim3(256), 0, s, B,
                         k, d, dxg, dxe, slot_pos, b.dx);
    else
      hipLaunchKernelGGL((dx_sum_kernel<false>), dim3(blocks_for(B * (d / 4))), dim3(256), 0, s, B,
                         k, d, dxg, dxe, slot_pos, b.dx);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
