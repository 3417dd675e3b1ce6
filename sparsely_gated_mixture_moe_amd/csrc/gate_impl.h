// Template of the gating kernel; instantiated per storage-type combination in
// gate_bf16.hip, gate_bf16x_f32w.hip and gate_f32.hip.
#pragma once

// Noisy top-k gating on gfx950 (section "Noisy top-k gating", eqs 3-5, with the
// noise floor of the explainer's code as a parameter), and the Load pass of
// "A differentiable count of examples" (eqs 8-10), which shares its main loop.
//
// One workgroup owns 128 token rows (8 waves x 16 rows) and sweeps all n
// experts in chunks: the clean-logit and noise-scale weight rows of a chunk
// are staged once in LDS (double-buffered, in matrix-core fragment order) and
// shared by the 8 waves; each wave keeps its 16 rows of x in registers as MFMA
// A operands for the whole sweep. The logits never reach HBM.
//
// Pass 1 epilogue, per (token, expert): sigma = Softplus(u) + floor,
// H = clean + eps * sigma; each lane keeps, for its 4 rows, the L best (H,
// expert) pairs of the experts it sees (expert = lane mod 16); at the end the
// 16 lanes of a row merge their lists (butterfly over lane bits 0-3), and the
// row's top k, their softmax gates and the k-th/(k+1)-th logits are written.
//
// Pass 2 epilogue: P = Phi((clean - v_k) / sigma) with v_k the row's k-th
// largest logit; column sums over the block's rows in a fixed order go to a
// per-block partial, reduced afterwards in block order. The selected pairs,
// whose threshold is the (k+1)-th logit instead, are corrected by a separate
// kernel over the routed rows. Pass 2 recomputes the matrix products instead
// of storing B x n logits.

#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace gate_detail {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
static_assert(kGateRows == kWaves * 16, "gate rows per block");

struct GateParams {
  const void* x;
  const void* wg;
  const void* wn;
  const float* bias;
  const float* eps;
  int64_t B;
  int n, k;
  float floor;
  int32_t* topk_idx;
  float* topk_gate;
  float* thresh;
  const float* sel_thr;  // pass 2: (k-th, (k+1)-th) logit of each row
  float* partial;
  // Gradient pass (the Load pass's products, another epilogue; 32x32 kernel
  // only): dload [n] is d loss / d Load; every pair's gradients with respect
  // to its clean logit and noise pre-activation, taken as unselected, go to
  // dcu in blocks of 16 experts: row r of block q (experts 16 q .. 16 q + 15)
  // is 32 floats at dcu + (q B + r) 32, the 16 clean-logit gradients then the
  // 16 noise ones. Null otherwise.
  const float* dload;
  float* dcu;
  // Selection of one expert range (gridDim.y ranges): each row's best L
  // (value, expert) go to [(row * gridDim.y + blockIdx.y) * L + j] instead of
  // the outputs above; null when every workgroup sweeps all experts.
  float* cand_v;
  int32_t* cand_i;
  // with gate_order 1 each range also writes its rows' (max, sum of exp(H -
  // max)) pair to cand_ms [(row * gridDim.y + blockIdx.y) * 2]
  float* cand_ms;
  // Batchwise gating: every H goes to scores[e * sld + row] (expert-major,
  // one row of sld >= B per expert) instead of a selection; null otherwise.
  float* scores;
  int64_t sld;
  // Secondary gating of a hierarchical layer ("Hierarchical MoE"); all null
  // for a flat gate. The rows are those a primary route sent to each group:
  // workgroup u covers the rows seg_off[g] + first, ... of group g, with
  // (g, first) = (units[1 + 2u], units[2 + 2u]) and units[0] the number of
  // units. Routed row r reads x row row_token[r] and owns row row_slot[r] of
  // eps, of the outputs and of sel_thr; group g's gate weights are
  // rows g*n .. g*n + n - 1 of wg / wn, its biases entries g*n .. of bias.
  const int32_t* units;
  const int32_t* seg_off;
  const int32_t* row_token;
  const int32_t* row_slot;
};

// The rows of one workgroup: flat gating takes batch rows first .. first +
// ROWS - 1 (those below B); secondary gating takes routed rows first .. of one
// group (those below the group's segment end).
struct RowTile {
  int64_t first, end;
  bool grouped;
};

// Resolves this workgroup's rows; for secondary gating also moves the weight
// and bias pointers to the group's block. Returns false when a secondary
// gating workgroup has no unit (the grid covers the largest possible count).
template <int ROWS, typename WT, int D>
__device__ __forceinline__ bool resolve_tile(GateParams& p, RowTile& t) {
  if (p.units == nullptr) {
    t.first = (int64_t)blockIdx.x * ROWS;
    t.end = p.B;
    t.grouped = false;
    return true;
  }
  const int u = blockIdx.x;
  if (u >= p.units[0]) return false;
  const int g = p.units[1 + 2 * u];
  t.first = (int64_t)p.seg_off[g] + p.units[2 + 2 * u];
  t.end = p.seg_off[g + 1];
  t.grouped = true;
  const int64_t woff = (int64_t)g * p.n * D;
  p.wg = reinterpret_cast<const WT*>(p.wg) + woff;
  p.wn = reinterpret_cast<const WT*>(p.wn) + woff;
  if (p.bias) p.bias += (int64_t)g * p.n;
  return true;
}

// x row of local row i of the tile, or -1 past its end.
__device__ __forceinline__ int64_t tile_xrow(const GateParams& p, const RowTile& t, int i) {
  const int64_t r = t.first + i;
  if (r >= t.end) return -1;
  return t.grouped ? (int64_t)p.row_token[r] : r;
}

// Row of eps, of the outputs and of the selections owned by local row i, or -1.
__device__ __forceinline__ int64_t tile_iorow(const GateParams& p, const RowTile& t, int i) {
  const int64_t r = t.first + i;
  if (r >= t.end) return -1;
  return t.grouped ? (int64_t)p.row_slot[r] : r;
}

template <typename CT>
struct GateShape;
template <>
struct GateShape<bf16> {
  static constexpr int kChunk = 32;  // experts per LDS chunk
};
template <>
struct GateShape<float> {
  static constexpr int kChunk = 16;
};

// Loads the 16-byte unit of x (compute type CT) at element offset `off`.
template <typename XS, typename CT>
__device__ __forceinline__ U16 load_x_unit(const void* x, int64_t off) {
  if constexpr (sizeof(XS) == sizeof(CT)) {
    return ld_unit(reinterpret_cast<const char*>(x) + off * sizeof(XS));
  } else {
    return widen4_bf16(reinterpret_cast<const char*>(x) + off * sizeof(XS));  // bf16 -> fp32
  }
}

// L-entry descending list insertion of a (value, index) pair known to rank
// after every equal value already in the list (its index is larger).
template <int L>
__device__ __forceinline__ void insert_new(float (&lv)[L], int (&li)[L], float v, int id) {
  if (v > lv[L - 1]) {
    lv[L - 1] = v;
    li[L - 1] = id;
#pragma unroll
    for (int s = L - 1; s > 0; --s) {
      const bool sw = lv[s] > lv[s - 1];
      const float tv = lv[s];
      const int ti = li[s];
      lv[s] = sw ? lv[s - 1] : tv;
      li[s] = sw ? li[s - 1] : ti;
      lv[s - 1] = sw ? tv : lv[s - 1];
      li[s - 1] = sw ? ti : li[s - 1];
    }
  }
}

// Insertion with the full ranking order (used when merging lists).
template <int L>
__device__ __forceinline__ void insert_any(float (&lv)[L], int (&li)[L], float v, int id) {
  if (ranks_before(v, id, lv[L - 1], li[L - 1])) {
    lv[L - 1] = v;
    li[L - 1] = id;
#pragma unroll
    for (int s = L - 1; s > 0; --s) {
      const bool sw = ranks_before(lv[s], li[s], lv[s - 1], li[s - 1]);
      const float tv = lv[s];
      const int ti = li[s];
      lv[s] = sw ? lv[s - 1] : tv;
      li[s] = sw ? li[s - 1] : ti;
      lv[s - 1] = sw ? tv : lv[s - 1];
      li[s - 1] = sw ? ti : li[s - 1];
    }
  }
}

// Chunks [c0, c0 + count) of the nch chunks of n experts that workgroup
// (x, y) sweeps: gridDim.y consecutive ranges of ceil(nch / gridDim.y) chunks
// (the launcher picks gridDim.y so that none is empty).
struct ChunkRange {
  int c0, count;
};
__device__ __forceinline__ ChunkRange chunk_range(int nch) {
  const int per = (nch + (int)gridDim.y - 1) / (int)gridDim.y;
  const int c0 = (int)blockIdx.y * per;
  return ChunkRange{c0, min(per, nch - c0)};
}

// Softmax over all n logits (gate_order 1): each lane keeps the running
// maximum m of the logits it has seen and s = sum of exp(H - m) over them,
// rescaled when m grows; two such pairs combine the same way. A lane that
// has seen only -inf keeps (m, s) = (-inf, 0).
struct ExpSum {
  float m, s;
};
__device__ __forceinline__ ExpSum expsum_merge(ExpSum a, ExpSum b) {
  const float m = fmaxf(a.m, b.m);
  const float ref = m == -INFINITY ? 0.f : m;
  return ExpSum{m, a.s * expf(a.m - ref) + b.s * expf(b.m - ref)};
}
template <int N>
__device__ __forceinline__ ExpSum expsum_add(ExpSum a, const float (&h)[N]) {
  float mx = h[0];
#pragma unroll
  for (int i = 1; i < N; ++i) mx = fmaxf(mx, h[i]);
  const float m = fmaxf(a.m, mx);
  const float ref = m == -INFINITY ? 0.f : m;
  float add = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) add += expf(h[i] - ref);
  return ExpSum{m, fmaf(a.s, expf(a.m - ref), add)};
}

// A row's outputs from its best L (value, expert) in rank order: the first
// k experts, the softmax of their logits (over the kept k, or with gate_order
// 1 over all n, whose (max, sum) is `es`), and the k-th and (k+1)-th logits;
// or, for a split sweep, the list itself (and `es`) as this range's
// candidates.
template <int L>
__device__ __forceinline__ void write_selection(const GateParams& p, int64_t row,
                                                const float (&lv)[L], const int (&li)[L],
                                                ExpSum es = ExpSum{-INFINITY, 0.f}) {
  if (p.cand_v) {
    const int64_t o = (row * gridDim.y + blockIdx.y) * L;
#pragma unroll
    for (int j = 0; j < L; ++j) {
      p.cand_v[o + j] = lv[j];
      p.cand_i[o + j] = li[j];
    }
    if (p.cand_ms) {
      p.cand_ms[(row * gridDim.y + blockIdx.y) * 2] = es.m;
      p.cand_ms[(row * gridDim.y + blockIdx.y) * 2 + 1] = es.s;
    }
    return;
  }
  const int k = p.k;
  // softmax over the k kept logits (the rest are -inf, gate 0), or their
  // share of the softmax over all n
  const bool all_n = es.s > 0.f;
  const float top = all_n ? es.m : lv[0];
  float ex[L - 1];
  float z = 0.f;
#pragma unroll
  for (int j = 0; j < L - 1; ++j) {
    ex[j] = (j < k) ? expf(lv[j] - top) : 0.f;
    z += ex[j];
  }
  const float inv = 1.0f / (all_n ? es.s : z);
#pragma unroll
  for (int j = 0; j < L - 1; ++j) {
    if (j < k) {
      p.topk_idx[row * k + j] = li[j];
      p.topk_gate[row * k + j] = ex[j] * inv;
    }
  }
  float vk = lv[0], vk1 = lv[1];
#pragma unroll
  for (int j = 1; j < L; ++j) {
    if (j == k - 1) vk = lv[j];
    if (j == k) vk1 = lv[j];
  }
  p.thresh[row * 2] = vk;
  p.thresh[row * 2 + 1] = vk1;
}

template <typename XS, typename CT, int D, int L, bool TRAIN, bool PASS2, bool SMX = false,
          bool SCORES = false>
__global__ __launch_bounds__(kThreads) void gate_kernel(GateParams p) {
  RowTile tile;
  if (!resolve_tile<kGateRows, CT, D>(p, tile)) return;
  constexpr int UE = Elem<CT>::kPerUnit;
  constexpr int KB = 4 * UE;  // K-block of the 16x16 tiles
  static_assert(D % KB == 0, "d must be a multiple of the K-block");
  constexpr int NKB = D / KB;
  // bf16 x with fp32 weights: x stays packed as bf16 in registers (half the
  // registers of fp32, which would not fit beside the rest with two waves per
  // SIMD) and each value is widened exactly as it feeds its fp32 product. A
  // lane then holds 8 consecutive K values per 16-byte unit, so K-block kb
  // takes K values (kb / 2) * 32 + 8 q + 4 (kb % 2) + s at product step s (the
  // weight fragments are staged in the same order).
  constexpr bool XPACK = sizeof(XS) == 2 && sizeof(CT) == 4;
  static_assert(!XPACK || NKB % 2 == 0, "packed x takes K-blocks in pairs");
  constexpr int NXU = XPACK ? NKB / 2 : NKB;  // x units per lane
  constexpr int EC = GateShape<CT>::kChunk;
  constexpr int NT = EC / 16;
  constexpr int NM = TRAIN ? 2 : 1;
  constexpr int UROW = D / UE;  // units per weight row
  constexpr int CHUNK_UNITS = NM * EC * UROW;
  constexpr int LOAD_ITERS = (CHUNK_UNITS + kThreads - 1) / kThreads;
  static_assert(!PASS2 || TRAIN, "the load pass is only needed with noise");

  __shared__ U16 wbuf[2][CHUNK_UNITS];
  __shared__ float red[PASS2 ? 2 : 1][kWaves][EC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;  // A-operand row / C column within a 16x16 tile
  const int q = lane >> 4;   // K unit of the A/B operands; C row group
  const int n = p.n;
  const int wrow0 = wave * 16;  // first local row of this wave
  // this workgroup's range of expert chunks (all of them unless split)
  const ChunkRange cr = chunk_range((n + EC - 1) / EC);
  const int cbase = cr.c0 * EC;
  const int nchunks = cr.count;

  // x rows of this wave as A operands for every K-block.
  U16 xa[NXU];
  {
    const int64_t r = tile_xrow(p, tile, wrow0 + lr);
#pragma unroll
    for (int u = 0; u < NXU; ++u) {
      if constexpr (XPACK)
        xa[u] = (r >= 0) ? ld_unit(reinterpret_cast<const XS*>(p.x) + r * D + u * 32 + q * 8)
                         : zero_unit();
      else
        xa[u] = (r >= 0) ? load_x_unit<XS, CT>(p.x, r * D + u * KB + q * UE) : zero_unit();
    }
  }
  // The A operand of K-block kb.
  auto x_operand = [&](int kb) __attribute__((always_inline)) -> U16 {
    if constexpr (XPACK) {
      // opaque copies: the widened values are loop-invariant, and hoisting
      // them out of the chunk loop would rebuild the fp32 copy of x
      uint32_t lo = xa[kb >> 1].w[(kb & 1) * 2], hi = xa[kb >> 1].w[(kb & 1) * 2 + 1];
      asm volatile("" : "+v"(lo), "+v"(hi));
      U16 a;
      a.w[0] = lo << 16;
      a.w[1] = lo & 0xFFFF0000u;
      a.w[2] = hi << 16;
      a.w[3] = hi & 0xFFFF0000u;
      return a;
    } else {
      return xa[kb];
    }
  };

  // Per-lane state for the C rows wrow0 + 4q + r, r < 4: validity and the row
  // of eps / outputs they own (invalid rows read the tile's first row's noise,
  // which is masked).
  bool row_ok[4];
  int64_t iorow[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    iorow[r] = tile_iorow(p, tile, wrow0 + 4 * q + r);
    row_ok[r] = iorow[r] >= 0;
  }
  const int64_t iorow_any = tile_iorow(p, tile, 0);
  float lv[4][L];
  int li[4][L];
  ExpSum es[4];  // SMX: this lane's part of each row's softmax over all n
#pragma unroll
  for (int r = 0; r < 4; ++r) es[r] = ExpSum{-INFINITY, 0.f};
  float shared_thr[4];  // max over the row's 16 lanes of their L-th best: a lower
                        // bound of the row's L-th best logit
  float thr_k[4];
  if constexpr (!PASS2) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      shared_thr[r] = -INFINITY;
#pragma unroll
      for (int j = 0; j < L; ++j) {
        lv[r][j] = -INFINITY;
        li[r][j] = 0x7FFFFFFF;
      }
    }
  } else {
    // Every pair is evaluated against the row's k-th largest logit; the
    // selected pairs' difference (threshold (k+1)-th) is added separately.
#pragma unroll
    for (int r = 0; r < 4; ++r) thr_k[r] = row_ok[r] ? p.sel_thr[iorow[r] * 2] : 0.f;
  }

  // Chunk staging. Unit u of a chunk is stored at LDS unit u in fragment order
  // (u = ((kb * NM + m) * NT + nt) * 64 + fragment lane), so each wave writes
  // one contiguous kilobyte per instruction and the MFMA B-operand reads are
  // contiguous too. Fragment lane fl holds expert column nt * 16 + (fl & 15),
  // K unit kb * 4 + (fl >> 4).
  U16 stage[LOAD_ITERS];
  auto gload = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < LOAD_ITERS; ++it) {
      const int u = tid + it * kThreads;
      if (CHUNK_UNITS % kThreads == 0 || u < CHUNK_UNITS) {
        const int fl = u & 63;
        const int rest = u >> 6;
        const int nt = rest % NT;
        const int m = (rest / NT) % NM;
        const int kb = rest / (NT * NM);
        // experts past n read row n - 1; their logits are masked in the epilogue
        const int e = min(cbase + c * EC + nt * 16 + (fl & 15), n - 1);
        const CT* w = reinterpret_cast<const CT*>(m ? p.wn : p.wg);
        const int koff = XPACK ? (kb >> 1) * 32 + (fl >> 4) * 8 + (kb & 1) * 4
                               : (kb * 4 + (fl >> 4)) * UE;
        stage[it] = ld_unit(w + (int64_t)e * D + koff);
      }
    }
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < LOAD_ITERS; ++it) {
      const int u = tid + it * kThreads;
      if (CHUNK_UNITS % kThreads == 0 || u < CHUNK_UNITS) wbuf[buf][u] = stage[it];
    }
  };
  auto mfma_chunk = [&](int buf, f32x4 (&acc)[NM][NT]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          Mfma<CT>::k16(acc[m][nt], x_operand(kb),
                        wbuf[buf][((kb * NM + m) * NT + nt) * 64 + lane]);
  };
  // Noise draws and biases of a chunk. Addresses are clamped into range and
  // invalid entries are masked later by selects, so no branch splits the block
  // that overlaps the matrix products with the epilogue.
  const bool has_bias = p.bias != nullptr;
  const float* bias_src = has_bias ? p.bias : reinterpret_cast<const float*>(p.wg);
  auto load_eps = [&](int c, float (&ev)[NT][4], float (&bv)[NT]) __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int e = min(cbase + c * EC + nt * 16 + lr, n - 1);
      bv[nt] = bias_src[e];
      if constexpr (TRAIN && !PASS2) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t row = row_ok[r] ? iorow[r] : iorow_any;
          ev[nt][r] = p.eps[row * n + e];
        }
      }
    }
  };

  // Software pipeline over expert chunks: the matrix products of chunk c + 1
  // and the epilogue of chunk c sit in one straight-line block, so the matrix
  // cores and the vector ALUs overlap; weights are staged two chunks ahead.
  f32x4 acc[NM][NT], acc_next[NM][NT];
  float ev[NT][4], ev_next[NT][4], bv[NT], bv_next[NT];
  gload(0);
  lstore(0);
  if (nchunks > 1) gload(1);
  load_eps(0, ev, bv);
  __syncthreads();
  mfma_chunk(0, acc);
  if (nchunks > 1) lstore(1);
  __syncthreads();
  if (nchunks > 2) gload(2);

  for (int c = 0; c < nchunks; ++c) {
    const bool more = c + 1 < nchunks;
    // The two waves that share a SIMD (w and w + 4) run this chunk's two
    // halves in opposite order -- one starts on the matrix core (next chunk's
    // products; after the last chunk they read a stale buffer and are
    // discarded) while the other starts on the vector ALUs (this chunk's
    // epilogue) -- so the two units overlap.
    float hv[NT][4];
    bool cand_any = false;
    float colsum[NT];
    auto products = [&]() __attribute__((always_inline)) {
      load_eps(more ? c + 1 : c, ev_next, bv_next);
      mfma_chunk((c + 1) & 1, acc_next);
    };
    auto epilogue = [&]() __attribute__((always_inline)) {
      // branch-free: invalid rows/experts are masked by selects
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        colsum[nt] = 0.f;
        const int e = cbase + c * EC + nt * 16 + lr;
        const bool e_ok = e < n;
        const float bias = has_bias ? bv[nt] : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = e_ok && row_ok[r];
          const float clean = acc[0][nt][r] + bias;
          if constexpr (!PASS2) {
            float H = clean;
            if constexpr (TRAIN) H = fmaf(ev[nt][r], softplus_f(acc[NM - 1][nt][r]) + p.floor, clean);
            H = ok ? H : -INFINITY;
            hv[nt][r] = H;
            cand_any |= (H > lv[r][L - 1]) && (H >= shared_thr[r]);
          } else {
            const float sigma = softplus_f(acc[NM - 1][nt][r]) + p.floor;
            const float P = phi_f((clean - thr_k[r]) * rcp_f(sigma));
            colsum[nt] += ok ? P : 0.f;
          }
        }
      }
    };
    if (wave & 4) {
      epilogue();
      __builtin_amdgcn_sched_barrier(0);
      products();
    } else {
      products();
      __builtin_amdgcn_sched_barrier(0);
      epilogue();
    }

    if constexpr (PASS2) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float s = colsum[nt];
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        if (q == 0) red[c & 1][wave][nt * 16 + lr] = s;
      }
    } else if constexpr (SCORES) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int e = cbase + c * EC + nt * 16 + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (e < n && row_ok[r]) p.scores[(int64_t)e * p.sld + iorow[r]] = hv[nt][r];
      }
    } else {
      if constexpr (SMX) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float h[NT];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) h[nt] = hv[nt][r];
          es[r] = expsum_add(es[r], h);
        }
      }
      // Rare path: candidates above both the lane's own L-th best and the
      // row's shared bound. Experts reach a lane in increasing index order.
      if (__any(cand_any)) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (hv[nt][r] >= shared_thr[r])
              insert_new<L>(lv[r], li[r], hv[nt][r], cbase + c * EC + nt * 16 + lr);
      }
    }

    if (c + 2 < nchunks) lstore(c & 1);
    __syncthreads();
    if (c + 3 < nchunks) gload(c + 3);

    if constexpr (!PASS2) {
      if ((c & 3) == 3) {
        // Refresh the shared bound: max over the 16 lanes of each row.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float t = lv[r][L - 1];
          t = fmaxf(t, __shfl_xor(t, 1));
          t = fmaxf(t, __shfl_xor(t, 2));
          t = fmaxf(t, __shfl_xor(t, 4));
          t = fmaxf(t, __shfl_xor(t, 8));
          shared_thr[r] = t;
        }
      }
    } else {
      if (tid < EC) {
        const int e = cbase + c * EC + tid;
        if (e < n) {
          float s = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) s += red[c & 1][w][tid];
          p.partial[(int64_t)blockIdx.x * n + e] = s;
        }
      }
    }

#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[m][nt] = acc_next[m][nt];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bv[nt] = bv_next[nt];
#pragma unroll
      for (int r = 0; r < 4; ++r) ev[nt][r] = ev_next[nt][r];
    }
  }

  if constexpr (!PASS2 && !SCORES) {
    // Merge the 16 lanes that share each row.
#pragma unroll
    for (int s = 1; s < 16; s <<= 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float ov[L];
        int oi[L];
#pragma unroll
        for (int j = 0; j < L; ++j) {
          ov[j] = __shfl_xor(lv[r][j], s);
          oi[j] = __shfl_xor(li[r][j], s);
        }
#pragma unroll
        for (int j = 0; j < L; ++j) insert_any<L>(lv[r], li[r], ov[j], oi[j]);
      }
    }
    if constexpr (SMX) {
#pragma unroll
      for (int s = 1; s < 16; s <<= 1)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          es[r] = expsum_merge(es[r], ExpSum{__shfl_xor(es[r].m, s), __shfl_xor(es[r].s, s)});
    }
    if (lr == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (row_ok[r]) write_selection<L>(p, iorow[r], lv[r], li[r], es[r]);
    }
  }
}

// Workgroups of a launch: one per tile of `rows` batch rows, or for secondary
// gating one per possible work unit (those past the unit count exit at once).
inline dim3 gate_grid(const GateLaunch& g, int rows) {
  return dim3((unsigned)(g.units ? g.max_units : (g.tokens + rows - 1) / rows),
              (unsigned)(g.units ? 1 : g.ranges));
}

template <typename XS, typename CT, int D, int L>
hipError_t gate_dispatch_train(const GateLaunch& g, const GateParams& p, bool pass2, hipStream_t s) {
  const dim3 grid = gate_grid(g, kGateRows);
  if (p.scores) {
    if (g.train)
      hipLaunchKernelGGL((gate_kernel<XS, CT, D, 5, true, false, false, true>), grid,
                         dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL((gate_kernel<XS, CT, D, 5, false, false, false, true>), grid,
                         dim3(kThreads), 0, s, p);
  } else if (pass2) {
    hipLaunchKernelGGL((gate_kernel<XS, CT, D, L, true, true>), grid, dim3(kThreads), 0, s, p);
  } else if (g.gate_order) {
    if (g.train)
      hipLaunchKernelGGL((gate_kernel<XS, CT, D, L, true, false, true>), grid, dim3(kThreads), 0,
                         s, p);
    else
      hipLaunchKernelGGL((gate_kernel<XS, CT, D, L, false, false, true>), grid, dim3(kThreads), 0,
                         s, p);
  } else if (g.train) {
    hipLaunchKernelGGL((gate_kernel<XS, CT, D, L, true, false>), grid, dim3(kThreads), 0, s, p);
  } else {
    hipLaunchKernelGGL((gate_kernel<XS, CT, D, L, false, false>), grid, dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

template <typename XS, typename CT, int D>
hipError_t gate_dispatch_l(const GateLaunch& g, const GateParams& p, bool pass2, hipStream_t s) {
  if (g.k <= 4 || p.scores) return gate_dispatch_train<XS, CT, D, 5>(g, p, pass2, s);
  return gate_dispatch_train<XS, CT, D, 9>(g, p, pass2, s);
}

template <typename XS, typename CT>
hipError_t gate_dispatch_d(const GateLaunch& g, const GateParams& p, bool pass2, hipStream_t s) {
  switch (g.d) {
    case 64: return gate_dispatch_l<XS, CT, 64>(g, p, pass2, s);
    case 128: return gate_dispatch_l<XS, CT, 128>(g, p, pass2, s);
    case 256: return gate_dispatch_l<XS, CT, 256>(g, p, pass2, s);
    case 512: return gate_dispatch_l<XS, CT, 512>(g, p, pass2, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gate_detail

// The 32x32 kernel (gate32_impl.h) takes bf16 x and weights, d in {128, 256,
// 512}, and n a multiple of 16 in training mode or of 32 in inference (chunks
// of 32 experts' clean rows); it uses 256-row blocks instead of 128.
inline bool gate_uses_g32(const GateLaunch& g) {
  return g.x_dt == kBF16 && g.w_dt == kBF16 && (g.d == 128 || g.d == 256 || g.d == 512) &&
         g.n % (g.train ? 16 : 32) == 0;
}

hipError_t gate_dispatch_bf16(const GateLaunch& g, const gate_detail::GateParams& p, bool pass2, hipStream_t s);
hipError_t gate_dispatch_bf16x_f32w(const GateLaunch& g, const gate_detail::GateParams& p, bool pass2, hipStream_t s);
hipError_t gate_dispatch_f32(const GateLaunch& g, const gate_detail::GateParams& p, bool pass2, hipStream_t s);

}  // namespace moe
