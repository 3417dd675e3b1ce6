// Noisy top-k gating and the Load pass on 32x32x16 bf16 matrix-core tiles,
// for bf16 x and gate weights with d_model >= 128 in training mode (the
// configuration of the large workloads). Same mathematics as gate_impl.h
// (sections "Noisy top-k gating", eqs 3-5, and "A differentiable count of
// examples", eqs 8-10); different data movement:
//
//  * a workgroup owns 256 token rows, 32 per wave; each wave keeps its rows of
//    x in registers as the A operands of every K-block;
//  * experts are swept in chunks of 16; a chunk's B tile has 32 columns: the 16
//    clean-logit weight rows and the 16 noise weight rows of those experts. It
//    is copied HBM/L2 -> LDS with global_load_lds_dwordx4 (no staging
//    registers) into a double buffer, each 1 KB fragment in lane order;
//  * every fragment read from LDS feeds one 32x32x16 MFMA (32 flop per LDS byte);
//  * the two waves that share a SIMD run each chunk's halves (next chunk's
//    products, this chunk's epilogue) in opposite order so the matrix cores
//    and the vector ALUs overlap.
//
// Epilogue. In the 32x32 C layout lane l holds column l % 32 for 16 rows: the
// clean logit (columns 0-15) or the noise pre-activation (16-31) of one expert.
// Lanes l and l ^ 16 swap half of their rows so each holds (clean, noise) pairs
// for 8 rows of one expert. Pass 1 forms H = clean + eps * (Softplus(u) +
// floor), transposes it through LDS and lets each lane own one row's half of
// the chunk: a lane sees every 8th-block of its row's experts in increasing
// order, keeps the row's L best (H, expert), and rarely needs to insert once
// its list is warm. Lanes l and l ^ 32 (the two halves of a row) merge at the
// end. Pass 2 evaluates P = Phi((clean - thr) / sigma) in place and sums each
// expert's column over the block's rows in a fixed order.
#pragma once

#include "gate_impl.h"

namespace moe {
namespace gate_detail {

constexpr int kG32Waves = 8;
constexpr int kG32Threads = kG32Waves * 64;
constexpr int kG32Rows = kG32Waves * 32;
constexpr int kG32Chunk = 16;
constexpr int kG32HStride = 20;  // padded row stride (floats) of the transpose tile

template <int D, int L, bool PASS2>
__global__ __launch_bounds__(kG32Threads) void gate32_kernel(GateParams p) {
  constexpr int UE = 8;          // bf16 per 16-byte unit
  constexpr int NKB = D / 16;    // 32x32x16 K-blocks
  static_assert(NKB % kG32Waves == 0, "each wave copies whole fragments");
  constexpr int DMA_PER_WAVE = NKB / kG32Waves;
  constexpr int EC = kG32Chunk;

  __shared__ U16 wbuf[2][NKB * 64];
  __shared__ float hbuf[PASS2 ? 1 : kG32Waves][32 * kG32HStride];
  __shared__ int selbuf[PASS2 ? kG32Rows : 1][L - 1];
  __shared__ float thrbuf[PASS2 ? kG32Rows : 1][2];
  __shared__ float red[PASS2 ? 2 : 1][kG32Waves][EC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bool clean_lane = l32 < 16;
  const int64_t B = p.B;
  const int n = p.n;
  const int64_t blk_row0 = (int64_t)blockIdx.x * kG32Rows;
  const int64_t row0 = blk_row0 + wave * 32;
  const bf16* wg = reinterpret_cast<const bf16*>(p.wg);
  const bf16* wn = reinterpret_cast<const bf16*>(p.wn);

  // x rows of this wave as A operands: lane supplies row l32, unit 2 kb + hi.
  U16 xa[NKB];
  {
    const int64_t r = row0 + l32;
    const bf16* x = reinterpret_cast<const bf16*>(p.x);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      xa[kb] = (r < B) ? ld_unit(x + r * D + (kb * 2 + hi) * UE) : zero_unit();
  }

  // Rows of this lane's (clean, noise) pairs after the exchange: element i is
  // C-layout register j = i (clean lanes) or 8 + i (noise lanes).
  int rr[8];
  bool row_ok[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    rr[i] = (clean_lane ? 0 : 16) + 8 * (i / 4) + 4 * hi + (i % 4);
    row_ok[i] = row0 + rr[i] < B;
  }

  if constexpr (PASS2) {
    for (int t = tid; t < kG32Rows; t += kG32Threads) {
      const int64_t row = blk_row0 + t;
      const bool ok = row < B;
#pragma unroll
      for (int j = 0; j < L - 1; ++j) selbuf[t][j] = (ok && j < p.k) ? p.sel_idx[row * p.k + j] : -1;
      thrbuf[t][0] = ok ? p.sel_thr[row * 2] : 0.f;
      thrbuf[t][1] = ok ? p.sel_thr[row * 2 + 1] : 0.f;
    }
  }

  // Row-owner state (pass 1): lane owns row l32 of the wave, half hi of each chunk.
  float lv[L];
  int li[L];
#pragma unroll
  for (int j = 0; j < L; ++j) {
    lv[j] = -INFINITY;
    li[j] = 0x7FFFFFFF;
  }

  // Chunk c -> LDS buffer b. Wave w copies fragments kb = w + 8 i; lane l's
  // 16 bytes are B column l32 (clean row of expert 16 c + l32, or the noise row
  // of expert 16 c + l32 - 16), K unit 2 kb + hi. Experts past n read row n - 1
  // and are masked in the epilogue.
  auto dma = [&](int c, int b) {
    const int e = min(c * EC + (l32 & 15), n - 1);
    const bf16* w = clean_lane ? wg : wn;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      const int kb = wave + kG32Waves * i;
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(w + (int64_t)e * D + (kb * 2 + hi) * UE),
          (__attribute__((address_space(3))) void*)(&wbuf[b][kb * 64]), 16, 0, 0);
    }
  };
  auto mfma_chunk = [&](int b, f32x16& acc) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) Mfma<bf16>::k32(acc, xa[kb], wbuf[b][kb * 64 + lane]);
  };
  const bool has_bias = p.bias != nullptr;
  const float* bias_src = has_bias ? p.bias : reinterpret_cast<const float*>(p.wg);
  auto load_chunk_inputs = [&](int c, float (&ev)[8], float& bv) {
    const int e = min(c * EC + (l32 & 15), n - 1);
    bv = bias_src[e];
    if constexpr (!PASS2) {
#pragma unroll
      for (int i = 0; i < 8; ++i) ev[i] = p.eps[min(row0 + rr[i], B - 1) * n + e];
    }
  };

  const int nchunks = (n + EC - 1) / EC;
  f32x16 acc, acc_next;
  float ev[8], ev_next[8], bv, bv_next;
  dma(0, 0);
  if (nchunks > 1) dma(1, 1);
  load_chunk_inputs(0, ev, bv);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  mfma_chunk(0, acc);
  __syncthreads();  // every wave has read chunk 0 before buffer 0 is refilled

  for (int c = 0; c < nchunks; ++c) {
    // Buffer c & 1 held chunk c, whose products every wave formed before the
    // last barrier; refill it with chunk c + 2 (ready by the end of this pass).
    if (c + 2 < nchunks) dma(c + 2, c & 1);

    float colsum = 0.f;
    float hpair[8];
    auto products = [&]() {
      load_chunk_inputs(c + 1 < nchunks ? c + 1 : c, ev_next, bv_next);
      mfma_chunk((c + 1) & 1, acc_next);
    };
    auto epilogue = [&]() {
      // exchange: clean lanes send clean rows j = 8..15, noise lanes send noise rows j = 0..7
      float recv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) recv[i] = __shfl_xor(clean_lane ? acc[8 + i] : acc[i], 16);
      const int e = c * EC + (l32 & 15);
      const bool e_ok = e < n;
      const float bias = has_bias ? bv : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float clean = (clean_lane ? acc[i] : recv[i]) + bias;
        const float u = clean_lane ? recv[i] : acc[8 + i];
        const bool ok = e_ok && row_ok[i];
        if constexpr (!PASS2) {
          const float H = fmaf(ev[i], softplus_f(u) + p.floor, clean);
          hpair[i] = ok ? H : -INFINITY;
        } else {
          const float sigma = softplus_f(u) + p.floor;
          const int row = wave * 32 + rr[i];
          bool member = false;
#pragma unroll
          for (int j = 0; j < L - 1; ++j) member |= (selbuf[row][j] == e);
          const float thr = member ? thrbuf[row][1] : thrbuf[row][0];
          const float P = phi_f((clean - thr) * rcp_f(sigma));
          colsum += ok ? P : 0.f;
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

    if constexpr (!PASS2) {
      // Transpose H through this wave's LDS tile, then each lane scans its row.
      float* hb = hbuf[wave];
      const int ecol = l32 & 15;
#pragma unroll
      for (int i = 0; i < 8; ++i) hb[rr[i] * kG32HStride + ecol] = hpair[i];
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      const float4 h0 = *reinterpret_cast<const float4*>(&hb[l32 * kG32HStride + hi * 8]);
      const float4 h1 = *reinterpret_cast<const float4*>(&hb[l32 * kG32HStride + hi * 8 + 4]);
      const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
      bool cand = false;
#pragma unroll
      for (int i = 0; i < 8; ++i) cand |= hv[i] > lv[L - 1];
      if (__any(cand)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) insert_new<L>(lv, li, hv[i], c * EC + hi * 8 + i);
      }
      __builtin_amdgcn_wave_barrier();
    } else {
      // column sums: lanes l, l ^ 16 (same expert, other rows) and l ^ 32
      colsum += __shfl_xor(colsum, 16);
      colsum += __shfl_xor(colsum, 32);
      if (lane < 16) red[c & 1][wave][lane] = colsum;
    }

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    if constexpr (PASS2) {
      if (tid < EC) {
        const int e = c * EC + tid;
        if (e < n) {
          float s = 0.f;
#pragma unroll
          for (int w = 0; w < kG32Waves; ++w) s += red[c & 1][w][tid];
          p.partial[(int64_t)blockIdx.x * n + e] = s;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = acc_next[j];
    bv = bv_next;
#pragma unroll
    for (int i = 0; i < 8; ++i) ev[i] = ev_next[i];
  }

  if constexpr (!PASS2) {
    // The two halves of a row (lanes l and l ^ 32) merge, then lanes 0-31 write.
    float ov[L];
    int oi[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
      ov[j] = __shfl_xor(lv[j], 32);
      oi[j] = __shfl_xor(li[j], 32);
    }
#pragma unroll
    for (int j = 0; j < L; ++j) insert_any<L>(lv, li, ov[j], oi[j]);
    const int64_t row = row0 + l32;
    if (hi == 0 && row < B) {
      const int k = p.k;
      const float top = lv[0];
      float ex[L - 1];
      float z = 0.f;
#pragma unroll
      for (int j = 0; j < L - 1; ++j) {
        ex[j] = (j < k) ? expf(lv[j] - top) : 0.f;
        z += ex[j];
      }
      const float inv = 1.0f / z;
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
  }
}

}  // namespace gate_detail
}  // namespace moe
