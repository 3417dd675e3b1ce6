// Noisy top-k gating and the Load pass on 32x32x16 bf16 matrix-core tiles,
// for bf16 x and gate weights with d_model >= 128: training mode with n a
// multiple of 16, or the noise-free selection (inference) with n a multiple
// of 32, where a chunk is 32 experts' clean rows (template flag CL). Same mathematics
// as gate_impl.h (sections "Noisy top-k gating", eqs 3-5, and "A differentiable count of
// examples", eqs 8-10); different data movement:
//
//  * a workgroup owns 256 token rows, 32 per wave; each wave keeps its rows of
//    x in registers as the A operands of every K-block;
//  * experts are swept in chunks of 16; a chunk's B tile has 32 columns: the 16
//    clean-logit weight rows and the 16 noise weight rows of those experts. It
//    is copied HBM/L2 -> LDS with global_load_lds_dwordx4 (no staging
//    registers) into a double buffer, each 1 KB fragment in lane order;
//  * every fragment read from LDS feeds one 32x32x16 MFMA (32 flop per LDS byte);
//  * each pass computes the next chunk's matrix products while this chunk's
//    epilogue runs on the vector ALUs: pass 1 issues the products first, pass
//    2 weaves its per-pair work between them (measured faster for pass 2's
//    longer per-pair work; pass 1's epilogue reads LDS and branches).
//
// Epilogue. Both passes multiply weights (A operand, from LDS) by x (B
// operand, in registers), so in the 32x32 C layout lane l holds token l % 32 and rows
// 8 (j / 4) + 4 (l / 32) + j % 4 of the weight tile: registers j < 8 are the
// clean logits of experts 4 (l / 32) + (0..3) and 8 + 4 (l / 32) + (0..3) of
// the chunk, registers 8 + j the noise pre-activations of the same experts.
// Each lane forms H = clean + eps * (Softplus(u) + floor) for its token and 8
// experts and keeps the token's L best (H, expert) of the experts it sees (in
// increasing order, so it rarely needs to insert once its list is warm); lanes
// l and l ^ 32 (the two halves of a token's experts) merge at the end. The
// noise draws and biases ride a five-slot LDS ring four chunks ahead, copied
// by waves 4-7 while waves 0-3 copy the weights.
// Pass 2 evaluates P = Phi((clean - v_k) / sigma) for the same 8 (token,
// expert) pairs of each lane and sums every expert's column over the wave's
// 32 tokens with a transposing reduction across lanes (lane swaps and DPP
// moves, each step halving the values a lane holds), then over the block's
// waves, in a fixed order (the selected pairs are corrected to the (k+1)-th
// threshold separately).
// The gradient pass (BWD) runs pass 2's products and, per pair, the
// derivatives of its Load term P = Phi((clean - v_k) / sigma) times d loss /
// d Load_i: with phi the normal density and z = (clean - v_k) / sigma,
// d/d clean = phi(z) / sigma and d/d u = -phi(z) z / sigma Softplus'(u),
// Softplus' the logistic function. They go to global memory one chunk late
// (so that the stores have a whole chunk's work to complete before the
// chunk's barrier, which waits for every memory operation in flight); the
// selected pairs are rewritten separately.
#pragma once

#include "gate_impl.h"

namespace moe {
namespace gate_detail {

constexpr int kG32Waves = 8;
constexpr int kG32Threads = kG32Waves * 64;
constexpr int kG32Rows = kG32Waves * 32;
static_assert(kG32Rows == kGate32Rows, "rows per block of the 32x32 gate kernel");
constexpr int kG32Chunk = kGate32Chunk;

template <int V>
struct IntConst {
  static constexpr int value = V;
};

// Biases of a gate without one: every chunk copies these zeros (16, or 32 in
// the clean-only mode).
__device__ const float kZeroBias[2 * kG32Chunk] = {};

// Vector instructions of one Load-pass pair (Softplus, Phi) and of one noisy
// logit of the selection pass (Softplus, noise, bias): the scheduler spreads
// this many over the matrix products that precede it.
constexpr int kG32PhiValu = 30;
constexpr int kG32HValu = 12;

template <int D, int L, bool PASS2, bool SMX = false, bool SCORES = false, bool CL = false,
          bool BWD = false>
__global__ __launch_bounds__(kG32Threads) void gate32_kernel(GateParams p) {
  static_assert(!BWD || PASS2, "the gradient pass is a variant of the Load pass");
  RowTile tile;
  if (!resolve_tile<kG32Rows, bf16, D>(p, tile)) return;
  constexpr int UE = 8;          // bf16 per 16-byte unit
  constexpr int NKB = D / 16;    // 32x32x16 K-blocks
  static_assert(NKB % kG32Waves == 0, "each wave copies whole fragments");
  constexpr int DMA_PER_WAVE = NKB / kG32Waves;
  constexpr int EC = kG32Chunk;
  // CL (noise-free selection pass without gate bias): a chunk's 32 tile
  // columns are 32 experts' clean rows instead of 16 clean and 16 noise rows
  static_assert(!(CL && PASS2), "the Load pass needs the noise rows");
  constexpr int EX = CL ? 2 * EC : EC;  // experts per chunk

  // weight double buffer as two objects, so that the compiler can tell a read
  // of one from a copy in flight into the other
  __shared__ U16 wbuf0[NKB * 64];
  __shared__ U16 wbuf1[NKB * 64];
  // pass 1: noise draws of a chunk, [256 rows][16 experts] fp32, then one copy
  // of the chunk's 16 biases per wave; a ring of NE slots, NE - 1 chunks ahead
  constexpr int ESLOT = kG32Rows * kG32Chunk + kG32Waves * kG32Chunk;
  constexpr int NE = 5;
  __shared__ float ebuf[PASS2 || CL ? 1 : NE][PASS2 || CL ? 1 : ESLOT];
  __shared__ float thrbuf[PASS2 ? kG32Rows : 1];  // pass 2: each row's k-th logit
  // pass 2: each wave's copy of a chunk's 16 biases, double-buffered by chunk parity
  // (CL: the same for a chunk's 32 biases; BWD: the 16 biases, then the 16 d loss / d Load)
  constexpr int BW = BWD ? 2 * EX : EX;
  __shared__ __attribute__((aligned(16))) float bbuf[PASS2 || CL ? 2 : 1][PASS2 || CL ? kG32Waves * BW : 1];
  __shared__ float red[PASS2 && !BWD ? 2 : 1][kG32Waves][EC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar addressing
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bool clean_lane = l32 < 16;
  const int n = p.n;
  const int wrow0 = wave * 32;  // first local row of this wave
  const bf16* wg = reinterpret_cast<const bf16*>(p.wg);
  const bf16* wn = reinterpret_cast<const bf16*>(p.wn);

  // x rows of this wave as the B operands of the matrix products: lane
  // supplies row l32, unit 2 kb + hi.
  U16 xa[NKB];
  {
    const int64_t r = tile_xrow(p, tile, wrow0 + l32);
    const bf16* x = reinterpret_cast<const bf16*>(p.x);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      xa[kb] = (r >= 0) ? ld_unit(x + r * D + (kb * 2 + hi) * UE) : zero_unit();
  }

  // Rows past the tile's end compute finite garbage (zero x, the first row's
  // noise): pass 1 never writes them out, pass 2 gives them thresholds of
  // +inf, so their P is exactly 0. n is a multiple of 16, so every expert is
  // valid.
  if constexpr (PASS2) {
    for (int t = tid; t < kG32Rows; t += kG32Threads) {
      const int64_t row = tile_iorow(p, tile, t);
      thrbuf[t] = row >= 0 ? p.sel_thr[row * 2] : INFINITY;
    }
  }

  // Pass 1: lane (l32, hi) owns token l32 of the wave and experts 4 hi + (0..3)
  // and 8 + 4 hi + (0..3) of every chunk.
  float lv[L];
  int li[L];
#pragma unroll
  for (int j = 0; j < L; ++j) {
    lv[j] = -INFINITY;
    li[j] = 0x7FFFFFFF;
  }
  ExpSum es{-INFINITY, 0.f};  // SMX: this lane's part of the softmax over all n
  // SCORES: the batch row of this lane's token (-1 past the tile's end)
  const int64_t srow = SCORES ? tile_iorow(p, tile, wrow0 + l32) : -1;

  // Chunk c -> LDS buffer dst: lane l's 16 bytes are column l32 (clean row of
  // expert 16 c + l32, or the noise row of expert 16 c + l32 - 16), K unit
  // 2 kb + hi, a fixed per-lane source plus a chunk offset common to the
  // wave. Pass 2: wave w copies fragments kb = w + 8 i. Pass 1: waves 0-3 copy
  // all fragments (kb = w + 4 i) and waves 4-7 all noise draws, so that each
  // wave's in-order copy counter waits on one stream only: the weights must
  // land within a pass, the noise draws have NE - 2 more.
  // this workgroup's range of expert chunks (all of them unless split); the
  // copy sources below start at its first chunk, c counts from there
  const ChunkRange cr = chunk_range((n + EX - 1) / EX);
  const int nchunks = cr.count;
  const bf16* wlane =
      CL ? wg + ((int64_t)cr.c0 * EX + l32) * D + hi * UE
         : (clean_lane ? wg : wn) + ((int64_t)cr.c0 * EC + (l32 & 15)) * D + hi * UE;
  auto dma = [&](int c, U16* dst) {
    const bf16* src = wlane + (int64_t)c * EX * D;
    if constexpr (PASS2 || CL) {
#pragma unroll
      for (int i = 0; i < DMA_PER_WAVE; ++i) {
        const int kb = wave + kG32Waves * i;
        copy16_to_lds(src + kb * 2 * UE, &dst[kb * 64]);
      }
    } else if (wave < 4) {
#pragma unroll
      for (int i = 0; i < 2 * DMA_PER_WAVE; ++i) {
        const int kb = wave + 4 * i;
        copy16_to_lds(src + kb * 2 * UE, &dst[kb * 64]);
      }
    }
  };
  const bool has_bias = p.bias != nullptr;
  // chunk c's biases: bias_src + c * bias_step
  const int bias_step = has_bias ? EX : 0;
  const float* bias_src = has_bias ? p.bias + cr.c0 * bias_step : kZeroBias;
  // Pass 2: lanes 0-3 copy chunk c's 16 biases into this wave's slot. A
  // copy, not a register load, so
  // that no compiler-inserted wait on the memory counter stalls the epilogue
  // behind the weight copies in flight.
  auto dma_bias = [&](int c, int slot) {
    if constexpr (BWD) {
      // lanes 0-3 the biases, lanes 4-7 d loss / d Load of the chunk's experts
      if (lane < 2 * EX / 4)
        copy16_to_lds(lane < EX / 4 ? bias_src + c * bias_step + 4 * lane
                                    : p.dload + (int64_t)(cr.c0 + c) * EX + 4 * (lane - EX / 4),
                      &bbuf[slot][wave * BW]);
    } else {
      if (lane < EX / 4) copy16_to_lds(bias_src + c * bias_step + 4 * lane, &bbuf[slot][wave * EX]);
    }
  };
  // One chunk's products: 32 x 32 tile of (rows, clean|noise columns) over
  // the K-blocks. Fragments are read four ahead of their matrix product; the
  // base address is kept in a register so each read's offset within the
  // buffer fits the instruction's immediate field.
  constexpr int FPF = NKB < 4 ? NKB : 4;
  auto mfma_chunk = [&](const U16* src, f32x16& acc) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef const __attribute__((address_space(3))) u32x4* LdsPtr;
    uint32_t base = (uint32_t)(uintptr_t)(src + lane);
    asm("" : "+v"(base));
    const LdsPtr bl = (LdsPtr)base;
    u32x4 f[FPF];
#pragma unroll
    for (int j = 0; j < FPF; ++j) f[j] = bl[j * 64];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      U16 cur;
      __builtin_memcpy(&cur, &f[kb % FPF], 16);
      if (kb + FPF < NKB) f[kb % FPF] = bl[(kb + FPF) * 64];
      Mfma<bf16>::k32(acc, cur, xa[kb]);  // rows: weights, columns: tokens
    }
    // Keep that order (the scheduler would otherwise pull the reads down next
    // to their use): FPF reads, then matrix product / read pairs, then the
    // last FPF products.
    __builtin_amdgcn_sched_group_barrier(0x100, FPF, 0);
#pragma unroll
    for (int kb = 0; kb + FPF < NKB; ++kb) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, FPF, 0);
  };
  // Noise draws of chunk c -> ring slot b (pass 1, waves 4-7): wave 4 + v
  // copies local rows 64 v + 16 i + (l / 4), so the slot holds the block's
  // [256][16] tile with each row's four 16-byte groups swizzled: group g of
  // row R sits at position g ^ ((R / 2) % 4), so that the reads of eight
  // consecutive rows' group fall in distinct banks. This kernel runs only when
  // n is a multiple of 16, so every 16-byte group is aligned and inside its
  // row; rows past the tile's end read the tile's first row and are masked in
  // the epilogue.
  const int ev = wave & 3;
  const float* elane[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t r = tile_iorow(p, tile, 64 * ev + 16 * i + (lane >> 2));
    if (r < 0) r = tile_iorow(p, tile, 0);
    elane[i] = p.eps + r * n + cr.c0 * EC + 4 * ((lane & 3) ^ ((lane >> 3) & 3));
  }
  constexpr int EPS_COPIES = 5;  // per wave and chunk: 4 row groups, 1 bias copy
  auto dma_eps = [&](int c, int b) {
    if (!CL && wave >= 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* src = elane[i] + c * EC;
        copy16_to_lds(src, &ebuf[b][(64 * ev + 16 * i) * EC]);
      }
      // lanes 0-7 copy the chunk's biases into the slots of waves 2 v and 2 v + 1
      if (lane < 8)
        copy16_to_lds(bias_src + c * bias_step + 4 * (lane & 3),
                      &ebuf[b][kG32Rows * EC + 2 * ev * EC]);
    }
  };

  // Pass 1: insert the lane's 8 values of chunk `chunk` (experts in
  // increasing order) into its token's list. Once the lists are warm (from
  // the range's fifth chunk on), each lane marks the values that beat its
  // list's last entry and inserts them lowest first, one per trip of a loop
  // that the wave runs as often as its busiest lane needs (once or twice),
  // the value picked by a select tree on the bits of its position; a marked
  // value that an earlier insertion has since outranked is dropped by
  // insert_new's own test, so the list is the one that inserting all values
  // in order gives. In the first chunks nearly every value is a candidate,
  // and inserting each value in turn (a branch the wave takes when any lane
  // needs it) is cheaper than a trip per value.
  auto insert_pairs = [&](const auto& hv, int chunk, auto warm) {
    constexpr int NV = CL ? 16 : 8;
    if constexpr (!decltype(warm)::value) {
#pragma unroll
      for (int i = 0; i < NV; ++i)
        insert_new<L>(lv, li, hv[i], (cr.c0 + chunk) * EX + 8 * (i / 4) + 4 * hi + (i % 4));
      return;
    }
    uint32_t marks = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) marks |= (hv[i] > lv[L - 1] ? 1u : 0u) << i;
    while (marks) {
      const int j = __builtin_ctz(marks);
      marks &= marks - 1;
      float t[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) t[i] = hv[i];
#pragma unroll
      for (int w = NV / 2, b = 1; w >= 1; w /= 2, b *= 2) {
#pragma unroll
        for (int i = 0; i < w; ++i) t[i] = (j & b) ? t[2 * i + 1] : t[2 * i];
      }
      insert_new<L>(lv, li, t[0], (cr.c0 + chunk) * EX + 8 * (j >> 2) + 4 * hi + (j & 3));
    }
  };

  // Accumulators of two consecutive chunks: pass P reads accs[P] (its own
  // chunk's products) and fills accs[P ^ 1] (the next chunk's); the same for
  // pass 2's bias slots.
  f32x16 accs[2];
  // BWD: the last chunk's gradients of this lane's 8 pairs, written one chunk
  // late (dc then du); the lane's batch row (-1 past the tile's end)
  float gdc[BWD ? 8 : 1], gdu[BWD ? 8 : 1];
  const int64_t grow = BWD ? tile_iorow(p, tile, wrow0 + l32) : -1;
  auto store_grads = [&](int c) __attribute__((always_inline)) {
    if constexpr (BWD) {
      if (grow >= 0) {
        // the chunk's block: row grow's 16 clean-logit gradients, then its 16
        // noise ones; a wave's four stores fill 32 consecutive 128-byte rows
        float* dst = p.dcu + ((int64_t)(cr.c0 + c) * p.B + grow) * 32 + 4 * hi;
        *reinterpret_cast<f32x4*>(dst) = f32x4{gdc[0], gdc[1], gdc[2], gdc[3]};
        *reinterpret_cast<f32x4*>(dst + 8) = f32x4{gdc[4], gdc[5], gdc[6], gdc[7]};
        *reinterpret_cast<f32x4*>(dst + 16) = f32x4{gdu[0], gdu[1], gdu[2], gdu[3]};
        *reinterpret_cast<f32x4*>(dst + 24) = f32x4{gdu[4], gdu[5], gdu[6], gdu[7]};
      }
    }
  };
  dma(0, wbuf0);
  if (nchunks > 1) dma(1, wbuf1);
  if constexpr (!PASS2 && !CL) {
    for (int c = 0; c < NE - 1 && c < nchunks; ++c) dma_eps(c, c);
  }
  if constexpr (PASS2 || CL) dma_bias(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  mfma_chunk(wbuf0, accs[0]);
  __syncthreads();  // every wave has read chunk 0 before buffer 0 is refilled

  // Pass 2 evaluates every pair against its row's k-th largest logit (+inf
  // for rows past the tile's end, so their P is 0); the selected pairs'
  // difference (threshold (k+1)-th) is added by a separate kernel.
  float thrk = 0.f;
  if constexpr (PASS2) thrk = thrbuf[wave * 32 + l32];
  const bool thr_fin = !isinf(thrk);

  // One pass per chunk; P = c & 1 is a compile-time constant (the loop below
  // is unrolled by two) so each pass names its buffers statically.
  auto chunk_pass = [&](const int c, auto parity, auto warm) {
    constexpr int P = decltype(parity)::value;
    U16* const wfill = P ? wbuf1 : wbuf0;       // buffer c & 1: chunk c + 2 goes here
    const U16* const wnext = P ? wbuf0 : wbuf1;  // buffer (c + 1) & 1: chunk c + 1
    f32x16& acc = accs[P];
    // Copies issued this pass: (pass 2) chunk c + 1's biases into bias slot
    // P ^ 1, chunk c + 2's weights into buffer c & 1 (whose chunk c every wave
    // used before the last barrier), and (pass 1) chunk c + NE - 1's noise
    // draws and biases into ring slot (c + NE - 1) % NE (chunk c - 1's, used
    // in the last pass). The weights must land by the end of this pass; the
    // noise draws of chunk c + 1 too, those of later chunks may stay in flight.
    if constexpr (PASS2 || CL) {
      if (c + 1 < nchunks) dma_bias(c + 1, P ^ 1);
    }
    if (c + 2 < nchunks) dma(c + 2, wfill);
    asm volatile("" ::: "memory");
    if constexpr (BWD) {
      if (c > 0) store_grads(c - 1);
    }
    if constexpr (!PASS2 && !CL) {
      if (c + NE - 1 < nchunks) dma_eps(c + NE - 1, (c + NE - 1) % NE);
    }

    if constexpr (PASS2) {
      // Load pass: the next chunk's products with this chunk's pairs woven
      // in, one pair after every eighth of the products, so that each pair's
      // vector work issues while the matrix core is busy.
      // This lane's 8 biases and the first reads ahead are issued before the
      // woven region below: the scheduler keeps the weave's pattern only
      // when that region starts with the products and reads of K-blocks.
      const float* br = &bbuf[P][wave * BW + 4 * hi];
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(br);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(br + 8);
      f32x4 dl0{}, dl1{};
      if constexpr (BWD) {
        dl0 = *reinterpret_cast<const f32x4*>(br + EC);
        dl1 = *reinterpret_cast<const f32x4*>(br + EC + 8);
      }
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      typedef const __attribute__((address_space(3))) u32x4* LdsPtr;
      uint32_t base = (uint32_t)(uintptr_t)(wnext + lane);
      asm("" : "+v"(base));
      const LdsPtr bl = (LdsPtr)base;
      u32x4 f[FPF];
#pragma unroll
      for (int j = 0; j < FPF; ++j) f[j] = bl[j * 64];
      __builtin_amdgcn_sched_barrier(0);
      f32x16& an = accs[P ^ 1];
#pragma unroll
      for (int j = 0; j < 16; ++j) an[j] = 0.f;
      constexpr int MPE = NKB / 8;
      static_assert(NKB % 8 == 0, "whole K-blocks per pair");
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < MPE; ++j) {
          const int kb = i * MPE + j;
          U16 cur;
          __builtin_memcpy(&cur, &f[kb % FPF], 16);
          if (kb + FPF < NKB) f[kb % FPF] = bl[(kb + FPF) * 64];
          Mfma<bf16>::k32(an, cur, xa[kb]);
        }
        // pairs in the order 0, 4, 1, 5, ...: the reduction's first step
        // pairs values i and i + 4, so it can start inside the weave
        const int e = (i >> 1) + 4 * (i & 1);
        const float clean = acc[e] + (e < 4 ? b0[e] : b1[e - 4]);
        if constexpr (BWD) {
          const float u = acc[8 + e];
          const float t = exp_native(-fabsf(u));
          const float sigma = fmaf(u + fabsf(u), 0.5f, log1p_small(t)) + p.floor;
          const float rs = rcp_f(sigma);
          const float z = (clean - thrk) * rs;
          const float dl = e < 4 ? dl0[e] : dl1[e - 4];
          // d loss / d clean = dl phi(z) / sigma; no threshold: no Load term
          const float a = thr_fin ? dl * exp_native(-0.5f * z * z) * 0.3989422804014327f * rs : 0.f;
          gdc[e] = a;
          gdu[e] = thr_fin ? -a * z * (u >= 0.f ? 1.f : t) * rcp_f(1.f + t) : 0.f;
        } else {
          const float sigma = softplus_f(acc[8 + e]) + p.floor;
          pv[e] = phi_f((clean - thrk) * rcp_f(sigma));
        }
      }
      // reads ahead, then (product, read, vector work) triples
      constexpr int V = (kG32PhiValu + MPE - 1) / MPE;
      __builtin_amdgcn_sched_group_barrier(0x100, FPF, 0);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (kb + FPF < NKB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!BWD) {
      // Column sums over the wave's 32 tokens (lanes of equal hi). Lane l
      // holds value j for expert 8 (j / 4) + 4 hi + j % 4. Each step pairs
      // lanes that hold the same values, keeps half of them and adds the
      // partner's copy of that half: lanes l, l ^ 16 (v_permlane16_swap
      // exchanges the upper row's j with the lower row's j + 4), then l, l ^ 8
      // (DPP row rotation by 8), then the lanes mirrored within each 8-lane
      // half-row (which differ in bit 2), then the quad. Afterwards lane l
      // holds the total of value j = (l / 4) % 8 for its half.
      float s4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(pv[i]),
                                                          __float_as_uint(pv[i + 4]), false, false);
        s4[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      const bool b3 = (lane & 8) != 0, b2 = (lane & 4) != 0;
      float s2[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float keep = b3 ? s4[i + 2] : s4[i];
        const float send = b3 ? s4[i] : s4[i + 2];
        s2[i] = keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), 0x128, 0xF, 0xF, true));
      }
      float s1;
      {
        const float keep = b2 ? s2[1] : s2[0];
        const float send = b2 ? s2[0] : s2[1];
        s1 = keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), 0x141, 0xF, 0xF, true));
      }
      s1 += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s1), 0xB1, 0xF, 0xF, true));
      s1 += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s1), 0x4E, 0xF, 0xF, true));
      if ((lane & 3) == 0) {
        const int j = (lane >> 2) & 7;
        red[P][wave][8 * (j >> 2) + 4 * hi + (j & 3)] = s1;
      }
      }
    } else {
      // Selection pass: this chunk's noise draws and biases are read first,
      // then the next chunk's products with this chunk's noisy logits woven
      // in (one after every eighth of the products); the insertions, which
      // branch, follow the products.
      f32x4 e0{}, e1{}, b0{}, b1{}, b2{}, b3{};
      if constexpr (CL) {
        // this lane's 16 biases: experts 4 hi + (0..3) of each group of 8
        const float* br = &bbuf[P][wave * EX + 4 * hi];
        b0 = *reinterpret_cast<const f32x4*>(br);
        b1 = *reinterpret_cast<const f32x4*>(br + 8);
        b2 = *reinterpret_cast<const f32x4*>(br + 16);
        b3 = *reinterpret_cast<const f32x4*>(br + 24);
      } else {
        const float* er = &ebuf[c % NE][(wave * 32 + l32) * EC];
        const int sw = (l32 >> 1) & 3;  // the row's group swizzle
        e0 = *reinterpret_cast<const f32x4*>(er + 4 * (hi ^ sw));
        e1 = *reinterpret_cast<const f32x4*>(er + 4 * ((2 + hi) ^ sw));
        const float* bp = &ebuf[c % NE][kG32Rows * EC + wave * EC + 4 * hi];
        b0 = *reinterpret_cast<const f32x4*>(bp);
        b1 = *reinterpret_cast<const f32x4*>(bp + 8);
      }
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      typedef const __attribute__((address_space(3))) u32x4* LdsPtr;
      uint32_t base = (uint32_t)(uintptr_t)(wnext + lane);
      asm("" : "+v"(base));
      const LdsPtr bl = (LdsPtr)base;
      u32x4 f[FPF];
#pragma unroll
      for (int j = 0; j < FPF; ++j) f[j] = bl[j * 64];
      __builtin_amdgcn_sched_barrier(0);
      f32x16& an = accs[P ^ 1];
#pragma unroll
      for (int j = 0; j < 16; ++j) an[j] = 0.f;
      constexpr int MPE = NKB / 8;
      static_assert(NKB % 8 == 0, "whole K-blocks per noisy logit");
      float hv[CL ? 16 : 8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < MPE; ++j) {
          const int kb = i * MPE + j;
          U16 cur;
          __builtin_memcpy(&cur, &f[kb % FPF], 16);
          if (kb + FPF < NKB) f[kb % FPF] = bl[(kb + FPF) * 64];
          Mfma<bf16>::k32(an, cur, xa[kb]);
        }
        if constexpr (!CL) {
          const float eps = i < 4 ? e0[i] : e1[i - 4];
          const float bias = i < 4 ? b0[i] : b1[i - 4];
          hv[i] = fmaf(eps, softplus_f(acc[8 + i]) + p.floor, acc[i] + bias);
        }
      }
      if constexpr (CL) {
        // noise-free: H is the clean logit plus the bias
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const f32x4& bq = i < 4 ? b0 : (i < 8 ? b1 : (i < 12 ? b2 : b3));
          hv[i] = acc[i] + bq[i % 4];
        }
        __builtin_amdgcn_sched_group_barrier(0x100, FPF, 0);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (kb + FPF < NKB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      } else {
        constexpr int V = (kG32HValu + MPE - 1) / MPE;
        __builtin_amdgcn_sched_group_barrier(0x100, FPF, 0);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (kb + FPF < NKB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (SCORES) {
        // batchwise gating: the 8 scores to their experts' rows; the 32 lanes
        // of each half write 128 contiguous bytes per expert
        if (srow >= 0) {
          float* dst = p.scores + (int64_t)((cr.c0 + c) * EX + 4 * hi) * p.sld + srow;
#pragma unroll
          for (int i = 0; i < (CL ? 16 : 8); ++i)
            dst[(int64_t)(8 * (i / 4) + (i % 4)) * p.sld] = hv[i];
        }
      } else {
        if constexpr (SMX) es = expsum_add(es, hv);
        insert_pairs(hv, c, warm);
      }
    }

    // Block barrier without a release fence (which would wait for every copy
    // in flight): each wave first waits for its LDS traffic and for its
    // copies; in pass 1 the noise waves leave the copies of chunks c + 2 ..
    // c + NE - 1 in flight (copies complete in issue order, so the count
    // covers everything older).
    static_assert(NE == 5, "the waits below count NE - 2 chunks of noise copies");
    if (!PASS2 && !CL && wave >= 4 && c + 4 < nchunks) {
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(3 * EPS_COPIES) : "memory");
    } else if (!PASS2 && !CL && wave >= 4 && c + 3 < nchunks) {
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * EPS_COPIES) : "memory");
    } else if (!PASS2 && !CL && wave >= 4 && c + 2 < nchunks) {
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(EPS_COPIES) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }

    if constexpr (PASS2 && !BWD) {
      if (tid < EC) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kG32Waves; ++w) s += red[P][w][tid];
        p.partial[(int64_t)blockIdx.x * n + (cr.c0 + c) * EC + tid] = s;
      }
    }
  };
  // the first kCold chunks of the range with the cold-list insertion (pass 1
  // only; the other passes compile the same loop once)
  constexpr int kCold = (PASS2 || SCORES) ? 0 : 4;
  const int ncold = nchunks < kCold ? nchunks : kCold;
  int c = 0;
  for (; c < ncold; c += 2) {
    chunk_pass(c, IntConst<0>{}, IntConst<0>{});
    if (c + 1 < nchunks) chunk_pass(c + 1, IntConst<1>{}, IntConst<0>{});
  }
  for (; c < nchunks; c += 2) {
    chunk_pass(c, IntConst<0>{}, IntConst<1>{});
    if (c + 1 < nchunks) chunk_pass(c + 1, IntConst<1>{}, IntConst<1>{});
  }
  if constexpr (BWD) {
    if (nchunks > 0) store_grads(nchunks - 1);
  }
  if constexpr (!PASS2 && !SCORES) {
    // The two halves of a token's experts (lanes l and l ^ 32) merge, then
    // lanes 0-31 write.
    float ov[L];
    int oi[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
      ov[j] = __shfl_xor(lv[j], 32);
      oi[j] = __shfl_xor(li[j], 32);
    }
#pragma unroll
    for (int j = 0; j < L; ++j) insert_any<L>(lv, li, ov[j], oi[j]);
    if constexpr (SMX) es = expsum_merge(es, ExpSum{__shfl_xor(es.m, 32), __shfl_xor(es.s, 32)});
    const int64_t row = tile_iorow(p, tile, wrow0 + l32);
    if (hi == 0 && row >= 0) write_selection<L>(p, row, lv, li, es);
  }
}

}  // namespace gate_detail
}  // namespace moe
