// Expert FFNs on their routed rows (section "How a mixture-of-experts layer
// works": each expert is input layer -> ReLU hidden layer -> output layer, and
// is evaluated only on the inputs whose gate is nonzero) as a grouped matrix
// product over the contiguous per-expert segments that routing produced.
//
// Work unit: (expert e, up to BM consecutive rows of its segment). A small
// planning kernel lists these units from the segment offsets; one workgroup
// takes one unit:
//   * gather its BM rows of x into LDS (16-byte units, XOR-swizzled by row so
//     the matrix-core operand reads are conflict-free);
//   * for each chunk of HC hidden units:
//       GEMM1  Hc^T = W1[chunk] . X^T   W1 rows stream from HBM straight into
//                                      the A operands (16 contiguous bytes per
//                                      lane), X^T comes from LDS;
//       bias + ReLU, round to the storage type, stage Hc in LDS;
//       GEMM2  Out += Hc . W2[:, chunk]^T  W2 rows stream from HBM into the B
//                                         operands (64 contiguous bytes per lane
//                                         per load); Out stays in registers;
//   * add b2 and write the rows to expert_out in segment order.
// Every expert weight is read from HBM once per work unit; with ~64 rows per
// expert (4096 experts, k = 4, 65536 tokens) the kernel is bound by streaming
// the expert weights, the shrinking-batch regime of "Keeping each expert's
// batch large".
#include <algorithm>

#include "device_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

template <typename T, int D>
struct FfnShape {
  static constexpr int NW = D / 64 < 2 ? 2 : (D / 64 > 8 ? 8 : D / 64);  // waves
  static constexpr int HC = 16 * NW;                     // hidden units per chunk
  // rows per work unit: 96 for bf16, so that an expert with up to 96 rows streams its
  // weights once; fp32 keeps its x tile within 64 KB of LDS
  static constexpr int BM = sizeof(T) == 2 ? 96 : (D >= 512 ? 32 : 64);
  static constexpr int T16 = BM / 16;                    // 16-row token tiles (GEMM1)
  static constexpr int CT2 = D / 16 / NW;                // 16-col output tiles per wave
  static constexpr int UE = Elem<T>::kPerUnit;
  static constexpr int XU = D / UE;                      // 16-byte units per x row
  static constexpr int HU = HC / UE;                     // units per hidden-chunk row
  static constexpr int XSW = XU >= 16 ? 16 : XU;
  static constexpr int HSW = HU >= 16 ? 16 : HU;
  static_assert(CT2 >= 1, "output tiles per wave");
  static_assert(HU >= 2, "hidden chunk of at least two units");
};

struct FfnParams {
  const void* x;
  const int32_t* offsets;
  const int32_t* perm_token;
  const void* w1;
  const void* b1;
  const void* w2;
  const void* b2;
  void* out;
  const int32_t* blocks;  // [0] = count; from [4] on, 16 bytes per unit (FfnUnit)
  int h;
  // split over the hidden units: unit u writes its fp32 partial output rows
  // (no b2) to part + u * part_rows * D; null when units are whole
  float* part;
  int part_rows;
};

// Global-memory byte pointer: loads through it are global (not flat) loads
// even after the pointer has passed through an asm statement.
typedef const __attribute__((address_space(1))) char* GPtr;
__device__ __forceinline__ GPtr gptr(const void* p) { return (GPtr)(p); }
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ U16 ld_unit_g(GPtr p) {
  const u32x4 v = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(p);
  U16 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}
__device__ __forceinline__ U16 ld_unit_g_stream(GPtr p) {
  const u32x4 v =
      __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(p));
  U16 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

template <typename T>
__device__ __forceinline__ float load_scalar(const void* p, int64_t i) {
  if constexpr (sizeof(T) == 2) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  } else {
    return reinterpret_cast<const float*>(p)[i];
  }
}

template <typename T>
__device__ __forceinline__ void store_scalar(void* p, int64_t i, float v) {
  if constexpr (sizeof(T) == 2) {
    reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16_bits(v);
  } else {
    reinterpret_cast<float*>(p)[i] = v;
  }
}

// DPP quad permutation (lanes 4m..4m+3 exchange values): xor 1 and xor 2.
__device__ __forceinline__ float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// 4x4 transpose within each quad of lanes: lane c of the quad holds x[j] =
// M[c][j] before and M[j][c] after.
__device__ __forceinline__ void quad_transpose(f32x4& x, int c) {
  const bool odd = c & 1, hi = c & 2;
  const float r0 = quad_xor1(odd ? x[0] : x[1]);
  const float r2 = quad_xor1(odd ? x[2] : x[3]);
  if (odd) {
    x[0] = r0;
    x[2] = r2;
  } else {
    x[1] = r0;
    x[3] = r2;
  }
  const float s0 = quad_xor2(hi ? x[0] : x[2]);
  const float s1 = quad_xor2(hi ? x[1] : x[3]);
  if (hi) {
    x[0] = s0;
    x[1] = s1;
  } else {
    x[2] = s0;
    x[3] = s1;
  }
}

// A work unit as the planning kernel lists it (16 bytes). hr = 0: every
// hidden chunk; otherwise chunks [hr & 0xFFFF, + (hr >> 16)) only, the unit's
// output then being a partial sum (a small batch split over the hidden units).
struct FfnUnit {
  int32_t e, seg, rows, hr;
};

// PK: the expert weights are in the packed layout (pack_weights_kernel below):
// each 16-row x 64-byte operand block is one contiguous kilobyte in lane
// order, so every wave load reads eight whole 128-byte lines. NT (packed
// only): the weight loads are non-temporal, for batches in which each
// expert's weights are read about once (no unit of the same expert follows
// to find them in the caches).
template <typename T, int D, bool PK, bool NT>
__global__ __launch_bounds__((FfnShape<T, D>::NW * 64))
__attribute__((amdgpu_waves_per_eu(2, 2))) void ffn_kernel(FfnParams p) {
  using S = FfnShape<T, D>;
  constexpr int UE = S::UE;
  __shared__ U16 xs[S::BM * S::XU];
  __shared__ U16 hs[S::BM * S::HU];
  __shared__ int32_t tokbuf[S::BM];  // token of each row of the unit whose rows come next

  // Persistent workgroups. Workgroups are dealt to the 8 XCDs round-robin, so
  // workgroup b runs on XCD b % 8; it takes every (G / 8)-th unit of that
  // XCD's eighth of the unit list, starting at b / 8. The units of one expert
  // are adjacent in the list, so they run at the same time on one L2.
  const int count = p.blocks[0];
  const int per_xcd = (count + 7) / 8;
  const int xcd = blockIdx.x % 8;
  const int nslot = gridDim.x / 8;
  auto valid = [&](int j) { return j < per_xcd && xcd * per_xcd + j < count; };
  const FfnUnit* units = reinterpret_cast<const FfnUnit*>(p.blocks + 4);
  // a unit's description, loaded by every lane, moved to scalar registers
  auto uniform_unit = [&](const FfnUnit& v) {
    FfnUnit u;
    u.e = __builtin_amdgcn_readfirstlane(v.e);
    u.seg = __builtin_amdgcn_readfirstlane(v.seg);
    u.rows = __builtin_amdgcn_readfirstlane(v.rows);
    u.hr = __builtin_amdgcn_readfirstlane(v.hr);
    return u;
  };
  int j = blockIdx.x / 8;
  if (!valid(j)) return;
  const int h = p.h;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Weight streaming: W1/W2 fragments go from HBM straight into registers
  // through two prefetch rings (PF1 K-blocks of W1, PF2 K-blocks of W2 ahead
  // of use). The next phase's first fragments (across units too) are
  // requested before each barrier, so the loads stay in flight across the
  // barriers.
  //
  // GEMM1 runs on 16x16 tiles: wave w owns hidden units hc + 16 w + (0..15)
  // (A operand, a row of W1 per lane) against all BM tokens (B operand from the
  // x tile); GEMM2 runs on 16x16 tiles too: wave w owns output columns
  // [16 CT2 w, 16 CT2 (w + 1)) for all tokens (B operand: a W2 row per lane,
  // 64 contiguous bytes of it per load), Hc tiles from LDS as A operands.
  constexpr int NKB1 = D / (4 * UE);
  constexpr int NKB2 = S::HC / (4 * UE);
  constexpr int PF1 = NKB1 < 5 ? NKB1 : 5;
  constexpr int PF2 = NKB2 < 2 ? NKB2 : 2;
  const int l16 = lane & 15;
  const int q = lane >> 4;
  const int nch = h / S::HC;
  // a unit's first hidden chunk and chunk count
  auto chunk0 = [&](const FfnUnit& v) { return v.hr & 0xFFFF; };
  auto nchunks = [&](const FfnUnit& v) { return (v.hr >> 16) ? (v.hr >> 16) : nch; };
  // Addresses: a wave-uniform base (scalar registers) plus one 32-bit byte
  // offset per lane and stream, so the prefetch rings cost no 64-bit vector
  // address registers.
  auto w1_base = [&](int e) {
    return gptr(reinterpret_cast<const T*>(p.w1) + ((int64_t)e * h + 16 * wave) * D);
  };
  auto w2_base = [&](int e) {
    return gptr(reinterpret_cast<const T*>(p.w2) + ((int64_t)e * D + 16 * S::CT2 * wave) * h);
  };
  // Natural layout: lane (q, l16) reads row l16, elements [UE q, UE q + UE)
  // of a 64-byte K-block. Packed: the same 16 bytes sit at lane * 16 of the
  // block's kilobyte, and one element step along K is 16 elements in memory.
  const uint32_t o1 = PK ? (uint32_t)(lane * 16) : (uint32_t)((l16 * D + q * UE) * (int)sizeof(T));
  const uint32_t o2 = PK ? (uint32_t)(lane * 16) : (uint32_t)((l16 * h + q * UE) * (int)sizeof(T));
  constexpr int64_t KSTEP = PK ? 16 * (int64_t)sizeof(T) : (int64_t)sizeof(T);  // bytes per K element
  static_assert(PK || !NT, "non-temporal weight loads read whole lines only when packed");
  auto ld_w = [&](GPtr a) { return NT ? ld_unit_g_stream(a) : ld_unit_g(a); };
  auto w1_at = [&](GPtr w1w, int hc, int kb) {
    return ld_w(w1w + (int64_t)hc * D * (int64_t)sizeof(T) + kb * 4 * UE * KSTEP + o1);
  };
  auto w2_at = [&](GPtr w2w, int hc, int kb, int i) {
    return ld_w(w2w + (int64_t)i * 16 * h * (int64_t)sizeof(T) + ((int64_t)hc + kb * 4 * UE) * KSTEP + o2);
  };
  // b1 of the lane's 4 hidden units of a chunk travels with the chunk's first
  // W1 fragments, so the bias never waits on a load issued next to its use.
  // Without b1 the same loads read the start of W1 (always there) and the
  // values are not used, so that no branch separates the prefetches.
  constexpr int BW = sizeof(T) == 2 ? 2 : 4;
  struct B1 {
    uint32_t w[BW];
  };
  const bool has_b1 = p.b1 != nullptr;
  const uint32_t ob1 = (uint32_t)(4 * q * (int)sizeof(T));
  auto b1_at = [&](int e, int hc) {
    const GPtr b1w = has_b1 ? gptr(reinterpret_cast<const T*>(p.b1) + (int64_t)e * h + 16 * wave + hc)
                            : gptr(p.w1);
    B1 v;
    if constexpr (BW == 2) {
      const u32x2 u = *reinterpret_cast<const __attribute__((address_space(1))) u32x2*>(b1w + ob1);
      v.w[0] = u[0];
      v.w[1] = u[1];
    } else {
      const U16 u = ld_unit_g(b1w + ob1);
#pragma unroll
      for (int i = 0; i < 4; ++i) v.w[i] = u.w[i];
    }
    return v;
  };
  // Rows of x of a unit -> the x tile, by global -> LDS copies (no staging
  // registers): copy g (of BM XU / 64) fills tile units [64 g, 64 g + 64);
  // lane l's unit is row r = (64 g + l) / XU, slot (64 g + l) % XU, which
  // holds column slot ^ (r % XSW) of the row (the swizzle of the operand
  // reads). Rows past the unit's end are not copied: they keep finite values
  // of an earlier unit (or whatever the tile held), which only reach output
  // rows that are never written.
  constexpr int NG = S::BM * S::XU / 64 / S::NW;
  static_assert(S::BM * S::XU % (64 * S::NW) == 0, "whole copies per wave");
  auto gather = [&](int rows) {
    // lane index made opaque, so that the per-copy indexes are recomputed
    // here rather than kept in registers across units
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int g = wave + S::NW * i;
      const int u = 64 * g + ln;
      const int r = u / S::XU;
      const int slot = u - r * S::XU;
      if (r < rows) {
        const int64_t tok = tokbuf[r];
        copy16_to_lds(reinterpret_cast<const T*>(p.x) + tok * D + (slot ^ (r & (S::XSW - 1))) * UE,
                      &xs[64 * g]);
      }
    }
  };
  // Token ids of a unit's rows -> tokbuf, by 4-byte global -> LDS copies
  // issued by the first (BM + 63) / 64 waves.
  auto copy_tokens = [&](const FfnUnit& u) {
    if (wave * 64 < S::BM) {
      int ln = lane;  // opaque, as in gather()
      asm volatile("" : "+v"(ln));
      const int r = wave * 64 + ln;
      if (r < u.rows) copy4_to_lds(p.perm_token + u.seg + r, &tokbuf[wave * 64]);
    }
  };
  // Waits for this wave's copies: everything older than the last PF1 + 1
  // loads (the next unit's first W1 fragments and b1), which complete in
  // issue order.
  auto wait_copies = [&]() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PF1 + 1) : "memory"); };

  FfnUnit u = uniform_unit(units[xcd * per_xcd + j]);
  GPtr w1w = w1_base(u.e);
  B1 b1r{};
  U16 pa[PF1];
  U16 pb[PF2][S::CT2];
  // first unit: its tokens, then its rows of x and its first W1 fragments
  if (tid < u.rows) tokbuf[tid] = p.perm_token[u.seg + tid];
  __syncthreads();
  gather(u.rows);
#pragma unroll
  for (int jj = 0; jj < PF1; ++jj) pa[jj] = w1_at(w1w, chunk0(u) * S::HC, jj);
  b1r = b1_at(u.e, chunk0(u) * S::HC);
  wait_copies();
  __syncthreads();

  for (;;) {
    const bool has_next = valid(j + nslot);
    const int jn = has_next ? j + nslot : j;
    // the next unit's description: requested now, used after chunk 0's GEMM1
    const FfnUnit un_raw = units[xcd * per_xcd + jn];
    FfnUnit un = u;
    const GPtr w2w = w2_base(u.e);
    GPtr w1n = w1w;

    f32x4 acc2[S::T16][S::CT2];
#pragma unroll
    for (int tt = 0; tt < S::T16; ++tt)
#pragma unroll
      for (int i = 0; i < S::CT2; ++i) acc2[tt][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nchu = nchunks(u);
    for (int ch = 0; ch < nchu; ++ch) {
      const int hc = (chunk0(u) + ch) * S::HC;
      const bool last = ch + 1 == nchu;
      // this chunk's weight bases, opaque to the compiler so that it forms
      // each load's address from one base and an immediate offset instead of
      // keeping a pointer per K-block live across chunks and units
      GPtr w1c = w1w + (int64_t)hc * D * (int64_t)sizeof(T);
      GPtr w2c = w2w + (int64_t)hc * KSTEP;
      asm volatile("" : "+s"(w1c), "+s"(w2c));
      f32x4 acc1[S::T16];
#pragma unroll
      for (int tt = 0; tt < S::T16; ++tt) acc1[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB1; ++kb) {
        const U16 a = pa[kb % PF1];
        if (kb + PF1 < NKB1) pa[kb % PF1] = w1_at(w1c, 0, kb + PF1);
        // keep the prefetches where they are issued (the scheduler would
        // otherwise sink them next to their use under register pressure)
        __builtin_amdgcn_sched_barrier(0);
        if (kb == (NKB1 > PF1 ? NKB1 - PF1 : 0)) {
#pragma unroll
          for (int jj = 0; jj < PF2; ++jj)
#pragma unroll
            for (int i = 0; i < S::CT2; ++i) pb[jj][i] = w2_at(w2c, 0, jj, i);
        }
        const int c = kb * 4 + q;
#pragma unroll
        for (int tt = 0; tt < S::T16; ++tt) {
          const int r = tt * 16 + l16;
          Mfma<T>::k16(acc1[tt], a, xs[r * S::XU + (c ^ (r & (S::XSW - 1)))]);
        }
      }
      if (ch == 0) {
        // the next unit: its description, and its tokens on their way to
        // tokbuf (read by its row copies at the end of this unit)
        un = uniform_unit(un_raw);
        w1n = w1_base(un.e);
        if (has_next) copy_tokens(un);
        if (nchu == 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __syncthreads();  // the previous chunk's GEMM2 has finished reading hs;
                        // after the last chunk, every wave is done with xs
      if (last && has_next) gather(un.rows);

      // bias + ReLU, round, stage Hc[token][hidden] in LDS: lane l holds token
      // 16 tt + l % 16 and the 4 consecutive hidden units 16 w + 4 (l / 16) + r.
      {
        const int hl = 16 * wave + 4 * q;
        float bias[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float b;
          if constexpr (BW == 2)
            b = bf16_bits_to_f32((b1r.w[i / 2] >> (16 * (i % 2))) & 0xffffu);
          else
            b = __uint_as_float(b1r.w[i]);
          bias[i] = has_b1 ? b : 0.f;
        }
        const int cu = hl / UE;
#pragma unroll
        for (int tt = 0; tt < S::T16; ++tt) {
          const int tok = tt * 16 + l16;
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a = acc1[tt][i] + bias[i];
            v[i] = a > 0.f ? a : 0.f;
          }
          char* dst = reinterpret_cast<char*>(&hs[tok * S::HU + (cu ^ (tok & (S::HSW - 1)))]);
          if constexpr (sizeof(T) == 2) {
            uint2 pk;
            pk.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
            pk.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
            *reinterpret_cast<uint2*>(dst + (hl % UE) * 2) = pk;
          } else {
            U16 pk;
#pragma unroll
            for (int i = 0; i < 4; ++i) pk.w[i] = __float_as_uint(v[i]);
            *reinterpret_cast<U16*>(dst) = pk;
          }
        }
      }
      __syncthreads();

      // GEMM2: Out[token][col] += Hc[token][:] . W2[col][hc:hc+HC]. Its last
      // K-blocks request the first W1 fragments and b1 of the next chunk, of
      // the next unit's first chunk, or (after the last unit) of this unit's
      // first chunk again, unused.
      const int hc_p = last ? chunk0(un) * S::HC : hc + S::HC;
      const GPtr w1p = !last ? w1c + (int64_t)S::HC * D * (int64_t)sizeof(T)
                             : w1n + (int64_t)hc_p * D * (int64_t)sizeof(T);
      const int e_p = last ? un.e : u.e;
#pragma unroll
      for (int kb = 0; kb < NKB2; ++kb) {
        U16 b[S::CT2];
#pragma unroll
        for (int i = 0; i < S::CT2; ++i) b[i] = pb[kb % PF2][i];
        if (kb + PF2 < NKB2) {
#pragma unroll
          for (int i = 0; i < S::CT2; ++i) pb[kb % PF2][i] = w2_at(w2c, 0, kb + PF2, i);
        }
        if (kb == (NKB2 > PF2 ? NKB2 - PF2 : 0)) {
#pragma unroll
          for (int jj = 0; jj < PF1; ++jj) pa[jj] = w1_at(w1p, 0, jj);
          b1r = b1_at(e_p, hc_p);
        }
        __builtin_amdgcn_sched_barrier(0);
        const int c = kb * 4 + q;
#pragma unroll
        for (int tt = 0; tt < S::T16; ++tt) {
          const int r = tt * 16 + l16;
          const U16 a = hs[r * S::HU + (c ^ (r & (S::HSW - 1)))];
#pragma unroll
          for (int i = 0; i < S::CT2; ++i) Mfma<T>::k16(acc2[tt][i], a, b[i]);
        }
      }
    }

    // the next unit's rows have landed in this wave's part of the tile (the
    // wait comes before the stores, so that the last loads issued are the
    // next unit's first W1 fragments and b1, which it leaves in flight)
    if (has_next) wait_copies();

    // Output rows in segment order. A 4x4 transpose inside each quad of lanes
    // turns the C layout (lane: one column, 4 consecutive rows) into one row
    // and 4 consecutive columns per lane, written with one 8-byte (bf16) or
    // 16-byte (fp32) store; b2 is added on the way. A unit of a split batch
    // writes its fp32 partial sums instead.
    if (p.part) {
      const int cq = lane & 3;
      const int col0 = wave * S::CT2 * 16 + (lane & 12);
      const int row0 = 4 * (lane >> 4) + cq;
      float* prow = p.part + ((int64_t)(xcd * per_xcd + j) * p.part_rows + row0) * D + col0;
      const int rleft = u.rows - row0;
#pragma unroll
      for (int i = 0; i < S::CT2; ++i) {
#pragma unroll
        for (int tt = 0; tt < S::T16; ++tt) {
          f32x4 v = acc2[tt][i];
          quad_transpose(v, cq);
          if (tt * 16 < rleft) *reinterpret_cast<f32x4*>(prow + (int64_t)tt * 16 * D + i * 16) = v;
        }
      }
    } else {
      int ln = lane;  // opaque, as in gather()
      asm volatile("" : "+v"(ln));
      const int cq = ln & 3;
      const int col0 = wave * S::CT2 * 16 + (ln & 12);
      const int row0 = 4 * (ln >> 4) + cq;
      // this unit's output from the lane's first element on, opaque (as for
      // the weights) so that no per-element address outlives the unit
      __attribute__((address_space(1))) T* orow =
          (__attribute__((address_space(1))) T*)(reinterpret_cast<T*>(p.out)) +
          (u.seg + row0) * D + col0;
      asm volatile("" : "+v"(orow));
      const int rleft = u.rows - row0;
#pragma unroll
      for (int i = 0; i < S::CT2; ++i) {
        float b2v[4] = {0.f, 0.f, 0.f, 0.f};
        if (p.b2) {
#pragma unroll
          for (int k = 0; k < 4; ++k) b2v[k] = load_scalar<T>(p.b2, (int64_t)u.e * D + col0 + i * 16 + k);
        }
#pragma unroll
        for (int tt = 0; tt < S::T16; ++tt) {
          f32x4 v = acc2[tt][i];
          quad_transpose(v, cq);
          if (tt * 16 < rleft) {
            __attribute__((address_space(1))) T* dst = orow + (int64_t)tt * 16 * D + i * 16;
            if constexpr (sizeof(T) == 2) {
              u32x2 pk;
              pk[0] = f32_to_bf16_bits(v[0] + b2v[0]) | (f32_to_bf16_bits(v[1] + b2v[1]) << 16);
              pk[1] = f32_to_bf16_bits(v[2] + b2v[2]) | (f32_to_bf16_bits(v[3] + b2v[3]) << 16);
              *reinterpret_cast<__attribute__((address_space(1))) u32x2*>(dst) = pk;
            } else {
              f32x4 o = {v[0] + b2v[0], v[1] + b2v[1], v[2] + b2v[2], v[3] + b2v[3]};
              *reinterpret_cast<__attribute__((address_space(1))) f32x4*>(dst) = o;
            }
          }
        }
      }
    }
    if (!has_next) break;
    __syncthreads();  // ... and in every wave's part
    u = un;
    w1w = w1n;
    j = jn;
  }
}

// Lists the work units: expert e gets ceil(count_e / BM) units, each written
// as (expert, first pair of its rows, rows) after the count. One workgroup;
// thread t owns a contiguous span of experts.
// Segments: expert e's rows start at offsets[e] and number offsets[e + 1] -
// offsets[e]; or, with seg_counts, start at e * seg_stride and number
// seg_counts[e] (fixed-stride segments with gaps, as batchwise gating lays
// them out).
__global__ __launch_bounds__(1024) void ffn_plan(const int32_t* __restrict__ offsets, int n, int bm,
                                                 int hsplit, int nch, int capacity,
                                                 const int32_t* __restrict__ seg_counts,
                                                 int seg_stride, int32_t* __restrict__ blocks) {
  // rows of expert e that are served: all, or the first `capacity`
  auto served = [&](int e) {
    const int c = seg_counts ? seg_counts[e] : offsets[e + 1] - offsets[e];
    return capacity > 0 ? min(c, capacity) : c;
  };
  auto seg_start = [&](int e) { return seg_counts ? e * seg_stride : offsets[e]; };
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int e0 = min(n, t * per), e1 = min(n, e0 + per);
  // hsplit > 1: each unit becomes hsplit consecutive units over hidden-chunk
  // ranges of hper chunks (the launcher picks hsplit so that none is empty)
  const int hper = (nch + hsplit - 1) / hsplit;
  int s = 0;
  for (int e = e0; e < e1; ++e) s += (served(e) + bm - 1) / bm * hsplit;
  part[t] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = (t >= o) ? part[t - o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int pos = part[t] - s;
  FfnUnit* units = reinterpret_cast<FfnUnit*>(blocks + 4);
  const int lane = t & 63;
  // unit u of an expert: row block u / hsplit, hidden range u % hsplit
  auto unit_at = [&](int e, int seg, int cnt, int u) {
    const int r = u / hsplit * bm, q = u % hsplit;
    const int hr = hsplit > 1 ? (q * hper) | (min(hper, nch - q * hper) << 16) : 0;
    return FfnUnit{e, seg + r, min(bm, cnt - r), hr};
  };
  // A thread lists the units of an expert with a few of them itself; an
  // expert with many (a popular one) has its units listed by the whole wave,
  // one such expert at a time, so that no thread writes hundreds in a row.
  // Every unit lands at the same position either way.
  for (int i = 0; i < per; ++i) {  // per is uniform over the workgroup
    const int e = e0 + i;
    const bool has = e < e1;
    const int cnt = has ? served(e) : 0;
    const int seg = has ? seg_start(e) : 0;
    const int nu = (cnt + bm - 1) / bm * hsplit;
    const bool many = nu > 8;
    if (!many)
      for (int u = 0; u < nu; ++u) units[pos + u] = unit_at(e, seg, cnt, u);
    uint64_t m = __ballot(many);
    while (m) {
      const int j = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      const int be = __shfl(e, j), bseg = __shfl(seg, j), bcnt = __shfl(cnt, j);
      const int bnu = __shfl(nu, j), bpos = __shfl(pos, j);
      for (int u = lane; u < bnu; u += 64) units[bpos + u] = unit_at(be, bseg, bcnt, u);
    }
    pos += nu;
  }
  if (t == 1023) blocks[0] = part[t];
}

// Sum of a split batch's partial outputs: workgroup b owns the b-th group of
// hsplit consecutive units (one row block of one expert) and writes its rows
// of expert_out = b2 + the hsplit partials in order, 4 columns per thread.
template <typename T, int D>
__global__ __launch_bounds__(256) void ffn_split_reduce(FfnParams p, int hsplit) {
  const int count = p.blocks[0];
  const int b = blockIdx.x;
  if (b * hsplit >= count) return;
  const FfnUnit u = reinterpret_cast<const FfnUnit*>(p.blocks + 4)[b * hsplit];
  for (int idx = threadIdx.x; idx < u.rows * (D / 4); idx += 256) {
    const int r = idx / (D / 4), c = (idx % (D / 4)) * 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (p.b2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = load_scalar<T>(p.b2, (int64_t)u.e * D + c + i);
    }
    for (int q = 0; q < hsplit; ++q) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(
          p.part + ((int64_t)(b * hsplit + q) * p.part_rows + r) * D + c);
      acc += v;
    }
    T* dst = reinterpret_cast<T*>(p.out) + (int64_t)(u.seg + r) * D + c;
    if constexpr (sizeof(T) == 2) {
      uint2 pk;
      pk.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
      pk.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
      *reinterpret_cast<uint2*>(dst) = pk;
    } else {
      *reinterpret_cast<f32x4*>(dst) = acc;
    }
  }
}


template <typename T, int D>
hipError_t ffn_launch_t(int64_t rows, int64_t max_blocks, const FfnParams& p, const int32_t* offsets, int n,
                        int hsplit, int capacity, const int32_t* seg_counts, int seg_stride,
                        hipStream_t s, hipEvent_t ev0, hipEvent_t ev1, bool packed) {
  using S = FfnShape<T, D>;
  hipLaunchKernelGGL(ffn_plan, dim3(1), dim3(1024), 0, s, offsets, n, S::BM, hsplit,
                     p.h / S::HC, capacity, seg_counts, seg_stride,
                     const_cast<int32_t*>(p.blocks));
  max_blocks *= hsplit;
  if (max_blocks <= 0) {  // no rows: an empty timed interval
    hipError_t er = hipGetLastError();
    if (er == hipSuccess && ev0) er = hipEventRecord(ev0, s);
    if (er == hipSuccess && ev1) er = hipEventRecord(ev1, s);
    return er;
  }
  // one persistent workgroup per compute unit (the LDS tile allows one), a
  // multiple of 8 so that every XCD gets the same number of slots, and no
  // more than the largest possible unit count needs
  int cus = 0;
  const hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  const int64_t want = (max_blocks + 7) / 8 * 8;
  const int64_t grid = std::min<int64_t>(want, std::max(8, cus / 8 * 8));
  if (ev0) {
    const hipError_t er = hipEventRecord(ev0, s);
    if (er != hipSuccess) return er;
  }
  // Streamed weights: at most one unit per expert on average (the rows the
  // workspace is sized for over the experts fit one unit each).
  const bool once = rows <= (int64_t)n * S::BM;
  if (packed && once)
    hipLaunchKernelGGL((ffn_kernel<T, D, true, true>), dim3((unsigned)grid), dim3(S::NW * 64), 0,
                       s, p);
  else if (packed)
    hipLaunchKernelGGL((ffn_kernel<T, D, true, false>), dim3((unsigned)grid), dim3(S::NW * 64), 0,
                       s, p);
  else
    hipLaunchKernelGGL((ffn_kernel<T, D, false, false>), dim3((unsigned)grid), dim3(S::NW * 64), 0,
                       s, p);
  if (hsplit > 1)
    hipLaunchKernelGGL((ffn_split_reduce<T, D>), dim3((unsigned)(max_blocks / hsplit)), dim3(256),
                       0, s, p, hsplit);
  const hipError_t el = hipGetLastError();
  if (el != hipSuccess || !ev1) return el;
  return hipEventRecord(ev1, s);
}

// Packed expert weights. A matrix of R rows (R a multiple of 16) and K
// columns (64-byte K-blocks of KB = 64 / sizeof(T) elements) is stored as
// blocks of 16 rows x one K-block, row block by row block and K-block by
// K-block, each block one kilobyte: lane c * 16 + r of the block holds the
// 16 bytes at row r, elements [c UE, c UE + UE) of the K-block, the operand
// a lane of the 16x16 products reads. One thread moves one 16-byte unit.
__global__ __launch_bounds__(256) void pack_weights_kernel(const char* __restrict__ src,
                                                           char* __restrict__ dst, int64_t units,
                                                           int64_t row_bytes) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int64_t lane = u & 63;
  const int64_t blk = u >> 6;                 // (row block, K-block), K-block fastest
  const int64_t kbs = row_bytes / 64;         // K-blocks per row
  const int64_t rb = blk / kbs, kb = blk - rb * kbs;
  const int64_t row = rb * 16 + (lane & 15);
  const int64_t off = row * row_bytes + kb * 64 + (lane >> 4) * 16;
  st_unit(dst + u * 16, ld_unit(src + off));
}

template <typename T>
int bm_for(int d) {
  switch (d) {
    case 64: return FfnShape<T, 64>::BM;
    case 128: return FfnShape<T, 128>::BM;
    case 256: return FfnShape<T, 256>::BM;
    case 512: return FfnShape<T, 512>::BM;
    default: return 0;
  }
}

}  // namespace

// Compute units of the current device (cached per device).
hipError_t device_cus(int* cus) {
  static int cache[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (cache[dev] == 0) {
    int v = 0;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cache[dev] = v > 0 ? v : 1;
  }
  *cus = cache[dev];
  return hipSuccess;
}

int ffn_rows_per_block(int d, Dt dt) { return dt == kBF16 ? bm_for<bf16>(d) : bm_for<float>(d); }

int64_t ffn_max_blocks(int64_t rows, int n, int d, Dt dt) {
  const int bm = ffn_rows_per_block(d, dt);
  if (bm <= 0) return 0;
  return (rows + bm - 1) / bm + n;
}

int ffn_hsplit(int64_t rows, int n, int d, int h, Dt dt) {
  // units are at most the rows and at most ffn_max_blocks; a batch of fewer
  // than 128 units splits each over up to 256 / units hidden-chunk ranges
  const int64_t ub = std::min<int64_t>(ffn_max_blocks(rows, n, d, dt), rows);
  const int hc = 16 * std::max(2, std::min(8, d / 64));  // hidden units per chunk
  const int nch = h / hc;
  if (ub <= 0 || ub >= 128 || nch < 2) return 1;
  const int want = (int)std::min<int64_t>(nch, 256 / ub);
  if (want <= 1) return 1;
  const int per = (nch + want - 1) / want;
  return (nch + per - 1) / per;  // no empty range
}

// Rows of a split unit's partial-output slot: a unit holds at most BM rows,
// and at most all rows of the batch.
static int ffn_part_rows(int64_t rows, int d, Dt dt) {
  return (int)std::min<int64_t>(ffn_rows_per_block(d, dt), rows);
}

// Units the plan can list: every unit has at least one row, so at most the
// rows as well as at most ffn_max_blocks (before the split over hidden ranges).
static int64_t ffn_units_max(int64_t rows, int n, int d, Dt dt) {
  return std::min<int64_t>(ffn_max_blocks(rows, n, d, dt), rows);
}

static size_t ffn_list_bytes(int64_t rows, int n, int d, int h, Dt dt) {
  const size_t b = (size_t)(4 + 4 * ffn_units_max(rows, n, d, dt) * ffn_hsplit(rows, n, d, h, dt)) *
                   sizeof(int32_t);
  return (b + 255) / 256 * 256;
}

size_t ffn_plan_bytes(int64_t rows, int n, int d, int h, Dt dt) {
  const int hs = ffn_hsplit(rows, n, d, h, dt);
  size_t b = ffn_list_bytes(rows, n, d, h, dt);
  if (hs > 1)
    b += (size_t)ffn_units_max(rows, n, d, dt) * hs * ffn_part_rows(rows, d, dt) * d *
         sizeof(float);
  return b;
}

bool ffn_supported(int d, int h, Dt dt) {
  (void)dt;
  return (d == 64 || d == 128 || d == 256 || d == 512) && h >= 128 && h % 128 == 0;
}

hipError_t launch_ffn(int64_t tokens, int k, int d, int h, int n, Dt dt, const void* x,
                      const int32_t* offsets, const int32_t* perm_token, const void* w1,
                      const void* b1, const void* w2, const void* b2, void* expert_out,
                      int32_t* blocks, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1,
                      int capacity, const int32_t* seg_counts, int seg_stride, bool packed) {
  const int64_t mb = ffn_max_blocks(tokens * k, n, d, dt);
  const int hs = ffn_hsplit(tokens * k, n, d, h, dt);
  FfnParams p{x, offsets, perm_token, w1, b1, w2, b2, expert_out, blocks, h, nullptr, 0};
  if (hs > 1) {
    p.part = reinterpret_cast<float*>(reinterpret_cast<char*>(blocks) +
                                      ffn_list_bytes(tokens * k, n, d, h, dt));
    p.part_rows = ffn_part_rows(tokens * k, d, dt);
  }
  if (dt == kBF16) {
    switch (d) {
      case 64: return ffn_launch_t<bf16, 64>(tokens * k, mb, p, offsets, n, hs, capacity, seg_counts, seg_stride, s, ev0, ev1, packed);
      case 128: return ffn_launch_t<bf16, 128>(tokens * k, mb, p, offsets, n, hs, capacity, seg_counts, seg_stride, s, ev0, ev1, packed);
      case 256: return ffn_launch_t<bf16, 256>(tokens * k, mb, p, offsets, n, hs, capacity, seg_counts, seg_stride, s, ev0, ev1, packed);
      case 512: return ffn_launch_t<bf16, 512>(tokens * k, mb, p, offsets, n, hs, capacity, seg_counts, seg_stride, s, ev0, ev1, packed);
    }
  } else {
    switch (d) {
      case 64: return ffn_launch_t<float, 64>(tokens * k, mb, p, offsets, n, hs, capacity, seg_counts, seg_stride, s, ev0, ev1, packed);
      case 128: return ffn_launch_t<float, 128>(tokens * k, mb, p, offsets, n, hs, capacity, seg_counts, seg_stride, s, ev0, ev1, packed);
      case 256: return ffn_launch_t<float, 256>(tokens * k, mb, p, offsets, n, hs, capacity, seg_counts, seg_stride, s, ev0, ev1, packed);
      case 512: return ffn_launch_t<float, 512>(tokens * k, mb, p, offsets, n, hs, capacity, seg_counts, seg_stride, s, ev0, ev1, packed);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_pack_weights(const void* src, void* dst, int64_t rows, int64_t row_bytes,
                               hipStream_t s) {
  const int64_t units = rows * row_bytes / 16;
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const char*>(src), reinterpret_cast<char*>(dst), units,
                     row_bytes);
  return hipGetLastError();
}

}  // namespace moe
