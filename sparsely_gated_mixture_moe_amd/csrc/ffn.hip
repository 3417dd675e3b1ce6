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
  const int32_t* blocks;  // [0] = count, then (expert, first row) pairs
  int h;
};

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

template <typename T, int D>
__global__ __launch_bounds__((FfnShape<T, D>::NW * 64))
__attribute__((amdgpu_waves_per_eu(2, 2))) void ffn_kernel(FfnParams p) {
  using S = FfnShape<T, D>;
  constexpr int NT = S::NW * 64;
  constexpr int UE = S::UE;
  __shared__ U16 xs[S::BM * S::XU];
  __shared__ U16 hs[S::BM * S::HU];

  // XCD-aware placement: workgroups are dealt to the 8 XCDs round-robin, so
  // XCD x = blockIdx % 8 takes the x-th eighth of the unit list in order and
  // the units of one expert run back to back on one L2.
  const int count = p.blocks[0];
  const int per_xcd = (count + 7) / 8;
  const int slot = blockIdx.x / 8;
  const int blk = (blockIdx.x % 8) * per_xcd + slot;
  if (slot >= per_xcd || blk >= count) return;
  const int e = p.blocks[1 + 2 * blk];
  const int row0 = p.blocks[2 + 2 * blk];
  const int seg0 = p.offsets[e];
  const int rows = min(S::BM, p.offsets[e + 1] - seg0 - row0);
  const int64_t seg = (int64_t)seg0 + row0;
  const int h = p.h;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const T* w1e = reinterpret_cast<const T*>(p.w1) + (int64_t)e * h * D;
  const T* w2e = reinterpret_cast<const T*>(p.w2) + (int64_t)e * D * h;

  f32x4 acc2[S::T16][S::CT2];
#pragma unroll
  for (int tt = 0; tt < S::T16; ++tt)
#pragma unroll
    for (int i = 0; i < S::CT2; ++i) acc2[tt][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Weight streaming: W1/W2 fragments go from HBM straight into registers
  // through two prefetch rings (PF1 K-blocks of W1, PF2 K-blocks of W2 ahead
  // of use). The next phase's first fragments are requested before each
  // barrier, so the loads stay in flight across the barriers.
  //
  // GEMM1 runs on 16x16 tiles: wave w owns hidden units hc + 16 w + (0..15)
  // (A operand, a row of W1 per lane) against all BM tokens (B operand from the
  // x tile); GEMM2 runs on 16x16 tiles too: wave w owns output columns
  // [16 CT2 w, 16 CT2 (w + 1)) for all tokens (B operand: a W2 row per lane,
  // 64 contiguous bytes of it per load), Hc tiles from LDS as A operands.
  constexpr int NKB1 = D / (4 * UE);
  constexpr int NKB2 = S::HC / (4 * UE);
  constexpr int PF1 = NKB1 < 7 ? NKB1 : 7;
  constexpr int PF2 = NKB2 < 2 ? NKB2 : 2;
  const int l16 = lane & 15;
  const int q = lane >> 4;
  const int nch = h / S::HC;
  // Addresses: a wave-uniform base (scalar registers) plus one 32-bit byte
  // offset per lane and stream, so the prefetch rings cost no 64-bit vector
  // address registers.
  const char* w1w = reinterpret_cast<const char*>(w1e + (int64_t)16 * wave * D);
  const char* w2w = reinterpret_cast<const char*>(w2e + (int64_t)16 * S::CT2 * wave * h);
  const uint32_t o1 = (uint32_t)((l16 * D + q * UE) * (int)sizeof(T));
  const uint32_t o2 = (uint32_t)((l16 * h + q * UE) * (int)sizeof(T));
  auto w1_at = [&](int hc, int kb) {
    return ld_unit(w1w + ((int64_t)hc * D + kb * 4 * UE) * (int64_t)sizeof(T) + o1);
  };
  auto w2_at = [&](int hc, int kb, int i) {
    return ld_unit(w2w + ((int64_t)i * 16 * h + hc + kb * 4 * UE) * (int64_t)sizeof(T) + o2);
  };
  // b1 of the lane's 4 hidden units of a chunk travels with the chunk's first
  // W1 fragments, so the bias never waits on a load issued next to its use.
  constexpr int BW = sizeof(T) == 2 ? 2 : 4;
  struct B1 { uint32_t w[BW]; };
  const bool has_b1 = p.b1 != nullptr;
  const char* b1w = has_b1 ? reinterpret_cast<const char*>(p.b1) +
                                ((int64_t)e * h + 16 * wave) * (int64_t)sizeof(T)
                          : nullptr;
  const uint32_t ob = (uint32_t)(4 * q * (int)sizeof(T));
  auto b1_at = [&](int hc) {
    B1 v;
    if constexpr (BW == 2) {
      const uint2 u = *reinterpret_cast<const uint2*>(b1w + (int64_t)hc * sizeof(T) + ob);
      v.w[0] = u.x;
      v.w[1] = u.y;
    } else {
      const U16 u = ld_unit(b1w + (int64_t)hc * sizeof(T) + ob);
#pragma unroll
      for (int i = 0; i < 4; ++i) v.w[i] = u.w[i];
    }
    return v;
  };
  B1 b1r{};
  U16 pa[PF1];
  U16 pb[PF2][S::CT2];
  // The first W1 fragments are requested before the gather, so the weight
  // stream is already in flight while the rows of x arrive.
#pragma unroll
  for (int j = 0; j < PF1; ++j) pa[j] = w1_at(0, j);
  if (has_b1) b1r = b1_at(0);

  // Gather the unit's rows of x.
  for (int u = tid; u < S::BM * S::XU; u += NT) {
    const int r = u / S::XU;
    const int c = u - r * S::XU;
    U16 v = zero_unit();
    if (r < rows) {
      const int64_t tok = p.perm_token[seg + r];
      v = ld_unit(reinterpret_cast<const T*>(p.x) + tok * D + c * UE);
    }
    xs[r * S::XU + (c ^ (r & (S::XSW - 1)))] = v;
  }
  __syncthreads();

  for (int ch = 0; ch < nch; ++ch) {
    const int hc = ch * S::HC;
    f32x4 acc1[S::T16];
#pragma unroll
    for (int tt = 0; tt < S::T16; ++tt) acc1[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB1; ++kb) {
      const U16 a = pa[kb % PF1];
      if (kb + PF1 < NKB1) pa[kb % PF1] = w1_at(hc, kb + PF1);
      // keep the prefetches where they are issued (the scheduler would
      // otherwise sink them next to their use under register pressure)
      __builtin_amdgcn_sched_barrier(0);
      if (kb == (NKB1 > PF1 ? NKB1 - PF1 : 0)) {
#pragma unroll
        for (int j = 0; j < PF2; ++j)
#pragma unroll
          for (int i = 0; i < S::CT2; ++i) pb[j][i] = w2_at(hc, j, i);
      }
      const int c = kb * 4 + q;
#pragma unroll
      for (int tt = 0; tt < S::T16; ++tt) {
        const int r = tt * 16 + l16;
        Mfma<T>::k16(acc1[tt], a, xs[r * S::XU + (c ^ (r & (S::XSW - 1)))]);
      }
    }
    __syncthreads();  // the previous chunk's GEMM2 has finished reading hs

    // bias + ReLU, round, stage Hc[token][hidden] in LDS: lane l holds token
    // 16 tt + l % 16 and the 4 consecutive hidden units 16 w + 4 (l / 16) + r.
    {
      const int hl = 16 * wave + 4 * q;
      float bias[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (BW == 2)
          bias[i] = bf16_bits_to_f32((b1r.w[i / 2] >> (16 * (i % 2))) & 0xffffu);
        else
          bias[i] = __uint_as_float(b1r.w[i]);
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

    // GEMM2: Out[token][col] += Hc[token][:] . W2[col][hc:hc+HC].
#pragma unroll
    for (int kb = 0; kb < NKB2; ++kb) {
      U16 b[S::CT2];
#pragma unroll
      for (int i = 0; i < S::CT2; ++i) b[i] = pb[kb % PF2][i];
      if (kb + PF2 < NKB2) {
#pragma unroll
        for (int i = 0; i < S::CT2; ++i) pb[kb % PF2][i] = w2_at(hc, kb + PF2, i);
      }
      if (kb == (NKB2 > PF2 ? NKB2 - PF2 : 0) && ch + 1 < nch) {
#pragma unroll
        for (int j = 0; j < PF1; ++j) pa[j] = w1_at(hc + S::HC, j);
        if (has_b1) b1r = b1_at(hc + S::HC);
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

  // b2, then write the rows in segment order (lane: column l % 16 of each tile,
  // token rows 4 (l / 16) + j).
#pragma unroll
  for (int i = 0; i < S::CT2; ++i) {
    const int col = (wave * S::CT2 + i) * 16 + l16;
    const float bias = p.b2 ? load_scalar<T>(p.b2, (int64_t)e * D + col) : 0.f;
#pragma unroll
    for (int tt = 0; tt < S::T16; ++tt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tok = tt * 16 + 4 * q + j;
        if (tok < rows) store_scalar<T>(p.out, (seg + tok) * D + col, acc2[tt][i][j] + bias);
      }
  }
}

// Lists the work units: expert e gets ceil(count_e / BM) units. One workgroup;
// thread t owns a contiguous span of experts.
__global__ __launch_bounds__(1024) void ffn_plan(const int32_t* __restrict__ offsets, int n, int bm,
                                                 int32_t* __restrict__ blocks) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int e0 = min(n, t * per), e1 = min(n, e0 + per);
  int s = 0;
  for (int e = e0; e < e1; ++e) s += (offsets[e + 1] - offsets[e] + bm - 1) / bm;
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
    const int cnt = offsets[e + 1] - offsets[e];
    for (int r = 0; r < cnt; r += bm) {
      blocks[1 + 2 * pos] = e;
      blocks[2 + 2 * pos] = r;
      ++pos;
    }
  }
  if (t == 1023) blocks[0] = part[t];
}

template <typename T, int D>
hipError_t ffn_launch_t(int64_t max_blocks, const FfnParams& p, const int32_t* offsets, int n,
                        hipStream_t s) {
  using S = FfnShape<T, D>;
  hipLaunchKernelGGL(ffn_plan, dim3(1), dim3(1024), 0, s, offsets, n, S::BM,
                     const_cast<int32_t*>(p.blocks));
  // every XCD gets ceil(count / 8) slots; the grid covers the largest possible count
  const int64_t grid = (max_blocks + 7) / 8 * 8;
  if (max_blocks > 0)
    hipLaunchKernelGGL((ffn_kernel<T, D>), dim3((unsigned)grid), dim3(S::NW * 64), 0, s, p);
  return hipGetLastError();
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

int ffn_rows_per_block(int d, Dt dt) { return dt == kBF16 ? bm_for<bf16>(d) : bm_for<float>(d); }

int64_t ffn_max_blocks(int64_t rows, int n, int d, Dt dt) {
  const int bm = ffn_rows_per_block(d, dt);
  if (bm <= 0) return 0;
  return (rows + bm - 1) / bm + n;
}

bool ffn_supported(int d, int h, Dt dt) {
  (void)dt;
  return (d == 64 || d == 128 || d == 256 || d == 512) && h >= 128 && h % 128 == 0;
}

hipError_t launch_ffn(int64_t tokens, int k, int d, int h, int n, Dt dt, const void* x,
                      const int32_t* offsets, const int32_t* perm_token, const void* w1,
                      const void* b1, const void* w2, const void* b2, void* expert_out,
                      int32_t* blocks, hipStream_t s) {
  FfnParams p{x, offsets, perm_token, w1, b1, w2, b2, expert_out, blocks, h};
  const int64_t mb = ffn_max_blocks(tokens * k, n, d, dt);
  if (dt == kBF16) {
    switch (d) {
      case 64: return ffn_launch_t<bf16, 64>(mb, p, offsets, n, s);
      case 128: return ffn_launch_t<bf16, 128>(mb, p, offsets, n, s);
      case 256: return ffn_launch_t<bf16, 256>(mb, p, offsets, n, s);
      case 512: return ffn_launch_t<bf16, 512>(mb, p, offsets, n, s);
    }
  } else {
    switch (d) {
      case 64: return ffn_launch_t<float, 64>(mb, p, offsets, n, s);
      case 128: return ffn_launch_t<float, 128>(mb, p, offsets, n, s);
      case 256: return ffn_launch_t<float, 256>(mb, p, offsets, n, s);
      case 512: return ffn_launch_t<float, 512>(mb, p, offsets, n, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
