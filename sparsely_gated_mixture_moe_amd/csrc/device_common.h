// Device-side building blocks shared by the gfx950 kernels: storage types,
// 16-byte operand units, the CDNA4 matrix-core (MFMA) wrappers and the scalar
// functions of the gate.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// bf16 is stored as its bit pattern.
struct bf16 {
  uint16_t bits;
};

typedef short short8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// A 16-byte operand unit: 8 bf16 or 4 fp32 consecutive elements of a row.
struct alignas(16) U16 {
  uint32_t w[4];
};

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kPerUnit = 4;
};
template <>
struct Elem<bf16> {
  static constexpr int kPerUnit = 8;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ U16 ld_unit(const void* p) { return *reinterpret_cast<const U16*>(p); }

// The same as a non-temporal load, for data read once in whole cache lines
// (each wave instruction covering full 128-byte lines) from beyond the caches.
__device__ __forceinline__ U16 ld_unit_stream(const void* p) {
  typedef uint32_t u32x4_ __attribute__((ext_vector_type(4)));
  const u32x4_ v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_*>(p));
  U16 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// Arrays larger than this many bytes do not stay in the 256 MB Infinity Cache
// between the kernel that writes them and the one that reads them once; those
// reads go to HBM and are faster as non-temporal loads.
constexpr int64_t kStreamBytes = (int64_t)192 << 20;
__device__ __forceinline__ void st_unit(void* p, const U16& v) { *reinterpret_cast<U16*>(p) = v; }
__device__ __forceinline__ U16 zero_unit() { return U16{{0u, 0u, 0u, 0u}}; }

// Four bf16 (8 bytes) widened to a unit of four fp32.
__device__ __forceinline__ U16 widen4_bf16(const void* p) {
  uint2 v = *reinterpret_cast<const uint2*>(p);
  U16 r;
  r.w[0] = v.x << 16;
  r.w[1] = v.x & 0xFFFF0000u;
  r.w[2] = v.y << 16;
  r.w[3] = v.y & 0xFFFF0000u;
  return r;
}

__device__ __forceinline__ short8 as_short8(const U16& u) {
  short8 s;
  __builtin_memcpy(&s, &u, 16);
  return s;
}

// ---------------------------------------------------------------------------
// Matrix-core K-blocks. A "K-block" is the K range that one 16-byte unit per
// lane covers across a wave.
//
// 16x16 tiles (v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x4_f32): lane l
// supplies row (A) or column (B) l % 16 and unit q = l / 16 of the K-block, so
// a K-block is 4 units: 32 bf16 or 16 fp32. For fp32 the four elements of a
// lane's unit feed four successive 16x16x4 steps; step s then contracts the K
// indices {4q + s}, which covers the K-block once because A and B use the same
// assignment. Output: lane l holds column l % 16, rows 4 (l / 16) + r, r < 4.
//
// 32x32 tiles (v_mfma_f32_32x32x16_bf16 / v_mfma_f32_32x32x2_f32): lane l
// supplies row/column l % 32 and unit l / 32, so a K-block is 2 units: 16 bf16
// or 8 fp32 (four 32x32x2 steps). Output: lane l holds column l % 32, rows
// 8 (j / 4) + 4 (l / 32) + j % 4 for j < 16.
// ---------------------------------------------------------------------------
template <typename T>
struct Mfma;

template <>
struct Mfma<bf16> {
  __device__ __forceinline__ static void k16(f32x4& acc, const U16& a, const U16& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_short8(a), as_short8(b), acc, 0, 0, 0);
  }
  __device__ __forceinline__ static void k32(f32x16& acc, const U16& a, const U16& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_short8(a), as_short8(b), acc, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  __device__ __forceinline__ static void k16(f32x4& acc, const U16& a, const U16& b) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w[s]), __uint_as_float(b.w[s]),
                                                 acc, 0, 0, 0);
  }
  __device__ __forceinline__ static void k32(f32x16& acc, const U16& a, const U16& b) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w[s]), __uint_as_float(b.w[s]),
                                                 acc, 0, 0, 0);
  }
};

// One 16-byte global -> LDS copy per active lane (global_load_lds_dwordx4):
// lane l's 16 bytes land at lds_base + 16 l; lds_base must be the same in
// every lane. The copy is issued from inline asm, so the compiler neither waits
// for it nor counts it: the caller must wait for it (s_waitcnt vmcnt, in issue
// order) before reading the destination. Untracked copies only make the
// compiler's own vmcnt waits stricter, never too weak. The compiler sets m0
// (the LDS base) for the asm; an SALU write of m0 needs one wait state before
// an LDS-DMA instruction reads it, hence the s_nop.
__device__ __forceinline__ void copy16_to_lds(const void* src, const void* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "{m0}"(m0)
      : "memory");
}

// The same with 4 bytes per lane (global_load_lds_dword): lane l's 4 bytes
// land at lds_base + 4 l.
__device__ __forceinline__ void copy4_to_lds(const void* src, const void* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(src), "{m0}"(m0)
      : "memory");
}

// Fast reciprocal (v_rcp_f32, about 1 ulp).
__device__ __forceinline__ float rcp_f(float x) { return __builtin_amdgcn_rcpf(x); }

// log(1 + t) for t in [0, 1] with one native log2: w = 1 + t is rounded, but
// w - 1 is exact (Sterbenz), so the rounding error d = t - (w - 1) is known
// exactly and log(1 + t) = log(w) + log(1 + d / w). Taking d for the last term
// errs by |d| (w - 1) / w <= 2^-24 t, a relative error below 2^-23 (the
// compensated-summation idea of Kahan; Goldberg, "What every computer
// scientist should know about floating-point arithmetic", 1991).
__device__ __forceinline__ float log1p_small(float t) {
  const float w = 1.0f + t;
  const float d = t - (w - 1.0f);
  return fmaf(__builtin_amdgcn_logf(w), 0.69314718055994531f, d);
}

// e^x through the native 2^x (v_exp_f32); arguments are <= 0 here.
__device__ __forceinline__ float exp_native(float x) {
  return __builtin_amdgcn_exp2f(x * 1.44269504088896341f);
}

// Softplus(u) = log(1 + e^u) = max(u, 0) + log(1 + e^-|u|), which cannot
// overflow; max(u, 0) = (u + |u|) / 2 rides on the final multiply-add. u must
// be finite.
__device__ __forceinline__ float softplus_f(float u) {
  return fmaf(u + fabsf(u), 0.5f, log1p_small(exp_native(-fabsf(u))));
}

// Standard normal CDF from the Chebyshev fit of erfc in Numerical Recipes
// (Press et al., 2nd ed., section 6.2, "erfcc"; fractional error below 1.2e-7
// everywhere): with a = |z| / sqrt 2 and t = 1 / (1 + a / 2),
// erfc(a) = t exp(-a^2 + P(t)). Here h = erfc(a) / 2 is evaluated as
// t 2^(Q(t) - z^2 log2(e) / 2) with Q = log2(e) P - 1 (the fit's coefficients
// times log2 e, the constant term lowered by one for the halving), and
// Phi(z) = h for z < 0, 1 - h otherwise (erfc(-a) = 2 - erfc(a)).
__device__ __forceinline__ float phi_f(float z) {
  constexpr float L2E = 1.44269504088896341f;
  const float t = rcp_f(fmaf(fabsf(z), 0.35355339059327376f, 1.0f));
  float q = 0.17087277f * L2E;
  q = fmaf(t, q, -0.82215223f * L2E);
  q = fmaf(t, q, 1.48851587f * L2E);
  q = fmaf(t, q, -1.13520398f * L2E);
  q = fmaf(t, q, 0.27886807f * L2E);
  q = fmaf(t, q, -0.18628806f * L2E);
  q = fmaf(t, q, 0.09678418f * L2E);
  q = fmaf(t, q, 0.37409196f * L2E);
  q = fmaf(t, q, 1.00002368f * L2E);
  q = fmaf(t, q, -1.26551223f * L2E - 1.0f);
  const float h = t * __builtin_amdgcn_exp2f(fmaf(z * (-0.5f * L2E), z, q));
  return z < 0.0f ? h : 1.0f - h;
}

// Ranking order of (logit, expert) pairs: larger logit first, equal logits to
// the lower expert index.
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

}  // namespace moe
