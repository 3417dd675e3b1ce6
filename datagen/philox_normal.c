/*
 * Seeded synthetic input generator shared by the oracle tests, the GPU parity
 * tests and the benchmark. It holds none of the MoE method's arithmetic: it
 * only turns (seed, tensor id, element index) into standard normal draws.
 *
 * Generator: Philox4x32-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11).
 * Ten rounds of the Philox S-box on a 128-bit counter with a 64-bit key, the
 * key bumped by the Weyl constants after every round.
 *
 * Normals: the Box-Muller transform (Box and Muller, 1958) in double
 * precision, two normals per Philox call; the 128 output bits give two 53-bit
 * uniforms u1 in (0,1] and u2 in [0,1).
 *
 * Element e of tensor `tid` uses counter (p_lo, p_hi, tid, 0) with p = e / 2
 * and key (seed, 0); even e takes the cosine branch, odd e the sine branch.
 * So any slice of any tensor can be regenerated independently.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox_round(uint32_t c[4], const uint32_t k[2]) {
  uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
  uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
  uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  uint32_t n0 = hi1 ^ c[1] ^ k[0];
  uint32_t n2 = hi0 ^ c[3] ^ k[1];
  c[0] = n0;
  c[1] = lo1;
  c[2] = n2;
  c[3] = lo0;
}

void dg_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  for (int r = 0; r < 10; ++r) {
    philox_round(c, k);
    k[0] += PHILOX_W0;
    k[1] += PHILOX_W1;
  }
  memcpy(out, c, sizeof(c));
}

static inline void normal_pair(uint32_t seed, uint32_t tid, uint64_t p, double* z0, double* z1) {
  uint32_t ctr[4] = {(uint32_t)p, (uint32_t)(p >> 32), tid, 0u};
  uint32_t key[2] = {seed, 0u};
  uint32_t r[4];
  dg_philox4x32_10(ctr, key, r);
  uint64_t a = ((uint64_t)r[1] << 32) | r[0];
  uint64_t b = ((uint64_t)r[3] << 32) | r[2];
  const double two_m53 = 1.0 / 9007199254740992.0;
  double u1 = (double)((a >> 11) + 1) * two_m53; /* (0, 1] */
  double u2 = (double)(b >> 11) * two_m53;       /* [0, 1) */
  double rad = sqrt(-2.0 * log(u1));
  double ang = 6.283185307179586476925286766559 * u2;
  *z0 = rad * cos(ang);
  *z1 = rad * sin(ang);
}

/* Round-to-nearest-even fp32 -> bf16 (finite inputs). */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t bias = 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)((u + bias) >> 16);
}

/* Standard normal draws z[e] for e in [offset, offset + count), scaled by `scale`
 * and rounded to fp32 (out_dtype 0 -> float*) or further to bf16 (out_dtype 1 ->
 * uint16_t*). Returns 0, or -1 on a bad dtype. */
int dg_normal(uint32_t seed, uint32_t tid, uint64_t offset, uint64_t count, double scale,
              int out_dtype, void* out) {
  if (out_dtype != 0 && out_dtype != 1) return -1;
  float* of = (float*)out;
  uint16_t* ob = (uint16_t*)out;
  const int64_t npair_lo = (int64_t)(offset / 2);
  const int64_t npair_hi = (int64_t)((offset + count + 1) / 2);
#pragma omp parallel for schedule(static)
  for (int64_t p = npair_lo; p < npair_hi; ++p) {
    double z[2];
    normal_pair(seed, tid, (uint64_t)p, &z[0], &z[1]);
    for (int s = 0; s < 2; ++s) {
      uint64_t e = (uint64_t)p * 2 + (uint64_t)s;
      if (e < offset || e >= offset + count) continue;
      float v = (float)(z[s] * scale);
      uint64_t o = e - offset;
      if (out_dtype == 0)
        of[o] = v;
      else
        ob[o] = f32_to_bf16_rne(v);
    }
  }
  return 0;
}

/* fp32 -> bf16 (RNE) conversion of an existing array, for inputs that are
 * built from generated draws by the workload recipes. */
void dg_f32_to_bf16(const float* in, uint16_t* out, uint64_t count) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)count; ++i) out[i] = f32_to_bf16_rne(in[i]);
}
