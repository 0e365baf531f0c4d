/* Host implementation of the synthetic-input generator (Philox4x32-10 +
 * Box-Muller in float64), the same draw recipe as synth/__init__.py:
 *   stream key = (seed, fnv1a32(name)); block j -> counter (j lo, j hi, 0, 0);
 *   element 4j+m takes word m; normals from word pairs (0,1), (2,3) with
 *   u = (x + 0.5) * 2^-32, r = sqrt(-2 ln u1), z = (r cos 2*pi*u2, r sin 2*pi*u2);
 *   value = fp32(z * std + mean), optionally rounded on to bf16 (nearest even).
 * Built with -ffp-contract=off so that no multiply-add is fused.
 * Philox4x32-10: Salmon et al., "Parallel random numbers: as easy as 1, 2, 3",
 * SC'11. */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static void philox(uint64_t j, uint32_t k0, uint32_t k1, uint32_t out[4]) {
  uint32_t c0 = (uint32_t)j, c1 = (uint32_t)(j >> 32), c2 = 0, c3 = 0;
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += PHILOX_W0; k1 += PHILOX_W1; }
    uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
    uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c0 = n0; c1 = (uint32_t)p1; c2 = n2; c3 = (uint32_t)p0;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static void block_normals(uint64_t j, uint32_t seed, uint32_t key, double z[4]) {
  uint32_t w[4];
  philox(j, seed, key, w);
  const double two32inv = 1.0 / 4294967296.0;
  for (int p = 0; p < 2; ++p) {
    double u1 = ((double)w[2 * p] + 0.5) * two32inv;
    double u2 = ((double)w[2 * p + 1] + 0.5) * two32inv;
    double r = sqrt(-2.0 * log(u1));
    double t = 2.0 * M_PI * u2;
    z[2 * p] = r * cos(t);
    z[2 * p + 1] = r * sin(t);
  }
}

static uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return (uint16_t)u;
}

void synth_u32(uint32_t seed, uint32_t key, int64_t start, int64_t n, uint32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint64_t e = (uint64_t)(start + i);
    uint32_t w[4];
    philox(e >> 2, seed, key, w);
    out[i] = w[e & 3];
  }
}

/* Elements start .. start+n-1 of the stream. */
void synth_normal(uint32_t seed, uint32_t key, int64_t start, int64_t n, double std,
                  double mean, int bf16, void* out) {
  int64_t j0 = start >> 2, j1 = (start + n + 3) >> 2;
#pragma omp parallel for schedule(static)
  for (int64_t j = j0; j < j1; ++j) {
    double z[4];
    block_normals((uint64_t)j, seed, key, z);
    for (int m = 0; m < 4; ++m) {
      int64_t e = 4 * j + m;
      if (e < start || e >= start + n) continue;
      float v = (float)(z[m] * std + mean);
      if (bf16) ((uint16_t*)out)[e - start] = f32_to_bf16(v);
      else ((float*)out)[e - start] = v;
    }
  }
}

void synth_token_ids(uint32_t seed, uint32_t key, int64_t n, uint32_t vocab, int32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint32_t w[4];
    philox((uint64_t)i >> 2, seed, key, w);
    out[i] = (int32_t)(((uint64_t)w[i & 3] * vocab) >> 32);
  }
}
