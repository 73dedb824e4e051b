/*
 * Seeded synthetic inputs: counter-based Philox4x32-10 (Salmon, Moraes, Dror,
 * Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11) turned into
 * N(mean, std) samples by the Box-Muller transform, written as fp32 or as
 * bf16 (round to nearest, ties to even).
 *
 * This module only manufactures inputs. It holds none of the arithmetic of
 * the weight-streaming method or of the DiT block, and is the one piece that
 * both the CPU oracle and the GPU path consume (as bytes).
 *
 * Stream layout: sample e of the sequence (seed, stream, a, b) comes from the
 * Philox block with key = (seed & 0xffffffff, stream) and counter
 * = (q & 0xffffffff, q >> 32, a, b), q = e / 4; lane e % 4 of that block.
 * Lanes (0,1) and (2,3) each form one Box-Muller pair.
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
  c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
}

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  for (int r = 0; r < 10; ++r) {
    if (r) { k[0] += PHILOX_W0; k[1] += PHILOX_W1; }
    philox_round(c, k);
  }
  memcpy(out, c, sizeof c);
}

/* uniform in (0,1): 24 high bits, centred in their bin so 0 and 1 never occur */
static inline float u01(uint32_t x) { return ((float)(x >> 8) + 0.5f) * (1.0f / 16777216.0f); }

/* 64 consecutive samples (16 Philox blocks) starting at sample 4*q0; written
 * as plain loops over lanes so the compiler can vectorise them. */
#define LANES 16
static inline void normals64(uint64_t seed, uint32_t stream, uint32_t a, uint32_t b, uint64_t q0,
                             float z[4 * LANES]) {
  uint32_t c0[LANES], c1[LANES], c2[LANES], c3[LANES];
  for (int j = 0; j < LANES; ++j) {
    uint64_t q = q0 + (uint64_t)j;
    c0[j] = (uint32_t)q; c1[j] = (uint32_t)(q >> 32); c2[j] = a; c3[j] = b;
  }
  uint32_t k0 = (uint32_t)seed, k1 = stream;
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += PHILOX_W0; k1 += PHILOX_W1; }
#pragma omp simd
    for (int j = 0; j < LANES; ++j) {
      uint64_t p0 = (uint64_t)PHILOX_M0 * c0[j];
      uint64_t p1 = (uint64_t)PHILOX_M1 * c2[j];
      uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1[j] ^ k0;
      uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3[j] ^ k1;
      c0[j] = n0; c1[j] = (uint32_t)p1; c2[j] = n2; c3[j] = (uint32_t)p0;
    }
  }
  /* Box-Muller: r = sqrt(-2 ln u1), z = (r cos 2 pi u2, r sin 2 pi u2).  The
   * sine is taken as cos(2 pi (u2 - 1/4)) so that each line is a plain cosf
   * that vectorises (a sinf/cosf pair of one argument would be fused into a
   * scalar sincosf call). */
  float rad0[LANES], u20[LANES], rad1[LANES], u21[LANES];
#pragma omp simd
  for (int j = 0; j < LANES; ++j) {
    rad0[j] = sqrtf(-2.0f * logf(u01(c0[j])));
    u20[j] = u01(c1[j]);
    rad1[j] = sqrtf(-2.0f * logf(u01(c2[j])));
    u21[j] = u01(c3[j]);
  }
  const float two_pi = 6.28318530717958647692f;
#pragma omp simd
  for (int j = 0; j < LANES; ++j) {
    z[4 * j + 0] = rad0[j] * cosf(two_pi * u20[j]);
    z[4 * j + 2] = rad1[j] * cosf(two_pi * u21[j]);
  }
#pragma omp simd
  for (int j = 0; j < LANES; ++j) {
    z[4 * j + 1] = rad0[j] * cosf(two_pi * (u20[j] - 0.25f));
    z[4 * j + 3] = rad1[j] * cosf(two_pi * (u21[j] - 0.25f));
  }
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

#define CHUNK 8192 /* samples per parallel work item (multiple of 64) */

void synth_normal_f32(uint64_t seed, uint32_t stream, uint32_t a, uint32_t b, int64_t n,
                      float mean, float std, float *out) {
  int64_t nchunks = (n + CHUNK - 1) / CHUNK;
#pragma omp parallel for schedule(static)
  for (int64_t ch = 0; ch < nchunks; ++ch) {
    int64_t e0 = ch * CHUNK, e1 = e0 + CHUNK < n ? e0 + CHUNK : n;
    for (int64_t e = e0; e < e1; e += 4 * LANES) {
      float z[4 * LANES];
      normals64(seed, stream, a, b, (uint64_t)(e >> 2), z);
      for (int j = 0; j < 4 * LANES && e + j < e1; ++j) out[e + j] = mean + std * z[j];
    }
  }
}

void synth_normal_bf16(uint64_t seed, uint32_t stream, uint32_t a, uint32_t b, int64_t n,
                       float mean, float std, uint16_t *out) {
  int64_t nchunks = (n + CHUNK - 1) / CHUNK;
#pragma omp parallel for schedule(static)
  for (int64_t ch = 0; ch < nchunks; ++ch) {
    int64_t e0 = ch * CHUNK, e1 = e0 + CHUNK < n ? e0 + CHUNK : n;
    for (int64_t e = e0; e < e1; e += 4 * LANES) {
      float z[4 * LANES];
      normals64(seed, stream, a, b, (uint64_t)(e >> 2), z);
      for (int j = 0; j < 4 * LANES && e + j < e1; ++j) out[e + j] = f32_to_bf16_rne(mean + std * z[j]);
    }
  }
}

/* fp32 -> bf16 (RNE) of an existing array, exposed so tests can pin the rounding rule */
void synth_f32_to_bf16(const float *in, int64_t n, uint16_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}
