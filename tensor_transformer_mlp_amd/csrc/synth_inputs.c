/*
 * Seeded synthetic inputs for the tensor-parallel MLP shard forward.
 *
 * This file generates random numbers and rounds them to the storage type; it
 * holds none of the MLP's arithmetic.  Both the GPU path and the CPU oracle are
 * fed from what it writes, so that they see bit-identical inputs.
 *
 * Bit source: Philox4x64-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11),
 * written here from that paper's definition (ten rounds of two 64x64->128-bit
 * multiplies, a key schedule bumped by the two Weyl constants).  Its raw
 * output is checked in the tests against numpy.random.Philox, an independent
 * implementation of the same generator.
 *
 * Element e of stream s under seed q takes Philox block counter (e / 4, 0, 0, 0)
 * with key (q, s).  The block's four 64-bit words give two uniform pairs in
 * (0, 1) (53-bit mantissa, offset by half an ulp so that 0 never occurs), and
 * each pair gives two standard normals by the Box-Muller transform
 * (Box & Muller, 1958).  Element e takes normal number (e % 4) of its block.
 * Because every element depends only on (q, s, e), any slice can be drawn on
 * its own and the result does not depend on the thread count.
 *
 * The normal is computed in double, multiplied by the standard deviation,
 * rounded to float32, and for bfloat16 storage rounded once more, to nearest
 * with ties to even, keeping the upper 16 bits of the float32 pattern.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2E7470EE14C6C93ULL
#define PHILOX_M1 0xCA5A826395121157ULL
#define PHILOX_W0 0x9E3779B97F4A7C15ULL
#define PHILOX_W1 0xBB67AE8584CAA73BULL

static inline void mul_hilo(uint64_t a, uint64_t b, uint64_t* hi, uint64_t* lo) {
  unsigned __int128 p = (unsigned __int128)a * (unsigned __int128)b;
  *hi = (uint64_t)(p >> 64);
  *lo = (uint64_t)p;
}

/* One Philox4x64 block with `rounds` rounds: ctr[4], key[2] -> out[4]. */
void synth_philox4x64(const uint64_t ctr[4], const uint64_t key[2], int rounds,
                      uint64_t out[4]) {
  uint64_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint64_t k0 = key[0], k1 = key[1];
  for (int r = 0; r < rounds; ++r) {
    if (r > 0) {
      k0 += PHILOX_W0;
      k1 += PHILOX_W1;
    }
    uint64_t hi0, lo0, hi1, lo1;
    mul_hilo(PHILOX_M0, c0, &hi0, &lo0);
    mul_hilo(PHILOX_M1, c2, &hi1, &lo1);
    uint64_t n0 = hi1 ^ c1 ^ k0;
    uint64_t n1 = lo1;
    uint64_t n2 = hi0 ^ c3 ^ k1;
    uint64_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline double u53(uint64_t x) {
  /* (0, 1): top 53 bits plus half an ulp. */
  return ((double)(x >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static void normals_of_block(uint64_t seed, uint64_t stream, uint64_t block, double z[4]) {
  const double two_pi = 6.283185307179586476925286766559;
  uint64_t ctr[4] = {block, 0, 0, 0};
  uint64_t key[2] = {seed, stream};
  uint64_t w[4];
  synth_philox4x64(ctr, key, 10, w);
  for (int p = 0; p < 2; ++p) {
    double u1 = u53(w[2 * p]);
    double u2 = u53(w[2 * p + 1]);
    double r = sqrt(-2.0 * log(u1));
    double t = two_pi * u2;
    z[2 * p] = r * cos(t);
    z[2 * p + 1] = r * sin(t);
  }
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Raw standard normals (double) for elements [first, first + n) of a stream. */
void synth_normal_f64(uint64_t seed, uint64_t stream, int64_t first, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int64_t e = first + i;
    double z[4];
    normals_of_block(seed, stream, (uint64_t)(e >> 2), z);
    out[i] = z[e & 3];
  }
}

/* N(0, std) rounded to float32, elements [first, first + n). */
void synth_normal_f32(uint64_t seed, uint64_t stream, int64_t first, int64_t n, double std_,
                      float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t blk = (first >> 2); blk <= ((first + n - 1) >> 2); ++blk) {
    double z[4];
    normals_of_block(seed, stream, (uint64_t)blk, z);
    for (int j = 0; j < 4; ++j) {
      int64_t e = blk * 4 + j;
      if (e < first || e >= first + n) continue;
      out[e - first] = (float)(z[j] * std_);
    }
  }
}

/* N(0, std) rounded to float32, then to bfloat16 (RNE); raw bit patterns. */
void synth_normal_bf16(uint64_t seed, uint64_t stream, int64_t first, int64_t n, double std_,
                       uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t blk = (first >> 2); blk <= ((first + n - 1) >> 2); ++blk) {
    double z[4];
    normals_of_block(seed, stream, (uint64_t)blk, z);
    for (int j = 0; j < 4; ++j) {
      int64_t e = blk * 4 + j;
      if (e < first || e >= first + n) continue;
      out[e - first] = f32_to_bf16_rne((float)(z[j] * std_));
    }
  }
}

/* float32 -> bfloat16 (RNE) over an array; exposed so the tests can check it. */
void synth_round_bf16(const float* in, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}

/* SHA-256 of this file's text, passed on the compiler command line by the
   build, so that the loader can refuse a library built from an older copy
   of the source. */
#ifndef SYNTH_SOURCE_SHA256
#define SYNTH_SOURCE_SHA256 "unknown"
#endif
const char* synth_source_sha256(void) { return SYNTH_SOURCE_SHA256; }
