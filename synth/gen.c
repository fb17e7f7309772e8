/*
 * Seeded synthetic input generator (host side).
 *
 * Test and benchmark infrastructure: it produces the input tensors that both
 * the GPU library and the CPU oracle consume, and holds none of the layer's
 * arithmetic.  A device twin lives in gen_gpu.hip; both follow the one
 * definition below, so a tensor (or any row block of it) is bit-identical no
 * matter which side, thread count or launch shape produced it.
 *
 * Definition (element e = r * cols + c of a tensor with key `seed`):
 *   SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
 *   generators", OOPSLA 2014): mix(z) = z ^ (z >> 31) after the two
 *   xor-shift-multiply rounds with the constants of that paper;
 *   stream value j of state s is mix(s + (j + 1) * GAMMA).
 *   key   = mix(seed + GAMMA)                       (first output of seed)
 *   h_j   = mix(key + (3e + j + 1) * GAMMA),  j = 0, 1, 2
 *   normal:  s = sum of the twelve 16-bit fields of h_0, h_1, h_2;
 *            z = (s - 393210) / 65536   (Irwin-Hall(12) - 6: mean 0, var 1,
 *            exact in fp64); v = z * sigma (fp64, round-to-nearest);
 *            f = (float)v (round-to-nearest-even); bf16 = RNE(f).
 *   ternary: t = ((h_0 >> 32) * 3) >> 32 in {0,1,2};  value t - 1 as bf16.
 *   f32 normal: (float)z.
 */
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_splitmix64_next(uint64_t *state) {
  *state += GAMMA;
  return mix64(*state);
}

static uint64_t key_of(uint64_t seed) { return mix64(seed + GAMMA); }

static double irwin_hall_z(uint64_t key, uint64_t e) {
  int64_t s = 0;
  for (uint64_t j = 0; j < 3; ++j) {
    uint64_t h = mix64(key + (3 * e + j + 1) * GAMMA);
    s += (int64_t)(h & 0xFFFF) + (int64_t)((h >> 16) & 0xFFFF) +
         (int64_t)((h >> 32) & 0xFFFF) + (int64_t)(h >> 48);
  }
  return (double)(s - 393210) * (1.0 / 65536.0);
}

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Rows [r0, r0 + nrows) of a (.. x cols) N(0, sigma^2)-like bf16 tensor, dense. */
void synth_normal_bf16_rows(uint16_t *out, uint64_t seed, double sigma, int64_t cols,
                            int64_t r0, int64_t nrows) {
  const uint64_t key = key_of(seed);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      uint64_t e = (uint64_t)(r0 + r) * (uint64_t)cols + (uint64_t)c;
      double v = irwin_hall_z(key, e) * sigma;
      out[r * cols + c] = f32_to_bf16_rne((float)v);
    }
}

/* Same index space, fp32 N(0,1)-like values (router logits). */
void synth_normal_f32_rows(float *out, uint64_t seed, int64_t cols, int64_t r0, int64_t nrows) {
  const uint64_t key = key_of(seed);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      uint64_t e = (uint64_t)(r0 + r) * (uint64_t)cols + (uint64_t)c;
      out[r * cols + c] = (float)irwin_hall_z(key, e);
    }
}

/* Same index space, values in {-1, 0, +1} (integer-exact GEMM cases). */
void synth_ternary_bf16_rows(uint16_t *out, uint64_t seed, int64_t cols, int64_t r0, int64_t nrows) {
  const uint64_t key = key_of(seed);
  static const uint16_t lut[3] = {0xBF80u, 0x0000u, 0x3F80u};
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      uint64_t e = (uint64_t)(r0 + r) * (uint64_t)cols + (uint64_t)c;
      uint64_t h = mix64(key + (3 * e + 1) * GAMMA);
      out[r * cols + c] = lut[((h >> 32) * 3) >> 32];
    }
}

/* Same index space, N(mean, sigma^2)-like bf16 values: (float)(mean + z * sigma) rounded to nearest even
 * (norm scales near one). */
void synth_affine_bf16_rows(uint16_t *out, uint64_t seed, double mean, double sigma, int64_t cols,
                            int64_t r0, int64_t nrows) {
  const uint64_t key = key_of(seed);
  for (int64_t r = 0; r < nrows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      uint64_t e = (uint64_t)(r0 + r) * (uint64_t)cols + (uint64_t)c;
      out[r * cols + c] = f32_to_bf16_rne((float)(mean + irwin_hall_z(key, e) * sigma));
    }
}

/* Dropout keep mask (the random draw of dropout, handed to both sides as an input): element e is kept iff
 * (h_0 >> 11) >= floor(p * 2^53), i.e. a 53-bit uniform at least p (kept with probability 1 - p).  Packed
 * eight columns to a byte, column c of row r in bit (c % 8) of byte r * ldk + c / 8; padding bytes are zero. */
void synth_keep_bits_rows(uint8_t *out, int64_t ldk, uint64_t seed, double p, int64_t cols, int64_t r0,
                          int64_t nrows) {
  const uint64_t key = key_of(seed);
  const uint64_t thr = (uint64_t)(p * 9007199254740992.0);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    memset(out + r * ldk, 0, (size_t)ldk);
    for (int64_t c = 0; c < cols; ++c) {
      uint64_t e = (uint64_t)(r0 + r) * (uint64_t)cols + (uint64_t)c;
      uint64_t h = mix64(key + (3 * e + 1) * GAMMA);
      if ((h >> 11) >= thr) out[r * ldk + c / 8] |= (uint8_t)(1u << (c % 8));
    }
  }
}
