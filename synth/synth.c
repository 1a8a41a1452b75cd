/*
 * synth.c - seeded, counter-based synthetic input generator.
 *
 * This module only draws numbers: it holds none of the NVFP4 method's
 * arithmetic. Both the HIP path and the CPU oracle are fed the identical bytes
 * it writes, so neither side depends on the other for its inputs.
 *
 * Definition (stable across machines; the only library calls are log, sqrt,
 * cos and sin from the C library of the machine that runs it):
 *
 *   mix64(z)        the splitmix64 output function (Steele, Lea and Flood,
 *                   "Fast splittable pseudorandom number generators", 2014).
 *   key(seed, tag)  = mix64(seed * G + mix64(tag + 1)),  G = 0x9E3779B97F4A7C15
 *   draw(key, i)    = mix64(key + (i + 1) * G)           (splitmix64 step i)
 *
 *   Normals come in Box-Muller pairs: pair p uses h = draw(key, p),
 *   u1 = ((h >> 32) + 0.5) / 2^32 in (0,1), u2 = (h & 0xffffffff) / 2^32,
 *   rad = sqrt(-2 ln u1); element 2p gets rad*cos(2 pi u2), element 2p+1 gets
 *   rad*sin(2 pi u2).  The flat element index i runs row-major over the
 *   logical [rows, cols] tensor.
 *
 *   Element value: v = (float)(sigma * n_i)  (round to nearest), then v *= 20
 *   in float when its column is an outlier channel, then round to nearest even
 *   to bfloat16.
 *
 *   Outlier channels: a Fisher-Yates shuffle of [0, cols) driven by
 *   draw(key(seed, tag), t) for t = 0, 1, ...; the first n_out entries of the
 *   shuffled order are the outlier columns.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tag) {
  return mix64(seed * GOLDEN + mix64(tag + 1));
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

static inline uint16_t float_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  /* finite inputs only: add 0x7fff plus the lsb of the kept half, then truncate */
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint64_t synth_draw(uint64_t seed, uint64_t tag, uint64_t i) {
  return draw(stream_key(seed, tag), i);
}

/* standard normal number i of stream (seed, tag), in double */
double synth_normal(uint64_t seed, uint64_t tag, uint64_t i) {
  uint64_t h = draw(stream_key(seed, tag), i >> 1);
  double u1 = ((double)(h >> 32) + 0.5) * (1.0 / 4294967296.0);
  double u2 = (double)(h & 0xFFFFFFFFu) * (1.0 / 4294967296.0);
  double rad = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? rad * sin(th) : rad * cos(th);
}

/* mask[c] = 1 for the first n_out columns of the seeded shuffle of [0, cols) */
int synth_outlier_mask(uint8_t* mask, int64_t cols, uint64_t seed, uint64_t tag, int64_t n_out) {
  if (!mask || cols <= 0 || n_out < 0 || n_out > cols) return -1;
  int64_t* perm = (int64_t*)malloc((size_t)cols * sizeof(int64_t));
  if (!perm) return -2;
  for (int64_t c = 0; c < cols; ++c) perm[c] = c;
  uint64_t key = stream_key(seed, tag);
  uint64_t t = 0;
  for (int64_t i = cols - 1; i >= 1; --i) {
    uint64_t j = draw(key, t++) % (uint64_t)(i + 1);
    int64_t tmp = perm[i];
    perm[i] = perm[j];
    perm[j] = tmp;
  }
  memset(mask, 0, (size_t)cols);
  for (int64_t c = 0; c < n_out; ++c) mask[perm[c]] = 1;
  free(perm);
  return 0;
}

/*
 * out[r * ld + c] for r < rows, c < cols: bf16 bits of the seeded normal with
 * standard deviation sigma, x20 on columns where mask[c] != 0 (mask may be
 * NULL). Elements of a row beyond cols (ld > cols) are left untouched.
 */
int synth_normal_bf16(uint16_t* out, int64_t rows, int64_t cols, int64_t ld, uint64_t seed,
                      uint64_t tag, float sigma, const uint8_t* mask, int nthreads) {
  if (!out || rows < 0 || cols < 0 || ld < cols) return -1;
  const uint64_t key = stream_key(seed, tag);
  const int64_t total = rows * cols;
  const int64_t npairs = (total + 1) / 2;
  (void)nthreads;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
  for (int64_t p = 0; p < npairs; ++p) {
    uint64_t h = draw(key, (uint64_t)p);
    double u1 = ((double)(h >> 32) + 0.5) * (1.0 / 4294967296.0);
    double u2 = (double)(h & 0xFFFFFFFFu) * (1.0 / 4294967296.0);
    double rad = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    double nv[2] = {rad * cos(th), rad * sin(th)};
    for (int s = 0; s < 2; ++s) {
      int64_t i = 2 * p + s;
      if (i >= total) break;
      int64_t r = i / cols, c = i - r * cols;
      float v = (float)((double)sigma * nv[s]);
      if (mask && mask[c]) v = v * 20.0f;
      out[r * ld + c] = float_to_bf16_rne(v);
    }
  }
  return 0;
}

/*
 * out[i] for i < n: seeded uniform bytes in [lo, hi] (inclusive), byte i from
 * draw(key(seed, tag), i). Used for synthetic packed operands.
 */
int synth_bytes(uint8_t* out, int64_t n, uint64_t seed, uint64_t tag, int lo, int hi, int nthreads) {
  if (!out || n < 0 || lo < 0 || hi > 255 || lo > hi) return -1;
  const uint64_t key = stream_key(seed, tag);
  const uint64_t span = (uint64_t)(hi - lo + 1);
  (void)nthreads;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)(lo + (int)(draw(key, (uint64_t)i) % span));
  return 0;
}
