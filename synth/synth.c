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
#include <pthread.h>
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
 * A parallel loop over [0, n) on nthreads threads (the caller included): fn runs on
 * contiguous slices; every thread is joined before returning, so no thread outlives
 * a call. Each element is a pure function of its index, so the thread count never
 * changes the result.
 */
typedef void (*slice_fn)(void* ctx, int64_t begin, int64_t end);
typedef struct {
  slice_fn fn;
  void* ctx;
  int64_t begin, end;
} slice_job;

static void* slice_main(void* arg) {
  slice_job* j = (slice_job*)arg;
  j->fn(j->ctx, j->begin, j->end);
  return NULL;
}

static void parallel_for(int64_t n, int nthreads, slice_fn fn, void* ctx) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if ((int64_t)nthreads > n) nthreads = n > 0 ? (int)n : 1;
  slice_job jobs[64];
  pthread_t tids[64];
  int started[64];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].begin = n * t / nthreads;
    jobs[t].end = n * (t + 1) / nthreads;
    started[t] = 0;
  }
  for (int t = 1; t < nthreads; ++t) started[t] = pthread_create(&tids[t], NULL, slice_main, &jobs[t]) == 0;
  slice_main(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) {
    if (started[t]) pthread_join(tids[t], NULL);
    else slice_main(&jobs[t]);  /* thread creation failed: run the slice here */
  }
}

typedef struct {
  uint16_t* out;
  int64_t total, cols, ld;
  uint64_t key;
  float sigma;
  const uint8_t* mask;
} normal_ctx;

static void normal_slice(void* vc, int64_t begin, int64_t end) {
  const normal_ctx* c = (const normal_ctx*)vc;
  for (int64_t p = begin; p < end; ++p) {
    uint64_t h = draw(c->key, (uint64_t)p);
    double u1 = ((double)(h >> 32) + 0.5) * (1.0 / 4294967296.0);
    double u2 = (double)(h & 0xFFFFFFFFu) * (1.0 / 4294967296.0);
    double rad = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    double nv[2] = {rad * cos(th), rad * sin(th)};
    for (int s = 0; s < 2; ++s) {
      int64_t i = 2 * p + s;
      if (i >= c->total) break;
      int64_t r = i / c->cols, col = i - r * c->cols;
      float v = (float)((double)c->sigma * nv[s]);
      if (c->mask && c->mask[col]) v = v * 20.0f;
      c->out[r * c->ld + col] = float_to_bf16_rne(v);
    }
  }
}

/*
 * out[r * ld + c] for r < rows, c < cols: bf16 bits of the seeded normal with
 * standard deviation sigma, x20 on columns where mask[c] != 0 (mask may be
 * NULL). Elements of a row beyond cols (ld > cols) are left untouched.
 */
int synth_normal_bf16(uint16_t* out, int64_t rows, int64_t cols, int64_t ld, uint64_t seed,
                      uint64_t tag, float sigma, const uint8_t* mask, int nthreads) {
  if (!out || rows < 0 || cols < 0 || ld < cols) return -1;
  normal_ctx c;
  c.out = out;
  c.total = rows * cols;
  c.cols = cols;
  c.ld = ld;
  c.key = stream_key(seed, tag);
  c.sigma = sigma;
  c.mask = mask;
  parallel_for((c.total + 1) / 2, nthreads, normal_slice, &c);
  return 0;
}

typedef struct {
  uint8_t* out;
  uint64_t key, span;
  int lo;
} bytes_ctx;

static void bytes_slice(void* vc, int64_t begin, int64_t end) {
  const bytes_ctx* c = (const bytes_ctx*)vc;
  for (int64_t i = begin; i < end; ++i) c->out[i] = (uint8_t)(c->lo + (int)(draw(c->key, (uint64_t)i) % c->span));
}

/*
 * out[i] for i < n: seeded uniform bytes in [lo, hi] (inclusive), byte i from
 * draw(key(seed, tag), i). Used for synthetic packed operands.
 */
int synth_bytes(uint8_t* out, int64_t n, uint64_t seed, uint64_t tag, int lo, int hi, int nthreads) {
  if (!out || n < 0 || lo < 0 || hi > 255 || lo > hi) return -1;
  bytes_ctx c;
  c.out = out;
  c.key = stream_key(seed, tag);
  c.span = (uint64_t)(hi - lo + 1);
  c.lo = lo;
  parallel_for(n, nthreads, bytes_slice, &c);
  return 0;
}
