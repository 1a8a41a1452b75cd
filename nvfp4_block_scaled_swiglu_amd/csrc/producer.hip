// producer.hip - the NVFP4 producer for gfx950: SwiGLU, plain and modulated inputs.
//
// Operation (component-2 NSYS summary: the pre-fusion chain silu -> multiply ->
// absmax_partial -> scale_finalize -> block_scale_zero -> activation_pack, whose
// "conclusion" notes that the global-scale dependency needs an explicit
// synchronisation design; "FC2 NVFP4 Scheduling Results", "Canonical Operation",
// for the formats and the 37,810 -> 37,824 row padding):
//
//   y       = RN_bf16(silu_bf16(gate) * up)          (SwiGLU mode)
//           = x                                      (plain mode)
//           = RN_bf16(fma_fp32(x, RN_fp32(1 + scale[k]), shift[k]))   (modulate mode)
//   amax    = max |y| over the logical rows, or the caller's value (GIVEN)
//   g       = amax / 2688 rounded up to fp32          (2688 = 6 * 448)
//   S[r,b]  = smallest UE4M3 byte with v(S) * 6 * g >= max_{16} |y|
//   code    = E2M1 nearest to |y| / (v(S) g), ties to even, sign of y
//   QDATA   = two codes per byte (even element low), rows [m, m_pad) zero
//   scales  = 512-byte tiles of 128 rows x 4 scale columns, padding zero
//
// Structure: two ordinary launches on the caller's stream. Each runs a persistent
// grid (one 16-wave workgroup per CU, the bf16 SiLU table in LDS) over work items of
// 64 rows x 512 columns; each lane owns one 16-element block of a row per step (a wave
// covers 2 rows x 32 blocks).
//  - The absmax launch reduces |y| with the next item's loads in flight (wavefront
//    shuffles, then LDS across waves) and writes one partial maximum per workgroup
//    into the caller's workspace.
//  - The kernel boundary is the grid-wide synchronisation the global scale needs.
//  - The quantize launch reduces the partials to amax, derives g, walks the items in
//    reverse order (so the rows the absmax launch read last, still in the memory-side
//    cache, are read first), recomputes y, and stores QDATA rows (32 lanes store one
//    full 256-byte row segment) and each scale byte at its place in its 512-byte
//    tile. It has no workgroup barrier, so the 16 waves drift apart and hide each
//    other's load latency.
// With GIVEN (amax from the caller) only the quantize launch runs: every input byte
// is read once.
//
// Exactness: every rounding decision equals the exact one.
//  - y: a product of two bf16 values is exact in fp32 when it is >= 2^-126; a block
//    with some |y| <= 2^-126 (or zero) has its nonzero subnormal products
//    recomputed in fp64 and rounded once.
//  - S: read off the bits of an fp32 estimate of bmax / 6g (relative error below
//    2^-22); estimates within 2^-17 of a grid point are settled by exact fp64
//    compares (v(e) * 6g has <= 30 significant bits).
//  - codes: the hardware fp32 -> E2M1 conversion (round to nearest even) is applied
//    to |y| * r_lo and |y| * r_hi, two brackets of the exact quotient built from a
//    1-ulp reciprocal with a 2^-20 margin; when the two codes agree the exact code
//    is that code (rounding is monotone), otherwise the element is decided by exact
//    fp64 compares against the seven midpoints.
#include "common.hpp"

namespace nvfp4 {

constexpr int kProdThreads = 1024;   // 16 waves, four per SIMD
constexpr int kWaves = kProdThreads / 64;
// A work item is 64 rows x 512 columns: each lane owns one 16-column block of a row
// per step, a wave covers 2 rows x 32 blocks (1 KB of each bf16 input row, one
// 256-byte QDATA row segment), and the 16 waves cover the 64 rows in 2 steps. Runs
// of 1 KB per row keep HBM page use and the spread of addresses over the XCDs even.
constexpr int kItemCols = 512;
constexpr int kLanesPerRow = kItemCols / 16;
constexpr int kWaveRows = 64 / kLanesPerRow;
constexpr int kRowsPerStep = kWaves * kWaveRows;
constexpr int kItemRows = 2 * kRowsPerStep;
constexpr int kRedBytes = 128;       // wave maxima and a broadcast slot
constexpr int kSteps = kItemRows / kRowsPerStep;

struct ProducerArgs {
  const uint16_t* x;  // gate (SwiGLU) or x (plain)
  const uint16_t* u;  // up (SwiGLU)
  int64_t ldx, ldu;   // row strides, elements
  int64_t m, k, m_pad;
  int64_t cpad;       // scale columns
  int items_m;        // scale row-tiles
  int items_k;        // 512-column segments
  uint8_t* qdata;
  uint8_t* scales;
  float* gout;
  const float* amax_in;  // caller-supplied amax (single-pass variant), else unused
  const uint16_t* mod_scale;  // modulation scale and shift, bf16 [k] (MODE kModulate)
  const uint16_t* mod_shift;
  uint32_t* partials;  // absmax launch: one slot per workgroup (the caller's workspace)
  int npart;           // quantize launch: slots to reduce (the absmax launch's grid)
  const uint16_t* silu_table;
};

// ---- small helpers ---------------------------------------------------------------------

__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  bf16x2_t r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

// smallest fp32 g with 2688 * g >= amax (products with 2688 = 21 * 2^7 are exact in fp64)
__device__ __forceinline__ float global_scale_from_amax(float amax) {
  if (!(amax > 0.0f)) return 0.0f;
  double a = (double)amax;
  float g = (float)(a / 2688.0);
  while ((double)g * 2688.0 < a) g = __uint_as_float(__float_as_uint(g) + 1u);
  for (;;) {
    float p = __uint_as_float(__float_as_uint(g) - 1u);
    if (p > 0.0f && (double)p * 2688.0 >= a) g = p;
    else break;
  }
  return g;
}

// Exact adjustment of a UE4M3 byte estimate e to the smallest e in [1, 126] with
// v(e) * g6 >= b (g6 = 6 g; v(e) * g6 has at most 30 significant bits, exact in fp64).
__device__ __noinline__ uint32_t block_scale_adjust(int e, double b, double g6) {
  e = e < 1 ? 1 : (e > 126 ? 126 : e);
  while (e < 126 && ue4m3_to_double((uint32_t)e) * g6 < b) ++e;
  while (e > 1 && ue4m3_to_double((uint32_t)(e - 1)) * g6 >= b) --e;
  return (uint32_t)e;
}

// Smallest UE4M3 byte e in [1, 126] with v(e) * 6g >= bmax (bmax > 0). q = bmax / (6g)
// is formed in fp32 as (bmax * bscale) * inv_f, inv_f = RN(bscale^-1 / 6g), with a
// relative error below 2^-22 whenever q is a normal number. The UE4M3 grid points are the fp32
// values whose mantissa has only its top three bits set (normal range, q >= 2^-6) and
// the multiples of 2^-9 below it, so the ceiling of q on the grid is read off q's
// bits. When q lies within 2^-17 (relative) of a grid point, or outside the range
// the method can produce, the estimate is settled by exact fp64 compares.
__device__ __forceinline__ uint32_t block_scale_byte(float bmax, float bscale, float inv_f, double g6) {
  const float q = (bmax * bscale) * inv_f;
  int e;
  bool near;
  if (q >= 0x1p-6f) {
    const uint32_t bits = __float_as_uint(q);
    const uint32_t rest = bits & 0xFFFFFu;
    // (biased exponent - 120) * 8 + top three mantissa bits, rounded up
    e = (int)((bits + 0xFFFFFu) >> 20) - 960;
    near = rest < 64u || rest > 0xFFFFFu - 64u || !(q < 0x1p+9f);
  } else {
    const float t = q * 512.0f;  // exact scaling: the grid points are the integers
    const float fl = floorf(t);
    e = (int)fl + 1;
    const float fr = t - fl;     // exact
    near = fr < 0x1p-16f || fr > 1.0f - 0x1p-16f;
  }
  if (near) return block_scale_adjust(e, (double)bmax, g6);
  return (uint32_t)(e > 126 ? 126 : e);
}

// E2M1 codes (hardware round-to-nearest-even) of the bf16 pair yb scaled by the two
// reciprocal brackets, into byte SEL of lo / hi
template <int SEL>
__device__ __forceinline__ void fp4_pair(uint32_t& lo, uint32_t& hi, uint32_t yb, float rlo, float rhi) {
  const float y0 = __uint_as_float(yb << 16);
  const float y1 = __uint_as_float(yb & 0xFFFF0000u);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, y0 * rlo, y1 * rlo, 1.0f, SEL);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, y0 * rhi, y1 * rhi, 1.0f, SEL);
}

// exact E2M1 code of a bf16 y in a block with scale byte s (> 0) and global scale g
__device__ __noinline__ uint32_t e2m1_code_exact(uint32_t y16, uint32_t s, float g) {
  uint32_t sign = (y16 >> 15) << 3;
  double a = (double)bf16_bits_to_float(y16 & 0x7FFFu);
  double unit = ue4m3_to_double(s) * (double)g;
  const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  uint32_t idx = 0;
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    double t = mid[j] * unit;  // exact
    bool up = (j & 1) ? (a >= t) : (a > t);  // ties go to the even neighbour
    if (up) idx = (uint32_t)(j + 1);
  }
  return sign | idx;
}

// Magnitude index il or il + 1 for a bf16 y whose |y| / unit lies next to the
// rounding boundary between E2M1 magnitudes il and il + 1: the exact comparison of
// |y| with that boundary times unit (exact in fp64), a tie going to the even index.
__device__ __forceinline__ uint32_t e2m1_step_exact(uint32_t y16, uint32_t s, float g, uint32_t il) {
  const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  const double a = (double)bf16_bits_to_float(y16 & 0x7FFFu);
  const double t = mid[il] * ue4m3_to_double(s) * (double)g;  // exact
  const bool up = (il & 1u) ? (a >= t) : (a > t);
  return up ? il + 1u : il;
}

// ---- the kernel ------------------------------------------------------------------------------

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// A nonzero product below 2^-126 may have been rounded in fp32: redo such products
// exactly. (A product that rounds to zero in fp32 is below 2^-149 and rounds to a
// zero of the same sign in bf16 as well.)
struct Y8 {
  uint32_t v[8];
};
__device__ __noinline__ Y8 block_y_fix(u32x4_t g0, u32x4_t g1, u32x4_t u0, u32x4_t u1, Y8 yb, const uint16_t* tab) {
  for (int j = 0; j < 16; ++j) {
    const u32x4_t& gq = j < 8 ? g0 : g1;
    const u32x4_t& uq = j < 8 ? u0 : u1;
    const uint32_t g16 = (gq[(j >> 1) & 3] >> (16 * (j & 1))) & 0xFFFFu;
    const uint32_t u16 = (uq[(j >> 1) & 3] >> (16 * (j & 1))) & 0xFFFFu;
    const float p = bf16_bits_to_float(tab[g16]) * bf16_bits_to_float(u16);
    if (fabsf(p) < 0x1p-126f && p != 0.0f) {
      const double pd = (double)bf16_bits_to_float(tab[g16]) * (double)bf16_bits_to_float(u16);
      const uint32_t y = rn_bf16_from_double(pd);
      const int sh = 16 * (j & 1);
      yb.v[j >> 1] = (yb.v[j >> 1] & ~(0xFFFFu << sh)) | (y << sh);
    }
  }
  return yb;
}

// What y is: x itself, RN_bf16(silu_bf16(gate) * up), or the adaLN-modulated
// RN_bf16(fma_fp32(x, RN_fp32(1 + scale), shift)).
constexpr int kPlain = 0, kSwiglu = 1, kModulate = 2;

// The modulated value of one bf16 element (as fp32 before the bf16 rounding).
__device__ __forceinline__ float modulate_f32(uint32_t x16, uint32_t scale16, uint32_t shift16) {
  const float m = 1.0f + bf16_bits_to_float(scale16);
  return __builtin_fmaf(bf16_bits_to_float(x16), m, bf16_bits_to_float(shift16));
}

// y for the 16 elements of one block, as 8 packed bf16 pairs. For kSwiglu, uv holds
// up; for kModulate, the item's scale (mv[0]) and shift (mv[1]) of the lane's 16
// columns. Products are formed in fp32 (exact whenever the result is a normal fp32
// number); the caller detects blocks that may hold a rounded subnormal product and
// repairs them with block_y_fix.
template <int MODE>
__device__ __forceinline__ void block_y(const u32x4_t (&gv)[2], const u32x4_t (&uv)[2],
                                        const u32x4_t (&mv)[2][2], const uint16_t* tab, uint32_t (&yb)[8]) {
  if (MODE == kModulate) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t xw = gv[w >> 2][w & 3], sw = mv[0][w >> 2][w & 3], bw = mv[1][w >> 2][w & 3];
      yb[w] = cvt_pk_bf16(modulate_f32(xw & 0xFFFFu, sw & 0xFFFFu, bw & 0xFFFFu),
                          modulate_f32(xw >> 16, sw >> 16, bw >> 16));
    }
  } else if (MODE == kSwiglu) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t gw = gv[w >> 2][w & 3], uw = uv[w >> 2][w & 3];
      const float p0 = __uint_as_float((uint32_t)tab[gw & 0xFFFFu] << 16) * __uint_as_float(uw << 16);
      const float p1 = __uint_as_float((uint32_t)tab[gw >> 16] << 16) * __uint_as_float(uw & 0xFFFF0000u);
      yb[w] = cvt_pk_bf16(p0, p1);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 8; ++w) yb[w] = gv[w >> 2][w & 3];
  }
}

typedef __attribute__((ext_vector_type(2))) unsigned short u16x2_t;

__device__ __forceinline__ u16x2_t as_u16x2(uint32_t v) {
  u16x2_t r;
  __builtin_memcpy(&r, &v, 4);
  return r;
}

// largest and smallest bf16 magnitude (bits) among the 16 elements, packed 16-bit ops
__device__ __forceinline__ void block_mag_range(const uint32_t (&yb)[8], uint32_t& mx, uint32_t& mn) {
  u16x2_t hi = as_u16x2(yb[0] & 0x7FFF7FFFu), lo = hi;
#pragma unroll
  for (int w = 1; w < 8; ++w) {
    const u16x2_t m = as_u16x2(yb[w] & 0x7FFF7FFFu);
    hi = __builtin_elementwise_max(hi, m);
    lo = __builtin_elementwise_min(lo, m);
  }
  mx = hi.x > hi.y ? hi.x : hi.y;
  mn = lo.x < lo.y ? lo.x : lo.y;
}

// The 16 bf16 values of this lane's block in each step of an item (zero outside the
// logical rows and columns). For kModulate the up slots carry the item's modulation
// instead: uv[0] = the scale and uv[1] = the shift of the lane's 16 columns.
static_assert(kSteps == 2, "modulation vectors ride in the two up slots");
template <int MODE>
__device__ __forceinline__ void load_item(const ProducerArgs& a, int item, int wave, int r4, int blk,
                                          u32x4_t (&gv)[kSteps][2], u32x4_t (&uv)[kSteps][2]) {
  const int rt = item / a.items_k, kt = item - rt * a.items_k;
  const int64_t col = (int64_t)kt * kItemCols + blk * 16;
  const u32x4_t z = {0u, 0u, 0u, 0u};
  if (MODE == kModulate) {
    const bool cok = col < a.k;
    const u32x4_t* ps = (const u32x4_t*)(a.mod_scale + col);
    const u32x4_t* pb = (const u32x4_t*)(a.mod_shift + col);
    uv[0][0] = cok ? ps[0] : z;
    uv[0][1] = cok ? ps[1] : z;
    uv[1][0] = cok ? pb[0] : z;
    uv[1][1] = cok ? pb[1] : z;
  }
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int64_t row = (int64_t)rt * kItemRows + s * kRowsPerStep + wave * kWaveRows + r4;
    const bool ok = row < a.m && col < a.k;
    const u32x4_t* px = (const u32x4_t*)(a.x + row * a.ldx + col);
    gv[s][0] = ok ? px[0] : z;
    gv[s][1] = ok ? px[1] : z;
    if (MODE == kSwiglu) {
      const u32x4_t* pu = (const u32x4_t*)(a.u + row * a.ldu + col);
      uv[s][0] = ok ? pu[0] : z;
      uv[s][1] = ok ? pu[1] : z;
    }
  }
}

// The bf16 silu table into LDS (SwiGLU only).
__device__ __forceinline__ void stage_silu_table(const uint16_t* src_tab, uint16_t* tab, int tid) {
  const u32x4_t* src = (const u32x4_t*)src_tab;
  u32x4_t* dst = (u32x4_t*)tab;
  for (int i = tid; i < 65536 * 2 / 16; i += kProdThreads) dst[i] = src[i];
  __syncthreads();
}

// Workgroup maximum of v (unsigned), returned to every thread. Uses red[0 .. kWaves].
__device__ __forceinline__ uint32_t workgroup_max_u32(uint32_t v, uint32_t* red, int tid) {
  const uint32_t wmax = wave_max_u32(v);
  if ((tid & 63) == 0) red[tid >> 6] = wmax;
  __syncthreads();
  if (tid == 0) {
    uint32_t r = 0;
    for (int i = 0; i < kWaves; ++i) r = red[i] > r ? red[i] : r;
    red[kWaves] = r;
  }
  __syncthreads();
  const uint32_t r = red[kWaves];
  __syncthreads();
  return r;
}

// ---- pass 1: the tensor absmax ------------------------------------------------------------------
//
// Each workgroup reduces max |y| over its items (every gridDim.x-th item, the next
// item's loads in flight while the current one is reduced) and writes it to its own
// slot of the workspace: the bits of a bf16 magnitude shifted into fp32 position.
// The quantize launch that follows on the same stream reduces the slots; the kernel
// boundary between the two launches is the grid-wide synchronisation the global
// scale needs.
template <int MODE>
__global__ void __launch_bounds__(kProdThreads) producer_absmax_kernel(ProducerArgs a) {
  constexpr bool SWIGLU = MODE == kSwiglu, MOD = MODE == kModulate;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint32_t* red = (uint32_t*)smem;
  uint16_t* tab = (uint16_t*)(smem + kRedBytes);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r4 = lane / kLanesPerRow;
  const int blk = lane % kLanesPerRow;
  const int nitems = a.items_m * a.items_k;
  if (SWIGLU) stage_silu_table(a.silu_table, tab, tid);

  uint32_t local_bits = 0;  // fp32 bits of a non-negative value
  // rows past m read zeros; only the modulation would turn them into nonzero y
  auto absmax_item = [&](int item, const u32x4_t (&gv)[kSteps][2], const u32x4_t (&uv)[kSteps][2]) {
    const int64_t row0 = (int64_t)(item / a.items_k) * kItemRows + wave * kWaveRows + r4;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      if (MOD && row0 + s * kRowsPerStep >= a.m) continue;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const uint32_t gw = gv[s][w >> 2][w & 3];
        if (MOD) {
          const uint32_t sw = uv[0][w >> 2][w & 3], bw = uv[1][w >> 2][w & 3];
          const float p0 = fabsf(modulate_f32(gw & 0xFFFFu, sw & 0xFFFFu, bw & 0xFFFFu));
          const float p1 = fabsf(modulate_f32(gw >> 16, sw >> 16, bw >> 16));
          const uint32_t b = __float_as_uint(fmaxf(p0, p1));
          local_bits = b > local_bits ? b : local_bits;
        } else if (SWIGLU) {
          const uint32_t uw = uv[s][w >> 2][w & 3];
          const float s0 = __uint_as_float((uint32_t)tab[gw & 0xFFFFu] << 16);
          const float s1 = __uint_as_float((uint32_t)tab[gw >> 16] << 16);
          const float p0 = fabsf(s0 * __uint_as_float(uw << 16));
          const float p1 = fabsf(s1 * __uint_as_float(uw & 0xFFFF0000u));
          const uint32_t b = __float_as_uint(fmaxf(p0, p1));
          local_bits = b > local_bits ? b : local_bits;
        } else {
          const uint32_t m0 = gw & 0x7FFFu, m1 = (gw >> 16) & 0x7FFFu;
          const uint32_t b = (m0 > m1 ? m0 : m1) << 16;
          local_bits = b > local_bits ? b : local_bits;
        }
      }
    }
  };
  {
    u32x4_t gA[kSteps][2], uA[kSteps][2], gB[kSteps][2], uB[kSteps][2];
    int item = blockIdx.x;
    if (item < nitems) load_item<MODE>(a, item, wave, r4, blk, gA, uA);
    while (item < nitems) {
      const int n1 = item + (int)gridDim.x;
      if (n1 < nitems) load_item<MODE>(a, n1, wave, r4, blk, gB, uB);
      absmax_item(item, gA, uA);
      item = n1;
      if (item >= nitems) break;
      const int n2 = item + (int)gridDim.x;
      if (n2 < nitems) load_item<MODE>(a, n2, wave, r4, blk, gA, uA);
      absmax_item(item, gB, uB);
      item = n2;
    }
  }
  // workgroup max of the unrounded |products| (SwiGLU) or of |x|
  local_bits = workgroup_max_u32(local_bits, red, tid);
  // A product below 2^-126 may have been rounded in fp32; if this workgroup's maximum
  // is such a product, redo its elements exactly (never taken for inputs whose absmax
  // is a normal number).
  if (SWIGLU && local_bits != 0 && local_bits < 0x00800000u) {
    uint32_t best = 0;  // bf16 magnitude bits
    for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
      u32x4_t gv[kSteps][2], uv[kSteps][2];
      load_item<MODE>(a, item, wave, r4, blk, gv, uv);
      for (int s = 0; s < kSteps; ++s)
        for (int j = 0; j < 16; ++j) {
          const uint32_t g16 = (gv[s][j >> 3][(j >> 1) & 3] >> (16 * (j & 1))) & 0xFFFFu;
          const uint32_t u16 = (uv[s][j >> 3][(j >> 1) & 3] >> (16 * (j & 1))) & 0xFFFFu;
          const double p = (double)bf16_bits_to_float(tab[g16]) * (double)bf16_bits_to_float(u16);
          const uint32_t y = rn_bf16_from_double(p) & 0x7FFFu;
          best = y > best ? y : best;
        }
    }
    local_bits = workgroup_max_u32(best, red, tid) << 16;
  } else if (SWIGLU || MOD) {
    // RN_bf16 is monotone, so the rounded maximum is the maximum of the rounded values.
    local_bits = (cvt_pk_bf16(__uint_as_float(local_bits), 0.0f) & 0xFFFFu) << 16;
  }
  if (tid == 0) a.partials[blockIdx.x] = local_bits;
}

// ---- pass 2: scales, codes, pack, swizzle ---------------------------------------------------------
//
// GIVEN: the tensor amax comes from the caller (a device float). Otherwise it is the
// maximum of the absmax launch's a.npart workgroup partials.
template <int MODE, bool GIVEN>
__global__ void __launch_bounds__(kProdThreads) producer_kernel(ProducerArgs a) {
  constexpr bool SWIGLU = MODE == kSwiglu, MOD = MODE == kModulate;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint32_t* red = (uint32_t*)smem;                          // wave maxima + a broadcast slot
  uint16_t* tab = (uint16_t*)(smem + kRedBytes);            // 65,536 entries (SwiGLU only)

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r4 = lane / kLanesPerRow;   // row within the wave's rows of a step
  const int blk = lane % kLanesPerRow;  // 16-column block of the item's column segment
  const int nitems = a.items_m * a.items_k;
  if (SWIGLU) stage_silu_table(a.silu_table, tab, tid);

  float amax;
  if constexpr (GIVEN) {
    amax = a.amax_in[0];
  } else {
    uint32_t v = 0;
    for (int i = tid; i < a.npart; i += kProdThreads) {
      const uint32_t p = a.partials[i];
      v = p > v ? p : v;
    }
    amax = __uint_as_float(workgroup_max_u32(v, red, tid));
  }
  const float g = global_scale_from_amax(amax);
  const double g6 = 6.0 * (double)g;
  // 1 / (6g) in fp32; for a tiny g both factors of bmax / (6g) are scaled by 2^64 (exact)
  double inv_g6 = g6 > 0.0 ? 1.0 / g6 : 0.0;
  float bscale = 1.0f;
  if (inv_g6 > 0x1p+100) {
    inv_g6 *= 0x1p-64;
    bscale = 0x1p+64f;
  }
  const float inv_f = (float)inv_g6;
  if (blockIdx.x == 0 && tid == 0) *a.gout = g;

  const int64_t qrow_bytes = a.k / 2;
  auto quantize_item = [&](int item, const u32x4_t (&gv)[kSteps][2], const u32x4_t (&uv)[kSteps][2]) {
    const int rt = item / a.items_k, kt = item - rt * a.items_k;
    const int64_t col = (int64_t)kt * kItemCols + blk * 16;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int lrow = s * kRowsPerStep + wave * kWaveRows + r4;
      const int64_t row = (int64_t)rt * kItemRows + lrow;
      uint32_t yb[8];
      block_y<MODE>(gv[s], uv[s], uv, tab, yb);
      if (MOD && row >= a.m) {
#pragma unroll
        for (int w = 0; w < 8; ++w) yb[w] = 0u;  // padding rows are zero, not the shift
      }
      // block maximum of |y| (bf16 magnitudes compare as integers)
      uint32_t mx, mn;
      block_mag_range(yb, mx, mn);
      if (SWIGLU && mn <= 0x0080u) {
        // some |y| <= 2^-126 (or zero): its fp32 product may have been subnormal and
        // rounded; redo such products exactly
        Y8 y;
#pragma unroll
        for (int w = 0; w < 8; ++w) y.v[w] = yb[w];
        y = block_y_fix(gv[s][0], gv[s][1], uv[s][0], uv[s][1], y, tab);
#pragma unroll
        for (int w = 0; w < 8; ++w) yb[w] = y.v[w];
        block_mag_range(yb, mx, mn);
      }
      const uint32_t S = (mx == 0) ? 0u : block_scale_byte(bf16_bits_to_float(mx), bscale, inv_f, g6);

      // E2M1 codes of the 16 elements
      const float unit = ue4m3_to_float(S) * g;
      const bool exact_block = (S != 0) && !(unit >= 0x1p-100f);
      const float rcp = (S == 0) ? 1.0f : __builtin_amdgcn_rcpf(unit);
      const float rlo = rcp * (1.0f - 0x1p-20f);
      const float rhi = rcp * (1.0f + 0x1p-20f);
      uint32_t clo0 = 0, chi0 = 0, clo1 = 0, chi1 = 0;
      fp4_pair<0>(clo0, chi0, yb[0], rlo, rhi);
      fp4_pair<1>(clo0, chi0, yb[1], rlo, rhi);
      fp4_pair<2>(clo0, chi0, yb[2], rlo, rhi);
      fp4_pair<3>(clo0, chi0, yb[3], rlo, rhi);
      fp4_pair<0>(clo1, chi1, yb[4], rlo, rhi);
      fp4_pair<1>(clo1, chi1, yb[5], rlo, rhi);
      fp4_pair<2>(clo1, chi1, yb[6], rlo, rhi);
      fp4_pair<3>(clo1, chi1, yb[7], rlo, rhi);
      if (exact_block) {
        uint32_t c[2] = {0u, 0u};
        for (int j = 0; j < 16; ++j) {
          const uint32_t y16 = (yb[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
          c[j >> 3] |= e2m1_code_exact(y16, S, g) << (4 * (j & 7));
        }
        clo0 = c[0];
        clo1 = c[1];
      } else if ((clo0 ^ chi0) | (clo1 ^ chi1)) {
        // The two bracket codes differ only where |y| / unit lies within the bracket of
        // an E2M1 rounding boundary: there the code is one of two neighbours, decided
        // by one exact comparison with that boundary (the other elements keep theirs).
        uint64_t d = ((uint64_t)(clo1 ^ chi1) << 32) | (clo0 ^ chi0);
        while (d) {
          const int j = (int)(__builtin_ctzll(d) >> 2);  // element 0..15
          d &= ~(0xFull << (4 * j));
          const uint32_t y16 = (yb[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
          const uint32_t sh = 4 * (j & 7);
          const uint32_t nl = ((j < 8 ? clo0 : clo1) >> sh) & 15u, nh = ((j < 8 ? chi0 : chi1) >> sh) & 15u;
          const uint32_t il = nl & 7u, ih = nh & 7u;
          uint32_t code;
          if (ih == il + 1u) {
            code = ((y16 >> 15) << 3) | e2m1_step_exact(y16, S, g, il);
          } else {
            code = e2m1_code_exact(y16, S, g);
          }
          if (j < 8) clo0 = (clo0 & ~(15u << sh)) | (code << sh);
          else clo1 = (clo1 & ~(15u << sh)) | (code << sh);
        }
      }
      if (row < a.m_pad && col < a.k) {
        const u32x2_t v = {clo0, clo1};
        *(u32x2_t*)(a.qdata + row * qrow_bytes + col / 2) = v;
      }
      // the scale byte at its place in its 128 x 4 tile (rows past m_pad hold zero)
      if (col < a.k) {
        const int64_t bc = (int64_t)kt * kLanesPerRow + blk;  // block column
        const int64_t tile = (row >> 7) * (a.cpad / 4) + (bc >> 2);
        a.scales[tile * 512 + (row & 31) * 16 + ((row >> 5) & 3) * 4 + (bc & 3)] = (uint8_t)S;
      }
    }
  };
  // Items in reverse order: the rows the absmax launch read last, still in the
  // memory-side cache, are read first. No workgroup barrier: the 16 waves drift apart
  // and hide each other's load latency.
  for (int item = nitems - 1 - (int)blockIdx.x; item >= 0; item -= (int)gridDim.x) {
    u32x4_t gv[kSteps][2], uv[kSteps][2];
    load_item<MODE>(a, item, wave, r4, blk, gv, uv);
    quantize_item(item, gv, uv);
  }
}

// ---- host side --------------------------------------------------------------------------------

size_t producer_smem_bytes(int mode) {
  return kRedBytes + (mode == kSwiglu ? 65536 * 2 : 0);
}

const void* producer_kernel_ptr(int mode, bool given) {
  if (mode == kSwiglu)
    return given ? (const void*)producer_kernel<kSwiglu, true> : (const void*)producer_kernel<kSwiglu, false>;
  if (mode == kModulate)
    return given ? (const void*)producer_kernel<kModulate, true> : (const void*)producer_kernel<kModulate, false>;
  return given ? (const void*)producer_kernel<kPlain, true> : (const void*)producer_kernel<kPlain, false>;
}

const void* producer_absmax_kernel_ptr(int mode) {
  if (mode == kSwiglu) return (const void*)producer_absmax_kernel<kSwiglu>;
  if (mode == kModulate) return (const void*)producer_absmax_kernel<kModulate>;
  return (const void*)producer_absmax_kernel<kPlain>;
}

int producer_block_threads() { return kProdThreads; }

// amax_in == nullptr: the two-pass producer (absmax launch into the workspace's
// partials, then the quantize launch); otherwise the single-read producer with the
// caller's amax (the quantize launch alone). Both are ordinary launches of at most
// max_blocks (<= kMaxPartials) workgroups.
hipError_t launch_producer(int mode, const uint16_t* x, int64_t ldx, const uint16_t* u, int64_t ldu,
                           const uint16_t* mod_scale, const uint16_t* mod_shift, int64_t m, int64_t k,
                           uint8_t* qdata, uint8_t* scales, float* gout, const float* amax_in, void* workspace,
                           const uint16_t* silu_table, int max_blocks, hipStream_t stream) {
  ProducerArgs args;
  args.x = x;
  args.u = u;
  args.ldx = ldx;
  args.ldu = ldu;
  args.m = m;
  args.k = k;
  args.m_pad = (m + 15) / 16 * 16;
  args.cpad = (k / 16 + 3) / 4 * 4;
  const int64_t scale_rows = (args.m_pad + 127) / 128 * 128;
  args.items_m = (int)(scale_rows / kItemRows);
  args.items_k = (int)((k + kItemCols - 1) / kItemCols);
  args.qdata = qdata;
  args.scales = scales;
  args.gout = gout;
  args.amax_in = amax_in;
  args.mod_scale = mod_scale;
  args.mod_shift = mod_shift;
  args.partials = workspace ? ((ProducerWorkspace*)workspace)->partial : nullptr;
  args.npart = 0;
  args.silu_table = silu_table;
  const int64_t nitems = (int64_t)args.items_m * args.items_k;
  if (max_blocks > kMaxPartials) max_blocks = kMaxPartials;
  int blocks = (int)(nitems < max_blocks ? nitems : max_blocks);
  if (blocks < 1) blocks = 1;
  const size_t smem = producer_smem_bytes(mode);
  if (amax_in) {
    void* kargs[] = {&args};
    return hipLaunchKernel(producer_kernel_ptr(mode, true), dim3(blocks), dim3(kProdThreads), kargs, smem, stream);
  }
  {
    void* kargs[] = {&args};
    hipError_t e = hipLaunchKernel(producer_absmax_kernel_ptr(mode), dim3(blocks), dim3(kProdThreads), kargs, smem,
                                   stream);
    if (e != hipSuccess) return e;
  }
  args.npart = blocks;
  void* kargs[] = {&args};
  return hipLaunchKernel(producer_kernel_ptr(mode, false), dim3(blocks), dim3(kProdThreads), kargs, smem, stream);
}

}  // namespace nvfp4
