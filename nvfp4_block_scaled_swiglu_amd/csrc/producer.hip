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
// Work is cut into units of 4 rows x 512 columns; a wave takes a unit in two steps
// of 2 rows, each lane owning one 16-element block of a row per step (1 KB runs of
// each input row per step).
//
// Two ordinary launches on the caller's stream:
//  - The absmax launch is a one-shot grid of 8-wave workgroups (one unit per wave),
//    dispatched in address order. It keeps no table in LDS: for SwiGLU, every |y| is
//    bounded by max(gate, 0.28125) * |up|, and silu_bf16 is the identity for
//    gate >= 8, so a log-domain screen on the bits leaves only the elements whose
//    bound can reach the wave's exact maximum to be looked up in the device silu
//    table in global memory. Each workgroup folds its maximum into one of the
//    workspace's 64 slots by atomic max.
//  - The kernel boundary is the grid-wide synchronisation the global scale needs.
//  - The quantize launch runs one persistent 12-wave workgroup per CU with the bf16
//    silu table in LDS. Its waves work through pieces (groups of 4 units, or half
//    groups near the end): a fixed one each, then pieces taken from 32 interleaved
//    run-time counters (takes issued one piece ahead), in reverse address order, so
//    that the rows the absmax launch read last come first and the whole grid moves
//    through memory together. It reduces the slots to amax, derives g, recomputes y,
//    and stores QDATA rows (32 lanes store one 256-byte row segment) and, per group,
//    each row's 16 scale bytes of each tile (gathered from the tile's 4 lanes) with
//    one store (8 bytes per half piece). Its last workgroup clears the counters and
//    the slots for the next call.
// With GIVEN (amax from the caller) only the quantize launch runs: every input byte
// is read once.
//
// Exactness: every rounding decision equals the exact one.
//  - y: a product of two bf16 values is exact in fp32 when it is >= 2^-126; smaller
//    nonzero products are recomputed in fp64 and rounded once.
//  - S: read off the bits of an fp32 estimate of bmax / 6g (relative error below
//    2^-22); estimates within 2^-17 of a grid point are settled by exact fp64
//    compares (v(e) * 6g has <= 30 significant bits).
//  - codes: the hardware fp32 -> E2M1 conversion (round to nearest even) is applied
//    to |y| * r_lo and |y| * r_hi, two brackets of the exact quotient built from a
//    1-ulp reciprocal with a 2^-20 margin; when the two codes agree the exact code
//    is that code (rounding is monotone). Otherwise the codes are neighbours i and
//    i + 1, and the sign of fma(mid_i * v(S), g, -|y|) decides (mid_i * v(S) has at
//    most 7 significant bits, and for unit >= 2^-90 the exact difference, when not
//    zero, is a normal fp32 number, so the fused result has the exact sign); a tie
//    goes to the even code. Smaller units use exact fp64 compares.
#include "common.hpp"

namespace nvfp4 {

constexpr int kUnitRows = 4;
constexpr int kUnitCols = 512;
constexpr int kSteps = 2;                   // steps of 2 rows per unit
constexpr int kLanesPerRow = kUnitCols / 16;
constexpr int kAbsWaves = 8;                // absmax workgroup: 8 waves, one unit each
constexpr int kQuantWaves = 12;             // quantize workgroup: 12 waves, persistent
constexpr int kGroupUnits = 4;              // units per queue take (one 64-byte scale line's rows)
static_assert(kLanesPerRow * 2 == 64 && kSteps * 2 == kUnitRows, "unit geometry");

struct ProducerArgs {
  const uint16_t* x;  // gate (SwiGLU) or x (plain, modulate)
  const uint16_t* u;  // up (SwiGLU)
  int64_t ldx, ldu;   // row strides, elements
  int64_t m, k, m_pad;
  int64_t cpad;       // scale columns
  int items_k;        // 512-column segments
  int nunits;         // (scale rows / 4) * items_k
  uint8_t* qdata;
  uint8_t* scales;
  float* gout;
  const float* amax_in;       // caller-supplied amax (GIVEN), else unused
  const uint16_t* mod_scale;  // modulation scale and shift, bf16 [k] (MODE kModulate)
  const uint16_t* mod_shift;
  uint32_t* slots;            // the workspace's absmax slots (two-pass), else null
  uint32_t* queue;            // the quantize launch's counter set
  const uint16_t* silu_table; // the device silu table (65,536 bf16)
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


// ---- unit loads ------------------------------------------------------------------------
//
// Where a lane works in the quantize launch: after the lane swaps, lane l holds the
// 16-element block l mod 32 of row l / 32 of each step.
struct LaneGeom {
  int r4, blk;  // row within a step (0, 1), 16-column block of the unit (0 .. 31)
};

__device__ __forceinline__ LaneGeom lane_geom(int lane) {
  LaneGeom L;
  L.r4 = lane / kLanesPerRow;
  L.blk = lane % kLanesPerRow;
  return L;
}

template <int MODE>
__device__ __forceinline__ void load_unit(const ProducerArgs& a, const LaneGeom& L, int uu, u32x4_t (&gv)[kSteps][2],
                                          u32x4_t (&uv)[kSteps][2]) {
  constexpr bool SWIGLU = MODE == kSwiglu;
  const int rt = uu / a.items_k, kt = uu - rt * a.items_k;
  const int64_t row0 = (int64_t)rt * kUnitRows;
  const int64_t col0 = (int64_t)kt * kUnitCols;
  // Each load instruction reads one row's whole 1 KB segment of the unit, non-temporal:
  // lane l takes bytes [32 (l mod 32) + 16 (l / 32), +16), the first or second half of
  // the 16-element block l mod 32. Row r lands in gv[r / 2][r % 2] as loaded;
  // arrange_unit later hands every lane its whole blocks.
  // The eight loads have no condition: rows past the tensor read its last row and
  // columns past it its last 8 columns (the caller zeroes such rows and stores nothing
  // for such columns). With no branch around them, the compiler knows how many loads
  // are in flight behind each one and waits for no more than it needs.
  int64_t col = col0 + L.blk * 16 + L.r4 * 8;
  col = col < a.k - 8 ? col : a.k - 8;
#pragma unroll
  for (int r = 0; r < kUnitRows; ++r) {
    const int64_t row = row0 + r < a.m ? row0 + r : a.m - 1;  // wave-uniform
    gv[r >> 1][r & 1] = __builtin_nontemporal_load((const u32x4_t*)(a.x + row * a.ldx + col));
    if (SWIGLU) uv[r >> 1][r & 1] = __builtin_nontemporal_load((const u32x4_t*)(a.u + row * a.ldu + col));
  }
}

// One permlane32 swap per dword between the two rows of a step turns load_unit's rows
// into blocks: afterwards gv[s][h] holds, in lanes 0-31, the step's first row and, in
// lanes 32-63, its second, 16 whole elements per lane (h: first or second 8). Done when
// the unit is about to be quantized, so that the wait for its loads comes as late as
// possible.
template <int MODE>
__device__ __forceinline__ void arrange_unit(u32x4_t (&gv)[kSteps][2], u32x4_t (&uv)[kSteps][2]) {
#pragma unroll
  for (int s = 0; s < kSteps; ++s)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const auto px = __builtin_amdgcn_permlane32_swap(gv[s][0][d], gv[s][1][d], false, false);
      gv[s][0][d] = px[0];
      gv[s][1][d] = px[1];
      if (MODE == kSwiglu) {
        const auto pu = __builtin_amdgcn_permlane32_swap(uv[s][0][d], uv[s][1][d], false, false);
        uv[s][0][d] = pu[0];
        uv[s][1][d] = pu[1];
      }
    }
}

// Zero the arranged blocks of the rows at or past m (row0: the unit's first row; lanes
// 32-63 hold the second row of each step).
template <int MODE>
__device__ __forceinline__ void zero_tail_rows(const ProducerArgs& a, int64_t row0, int lane,
                                               u32x4_t (&gv)[kSteps][2], u32x4_t (&uv)[kSteps][2]) {
  const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int s = 0; s < kSteps; ++s)
    if (row0 + 2 * s + (lane >> 5) >= a.m) {
      gv[s][0] = z;
      gv[s][1] = z;
      if (MODE == kSwiglu) {
        uv[s][0] = z;
        uv[s][1] = z;
      }
    }
}

// The modulation scale (mv[0]) and shift (mv[1]) of the lane's 16 columns of unit uu.
__device__ __forceinline__ void load_modulation(const ProducerArgs& a, const LaneGeom& L, int uu,
                                                u32x4_t (&mv)[2][2]) {
  const int kt = uu % a.items_k;
  int64_t col = (int64_t)kt * kUnitCols + L.blk * 16;
  col = col < a.k - 16 ? col : a.k - 16;  // blocks past the columns are never stored
  const u32x4_t* ps = (const u32x4_t*)(a.mod_scale + col);
  const u32x4_t* pb = (const u32x4_t*)(a.mod_shift + col);
  mv[0][0] = ps[0];
  mv[0][1] = ps[1];
  mv[1][0] = pb[0];
  mv[1][1] = pb[1];
}

// ---- pass 1: the tensor absmax -----------------------------------------------------------

// |y| of one SwiGLU element exactly, as the fp32 bits of a bf16 magnitude. For
// gate >= 8, silu_bf16(gate) = gate (1 - sigma(8) < 3.4e-4, under half a bf16 ulp of 8),
// so the table is not read; a product below 2^-126 is formed in fp64 and rounded once.
__device__ __forceinline__ uint32_t swiglu_abs_bits(const uint16_t* __restrict__ tab, uint32_t g16, uint32_t u16) {
  const float gf = bf16_bits_to_float(g16);
  const float s = gf >= 8.0f ? gf : bf16_bits_to_float(tab[g16]);
  const float uf = bf16_bits_to_float(u16);
  const float p = fabsf(s * uf);
  if (p != 0.0f && p < 0x1p-126f) return (rn_bf16_from_double((double)s * (double)uf) & 0x7FFFu) << 16;
  return (cvt_pk_bf16(p, 0.0f) & 0x7FFFu) << 16;
}

typedef __attribute__((ext_vector_type(2))) short i16x2_t;

// The screening key of each element pair: S = bits(G) + bits(|u|) per half, with
// G = max(gate, 0.28125) (bf16 bits; a signed 16-bit max, since 0.28125 > 0 and
// negative bf16 values are negative as int16). S fits 16 bits (<= 0x7F7F + 0x7F7F).
__device__ __forceinline__ uint32_t swiglu_key(uint32_t gw, uint32_t uw) {
  i16x2_t gi;
  __builtin_memcpy(&gi, &gw, 4);
  const i16x2_t floor_bits = {0x3E90, 0x3E90};  // 0.28125
  const i16x2_t G = __builtin_elementwise_max(gi, floor_bits);
  u16x2_t gu;
  __builtin_memcpy(&gu, &G, 4);
  const u16x2_t S = gu + as_u16x2(uw & 0x7FFF7FFFu);
  uint32_t r;
  __builtin_memcpy(&r, &S, 4);
  return r;
}

// Exact max |y| over the lane's elements whose key lies in [lo, hi).
__device__ __forceinline__ uint32_t swiglu_scan(const uint16_t* __restrict__ tab, const u32x4_t (&gv)[kSteps][2],
                                                const u32x4_t (&uv)[kSteps][2], const uint32_t (&key)[kSteps][8],
                                                uint32_t lo, uint32_t hi) {
  uint32_t m = 0;
#pragma unroll
  for (int s = 0; s < kSteps; ++s)
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t k0 = key[s][w] & 0xFFFFu, k1 = key[s][w] >> 16;
      const bool c0 = k0 >= lo && k0 < hi, c1 = k1 >= lo && k1 < hi;
      if (c0 || c1) {
        const uint32_t gw = gv[s][w >> 2][w & 3], uw = uv[s][w >> 2][w & 3];
        if (c0) {
          const uint32_t v = swiglu_abs_bits(tab, gw & 0xFFFFu, uw & 0xFFFFu);
          m = v > m ? v : m;
        }
        if (c1) {
          const uint32_t v = swiglu_abs_bits(tab, gw >> 16, uw >> 16);
          m = v > m ? v : m;
        }
      }
    }
  return m;
}

// max |y| of one SwiGLU unit held by a wave, exactly (fp32 bits of a bf16 magnitude;
// the same value in every lane), screened in the log domain:
//   |y| = RN_bf16(|silu_bf16(g)| |u|) <= RN_bf16(B), B = max(g, 0.28125) |u|, since
//   silu(g) < g for g > 0 and |silu(g)| <= 0.2785 for g <= 0, kept by the rounding.
//   For finite x, log2 x <= bits(x) / 128 - 127 + 0.0861 (0.0861 = max of
//   log2(1 + t) - t on [0, 1); bf16 subnormals and zero satisfy it without the term),
//   so log2 B <= S / 128 - 254 + 0.1722; and for a normal bf16 value M,
//   log2 M >= bits(M) / 128 - 127. Hence S <= bits(M) + 16233 implies B < M and
//   |y| <= M: such elements cannot raise an exact maximum M.
// The elements within 23 of the wave's largest key are evaluated exactly (the likely
// maximum); then every element whose key still reaches bits(M) + 16234 is; if M is
// below 2^-126 (or zero), every element is.
__device__ __forceinline__ uint32_t swiglu_unit_absmax(const uint16_t* __restrict__ tab, const u32x4_t (&gv)[kSteps][2],
                                                       const u32x4_t (&uv)[kSteps][2]) {
  uint32_t key[kSteps][8];
  u16x2_t kmax = {0, 0};
#pragma unroll
  for (int s = 0; s < kSteps; ++s)
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      key[s][w] = swiglu_key(gv[s][w >> 2][w & 3], uv[s][w >> 2][w & 3]);
      kmax = __builtin_elementwise_max(kmax, as_u16x2(key[s][w]));
    }
  const uint32_t lmax = kmax.x > kmax.y ? kmax.x : kmax.y;
  const uint32_t top = wave_max_u32(lmax);
  const uint32_t t1 = top - 23u;  // keys are >= 0x3E90, so no wrap
  uint32_t m = 0;
  if (lmax >= t1) m = swiglu_scan(tab, gv, uv, key, t1, 0x10000u);
  m = wave_max_u32(m);
  const uint32_t mb = m >> 16;  // bf16 bits of the exact maximum so far
  if (mb < 0x0080u) {
    // the maximum so far is subnormal or zero: the bound argument needs a normal M
    const uint32_t m2 = swiglu_scan(tab, gv, uv, key, 0u, t1);
    m = wave_max_u32(m2 > m ? m2 : m);
  } else {
    const uint32_t t2 = mb + 16234u;
    if (t2 < t1) {
      uint32_t m2 = 0;
      if (lmax >= t2) m2 = swiglu_scan(tab, gv, uv, key, t2, t1);
      m = wave_max_u32(m2 > m ? m2 : m);
    }
  }
  return m;
}

// The absmax launch reads a unit row by row: load instruction r takes row r's 1 KB
// segment of each input in one contiguous piece (lane L: columns 8L .. 8L + 7), with
// non-temporal loads, since nothing here is read twice. Measured on MI355X after the
// FC2 GEMM, this streams gate and up about 10 % faster than 32 bytes per lane in two
// interleaved loads; the maximum does not care which lane holds which element. gv[s][h]
// holds unit row 2s + h (zero outside the logical rows and columns); mv, for kModulate,
// the scale and shift of the lane's 8 columns.
template <int MODE>
__device__ __forceinline__ void load_unit_rows(const ProducerArgs& a, int lane, int uu, u32x4_t (&gv)[kSteps][2],
                                               u32x4_t (&uv)[kSteps][2], u32x4_t (&mv)[2]) {
  constexpr bool SWIGLU = MODE == kSwiglu, MOD = MODE == kModulate;
  const int rt = uu / a.items_k, kt = uu - rt * a.items_k;
  const int64_t row0 = (int64_t)rt * kUnitRows;
  const int64_t col0 = (int64_t)kt * kUnitCols;
  const int64_t col = col0 + lane * 8;
  const u32x4_t z = {0u, 0u, 0u, 0u};
  if (row0 + kUnitRows <= a.m && col0 + kUnitCols <= a.k) {  // the whole unit is inside (wave-uniform)
#pragma unroll
    for (int r = 0; r < kUnitRows; ++r) {
      gv[r >> 1][r & 1] = __builtin_nontemporal_load((const u32x4_t*)(a.x + (row0 + r) * a.ldx + col));
      if (SWIGLU) uv[r >> 1][r & 1] = __builtin_nontemporal_load((const u32x4_t*)(a.u + (row0 + r) * a.ldu + col));
    }
  } else {
    const bool cok = col < a.k;
#pragma unroll
    for (int r = 0; r < kUnitRows; ++r) {
      const bool ok = cok && row0 + r < a.m;
      gv[r >> 1][r & 1] = ok ? __builtin_nontemporal_load((const u32x4_t*)(a.x + (row0 + r) * a.ldx + col)) : z;
      if (SWIGLU)
        uv[r >> 1][r & 1] = ok ? __builtin_nontemporal_load((const u32x4_t*)(a.u + (row0 + r) * a.ldu + col)) : z;
    }
  }
  if (MOD) {
    const bool cok = col < a.k;
    mv[0] = cok ? *(const u32x4_t*)(a.mod_scale + col) : z;
    mv[1] = cok ? *(const u32x4_t*)(a.mod_shift + col) : z;
  }
}

// One-shot grid: workgroup b covers units 8b .. 8b + 7 (more only when the grid is
// capped), one per wave, in address order; its maximum goes to slot b % kAmaxSlots.
template <int MODE>
__global__ void __launch_bounds__(kAbsWaves * 64) producer_absmax_kernel(ProducerArgs a) {
  constexpr bool SWIGLU = MODE == kSwiglu, MOD = MODE == kModulate;
  __shared__ uint32_t red[kAbsWaves];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so unit arithmetic stays scalar
  const int lane = tid & 63;
  uint32_t mall = 0;  // fp32 bits of a bf16 magnitude
  const int groups = (a.nunits + kAbsWaves - 1) / kAbsWaves;
  for (int b = blockIdx.x; b < groups; b += gridDim.x) {
    const int uu = b * kAbsWaves + wave;
    if (uu >= a.nunits) break;
    u32x4_t gv[kSteps][2], uv[kSteps][2], mv[2];
    load_unit_rows<MODE>(a, lane, uu, gv, uv, mv);
    uint32_t m = 0;
    if (SWIGLU) {
      m = swiglu_unit_absmax(a.silu_table, gv, uv);
    } else if (MOD) {
      const int64_t row0 = (int64_t)(uu / a.items_k) * kUnitRows;
#pragma unroll
      for (int r = 0; r < kUnitRows; ++r) {
        if (row0 + r >= a.m) continue;  // padding rows are zero, not the shift
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t xw = gv[r >> 1][r & 1][w], sw = mv[0][w], bw = mv[1][w];
          const uint32_t yw = cvt_pk_bf16(modulate_f32(xw & 0xFFFFu, sw & 0xFFFFu, bw & 0xFFFFu),
                                          modulate_f32(xw >> 16, sw >> 16, bw >> 16));
          const uint32_t m0 = (yw & 0x7FFFu) << 16, m1 = (yw & 0x7FFF0000u);
          m = m0 > m ? m0 : m;
          m = m1 > m ? m1 : m;
        }
      }
    } else {
      u16x2_t pm = {0, 0};
#pragma unroll
      for (int s = 0; s < kSteps; ++s)
#pragma unroll
        for (int w = 0; w < 8; ++w) pm = __builtin_elementwise_max(pm, as_u16x2(gv[s][w >> 2][w & 3] & 0x7FFF7FFFu));
      m = (uint32_t)(pm.x > pm.y ? pm.x : pm.y) << 16;
    }
    mall = m > mall ? m : mall;
  }
  mall = wave_max_u32(mall);
  if (lane == 0) red[wave] = mall;
  __syncthreads();
  if (tid == 0) {
    uint32_t r = 0;
    for (int i = 0; i < kAbsWaves; ++i) r = red[i] > r ? red[i] : r;
    if (r != 0)
      __hip_atomic_fetch_max(a.slots + (blockIdx.x % kAmaxSlots) * kSlotStride, r, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---- pass 2: scales, codes, pack, swizzle ---------------------------------------------------

// y for the 16 elements of one block, as 8 packed bf16 pairs. For kSwiglu, uv holds
// up; for kModulate, mv the lane's scale (mv[0]) and shift (mv[1]). Products are formed
// in fp32 (exact whenever the result is a normal fp32 number); the caller detects
// blocks that may hold a rounded subnormal product and repairs them with block_y_fix.
template <int MODE>
__device__ __forceinline__ void block_y(const u32x4_t (&gv)[2], const u32x4_t (&uv)[2], const u32x4_t (&mv)[2][2],
                                        const uint16_t* tab, uint32_t (&yb)[8]) {
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

struct QuantCtx {
  float g, bscale, inv_f;
  double g6;
};

__device__ __forceinline__ QuantCtx quant_ctx(float amax) {
  QuantCtx c;
  c.g = global_scale_from_amax(amax);
  c.g6 = 6.0 * (double)c.g;
  // 1 / (6g) in fp32; for a tiny g both factors of bmax / (6g) are scaled by 2^64 (exact)
  double inv_g6 = c.g6 > 0.0 ? 1.0 / c.g6 : 0.0;
  c.bscale = 1.0f;
  if (inv_g6 > 0x1p+100) {
    inv_g6 *= 0x1p-64;
    c.bscale = 0x1p+64f;
  }
  c.inv_f = (float)inv_g6;
  return c;
}

// The 8 codes of one half-block, c from the lower bracket and ch from the upper one,
// where they differ: element j is the lower code il or the next one up. For unit >=
// 2^-90 the sign of fma(mid * v(S), g, -|y|) decides exactly (mid * v(S) = (4 mid) *
// (v(S) / 4) has at most 7 significant bits; the exact difference, when not zero, is a
// multiple of 2^-122, so the fused result keeps its sign); a tie goes to the even index.
// Smaller units use exact fp64 compares.
__device__ __forceinline__ uint32_t fix_half(uint32_t c, uint32_t ch, uint32_t y0, uint32_t y1, uint32_t y2, uint32_t y3,
                                             float vS4, float g, bool fma_ok, uint32_t S) {
  const uint32_t dall = c ^ ch;
  uint32_t d = dall;
  while (d) {
    const uint32_t j = (uint32_t)__builtin_ctz(d) >> 2;  // element 0..7 of the half
    const uint32_t sh = j << 2;
    d &= ~(0xFu << sh);
    const uint32_t yw = (j & 4u) ? ((j & 2u) ? y3 : y2) : ((j & 2u) ? y1 : y0);
    const uint32_t y16 = (j & 1u) ? (yw >> 16) : (yw & 0xFFFFu);
    const uint32_t il = (c >> sh) & 7u, ih = (ch >> sh) & 7u;
    if (ih == il + 1u) {
      bool up;
      if (fma_ok) {
        const float ay = __uint_as_float((y16 & 0x7FFFu) << 16);
        const uint64_t mids4 = 0x00140E0A07050301ull;  // 4 x the midpoint above index 0..6
        const float mid4 = (float)(uint32_t)((mids4 >> (8u * il)) & 0xFFu);
        const float dd = __builtin_fmaf(mid4 * vS4, g, -ay);
        up = (il & 1u) ? (dd <= 0.0f) : (dd < 0.0f);
      } else {
        up = e2m1_step_exact(y16, S, g, il) != il;
      }
      if (up) c ^= dall & (0xFu << sh);
    } else {
      c = (c & ~(0xFu << sh)) | (e2m1_code_exact(y16, S, g) << sh);
    }
  }
  return c;
}

// The 16 values y of the lane's block of row `row` as 8 packed bf16 pairs, and the
// largest magnitude among them (bf16 bits).
template <int MODE>
__device__ __forceinline__ void block_values(const ProducerArgs& a, const u32x4_t (&gv)[2], const u32x4_t (&uv)[2],
                                             const u32x4_t (&mv)[2][2], const uint16_t* tab, int64_t row,
                                             uint32_t (&yb)[8], uint32_t& mx) {
  constexpr bool SWIGLU = MODE == kSwiglu, MOD = MODE == kModulate;
  block_y<MODE>(gv, uv, mv, tab, yb);
  if (MOD && row >= a.m) {
#pragma unroll
    for (int w = 0; w < 8; ++w) yb[w] = 0u;  // padding rows are zero, not the shift
  }
  // block maximum of |y| (bf16 magnitudes compare as integers)
  uint32_t mn;
  block_mag_range(yb, mx, mn);
  if (SWIGLU && mn <= 0x0080u) {
    // some |y| <= 2^-126 (or zero): its fp32 product may have been subnormal and
    // rounded; redo such products exactly
    Y8 y;
#pragma unroll
    for (int w = 0; w < 8; ++w) y.v[w] = yb[w];
    y = block_y_fix(gv[0], gv[1], uv[0], uv[1], y, tab);
#pragma unroll
    for (int w = 0; w < 8; ++w) yb[w] = y.v[w];
    block_mag_range(yb, mx, mn);
  }
}

// The scale byte and the 16 codes of one block (values yb, largest magnitude mx): the
// codes are stored at qdst, the scale byte is returned. `store_q`: the row is below
// m_pad; `cok`: the block is inside the columns.
__device__ __forceinline__ uint32_t block_codes(const QuantCtx& c, const uint32_t (&yb)[8], uint32_t mx,
                                                bool store_q, bool cok, uint8_t* qdst) {
  const float g = c.g;
  const uint32_t S = (mx == 0) ? 0u : block_scale_byte(bf16_bits_to_float(mx), c.bscale, c.inv_f, c.g6);

  // E2M1 codes of the 16 elements
  const float vS = ue4m3_to_float(S);
  const float unit = vS * g;
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
    uint32_t cc[2] = {0u, 0u};
    for (int j = 0; j < 16; ++j) {
      const uint32_t y16 = (yb[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      cc[j >> 3] |= e2m1_code_exact(y16, S, g) << (4 * (j & 7));
    }
    clo0 = cc[0];
    clo1 = cc[1];
  } else if ((clo0 ^ chi0) | (clo1 ^ chi1)) {
    // The two bracket codes differ only where |y| / unit lies within the bracket of an
    // E2M1 rounding boundary: there the code is one of two neighbours, decided by one
    // exact comparison with that boundary (the other elements keep theirs).
    const bool fma_ok = unit >= 0x1p-90f;
    const float vS4 = vS * 0.25f;
    if (clo0 ^ chi0) clo0 = fix_half(clo0, chi0, yb[0], yb[1], yb[2], yb[3], vS4, g, fma_ok, S);
    if (clo1 ^ chi1) clo1 = fix_half(clo1, chi1, yb[4], yb[5], yb[6], yb[7], vS4, g, fma_ok, S);
  }
  if (store_q && cok) {
    // non-temporal: QDATA is written once and read by the next stage (measured: about 2 %
    // faster than plain stores)
    const u32x2_t v = {clo0, clo1};
    __builtin_nontemporal_store(v, (u32x2_t*)qdst);
  }
  return S;
}

// The scale bytes of a half group. Lane (r4, blk) holds, for one step, the bytes of the
// half's two units (sa: unit 2h, sb: unit 2h + 1) for its row and block column. In a
// 128 x 4 tile those bytes, for the tile's 4 block columns, are 8 consecutive bytes of
// the row's 16: unit 2h's 4 columns, then unit 2h + 1's. The 4 lanes of a tile
// (blk = 4t .. 4t + 3, one DPP quad) gather them, and the first writes them with one
// 8-byte store (plain: the L2 merges the group's pieces into whole lines;
// non-temporal stores of scale bytes were far slower). `cok` is the same for the 4
// lanes (k is a multiple of 64). All lanes of the wave must be active.
__device__ __forceinline__ void store_half_scales(uint32_t sa, uint32_t sb, int blk, bool cok, uint8_t* dst) {
  const uint32_t x = sa | (sb << 8);                                              // a_c, b_c
  const uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);  // lane c ^ 1
  const uint32_t pr = (blk & 1) ? (y | (x << 16)) : (x | (y << 16));             // a_e, b_e, a_o, b_o
  const uint32_t z = (uint32_t)__builtin_amdgcn_mov_dpp((int)pr, 0x4E, 0xF, 0xF, false); // lane c ^ 2
  if ((blk & 3) == 0 && cok) {
    u32x2_t v;
    v[0] = __builtin_amdgcn_perm(z, pr, 0x06040200u);  // a_0 a_1 a_2 a_3
    v[1] = __builtin_amdgcn_perm(z, pr, 0x07050301u);  // b_0 b_1 b_2 b_3
    *(u32x2_t*)dst = v;
  }
}

// The scale bytes of a whole group: lane (r4, blk) holds in x, for one step, the bytes
// of the group's units 0 .. 3 (byte q) for its row and block column. In a 128 x 4 tile
// they are the row's 16 bytes (unit q's 4 columns at 4q). The 4 lanes of a tile
// transpose them as a 4 x 4 byte matrix (two DPP quad moves each way), and the first
// writes them with one 16-byte store. All lanes of the wave must be active.
__device__ __forceinline__ void store_group_scales(uint32_t x, int blk, bool cok, uint8_t* dst) {
  const uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);  // lane c ^ 1
  const uint32_t lo = (blk & 1) ? y : x, hi = (blk & 1) ? x : y;                 // even, odd column
  const uint32_t pr = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // units 0, 1 of the lane pair
  const uint32_t rr = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // units 2, 3
  const uint32_t p2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)pr, 0x4E, 0xF, 0xF, false); // lane c ^ 2
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)rr, 0x4E, 0xF, 0xF, false);
  if ((blk & 3) == 0 && cok) {
    u32x4_t v;
    v[0] = __builtin_amdgcn_perm(p2, pr, 0x05040100u);  // unit 0, columns 0 .. 3
    v[1] = __builtin_amdgcn_perm(p2, pr, 0x07060302u);  // unit 1
    v[2] = __builtin_amdgcn_perm(r2, rr, 0x05040100u);  // unit 2
    v[3] = __builtin_amdgcn_perm(r2, rr, 0x07060302u);  // unit 3
    *(u32x4_t*)dst = v;
  }
}

// Persistent grid of G kQuantWaves-wave workgroups, W waves in all. Pieces of work
// (groups of units, and half groups at the end) are numbered from the end of the
// tensor. Wave v of workgroup b is wave w = v G + b (so that consecutive pieces go to
// different CUs); it starts with piece w, then takes pieces from counter
// j = (w / 8) % nq of the launch's set, the t-th take of counter j being piece
// W + t nq + j, where nq is kProdQueueCounters, or fewer on a grid too small to give each
// counter a wave. Each take is issued one piece ahead of its use. GIVEN: the tensor amax
// comes from the caller (a device float); otherwise it is the maximum of the workspace's
// slots, which the last workgroup clears together with the counters.
template <int MODE, bool GIVEN>
__global__ void __launch_bounds__(kQuantWaves * 64) producer_kernel(ProducerArgs a) {
  constexpr bool SWIGLU = MODE == kSwiglu, MOD = MODE == kModulate;
  __shared__ uint32_t red[kQuantWaves];  // wave maxima
  // The bf16 silu table (SwiGLU only) at a fixed LDS address, so that each lookup's
  // address is one shift of the gate bits.
  uint16_t* tab = nullptr;
  if constexpr (SWIGLU) {
    __shared__ __attribute__((aligned(16))) uint16_t silu_lds[65536];
    tab = silu_lds;
  }
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so unit arithmetic stays scalar
  const int lane = tid & 63;
  const LaneGeom L = lane_geom(lane);
  const int nwaves = gridDim.x * kQuantWaves;
  const int wg = wave * gridDim.x + blockIdx.x;  // global wave index, CU-minor
  // Counter j serves the waves of 8 consecutive workgroups, which sit on the 8 different
  // XCDs: counters serving a single XCD ran out at that XCD's pace, and the XCDs' clocks
  // differ.
  // (a grid of fewer than 8 * kProdQueueCounters waves uses as many counters as it has
  // groups of 8 waves, so that every counter in use serves at least one wave)
  const int nq = kProdQueueCounters < (nwaves + 7) / 8 ? kProdQueueCounters : (nwaves + 7) / 8;
  const int j = (wg >> 3) % nq;
  uint32_t* ctr = a.queue + j * kSlotStride;

  // A take hands out a group of kGroupUnits units: rows r, r + 32, r + 64 and r + 96
  // (r a multiple of 4) of one 128-row tile, 4 rows each, in one column segment. The 64-byte
  // lines of the scale tiles hold exactly these 16 rows, so each line is written whole by
  // one wave, and L2 merges its byte stores before the line goes to memory.
  const int ngroups = a.nunits / kGroupUnits;
  auto group_unit = [&](int grp, int jj) {  // unit index of member jj of group grp (reverse order)
    const int gg = ngroups - 1 - grp;
    const int kt = gg % a.items_k, rest = gg / a.items_k;
    const int rt = (rest / 8) * 32 + (rest % 8) + 8 * jj;
    return rt * a.items_k + kt;
  };
  // Work is handed out as pieces: whole groups, except that the last nsplit groups (the
  // start of the tensor, reached last) go out as halves (units 0, 1 or 2, 3 of a group),
  // so that when the counters run out no wave has more than half a group left to do.
  // Piece p is group p (p < nfull), else half (p - nfull) % 2 of group
  // nfull + (p - nfull) / 2.
  const int nsplit = ngroups < nwaves / 2 ? ngroups : nwaves / 2;
  const int nfull = ngroups - nsplit, npieces = nfull + 2 * nsplit;
  auto piece_group = [&](int p) { return p < nfull ? p : nfull + ((p - nfull) >> 1); };
  auto piece_half = [&](int p) { return p < nfull ? 0 : ((p - nfull) & 1); };        // first half
  auto piece_end = [&](int p) { return p < nfull ? 2 : ((p - nfull) & 1) + 1; };     // past its last half
  // the first piece needs no take: every wave starting with a take put 96 takes on
  // each counter before any load could be issued
  int p = wg, grp = piece_group(p), h = piece_half(p), hend = piece_end(p);
  // the first unit's loads are in flight while the table is staged and amax reduced
  u32x4_t gv[kSteps][2], uv[kSteps][2], mv[2][2];
  if (p < npieces) {
    load_unit<MODE>(a, L, group_unit(grp, 2 * h), gv, uv);
    if (MOD) load_modulation(a, L, group_unit(grp, 2 * h), mv);
  }
  uint32_t slot_max = 0;
  if (!GIVEN && tid < kAmaxSlots) slot_max = a.slots[tid * kSlotStride];
  if (SWIGLU) {
    const u32x4_t* src = (const u32x4_t*)a.silu_table;
    u32x4_t* dst = (u32x4_t*)tab;
    for (int i = tid; i < 65536 * 2 / 16; i += kQuantWaves * 64) dst[i] = src[i];
  }
  float amax;
  if constexpr (GIVEN) {
    amax = a.amax_in[0];
    if (SWIGLU) __syncthreads();
  } else {
    slot_max = wave_max_u32(slot_max);
    if (lane == 0) red[wave] = slot_max;
    __syncthreads();
    uint32_t r = 0;
    for (int i = 0; i < kQuantWaves; ++i) r = red[i] > r ? red[i] : r;
    amax = __uint_as_float(r);
  }
  const QuantCtx c = quant_ctx(amax);
  if (blockIdx.x == 0 && tid == 0) *a.gout = c.g;

  const int64_t qrow = a.k / 2;
  // quantizes unit uu; returns each step's scale byte in sc
  auto process = [&](int uu, u32x4_t (&xv)[kSteps][2], u32x4_t (&yv)[kSteps][2], const u32x4_t (&zv)[2][2],
                     uint32_t (&sc)[kSteps]) {
    arrange_unit<MODE>(xv, yv);
    const int rt = uu / a.items_k, kt = uu - rt * a.items_k;
    const int64_t row0 = (int64_t)rt * kUnitRows;
    if (row0 + kUnitRows > a.m) zero_tail_rows<MODE>(a, row0, lane, xv, yv);
    const bool cok = (int64_t)kt * kUnitCols + L.blk * 16 < a.k;
    const bool store_q = row0 < a.m_pad;  // units are 4-row aligned, m_pad 16-row aligned
    uint8_t* bq = a.qdata + row0 * qrow + kt * (kUnitCols / 2) + L.r4 * qrow + L.blk * 8;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      uint32_t yb[8], mx;
      block_values<MODE>(a, xv[s], yv[s], zv, tab, row0 + 2 * s + L.r4, yb, mx);
      sc[s] = block_codes(c, yb, mx, store_q, cok, bq + s * 2 * qrow);
    }
  };
  // Writes the scale bytes of the half group whose first unit is uu (sa) and second sb:
  // a half piece's at once, a whole group's first half kept in sx until its second.
  uint32_t sx[kSteps] = {0u, 0u};
  auto store_scales = [&](int uu, bool whole, int hh, const uint32_t (&sa)[kSteps], const uint32_t (&sb)[kSteps]) {
    const int rt = uu / a.items_k, kt = uu - rt * a.items_k;
    const int64_t row0 = (int64_t)rt * kUnitRows;
    const bool cok = (int64_t)kt * kUnitCols + L.blk * 16 < a.k;
    // the lane's row in its 128 x 4 tile (block column bc): row group (row0 & 31) + r4,
    // 4-byte column group (row0 >> 5) & 3, which is 2h for the half's first unit
    const int64_t bc = (int64_t)kt * kLanesPerRow + L.blk;
    uint8_t* bs = a.scales + ((row0 >> 7) * (a.cpad / 4) + (bc >> 2)) * 512 + (row0 & 31) * 16 +
                  ((row0 >> 5) & 3) * 4 + L.r4 * 16;
    if (!whole) {
#pragma unroll
      for (int s = 0; s < kSteps; ++s) store_half_scales(sa[s], sb[s], L.blk, cok, bs + s * 32);
    } else if (hh == 0) {
#pragma unroll
      for (int s = 0; s < kSteps; ++s) sx[s] = sa[s] | (sb[s] << 8);
    } else {
#pragma unroll
      for (int s = 0; s < kSteps; ++s)
        store_group_scales(sx[s] | (sa[s] << 16) | (sb[s] << 24), L.blk, cok, bs - 8 + s * 32);
    }
  };
  // Double-buffered: the next unit's loads are issued before the current unit is
  // quantized, so they are in flight during its arithmetic and stores.
  u32x4_t gw[kSteps][2], uw[kSteps][2], mw[2][2];
  // One iteration per half group. The take for the next piece is issued when a piece
  // starts and read in its last half, just after that half's first loads are issued
  // (before any store of the half, so that waiting for it waits for nothing newer):
  // one piece ahead.
  uint32_t tr = 0;
  bool fresh = true;  // the current half starts its piece
  while (p < npieces) {
    if (fresh && lane == 0) tr = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int n1 = group_unit(grp, 2 * h + 1);
    load_unit<MODE>(a, L, n1, gw, uw);
    if (MOD) load_modulation(a, L, n1, mw);
    // the next half: the piece's next one, or the next piece's first
    int np = p, ngrp = grp, nh = h + 1, nhend = hend;
    fresh = nh == hend;
    if (fresh) {
      np = nwaves + (int)__builtin_amdgcn_readfirstlane(tr) * nq + j;
      ngrp = piece_group(np);
      nh = piece_half(np);
      nhend = piece_end(np);
    }
    // nothing of the unit below may move above the next unit's loads (the scheduler
    // would otherwise start its lane swaps there and wait for those loads too)
    __builtin_amdgcn_sched_barrier(0);
    const int u0 = group_unit(grp, 2 * h);
    uint32_t sa[kSteps], sb[kSteps];
    process(u0, gv, uv, mv, sa);
    // (after the last piece, a load of unit 0 that is never used)
    const bool more = np < npieces;
    const int n2 = more ? group_unit(ngrp, 2 * nh) : 0;
    load_unit<MODE>(a, L, n2, gv, uv);
    if (MOD) load_modulation(a, L, n2, mv);
    __builtin_amdgcn_sched_barrier(0);
    process(n1, gw, uw, mw, sb);
    store_scales(u0, p < nfull, h, sa, sb);
    p = np;
    grp = ngrp;
    h = nh;
    hend = nhend;
  }
  // Every take of this wave has returned (its last value was read above). The waves of
  // the workgroup meet, and one lane counts the workgroup as done: one atomic per
  // workgroup, since one per wave (3,072 on one address, about 11 ns each) took some
  // 35 us at the end of every call. The last workgroup to count itself clears the
  // counter set and, after a two-pass call, the slots: every wave read the slots before
  // its loop.
  __syncthreads();
  if (wave == 0) {
    uint32_t done = 0;
    if (lane == 0)
      done = __hip_atomic_fetch_add(a.queue + kProdQueueCounters * kSlotStride, 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    done = __builtin_amdgcn_readfirstlane(done);
    if (done == gridDim.x - 1) {
      if (lane < kProdQueueCounters)
        __hip_atomic_store(a.queue + lane * kSlotStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (!GIVEN && lane < kAmaxSlots)
        __hip_atomic_store(a.slots + lane * kSlotStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0)
        __hip_atomic_store(a.queue + kProdQueueCounters * kSlotStride, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---- host side --------------------------------------------------------------------------------

// dynamic LDS of the quantize launch (its table and wave maxima are static)
size_t producer_smem_bytes(int) { return 0; }

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

int producer_block_threads() { return kQuantWaves * 64; }

int64_t producer_units(int64_t m, int64_t k) {
  const int64_t m_pad = (m + 15) / 16 * 16;
  const int64_t scale_rows = (m_pad + 127) / 128 * 128;
  return scale_rows / kUnitRows * ((k + kUnitCols - 1) / kUnitCols);
}

// amax_in == nullptr: the two-pass producer (absmax launch into the workspace's slots,
// then the quantize launch); otherwise the single-read producer with the caller's amax
// (the quantize launch alone). `queue` is a zeroed counter set of kProdQueueSetWords
// words; the quantize launch's grid is `quant_blocks` workgroups.
hipError_t launch_producer(int mode, const uint16_t* x, int64_t ldx, const uint16_t* u, int64_t ldu,
                           const uint16_t* mod_scale, const uint16_t* mod_shift, int64_t m, int64_t k,
                           uint8_t* qdata, uint8_t* scales, float* gout, const float* amax_in, void* workspace,
                           uint32_t* queue, const uint16_t* silu_table, int quant_blocks, hipStream_t stream) {
  ProducerArgs args;
  args.x = x;
  args.u = u;
  args.ldx = ldx;
  args.ldu = ldu;
  args.m = m;
  args.k = k;
  args.m_pad = (m + 15) / 16 * 16;
  args.cpad = (k / 16 + 3) / 4 * 4;
  args.items_k = (int)((k + kUnitCols - 1) / kUnitCols);
  args.nunits = (int)producer_units(m, k);
  args.qdata = qdata;
  args.scales = scales;
  args.gout = gout;
  args.amax_in = amax_in;
  args.mod_scale = mod_scale;
  args.mod_shift = mod_shift;
  args.slots = workspace ? ((ProducerWorkspace*)workspace)->slot : nullptr;
  args.queue = queue;
  args.silu_table = silu_table;
  const size_t smem = producer_smem_bytes(mode);
  if (!amax_in) {
    const int64_t groups = ((int64_t)args.nunits + kAbsWaves - 1) / kAbsWaves;
    const int grid = (int)(groups < ((int64_t)1 << 30) ? groups : ((int64_t)1 << 30));
    void* kargs[] = {&args};
    hipError_t e = hipLaunchKernel(producer_absmax_kernel_ptr(mode), dim3(grid < 1 ? 1 : grid), dim3(kAbsWaves * 64),
                                   kargs, 0, stream);
    if (e != hipSuccess) return e;
  }
  void* kargs[] = {&args};
  return hipLaunchKernel(producer_kernel_ptr(mode, amax_in != nullptr), dim3(quant_blocks < 1 ? 1 : quant_blocks),
                         dim3(kQuantWaves * 64), kargs, smem, stream);
}

}  // namespace nvfp4
