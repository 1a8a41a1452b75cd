// producer.hip - fused SwiGLU -> NVFP4 producer for gfx950 (one cooperative launch).
//
// Operation (component-2 NSYS summary: the pre-fusion chain silu -> multiply ->
// absmax_partial -> scale_finalize -> block_scale_zero -> activation_pack, whose
// "conclusion" notes that the global-scale dependency needs an explicit
// synchronisation design; "FC2 NVFP4 Scheduling Results", "Canonical Operation",
// for the formats and the 37,810 -> 37,824 row padding):
//
//   y       = RN_bf16(silu_bf16(gate) * up)          (plain variant: y = x)
//   amax    = max |y| over the logical rows
//   g       = amax / 2688 rounded up to fp32          (2688 = 6 * 448)
//   S[r,b]  = smallest UE4M3 byte with v(S) * 6 * g >= max_{16} |y|
//   code    = E2M1 nearest to |y| / (v(S) g), ties to even, sign of y
//   QDATA   = two codes per byte (even element low), rows [m, m_pad) zero
//   scales  = 512-byte tiles of 128 rows x 4 scale columns, padding zero
//
// Structure: a persistent grid (co-resident through a cooperative launch) walks
// work items of 128 rows x 256 columns. Pass 1 reduces |y| (wavefront shuffles,
// LDS across waves, one agent-scope atomic max per workgroup); a grid barrier
// publishes amax; pass 2 walks the items in reverse order (so the rows read
// last in pass 1, still in the memory-side cache, are read first), recomputes y,
// and writes coalesced QDATA rows (each wave instruction stores 2 full 128-byte
// rows) and whole 512-byte scale tiles staged in LDS.
//
// Exactness: every rounding decision equals the exact one.
//  - y: a product of two bf16 values is exact in fp32 when it is >= 2^-126; smaller
//    (or zero) products are recomputed in fp64 and rounded once.
//  - S: an fp64 estimate adjusted by exact fp64 compares (v(e) * 6g has <= 30
//    significant bits).
//  - codes: the hardware fp32 -> E2M1 conversion (round to nearest even) is applied
//    to |y| * r_lo and |y| * r_hi, two brackets of the exact quotient built from a
//    1-ulp reciprocal with a 2^-20 margin; when the two codes agree the exact code
//    is that code (rounding is monotone), otherwise the element is decided by exact
//    fp64 compares against the seven midpoints.
#include "common.hpp"

namespace nvfp4 {

constexpr int kProdThreads = 512;  // 8 waves
constexpr int kItemRows = 128;     // one scale row-tile
constexpr int kItemCols = 256;     // one 128-byte QDATA segment per row
constexpr int kSteps = 8;          // 128 rows / (8 waves * 2 rows per wave-step)
constexpr int kStagingBytes = 2048;  // four 512-byte scale tiles

struct ProducerArgs {
  const uint16_t* x;  // gate (SwiGLU) or x (plain)
  const uint16_t* u;  // up (SwiGLU)
  int64_t ldx, ldu;   // row strides, elements
  int64_t m, k, m_pad;
  int64_t cpad;       // scale columns
  int items_m;        // scale row-tiles
  int items_k;        // 256-column segments
  uint8_t* qdata;
  uint8_t* scales;
  float* gout;
  ProducerWorkspace* ws;
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

// smallest UE4M3 byte e with v(e) * g6 >= bmax (g6 = 6 g, exact in fp64); bmax > 0
__device__ __forceinline__ uint32_t block_scale_byte(float bmax, double g6) {
  double b = (double)bmax;
  double r = b / g6;
  int e;
  if (r >= 0x1p-6) {
    uint64_t u = (uint64_t)__double_as_longlong(r);
    int E = (int)((u >> 52) & 0x7FF) - 1023 + 7;
    if (E > 15) E = 15;
    int mant = (int)((u >> 49) & 7u);
    int rest = (u & ((1ull << 49) - 1)) != 0;
    e = ((E << 3) | mant) + rest;
  } else {
    e = (int)ceil(r * 512.0);
  }
  e = e < 1 ? 1 : (e > 126 ? 126 : e);
  while (e < 126 && ue4m3_to_double((uint32_t)e) * g6 < b) ++e;
  while (e > 1 && ue4m3_to_double((uint32_t)(e - 1)) * g6 >= b) --e;
  return (uint32_t)e;
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

// ---- the kernel ------------------------------------------------------------------------------

template <bool SWIGLU>
__global__ void __launch_bounds__(kProdThreads) producer_kernel(ProducerArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint8_t* staging = smem;                                  // kStagingBytes
  uint32_t* red = (uint32_t*)(smem + kStagingBytes);        // 8 wave maxima + broadcast
  uint16_t* tab = (uint16_t*)(smem + kStagingBytes + 64);   // 65,536 entries (SwiGLU only)

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int chunk = lane & 31;  // 8-element chunk of the 256-column segment
  const int nitems = a.items_m * a.items_k;

  if (SWIGLU) {
    const u32x4_t* src = (const u32x4_t*)a.silu_table;
    u32x4_t* dst = (u32x4_t*)tab;
    for (int i = tid; i < 65536 * 2 / 16; i += kProdThreads) dst[i] = src[i];
    __syncthreads();
  }

  auto load_item = [&](int item, u32x4_t (&gv)[kSteps], u32x4_t (&uv)[kSteps]) {
    const int rt = item / a.items_k, kt = item - rt * a.items_k;
    const int64_t col = (int64_t)kt * kItemCols + chunk * 8;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int64_t row = (int64_t)rt * kItemRows + s * 16 + wave * 2 + (lane >> 5);
      const bool ok = row < a.m && col < a.k;
      u32x4_t z = {0u, 0u, 0u, 0u};
      gv[s] = ok ? *(const u32x4_t*)(a.x + row * a.ldx + col) : z;
      if (SWIGLU) uv[s] = ok ? *(const u32x4_t*)(a.u + row * a.ldu + col) : z;
    }
  };

  // ---------------- pass 1: absmax ----------------
  uint32_t local_bits = 0;  // fp32 bits of a non-negative value
  bool needs_exact = false;
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    u32x4_t gv[kSteps], uv[kSteps];
    load_item(item, gv, uv);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (SWIGLU) {
          const uint32_t gw = gv[s][w], uw = uv[s][w];
          const float s0 = __uint_as_float((uint32_t)tab[gw & 0xFFFFu] << 16);
          const float s1 = __uint_as_float((uint32_t)tab[gw >> 16] << 16);
          const float p0 = fabsf(s0 * __uint_as_float(uw << 16));
          const float p1 = fabsf(s1 * __uint_as_float(uw & 0xFFFF0000u));
          const uint32_t b = __float_as_uint(fmaxf(p0, p1));
          local_bits = b > local_bits ? b : local_bits;
        } else {
          const uint32_t gw = gv[s][w];
          const uint32_t m0 = gw & 0x7FFFu, m1 = (gw >> 16) & 0x7FFFu;
          const uint32_t b = (m0 > m1 ? m0 : m1) << 16;
          local_bits = b > local_bits ? b : local_bits;
        }
      }
    }
  }
  // workgroup max of the unrounded |products| (SwiGLU) or of |x|
  {
    uint32_t wmax = wave_max_u32(local_bits);
    if (lane == 0) red[wave] = wmax;
    __syncthreads();
    if (tid == 0) {
      uint32_t v = 0;
      for (int i = 0; i < kProdThreads / 64; ++i) v = red[i] > v ? red[i] : v;
      red[8] = v;
    }
    __syncthreads();
    local_bits = red[8];
    // A product below 2^-126 may have been rounded in fp32; if this workgroup's
    // maximum is such a product, redo its elements exactly (never taken for
    // inputs whose absmax is a normal number).
    needs_exact = SWIGLU && local_bits != 0 && local_bits < 0x00800000u;
    __syncthreads();
  }
  if (SWIGLU && needs_exact) {
    uint32_t best = 0;  // bf16 magnitude bits
    for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
      u32x4_t gv[kSteps], uv[kSteps];
      load_item(item, gv, uv);
      for (int s = 0; s < kSteps; ++s)
        for (int j = 0; j < 8; ++j) {
          const uint32_t g16 = (gv[s][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
          const uint32_t u16 = (uv[s][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
          const double p = (double)bf16_bits_to_float(tab[g16]) * (double)bf16_bits_to_float(u16);
          const uint32_t y = rn_bf16_from_double(p) & 0x7FFFu;
          best = y > best ? y : best;
        }
    }
    uint32_t wmax = wave_max_u32(best);
    if (lane == 0) red[wave] = wmax;
    __syncthreads();
    if (tid == 0) {
      uint32_t v = 0;
      for (int i = 0; i < kProdThreads / 64; ++i) v = red[i] > v ? red[i] : v;
      red[8] = v << 16;
    }
    __syncthreads();
    local_bits = red[8];
  } else if (SWIGLU) {
    // RN_bf16 is monotone, so the rounded maximum is the maximum of the rounded values.
    local_bits = (cvt_pk_bf16(__uint_as_float(local_bits), 0.0f) & 0xFFFFu) << 16;
  }

  // ---------------- grid barrier: publish amax ----------------
  if (tid == 0) {
    ProducerWorkspace* ws = a.ws;
    __hip_atomic_fetch_max(&ws->amax_bits, local_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(&ws->arrived, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    while (__hip_atomic_load(&ws->arrived, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < gridDim.x)
      __builtin_amdgcn_s_sleep(2);
    const uint32_t amax = __hip_atomic_load(&ws->amax_bits, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    red[9] = amax;
    // the last workgroup to leave returns the workspace to zero for the next call
    const uint32_t d = __hip_atomic_fetch_add(&ws->departed, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (d == gridDim.x - 1) {
      __hip_atomic_store(&ws->amax_bits, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ws->arrived, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ws->departed, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  const float amax = __uint_as_float(red[9]);
  const float g = global_scale_from_amax(amax);
  const double g6 = 6.0 * (double)g;
  if (blockIdx.x == 0 && tid == 0) *a.gout = g;

  // ---------------- pass 2: scales, codes, pack, swizzle ----------------
  const int64_t qrow_bytes = a.k / 2;
  for (int item = nitems - 1 - (int)blockIdx.x; item >= 0; item -= gridDim.x) {
    const int rt = item / a.items_k, kt = item - rt * a.items_k;
    u32x4_t gv[kSteps], uv[kSteps];
    load_item(item, gv, uv);
    const int64_t col = (int64_t)kt * kItemCols + chunk * 8;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int lrow = s * 16 + wave * 2 + (lane >> 5);
      const int64_t row = (int64_t)rt * kItemRows + lrow;
      // y as four packed bf16 pairs
      uint32_t yb[4];
      if (SWIGLU) {
        float p[8];
        bool tiny = false;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t gw = gv[s][w], uw = uv[s][w];
          p[2 * w] = __uint_as_float((uint32_t)tab[gw & 0xFFFFu] << 16) * __uint_as_float(uw << 16);
          p[2 * w + 1] = __uint_as_float((uint32_t)tab[gw >> 16] << 16) * __uint_as_float(uw & 0xFFFF0000u);
          tiny |= fabsf(p[2 * w]) < 0x1p-126f;
          tiny |= fabsf(p[2 * w + 1]) < 0x1p-126f;
          yb[w] = cvt_pk_bf16(p[2 * w], p[2 * w + 1]);
        }
        if (tiny) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (fabsf(p[j]) < 0x1p-126f) {
              const uint32_t g16 = (gv[s][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
              const uint32_t u16 = (uv[s][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
              const double pd = (double)bf16_bits_to_float(tab[g16]) * (double)bf16_bits_to_float(u16);
              const uint32_t y = rn_bf16_from_double(pd);
              const int sh = 16 * (j & 1);
              yb[j >> 1] = (yb[j >> 1] & ~(0xFFFFu << sh)) | (y << sh);
            }
          }
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) yb[w] = gv[s][w];
      }
      // block maximum over the lane pair (16 elements)
      uint32_t mx = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t m0 = yb[w] & 0x7FFFu, m1 = (yb[w] >> 16) & 0x7FFFu;
        mx = m0 > mx ? m0 : mx;
        mx = m1 > mx ? m1 : mx;
      }
      const uint32_t other = (uint32_t)__shfl_xor((int)mx, 1, 64);
      mx = other > mx ? other : mx;
      const float bmax = bf16_bits_to_float(mx);
      const uint32_t S = (mx == 0) ? 0u : block_scale_byte(bmax, g6);

      // E2M1 codes of the 8 elements of this lane
      const float unit = ue4m3_to_float(S) * g;
      const bool exact_block = (S != 0) && !(unit >= 0x1p-100f);
      const float rcp = (S == 0) ? 1.0f : __builtin_amdgcn_rcpf(unit);
      const float rlo = rcp * (1.0f - 0x1p-20f);
      const float rhi = rcp * (1.0f + 0x1p-20f);
      uint32_t clo = 0, chi = 0;
      fp4_pair<0>(clo, chi, yb[0], rlo, rhi);
      fp4_pair<1>(clo, chi, yb[1], rlo, rhi);
      fp4_pair<2>(clo, chi, yb[2], rlo, rhi);
      fp4_pair<3>(clo, chi, yb[3], rlo, rhi);
      if (clo != chi || exact_block) {
        uint32_t c = 0;
        for (int j = 0; j < 8; ++j) {
          const uint32_t y16 = (yb[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
          const uint32_t nib_lo = (clo >> (4 * j)) & 15u, nib_hi = (chi >> (4 * j)) & 15u;
          const uint32_t code = (nib_lo == nib_hi && !exact_block) ? nib_lo : e2m1_code_exact(y16, S, g);
          c |= code << (4 * j);
        }
        clo = c;
      }
      if (row < a.m_pad && col < a.k)
        *(uint32_t*)(a.qdata + row * qrow_bytes + col / 2) = clo;
      if ((lane & 1) == 0) {
        const int b = chunk >> 1;  // block within the segment, 0..15
        staging[(b >> 2) * 512 + (lrow & 31) * 16 + ((lrow >> 5) & 3) * 4 + (b & 3)] = (uint8_t)S;
      }
    }
    __syncthreads();
    {
      // write the item's scale tiles: 4 tiles of 512 bytes, one dword per thread
      const int64_t seg_cols = a.k - (int64_t)kt * kItemCols;
      const int ntiles = (int)((seg_cols >= kItemCols ? kItemCols : seg_cols) / 64);
      const int tile = tid >> 7;
      if (tile < ntiles) {
        const int64_t off = ((int64_t)rt * (a.cpad / 4) + (int64_t)kt * 4 + tile) * 512 + (tid & 127) * 4;
        *(uint32_t*)(a.scales + off) = ((const uint32_t*)staging)[tid];
      }
    }
    __syncthreads();
  }
}

// ---- host side --------------------------------------------------------------------------------

size_t producer_smem_bytes(bool swiglu) {
  return kStagingBytes + 64 + (swiglu ? 65536 * 2 : 0);
}

const void* producer_kernel_ptr(bool swiglu) {
  return swiglu ? (const void*)producer_kernel<true> : (const void*)producer_kernel<false>;
}

int producer_block_threads() { return kProdThreads; }

hipError_t launch_producer(bool swiglu, const uint16_t* x, int64_t ldx, const uint16_t* u, int64_t ldu,
                           int64_t m, int64_t k, uint8_t* qdata, uint8_t* scales, float* gout,
                           void* workspace, const uint16_t* silu_table, int max_blocks,
                           hipStream_t stream) {
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
  args.ws = (ProducerWorkspace*)workspace;
  args.silu_table = silu_table;
  const int64_t nitems = (int64_t)args.items_m * args.items_k;
  int blocks = (int)(nitems < max_blocks ? nitems : max_blocks);
  if (blocks < 1) blocks = 1;
  void* kargs[] = {&args};
  return hipLaunchCooperativeKernel(producer_kernel_ptr(swiglu), dim3(blocks), dim3(kProdThreads), kargs,
                                    (unsigned)producer_smem_bytes(swiglu), stream);
}

}  // namespace nvfp4
