// gemm.hip - block-scaled NVFP4 GEMM with FP32 accumulation and BF16 output (gfx950).
//
// D[m, n] = RN_bf16(g_a g_w sum_k a[m,k] w[n,k]), a = e2m1(A) * v(SA), w = e2m1(W) * v(SW),
// E2M1 operands with vector-16 UE4M3 scales ("FC2 NVFP4 Scheduling Results",
// "Canonical Operation"). Like the split-K-1 schedule that page accepts, every
// output tile is owned by one workgroup that runs the whole K loop: no split-K,
// no workspace, no global reduction, one write of the padded output.
//
// Arithmetic: an E2M1 value times a UE4M3 scale has at most 6 significant bits
// and lies in [2^-10, 2688], so it is exact in fp16. gfx950 has no NVFP4 matrix
// instruction and its scaled fp4 conversions apply only the exponent of the scale,
// so each operand is dequantized in registers as
//     f16(e2m1 * 2^8) [v_cvt_scalef32_pk_f16_fp4, scale 256]  x  f16(S << 7)
// where the fp16 bit pattern S << 7 is exactly v(S) * 2^-8 for every UE4M3 byte S
// (normal and subnormal alike), and the packed fp16 product [v_pk_mul_f16] is exact.
// The exact fp16 operands feed v_mfma_f32_32x32x16_f16 with fp32 accumulation;
// the epilogue multiplies by g_a * g_w in fp32 and rounds to bf16 once.
//
// Tiling: a 256 x 256 output tile per workgroup of 4 waves (2 x 2), each wave
// 128 x 128 (4 x 4 MFMA tiles of 32 x 32, accumulators in AGPRs). K advances 128
// per step; the packed operands (64 bytes per row) and their four 512-byte scale
// tiles per operand are staged through double-buffered LDS. Within a K step the
// lane's k-half h covers k in [64h, 64h + 64), eight consecutive k per MFMA, the
// same assignment for both operands, so every lane reads 32 contiguous code bytes
// and one scale dword per 32-row fragment. Global loads are buffer loads whose
// range check returns zero past the end of A (rows >= m_padded) or W (rows >= n).
//
// Traversal: tiles are numbered m-band-major in bands of 8 M-tiles, and workgroup
// ids (dispatched round-robin over the 8 XCDs) are remapped so that each XCD owns
// one contiguous range of tiles; its 32 concurrent workgroups then share A row
// bands and W panels in that XCD's L2.
#include "common.hpp"

namespace nvfp4 {

constexpr int kTM = 256, kTN = 256, kTK = 128;
constexpr int kGemmThreads = 256;
constexpr int kRowStride = 80;                   // LDS bytes per staged row (64 data + 16 pad)
constexpr int kCodesBytes = 256 * kRowStride;    // one operand's codes per stage
constexpr int kScaleBytes = 2048;                // one operand's 4 scale tiles per stage
constexpr int kStageBytes = 2 * kCodesBytes + 2 * kScaleBytes;
constexpr int kBandM = 8;                        // M-tiles per traversal band

struct GemmArgs {
  const uint8_t* aq;
  const uint8_t* as;
  const float* ga;
  const uint8_t* wq;
  const uint8_t* ws;
  const float* gw;
  uint16_t* d;
  int64_t m_pad, n, k;
  int a_qbytes, w_qbytes, a_sbytes, w_sbytes;  // buffer sizes for the range checks
  int tiles_m, tiles_n;
  int cgroups;                                 // scale column groups = C / 4
  int ksteps;
};

__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

template <int SEL>
__device__ __forceinline__ f16x2_t dq2(uint32_t codes, f16x2_t sv) {
  f16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, SEL);
  return v * sv;
}

__device__ __forceinline__ f16x8_t dequant8(uint32_t codes, f16x2_t sv) {
  f16x2_t p0 = dq2<0>(codes, sv), p1 = dq2<1>(codes, sv), p2 = dq2<2>(codes, sv), p3 = dq2<3>(codes, sv);
  f16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// fp16 pair (v(S) * 2^-8, v(S) * 2^-8) for scale byte b of a scale dword
__device__ __forceinline__ f16x2_t scale_pair(uint32_t sdw, int b) {
  uint32_t h = ((sdw >> (8 * b)) & 0xFFu) << 7;
  uint32_t u = h | (h << 16);
  f16x2_t r;
  __builtin_memcpy(&r, &u, 4);
  return r;
}

__global__ void __launch_bounds__(kGemmThreads, 1) gemm_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  // ---- tile assignment: XCD-contiguous ranges, m-band-major order ----
  const int ntiles = a.tiles_m * a.tiles_n;
  const int b = blockIdx.x;
  const int nb = gridDim.x;
  const int per = nb / 8, rem = nb % 8;
  const int xcd = b % 8, idx = b / 8;
  const int t = xcd * per + (xcd < rem ? xcd : rem) + idx;
  if (t >= ntiles) return;
  const int band = t / (kBandM * a.tiles_n);
  const int in_band = t - band * kBandM * a.tiles_n;
  const int band_m = (a.tiles_m - band * kBandM) < kBandM ? (a.tiles_m - band * kBandM) : kBandM;
  const int tm = band * kBandM + in_band % band_m;
  const int tn = in_band / band_m;
  const int64_t m0 = (int64_t)tm * kTM, n0 = (int64_t)tn * kTN;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, h = lane >> 5;

  __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)a.aq, 0, a.a_qbytes, 0x00020000);
  __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc((void*)a.wq, 0, a.w_qbytes, 0x00020000);
  __amdgpu_buffer_rsrc_t rSA = __builtin_amdgcn_make_buffer_rsrc((void*)a.as, 0, a.a_sbytes, 0x00020000);
  __amdgpu_buffer_rsrc_t rSW = __builtin_amdgcn_make_buffer_rsrc((void*)a.ws, 0, a.w_sbytes, 0x00020000);
  const int krow = (int)(a.k / 2);

  // ---- global -> register prefetch of one K step ----
  // codes: 1024 chunks of 16 bytes per operand, 4 per thread: chunk c -> row c/4, part c%4
  // scales: threads 0..127 load A's 4 tiles, 128..255 W's (16 bytes each)
  u32x4_t pa[4], pw[4], ps;
  auto prefetch = [&](int ks) {
    const bool half = (int64_t)(ks + 1) * kTK > a.k;  // only k-half 0 is inside K
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * kGemmThreads;
      const int row = c >> 2, part = c & 3;
      const bool ok = !(half && part >= 2);
      const int offa = (int)((m0 + row) * krow) + ks * 64 + part * 16;
      const int offw = (int)((n0 + row) * krow) + ks * 64 + part * 16;
      u32x4_t z = {0u, 0u, 0u, 0u};
      pa[i] = ok ? buf_load16(rA, offa) : z;
      pw[i] = ok ? buf_load16(rW, offw) : z;
    }
    {
      const int c = tid & 127;
      const int rt = c >> 6, cg = (c >> 5) & 1, part = c & 31;
      const bool ok = !(half && cg == 1);
      const int64_t rt_g = (tid < 128 ? m0 : n0) / 128 + rt;
      const int off = (int)((rt_g * a.cgroups + (int64_t)ks * 2 + cg) * 512) + part * 16;
      u32x4_t z = {0u, 0u, 0u, 0u};
      ps = ok ? buf_load16(tid < 128 ? rSA : rSW, off) : z;
    }
  };
  auto stash = [&](int buf) {
    unsigned char* st = smem + buf * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * kGemmThreads;
      const int row = c >> 2, part = c & 3;
      *(u32x4_t*)(st + row * kRowStride + part * 16) = pa[i];
      *(u32x4_t*)(st + kCodesBytes + row * kRowStride + part * 16) = pw[i];
    }
    const int c = tid & 127;
    *(u32x4_t*)(st + 2 * kCodesBytes + (tid < 128 ? 0 : kScaleBytes) + c * 16) = ps;
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

  prefetch(0);
  stash(0);
  __syncthreads();

  for (int ks = 0; ks < a.ksteps; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < a.ksteps) prefetch(ks + 1);
    const unsigned char* st = smem + buf * kStageBytes;
    const unsigned char* stA = st;
    const unsigned char* stW = st + kCodesBytes;
    const unsigned char* ssA = st + 2 * kCodesBytes;
    const unsigned char* ssW = ssA + kScaleBytes;

    // scales: one dword per fragment (4 blocks of this lane's k-half)
    uint32_t sa[4], sw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] = *(const uint32_t*)(ssA + (wm * 2 + h) * 512 + lr * 16 + i * 4);
      sw[i] = *(const uint32_t*)(ssW + (wn * 2 + h) * 512 + lr * 16 + i * 4);
    }
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      u32x4_t ca[4], cw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ca[i] = *(const u32x4_t*)(stA + (wm * 128 + i * 32 + lr) * kRowStride + h * 32 + kq * 16);
        cw[i] = *(const u32x4_t*)(stW + (wn * 128 + i * 32 + lr) * kRowStride + h * 32 + kq * 16);
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int blk = kq * 2 + (kk >> 1);
        f16x8_t fa[4], fw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fa[i] = dequant8(ca[i][kk], scale_pair(sa[i], blk));
          fw[i] = dequant8(cw[i][kk], scale_pair(sw[i], blk));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fw[j], fa[i], acc[j][i], 0, 0, 0);
      }
    }
    if (ks + 1 < a.ksteps) stash(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: D[m, n] = RN_bf16(alpha * acc), alpha = g_a * g_w ----
  const float alpha = (*a.ga) * (*a.gw);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + wm * 128 + i * 32 + lr;
      if (m >= a.m_pad) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = n0 + wn * 128 + j * 32 + q * 8 + h * 4;
        if (n >= a.n) continue;
        bf16x2_t lo, hi;
        lo[0] = (__bf16)(acc[j][i][q * 4 + 0] * alpha);
        lo[1] = (__bf16)(acc[j][i][q * 4 + 1] * alpha);
        hi[0] = (__bf16)(acc[j][i][q * 4 + 2] * alpha);
        hi[1] = (__bf16)(acc[j][i][q * 4 + 3] * alpha);
        uint32_t ul, uh;
        __builtin_memcpy(&ul, &lo, 4);
        __builtin_memcpy(&uh, &hi, 4);
        typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
        u32x2_t v = {ul, uh};
        *(u32x2_t*)(a.d + m * a.n + n) = v;
      }
    }
  }
}

// ---- host side -----------------------------------------------------------------------------

size_t gemm_smem_bytes() { return 2 * (size_t)kStageBytes; }
const void* gemm_kernel_ptr() { return (const void*)gemm_kernel; }

hipError_t launch_gemm(const uint8_t* aq, const uint8_t* as, const float* ga, const uint8_t* wq,
                       const uint8_t* ws, const float* gw, uint16_t* d, int64_t m_pad, int64_t n, int64_t k,
                       hipStream_t stream) {
  GemmArgs args;
  args.aq = aq;
  args.as = as;
  args.ga = ga;
  args.wq = wq;
  args.ws = ws;
  args.gw = gw;
  args.d = d;
  args.m_pad = m_pad;
  args.n = n;
  args.k = k;
  const int64_t cpad = (k / 16 + 3) / 4 * 4;
  args.a_qbytes = (int)(m_pad * (k / 2));
  args.w_qbytes = (int)(n * (k / 2));
  args.a_sbytes = (int)(((m_pad + 127) / 128 * 128) * cpad);
  args.w_sbytes = (int)(((n + 127) / 128 * 128) * cpad);
  args.tiles_m = (int)((m_pad + kTM - 1) / kTM);
  args.tiles_n = (int)((n + kTN - 1) / kTN);
  args.cgroups = (int)(cpad / 4);
  args.ksteps = (int)((k + kTK - 1) / kTK);
  const int ntiles = args.tiles_m * args.tiles_n;
  if (ntiles == 0) return hipSuccess;
  gemm_kernel<<<dim3(ntiles), dim3(kGemmThreads), gemm_smem_bytes(), stream>>>(args);
  return hipGetLastError();
}

}  // namespace nvfp4
