// ceiling.hip - measurement aid, not a step of the method: the dense fp16 matrix-core
// rate this device sustains, and the shader clock it runs at while doing so.
//
// Each workgroup is 4 waves (one per SIMD, as in the GEMM); each wave issues `iters`
// rounds of 4 independent v_mfma_f32_32x32x16_f16 (four accumulator chains, so the
// matrix pipe never waits on a result) and nothing else in the loop. Lane 0 of each
// wave records the shader-clock cycle count (s_memtime) and the 100 MHz real-time
// count (s_memrealtime) around its loop, which gives the clock during the run.
#include "common.hpp"

namespace nvfp4 {

constexpr int kCeilThreads = 256;

__global__ void __launch_bounds__(kCeilThreads, 1) mfma_ceiling_kernel(uint64_t* out, int64_t iters) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f16x8_t a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (_Float16)(float)((lane + j) & 7);
    b[j] = (_Float16)(float)((lane * 3 + j) & 3);
  }
  f32x16_t acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[q][r] = 0.0f;
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[q], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[q][r];
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
  uint64_t* slot = out + ((int64_t)blockIdx.x * 4 + wave) * 2;
  // the sum is never negative (non-negative operands); the test keeps the MFMAs live
  if (lane == 0) {
    slot[0] = s < 0.0f ? 0 : c1 - c0;
    slot[1] = t1 - t0;
  }
}

hipError_t launch_mfma_ceiling(uint64_t* out, int64_t workgroups, int64_t iters, hipStream_t stream) {
  mfma_ceiling_kernel<<<dim3((unsigned)workgroups), dim3(kCeilThreads), 0, stream>>>(out, iters);
  return hipGetLastError();
}

}  // namespace nvfp4
