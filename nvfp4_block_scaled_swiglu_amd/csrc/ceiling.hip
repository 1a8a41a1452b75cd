// ceiling.hip - measurement aids, not steps of the method: the dense fp16 matrix-core
// rate this device sustains and the shader clock it runs at while doing so, and the
// HBM rate of a plain streaming kernel for a given mix of reads and writes.
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

// HBM streaming probe. The source is cut into chunks of kStreamChunk bytes and each
// workgroup streams one chunk and exits (a one-shot grid, dispatched in address order:
// the fastest form measured on this device, ahead of persistent grids that walk the
// chunks). Each thread loads 4 x 16 bytes of its chunk with all four loads in flight
// before their use. Loads and stores are non-temporal: measured on this device, that
// streams about 10 % more than plain accesses, read-only and at the quantize launch's
// write share alike, so it is the ceiling the producer is read against. For a write share w (bytes written per byte read, w <= 1), each chunk
// also stores its share of the destination, whole 16-byte pieces from the first threads:
// chunk c writes dst bytes [c * wpc, (c + 1) * wpc), wpc = write_bytes / chunks. The
// loaded words are folded into an XOR that is stored only if it equals a value the
// source never yields (so the loads stay live without extra traffic).
constexpr int kStreamThreads = 256;
constexpr int64_t kStreamChunk = kStreamThreads * 64;  // 16 KiB

__global__ void __launch_bounds__(kStreamThreads) hbm_stream_kernel(const u32x4_t* __restrict__ src,
                                                                  u32x4_t* __restrict__ dst, int64_t wpc16,
                                                                  uint32_t never) {
  const int t = threadIdx.x;
  const int64_t c = blockIdx.x;
  const u32x4_t* p = src + c * (kStreamChunk / 16);
  u32x4_t v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = __builtin_nontemporal_load(p + j * kStreamThreads + t);
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  for (int64_t i = t; i < wpc16; i += kStreamThreads) {
    const u32x4_t w = {acc, (uint32_t)i, (uint32_t)c, 0u};
    __builtin_nontemporal_store(w, dst + c * wpc16 + i);
  }
  if (acc == never) dst[0][0] = acc;
}

hipError_t launch_hbm_stream(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes, int /*workgroups*/,
                             hipStream_t stream) {
  const int64_t chunks = read_bytes / kStreamChunk;
  const int64_t wpc16 = write_bytes / 16 / chunks;
  hbm_stream_kernel<<<dim3((unsigned)chunks), dim3(kStreamThreads), 0, stream>>>((const u32x4_t*)src, (u32x4_t*)dst,
                                                                              wpc16, 0xFFFFFFFFu);
  return hipGetLastError();
}

int64_t hbm_stream_chunk_bytes() { return kStreamChunk; }

}  // namespace nvfp4
