// common.hpp - device helpers shared by the HIP kernels of the NVFP4 library (gfx950).
//
// Formats ("FC2 NVFP4 Scheduling Results", section "Canonical Operation"):
//   bf16   : 1 sign, 8 exponent (bias 127), 7 fraction bits.
//   UE4M3  : unsigned, 4 exponent (bias 7), 3 mantissa bits; E == 0 is subnormal
//            (m * 2^-9); the library never produces 0x7F.
//   E2M1   : 1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
//            {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// Workspace of the two-pass producer: kAmaxSlots slots, kSlotStride words apart (one
// per 256 bytes, so that the atomic maxima of the absmax launch spread over the memory
// channels). The absmax launch folds each workgroup's max |y| into slot
// (workgroup % kAmaxSlots) by atomic max (fp32 bits of a non-negative bf16 value, so
// unsigned order is value order); the quantize launch reads every slot and its last
// wave clears them. The workspace must therefore be zero before its first use, and
// every completed call leaves it zero.
constexpr int kAmaxSlots = 64;
constexpr int kSlotStride = 64;
struct ProducerWorkspace {
  uint32_t slot[kAmaxSlots * kSlotStride];
};
static_assert(sizeof(ProducerWorkspace) == 16384, "workspace layout");

// Unit queues of the producer's quantize launch: kProdQueueCounters counters
// kSlotStride words apart, then the word that counts the waves that have finished.
// Launch i on a device uses set i % kProdQueueSets (static device memory, zero at
// load); its last wave leaves the set zero again.
constexpr int kProdQueueCounters = 32;
constexpr int kProdQueueSetWords = (kProdQueueCounters + 1) * kSlotStride;
constexpr int kProdQueueSets = 64;

// Tile-queue words of the plain GEMM's persistent grid: one set of kGemmQueueWords
// per launch in flight, kGemmQueueSets sets per device (static device memory).
constexpr int kGemmQueueWords = 16;
constexpr int kGemmQueueSets = 64;

// What the GEMM does after its K loop (host -> launch_gemm).
//   kind 0: D = RN_bf16(alpha * acc)
//   kind 1: D1 = RN_bf16(alpha * acc + bias), D = RN_bf16(res + gate * D1)
//   kind 2: the SwiGLU pair: D1 as in kind 1 over gate/up rows interleaved in
//           chunks of 8, written to gate_out / up_out [m_pad, n / 2], and the
//           maximum of |RN_bf16(silu_bf16(gate) * up)| over rows < amax_rows
//           folded into *amax with an atomic max
struct GemmEpilogue {
  int kind = 0;
  const uint16_t* bias = nullptr;
  const uint16_t* gate = nullptr;
  const uint16_t* res = nullptr;
  uint16_t* gate_out = nullptr;
  uint16_t* up_out = nullptr;
  float* amax = nullptr;
  int64_t amax_rows = 0;
  const uint16_t* silu_table = nullptr;
  // measurement aid: workgroup b < clk_slots writes its shader-clock cycles and
  // 100 MHz ticks from start to end to clk[2b], clk[2b + 1] (null: nothing recorded)
  uint64_t* clk = nullptr;
  int clk_slots = 0;
};

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

__device__ __forceinline__ double ue4m3_to_double(uint32_t e) {
  uint32_t E = e >> 3, m = e & 7u;
  if (E == 0) return (double)m * 0x1p-9;
  uint64_t bits = ((uint64_t)(E - 7 + 1023) << 52) | ((uint64_t)m << 49);
  return __longlong_as_double((long long)bits);
}

__device__ __forceinline__ float ue4m3_to_float(uint32_t e) {
  uint32_t E = e >> 3, m = e & 7u;
  if (E == 0) return (float)m * 0x1p-9f;
  return __uint_as_float(((E - 7u + 127u) << 23) | (m << 20));
}

// Round a double to the nearest bf16 (ties to even): one rounding, subnormal
// results handled (quantum 2^-133 below 2^-126). Finite inputs.
__device__ __forceinline__ uint32_t rn_bf16_from_double(double v) {
  uint64_t u = (uint64_t)__double_as_longlong(v);
  uint32_t sign = (uint32_t)(u >> 63) << 15;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int ex = ((int)((u >> 52) & 0x7FF)) - 1023;  // a >= 2^-1022 for every product here
  int lead = ex < -126 ? -126 : ex;
  double q = ldexp(1.0, lead - 7);
  double n = rint(a * ldexp(1.0, 7 - lead));      // exact scaling; rint is ties-to-even
  double r = n * q;
  if (r >= 0x1p128) return sign | 0x7F80u;
  return sign | (__float_as_uint((float)r) >> 16);  // r has <= 8 significant bits: exact
}

}  // namespace nvfp4
