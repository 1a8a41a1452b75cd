// silu.hip - the correctly rounded bf16 silu table the producer uses.
//
// The component-2 NSYS summary (keys "swiglu_silu_total_ms" and
// "swiglu_multiply_total_ms") shows SwiGLU as a bf16 silu kernel followed by a
// bf16 multiply; the fused producer keeps that arithmetic: silu_bf16(x) is
// x / (1 + e^-x) rounded once to bf16, nearest-even. There are only 65,536 bf16
// inputs, so the library evaluates every one of them once per device, in fp64,
// into a table in device memory; the producer stages it in LDS.
//
// Accuracy argument: for |x| >= 1/16 the silu values of all bf16 inputs stay at
// least 9.5e-8 (relative) away from every bf16 rounding boundary, far above the
// few-ulp error of an fp64 evaluation. For |x| < 1/16 the value x/2 is exact and
// may itself lie on a boundary (x tiny), with silu(x) = x/2 + (x/2) tanh(x/2) just
// off it; the sum is formed with its exact rounding error (TwoSum) and the error's
// sign breaks such ties. The table is compared bit for bit with the CPU oracle's
// in the GPU tests.
#include "common.hpp"

namespace nvfp4 {

__device__ uint16_t g_silu_table[65536];

// Round hi + lo to bf16 where t = hi + lo (fp64) and err = (hi + lo) - t exactly.
__device__ static uint32_t rn_bf16_pair(double hi, double lo) {
  double t = (lo == 0.0) ? hi : hi + lo;
  double bb = t - hi;
  double err = (hi - (t - bb)) + (lo - bb);
  uint64_t u = (uint64_t)__double_as_longlong(t);
  uint32_t sign = (uint32_t)(u >> 63) << 15;
  double a = fabs(t);
  if (a == 0.0) return sign;
  double e_dir = (u >> 63) ? -err : err;
  int ex = ((int)((u >> 52) & 0x7FF)) - 1023;
  int lead = ex < -126 ? -126 : ex;
  double q = ldexp(1.0, lead - 7);
  double r = a / q;
  double fl = floor(r);
  double fr = r - fl;
  double n;
  if (fr > 0.5) n = fl + 1.0;
  else if (fr < 0.5) n = fl;
  else if (e_dir > 0.0) n = fl + 1.0;
  else if (e_dir < 0.0) n = fl;
  else n = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
  double rr = n * q;
  if (rr >= 0x1p128) return sign | 0x7F80u;
  return sign | (__float_as_uint((float)rr) >> 16);
}

__device__ static uint32_t silu_bf16_exact(uint32_t xb) {
  double x = (double)bf16_bits_to_float(xb);
  if (x == 0.0) return xb;                     // silu(+-0) = +-0
  if ((xb & 0x7F80u) == 0x7F80u) return xb;    // not reached for finite inputs
  if (fabs(x) < 0.0625) {
    double h = 0.5 * x;
    return rn_bf16_pair(h, h * tanh(h));
  }
  return rn_bf16_pair(x / (1.0 + exp(-x)), 0.0);
}

__global__ void __launch_bounds__(256) silu_table_init_kernel() {
  uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i < 65536u) g_silu_table[i] = (uint16_t)silu_bf16_exact(i);
}

__global__ void __launch_bounds__(256) silu_apply_kernel(const uint16_t* __restrict__ x,
                                                         uint16_t* __restrict__ y, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = g_silu_table[x[i]];
}

// Device address of the table on the current device (kernels in other
// translation units take it as an argument).
hipError_t silu_table_address(const uint16_t** p) {
  return hipGetSymbolAddress((void**)p, HIP_SYMBOL(g_silu_table));
}

hipError_t launch_silu_table_init(hipStream_t stream) {
  silu_table_init_kernel<<<256, 256, 0, stream>>>();
  return hipGetLastError();
}

hipError_t launch_silu_apply(const uint16_t* x, uint16_t* y, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  silu_apply_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(x, y, n);
  return hipGetLastError();
}

}  // namespace nvfp4
