// api.hip - the C ABI of the library (declared in include/nvfp4.h): argument
// validation, one-time device set-up, launch of the producer and GEMM kernels.
//
// Every entry point validates all arguments before it enqueues anything; on an
// error it returns a status, enqueues nothing and writes nothing, and records a
// per-thread message for nvfp4_last_error().
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "nvfp4.h"
#include "common.hpp"

namespace nvfp4 {
hipError_t silu_table_address(const uint16_t** p);
hipError_t launch_silu_table_init(hipStream_t stream);
hipError_t launch_silu_apply(const uint16_t* x, uint16_t* y, int64_t n, hipStream_t stream);
// producer modes: 0 plain, 1 SwiGLU, 2 modulated plain
size_t producer_smem_bytes(int mode);
const void* producer_kernel_ptr(int mode, bool given);
const void* producer_absmax_kernel_ptr(int mode);
int producer_block_threads();
int64_t producer_units(int64_t m, int64_t k);
hipError_t launch_producer(int mode, const uint16_t* x, int64_t ldx, const uint16_t* u, int64_t ldu,
                           const uint16_t* mod_scale, const uint16_t* mod_shift, int64_t m, int64_t k,
                           uint8_t* qdata, uint8_t* scales, float* gout, const float* amax_in, void* workspace,
                           uint32_t* queue, const uint16_t* silu_table, int quant_blocks, hipStream_t stream);
size_t gemm_smem_bytes(int kind);
const void* gemm_kernel_ptr(int kind);
hipError_t launch_gemm(const uint8_t* aq, const uint8_t* as, const float* ga, const uint8_t* wq,
                       const uint8_t* ws, const float* gw, uint16_t* d, int64_t m_pad, int64_t n, int64_t k,
                       const GemmEpilogue& ep, int cu_count, uint64_t* sched, hipStream_t stream);
hipError_t launch_mfma_ceiling(uint64_t* out, int64_t workgroups, int64_t iters, hipStream_t stream);
hipError_t launch_hbm_stream(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes, int workgroups,
                             hipStream_t stream);
int64_t hbm_stream_chunk_bytes();
}  // namespace nvfp4

namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kMaxBufferBytes = (int64_t)1 << 31;  // 32-bit buffer offsets in the kernels

// A device's set-up. `ready` is published with release order after every other
// field is written (under g_init_mutex) and read with acquire order, so a thread that
// sees it set also sees the finished state without taking the lock.
struct DeviceState {
  std::atomic<bool> ready{false};
  const uint16_t* silu_table = nullptr;
  void* scratch = nullptr;  // this device's copy of `scratch` (hipGetSymbolAddress)
  uint64_t* gemm_queues = nullptr;  // this device's copy of `gemm_queues`
  std::atomic<uint32_t> gemm_launches{0};  // picks the queue set of each plain GEMM launch
  uint32_t* producer_queues = nullptr;  // this device's copy of `producer_queues`
  std::atomic<uint32_t> producer_launches{0};  // picks the counter set of each quantize launch
  int producer_blocks[3] = {0, 0, 0};  // quantize launch's persistent grid per producer mode
  int cu_count = 0;
  char arch[64] = {0};
};

DeviceState g_dev[kMaxDevices];

}  // namespace

// Producer scratch of nvfp4_quantize_swiglu_noalloc: the absmax slots that the other
// two-pass entry points keep in the caller's workspace (16 KiB). Each GPU holds its own
// copy for the life of the process, zero at load; host code uses only the per-device
// address that set-up obtains with hipGetSymbolAddress (the name itself is a host-side
// stand-in). Every call on a GPU shares it; each call's quantize launch clears the slots
// after reading them, so every call starts from zero; calls that overlap in time on one
// GPU race.
static __device__ __align__(256) uint32_t scratch[sizeof(nvfp4::ProducerWorkspace) / 4];

// Unit counters of the producer's quantize launch (zero at load). Launch i on a device
// uses set i % kProdQueueSets; its last wave leaves the set zeroed again, so up to
// kProdQueueSets quantize launches may run at the same time on one GPU.
static __device__ __align__(256) uint32_t producer_queues[nvfp4::kProdQueueSets * nvfp4::kProdQueueSetWords];

// Tile queues of the plain GEMM's persistent grid (zero at load). Launch i on a device
// uses set i % kGemmQueueSets; its last workgroup leaves the set zeroed again, so up to
// kGemmQueueSets plain GEMM launches may run at the same time on one GPU.
static __device__ __align__(256) uint64_t gemm_queues[nvfp4::kGemmQueueSets * nvfp4::kGemmQueueWords];

namespace {
std::mutex g_init_mutex;
thread_local char t_last_error[512] = "";
thread_local char t_build_info[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(t_last_error, sizeof(t_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  t_last_error[0] = '\0';
  return NVFP4_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// One-time set-up of the current device (caller holds no lock).
int ensure_device(DeviceState** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) return fail(NVFP4_ERR_NO_DEVICE, "no HIP device (%s)", hipGetErrorString(e));
  if (dev >= kMaxDevices) return fail(NVFP4_ERR_NO_DEVICE, "device index %d out of range", dev);
  DeviceState& st = g_dev[dev];
  if (st.ready.load(std::memory_order_acquire)) {
    *out = &st;
    return NVFP4_OK;
  }
  std::lock_guard<std::mutex> lock(g_init_mutex);
  if (st.ready.load(std::memory_order_relaxed)) {
    *out = &st;
    return NVFP4_OK;
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(NVFP4_ERR_NO_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(NVFP4_ERR_NO_DEVICE, "device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
  snprintf(st.arch, sizeof(st.arch), "%s", prop.gcnArchName);
  st.cu_count = prop.multiProcessorCount;

  // kernels with more than 64 KiB of dynamic LDS must opt in; the quantize launch runs
  // as many persistent workgroups as fit on the device at once
  for (int mode = 0; mode < 3; ++mode) {
    for (int given = 0; given < 2; ++given) {
      e = hipFuncSetAttribute(nvfp4::producer_kernel_ptr(mode, given != 0),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)nvfp4::producer_smem_bytes(mode));
      if (e != hipSuccess) return fail(NVFP4_ERR_LAUNCH, "producer LDS attribute: %s", hipGetErrorString(e));
    }
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, nvfp4::producer_kernel_ptr(mode, false),
                                                     nvfp4::producer_block_threads(),
                                                     nvfp4::producer_smem_bytes(mode));
    if (e != hipSuccess || per_cu < 1)
      return fail(NVFP4_ERR_LAUNCH, "producer occupancy query: %s (%d)", hipGetErrorString(e), per_cu);
    st.producer_blocks[mode] = per_cu * st.cu_count;
  }
  for (int kind = 0; kind < 3; ++kind) {
    e = hipFuncSetAttribute(nvfp4::gemm_kernel_ptr(kind), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)nvfp4::gemm_smem_bytes(kind));
    if (e != hipSuccess) return fail(NVFP4_ERR_LAUNCH, "gemm LDS attribute: %s", hipGetErrorString(e));
  }

  e = nvfp4::silu_table_address(&st.silu_table);
  if (e != hipSuccess) return fail(NVFP4_ERR_LAUNCH, "silu table address: %s", hipGetErrorString(e));
  e = hipGetSymbolAddress(&st.scratch, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !st.scratch)
    return fail(NVFP4_ERR_LAUNCH, "producer scratch address: %s", hipGetErrorString(e));
  void* q = nullptr;
  e = hipGetSymbolAddress(&q, HIP_SYMBOL(gemm_queues));
  if (e != hipSuccess || !q) return fail(NVFP4_ERR_LAUNCH, "gemm queue address: %s", hipGetErrorString(e));
  st.gemm_queues = (uint64_t*)q;
  void* pq = nullptr;
  e = hipGetSymbolAddress(&pq, HIP_SYMBOL(producer_queues));
  if (e != hipSuccess || !pq) return fail(NVFP4_ERR_LAUNCH, "producer queue address: %s", hipGetErrorString(e));
  st.producer_queues = (uint32_t*)pq;
  hipStream_t s;
  e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
  if (e != hipSuccess) return fail(NVFP4_ERR_LAUNCH, "stream create: %s", hipGetErrorString(e));
  e = nvfp4::launch_silu_table_init(s);
  hipError_t e2 = hipStreamSynchronize(s);
  (void)hipStreamDestroy(s);
  if (e != hipSuccess || e2 != hipSuccess)
    return fail(NVFP4_ERR_LAUNCH, "silu table init: %s / %s", hipGetErrorString(e), hipGetErrorString(e2));
  st.ready.store(true, std::memory_order_release);
  *out = &st;
  return NVFP4_OK;
}

// The counter set of the next quantize launch on this device.
uint32_t* producer_queue_set(DeviceState& st) {
  const uint32_t set = st.producer_launches.fetch_add(1, std::memory_order_relaxed) % nvfp4::kProdQueueSets;
  return st.producer_queues + (size_t)set * nvfp4::kProdQueueSetWords;
}

// ws: the workspace of the two-pass producer, or the caller's amax of the single-pass
// one; with `scratch` (the library's own scratch stands in for the workspace) ws is unused
int check_quant_args(const void* x, int64_t ldx, const void* u, int64_t ldu, bool swiglu, int64_t m, int64_t k,
                     const void* qdata, const void* scales, const float* g, const void* ws, bool given,
                     bool scratch = false) {
  if (!g) return fail(NVFP4_ERR_INVALID_ARG, "null global-scale pointer");
  // with no rows nothing is read or written except the global scale
  if (m != 0 && (!x || (swiglu && !u) || !qdata || !scales))
    return fail(NVFP4_ERR_INVALID_ARG, "null input or output pointer");
  if (given && !ws) return fail(NVFP4_ERR_INVALID_ARG, "null amax pointer");
  if (!given && !scratch && !ws) return fail(NVFP4_ERR_WORKSPACE, "null workspace");
  if (m < 0 || k <= 0) return fail(NVFP4_ERR_INVALID_ARG, "bad shape m=%lld k=%lld", (long long)m, (long long)k);
  if (k % 64 != 0) return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "k=%lld is not a multiple of 64", (long long)k);
  if (ldx < k || (swiglu && ldu < k))
    return fail(NVFP4_ERR_INVALID_ARG, "row stride below k (ld=%lld, %lld, k=%lld)", (long long)ldx,
                (long long)ldu, (long long)k);
  // a documented limit that keeps every per-row count (512-column segments, scale
  // columns) far inside 32-bit integers
  if (k > ((int64_t)1 << 23) || ldx > ((int64_t)1 << 23) || (swiglu && ldu > ((int64_t)1 << 23)))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "k and row strides above 2^23 elements are not supported");
  if (ldx % 8 != 0 || (swiglu && ldu % 8 != 0))
    return fail(NVFP4_ERR_MISALIGNED, "row strides must be multiples of 8 elements");
  if (!aligned16(x) || (swiglu && !aligned16(u)) || !aligned16(qdata) || !aligned16(scales) || ((uintptr_t)g & 3u) ||
      (given ? ((uintptr_t)ws & 3u) != 0 : (!scratch && !aligned16(ws))))
    return fail(NVFP4_ERR_MISALIGNED, "pointers must be 16-byte aligned (global scale and amax 4-byte)");
  // units of 4 rows x 512 columns are numbered with 32-bit integers
  if (nvfp4::producer_units(m, k) > (int64_t)1 << 30) return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "tensor too large");
  return NVFP4_OK;
}

}  // namespace

extern "C" {

int64_t nvfp4_padded_rows(int64_t rows) { return rows < 0 ? -1 : (rows + 15) / 16 * 16; }
int64_t nvfp4_scale_rows(int64_t rows) { return rows < 0 ? -1 : (nvfp4_padded_rows(rows) + 127) / 128 * 128; }
int64_t nvfp4_scale_cols(int64_t k) { return k < 0 ? -1 : (k / 16 + 3) / 4 * 4; }
int64_t nvfp4_qdata_bytes(int64_t rows, int64_t k) {
  return (rows < 0 || k < 0) ? -1 : nvfp4_padded_rows(rows) * (k / 2);
}
int64_t nvfp4_scale_bytes(int64_t rows, int64_t k) {
  return (rows < 0 || k < 0) ? -1 : nvfp4_scale_rows(rows) * nvfp4_scale_cols(k);
}
int64_t nvfp4_quantize_workspace_bytes(void) { return (int64_t)sizeof(nvfp4::ProducerWorkspace); }

int nvfp4_init(void) {
  DeviceState* st = nullptr;
  int rc = ensure_device(&st);
  return rc == NVFP4_OK ? ok() : rc;
}

static int quantize_common(int mode, bool given, const void* x, int64_t ldx, const void* u, int64_t ldu,
                           const void* mod_scale, const void* mod_shift, int64_t m, int64_t k, void* qdata,
                           void* scales, float* g, const float* amax, void* ws, void* stream) {
  const bool swiglu = mode == 1;
  int rc = check_quant_args(x, ldx, u, ldu, swiglu, m, k, qdata, scales, g, given ? (const void*)amax : ws, given);
  if (rc != NVFP4_OK) return rc;
  if (mode == 2) {
    if (!mod_scale || !mod_shift) return fail(NVFP4_ERR_INVALID_ARG, "null modulation scale or shift");
    if (!aligned16(mod_scale) || !aligned16(mod_shift))
      return fail(NVFP4_ERR_MISALIGNED, "modulation scale and shift must be 16-byte aligned");
  }
  DeviceState* st = nullptr;
  rc = ensure_device(&st);
  if (rc != NVFP4_OK) return rc;
  hipError_t e = nvfp4::launch_producer(mode, (const uint16_t*)x, ldx, (const uint16_t*)u, ldu,
                                        (const uint16_t*)mod_scale, (const uint16_t*)mod_shift, m, k,
                                        (uint8_t*)qdata, (uint8_t*)scales, g, amax, given ? nullptr : ws,
                                        producer_queue_set(*st), st->silu_table, st->producer_blocks[mode],
                                        (hipStream_t)stream);
  if (e != hipSuccess) return fail(NVFP4_ERR_LAUNCH, "producer launch: %s", hipGetErrorString(e));
  return ok();
}

int nvfp4_quantize_swiglu(const void* gate_dev, int64_t ld_gate, const void* up_dev, int64_t ld_up, int64_t m,
                          int64_t k, void* qdata_dev, void* scales_dev, float* global_scale_dev, void* workspace_dev,
                          void* stream) {
  return quantize_common(1, false, gate_dev, ld_gate, up_dev, ld_up, nullptr, nullptr, m, k, qdata_dev, scales_dev,
                         global_scale_dev, nullptr, workspace_dev, stream);
}

int nvfp4_quantize_swiglu_noalloc(const void* gate_dev, int64_t ld_gate, const void* up_dev, int64_t ld_up, int64_t m,
                                  int64_t k, void* qdata_dev, void* scales_dev, float* global_scale_dev,
                                  void* stream) {
  // every argument is validated as for nvfp4_quantize_swiglu; the scratch is the workspace
  int rc = check_quant_args(gate_dev, ld_gate, up_dev, ld_up, true, m, k, qdata_dev, scales_dev, global_scale_dev,
                            nullptr, false, true);
  if (rc != NVFP4_OK) return rc;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(NVFP4_ERR_NO_DEVICE, "no HIP device (%s)", hipGetErrorString(e));
  DeviceState& st = g_dev[dev];
  // set-up allocates (a stream for the silu table build), so it is not done here
  if (!st.ready.load(std::memory_order_acquire))
    return fail(NVFP4_ERR_NO_DEVICE, "call nvfp4_init on device %d before nvfp4_quantize_swiglu_noalloc", dev);
  // the scratch is one workspace: a fixed set of absmax slots, whatever the shape
  static_assert(sizeof(scratch) == sizeof(nvfp4::ProducerWorkspace), "scratch holds one workspace");
  e = nvfp4::launch_producer(1, (const uint16_t*)gate_dev, ld_gate, (const uint16_t*)up_dev, ld_up, nullptr, nullptr,
                             m, k, (uint8_t*)qdata_dev, (uint8_t*)scales_dev, global_scale_dev, nullptr, st.scratch,
                             producer_queue_set(st), st.silu_table, st.producer_blocks[1], (hipStream_t)stream);
  if (e != hipSuccess) return fail(NVFP4_ERR_LAUNCH, "producer launch: %s", hipGetErrorString(e));
  return ok();
}

int nvfp4_quantize_swiglu_amax(const void* gate_dev, int64_t ld_gate, const void* up_dev, int64_t ld_up, int64_t m,
                               int64_t k, const float* amax_dev, void* qdata_dev, void* scales_dev,
                               float* global_scale_dev, void* stream) {
  return quantize_common(1, true, gate_dev, ld_gate, up_dev, ld_up, nullptr, nullptr, m, k, qdata_dev, scales_dev,
                         global_scale_dev, amax_dev, nullptr, stream);
}

int nvfp4_quantize(const void* x_dev, int64_t ld_x, int64_t rows, int64_t k, void* qdata_dev, void* scales_dev,
                   float* global_scale_dev, void* workspace_dev, void* stream) {
  return quantize_common(0, false, x_dev, ld_x, nullptr, 0, nullptr, nullptr, rows, k, qdata_dev, scales_dev,
                         global_scale_dev, nullptr, workspace_dev, stream);
}

int nvfp4_quantize_modulate(const void* x_dev, int64_t ld_x, int64_t rows, int64_t k, const void* scale_dev,
                            const void* shift_dev, void* qdata_dev, void* scales_dev, float* global_scale_dev,
                            void* workspace_dev, void* stream) {
  return quantize_common(2, false, x_dev, ld_x, nullptr, 0, scale_dev, shift_dev, rows, k, qdata_dev, scales_dev,
                         global_scale_dev, nullptr, workspace_dev, stream);
}

int nvfp4_quantize_amax(const void* x_dev, int64_t ld_x, int64_t rows, int64_t k, const float* amax_dev,
                        void* qdata_dev, void* scales_dev, float* global_scale_dev, void* stream) {
  return quantize_common(0, true, x_dev, ld_x, nullptr, 0, nullptr, nullptr, rows, k, qdata_dev, scales_dev,
                         global_scale_dev, amax_dev, nullptr, stream);
}

static int gemm_common(const void* a_qdata_dev, const void* a_scales_dev, const float* a_global_dev,
                       const void* w_qdata_dev, const void* w_scales_dev, const float* w_global_dev, void* d_dev,
                       int64_t m_padded, int64_t n, int64_t k, const nvfp4::GemmEpilogue& ep, void* stream) {
  if (!a_qdata_dev || !a_scales_dev || !a_global_dev || !w_qdata_dev || !w_scales_dev || !w_global_dev || !d_dev)
    return fail(NVFP4_ERR_INVALID_ARG, "null pointer argument");
  if (m_padded < 0 || n <= 0 || k <= 0)
    return fail(NVFP4_ERR_INVALID_ARG, "bad shape m_padded=%lld n=%lld k=%lld", (long long)m_padded, (long long)n,
                (long long)k);
  if (m_padded % 16 != 0 || n % 16 != 0 || k % 64 != 0)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "need m_padded %% 16 == 0, n %% 16 == 0, k %% 64 == 0 (got %lld, %lld, %lld)",
                (long long)m_padded, (long long)n, (long long)k);
  if (!aligned16(a_qdata_dev) || !aligned16(a_scales_dev) || !aligned16(w_qdata_dev) || !aligned16(w_scales_dev) ||
      !aligned16(d_dev) || ((uintptr_t)a_global_dev & 3u) || ((uintptr_t)w_global_dev & 3u))
    return fail(NVFP4_ERR_MISALIGNED, "pointers must be 16-byte aligned (global scales 4-byte)");
  if (ep.gate && !ep.res) return fail(NVFP4_ERR_INVALID_ARG, "a gate needs a residual");
  if (!aligned16(ep.bias) || !aligned16(ep.gate) || !aligned16(ep.res) || !aligned16(ep.gate_out) ||
      !aligned16(ep.up_out) || ((uintptr_t)ep.amax & 3u))
    return fail(NVFP4_ERR_MISALIGNED, "epilogue operands must be 16-byte aligned (amax 4-byte)");
  if (ep.kind == 2 && (!ep.gate_out || !ep.up_out))
    return fail(NVFP4_ERR_INVALID_ARG, "null gate or up output");
  if (ep.kind == 2 && (ep.amax_rows < 0 || ep.amax_rows > m_padded))
    return fail(NVFP4_ERR_INVALID_ARG, "amax_rows=%lld outside [0, m_padded]", (long long)ep.amax_rows);
  const int64_t mt = (m_padded + 255) / 256 * 256, nt = (n + 255) / 256 * 256;
  if (mt * (k / 2) >= kMaxBufferBytes || nt * (k / 2) >= kMaxBufferBytes ||
      (mt + 128) * nvfp4_scale_cols(k) >= kMaxBufferBytes || (nt + 128) * nvfp4_scale_cols(k) >= kMaxBufferBytes ||
      (mt / 256) * (nt / 256) >= ((int64_t)1 << 31))
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "operands beyond 2 GiB are not supported");
  DeviceState* st = nullptr;
  int rc = ensure_device(&st);
  if (rc != NVFP4_OK) return rc;
  if (m_padded == 0) return ok();
  nvfp4::GemmEpilogue ep2 = ep;
  ep2.silu_table = st->silu_table;
  const uint32_t set = st->gemm_launches.fetch_add(1, std::memory_order_relaxed) % nvfp4::kGemmQueueSets;
  uint64_t* queues = st->gemm_queues + (size_t)set * nvfp4::kGemmQueueWords;
  hipError_t e = nvfp4::launch_gemm((const uint8_t*)a_qdata_dev, (const uint8_t*)a_scales_dev, a_global_dev,
                                    (const uint8_t*)w_qdata_dev, (const uint8_t*)w_scales_dev, w_global_dev,
                                    (uint16_t*)d_dev, m_padded, n, k, ep2, st->cu_count, queues, (hipStream_t)stream);
  if (e != hipSuccess) return fail(NVFP4_ERR_LAUNCH, "gemm launch: %s", hipGetErrorString(e));
  return ok();
}

int nvfp4_gemm_bf16out(const void* a_qdata_dev, const void* a_scales_dev, const float* a_global_dev,
                       const void* w_qdata_dev, const void* w_scales_dev, const float* w_global_dev, void* d_dev,
                       int64_t m_padded, int64_t n, int64_t k, void* stream) {
  return gemm_common(a_qdata_dev, a_scales_dev, a_global_dev, w_qdata_dev, w_scales_dev, w_global_dev, d_dev,
                     m_padded, n, k, nvfp4::GemmEpilogue(), stream);
}

int nvfp4_gemm_bf16out_clock(const void* a_qdata_dev, const void* a_scales_dev, const float* a_global_dev,
                             const void* w_qdata_dev, const void* w_scales_dev, const float* w_global_dev,
                             void* d_dev, int64_t m_padded, int64_t n, int64_t k, void* clk_dev, int64_t slots,
                             void* stream) {
  if (!clk_dev || slots < 1 || slots > (int64_t)1 << 20)
    return fail(NVFP4_ERR_INVALID_ARG, "clock stamps need a buffer and 1..2^20 slots");
  if ((uintptr_t)clk_dev & 7u) return fail(NVFP4_ERR_MISALIGNED, "clock buffer must be 8-byte aligned");
  nvfp4::GemmEpilogue ep;
  ep.clk = (uint64_t*)clk_dev;
  ep.clk_slots = (int)slots;
  return gemm_common(a_qdata_dev, a_scales_dev, a_global_dev, w_qdata_dev, w_scales_dev, w_global_dev, d_dev,
                     m_padded, n, k, ep, stream);
}

int nvfp4_gemm_bf16out_fused(const void* a_qdata_dev, const void* a_scales_dev, const float* a_global_dev,
                             const void* w_qdata_dev, const void* w_scales_dev, const float* w_global_dev,
                             void* d_dev, int64_t m_padded, int64_t n, int64_t k, const void* bias_dev,
                             const void* gate_dev, const void* residual_dev, void* stream) {
  nvfp4::GemmEpilogue ep;
  ep.kind = 1;
  ep.bias = (const uint16_t*)bias_dev;
  ep.gate = (const uint16_t*)gate_dev;
  ep.res = (const uint16_t*)residual_dev;
  return gemm_common(a_qdata_dev, a_scales_dev, a_global_dev, w_qdata_dev, w_scales_dev, w_global_dev, d_dev,
                     m_padded, n, k, ep, stream);
}

int nvfp4_gemm_swiglu_pair(const void* a_qdata_dev, const void* a_scales_dev, const float* a_global_dev,
                           const void* w_qdata_dev, const void* w_scales_dev, const float* w_global_dev,
                           void* gate_dev, void* up_dev, int64_t m_padded, int64_t n_half, int64_t k,
                           const void* bias_dev, float* amax_dev, int64_t amax_rows, void* stream) {
  if (n_half <= 0 || n_half % 8 != 0)
    return fail(NVFP4_ERR_UNSUPPORTED_SHAPE, "n_half=%lld must be a positive multiple of 8", (long long)n_half);
  nvfp4::GemmEpilogue ep;
  ep.kind = 2;
  ep.bias = (const uint16_t*)bias_dev;
  ep.gate_out = (uint16_t*)gate_dev;
  ep.up_out = (uint16_t*)up_dev;
  ep.amax = amax_dev;
  ep.amax_rows = amax_rows;
  // d is unused by this epilogue; the gate output stands in for the pointer checks
  return gemm_common(a_qdata_dev, a_scales_dev, a_global_dev, w_qdata_dev, w_scales_dev, w_global_dev, gate_dev,
                     m_padded, 2 * n_half, k, ep, stream);
}

int nvfp4_silu_bf16(const void* x_dev, void* y_dev, int64_t count, void* stream) {
  if (count < 0) return fail(NVFP4_ERR_INVALID_ARG, "negative count");
  if (count > 0 && (!x_dev || !y_dev)) return fail(NVFP4_ERR_INVALID_ARG, "null pointer argument");
  if (((uintptr_t)x_dev & 1u) || ((uintptr_t)y_dev & 1u)) return fail(NVFP4_ERR_MISALIGNED, "2-byte alignment");
  DeviceState* st = nullptr;
  int rc = ensure_device(&st);
  if (rc != NVFP4_OK) return rc;
  hipError_t e = nvfp4::launch_silu_apply((const uint16_t*)x_dev, (uint16_t*)y_dev, count, (hipStream_t)stream);
  if (e != hipSuccess) return fail(NVFP4_ERR_LAUNCH, "silu launch: %s", hipGetErrorString(e));
  return ok();
}

int64_t nvfp4_mfma_ceiling_out_bytes(int64_t workgroups) { return workgroups > 0 ? workgroups * 4 * 16 : 0; }

int nvfp4_mfma_ceiling(int64_t workgroups, int64_t iters, void* out_dev, int64_t out_bytes, void* stream) {
  if (workgroups < 1 || workgroups > 65536) return fail(NVFP4_ERR_INVALID_ARG, "workgroups must be in [1, 65536]");
  if (iters < 1 || iters > ((int64_t)1 << 24)) return fail(NVFP4_ERR_INVALID_ARG, "iters must be in [1, 2^24]");
  if (!out_dev) return fail(NVFP4_ERR_INVALID_ARG, "null pointer argument");
  if ((uintptr_t)out_dev & 7u) return fail(NVFP4_ERR_MISALIGNED, "out must be 8-byte aligned");
  if (out_bytes < nvfp4_mfma_ceiling_out_bytes(workgroups))
    return fail(NVFP4_ERR_INVALID_ARG, "out holds %lld bytes; %lld needed", (long long)out_bytes,
                (long long)nvfp4_mfma_ceiling_out_bytes(workgroups));
  DeviceState* st = nullptr;
  int rc = ensure_device(&st);
  if (rc != NVFP4_OK) return rc;
  hipError_t e = nvfp4::launch_mfma_ceiling((uint64_t*)out_dev, workgroups, iters, (hipStream_t)stream);
  if (e != hipSuccess) return fail(NVFP4_ERR_LAUNCH, "ceiling launch: %s", hipGetErrorString(e));
  return ok();
}

int64_t nvfp4_hbm_stream_chunk_bytes(void) { return nvfp4::hbm_stream_chunk_bytes(); }

int nvfp4_hbm_stream_ceiling(const void* src_dev, int64_t read_bytes, void* dst_dev, int64_t write_bytes,
                             void* stream) {
  const int64_t chunk = nvfp4::hbm_stream_chunk_bytes();
  if (!src_dev || !dst_dev) return fail(NVFP4_ERR_INVALID_ARG, "null pointer argument");
  if (read_bytes <= 0 || read_bytes % chunk != 0 || read_bytes / chunk > 0x7FFFFFFF)
    return fail(NVFP4_ERR_INVALID_ARG, "read_bytes must be a positive multiple of %lld (at most 2^31 chunks)",
                (long long)chunk);
  if (write_bytes < 0 || write_bytes > read_bytes || write_bytes % 16 != 0)
    return fail(NVFP4_ERR_INVALID_ARG, "write_bytes must be a multiple of 16 in [0, read_bytes]");
  if (!aligned16(src_dev) || !aligned16(dst_dev)) return fail(NVFP4_ERR_MISALIGNED, "pointers must be 16-byte aligned");
  DeviceState* st = nullptr;
  int rc = ensure_device(&st);
  if (rc != NVFP4_OK) return rc;
  hipError_t e = nvfp4::launch_hbm_stream(src_dev, read_bytes, dst_dev, write_bytes, st->cu_count * 8,
                                          (hipStream_t)stream);
  if (e != hipSuccess) return fail(NVFP4_ERR_LAUNCH, "stream probe launch: %s", hipGetErrorString(e));
  return ok();
}

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_INVALID_ARG: return "invalid argument";
    case NVFP4_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case NVFP4_ERR_MISALIGNED: return "misaligned pointer or stride";
    case NVFP4_ERR_WORKSPACE: return "workspace missing";
    case NVFP4_ERR_NO_DEVICE: return "no usable gfx950 device";
    case NVFP4_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char* nvfp4_last_error(void) { return t_last_error; }

const char* nvfp4_build_info(void) {
  int rt = 0, drv = 0;
  (void)hipRuntimeGetVersion(&rt);
  (void)hipDriverGetVersion(&drv);
  int dev = -1;
  const char* arch = "";
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices &&
      g_dev[dev].ready.load(std::memory_order_acquire))
    arch = g_dev[dev].arch;
  snprintf(t_build_info, sizeof(t_build_info),
           "nvfp4 gfx950; HIP compile %d.%d.%d; HIP runtime %d; driver %d; device arch %s", HIP_VERSION_MAJOR,
           HIP_VERSION_MINOR, HIP_VERSION_PATCH, rt, drv, arch[0] ? arch : "(not initialised)");
  return t_build_info;
}

}  // extern "C"
