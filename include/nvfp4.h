/*
 * nvfp4.h - C ABI of the MI355X (gfx950) NVFP4 SwiGLU producer and block-scaled GEMM.
 *
 * The library implements the NVFP4 MLP projection described on the pages
 * "FC2 NVFP4 Scheduling Results" (section "Canonical Operation": E2M1 operands
 * with vector-16 UE4M3 block scales, FP32 global scales and accumulation, BF16
 * output; logical M = 37,810 padded to 37,824 rows, N = 5,376, K = 14,336) and
 * "gb10-component2-nsys-summary" (the fused SwiGLU producer replacing separate
 * silu, multiply, absmax, finalize, zero-fill and pack kernels; the 128-row by
 * 4-scale-column tiled block-scale layout).
 *
 * Conventions for every entry point:
 *  - Pointers named *_dev are device pointers on the current HIP device; the
 *    caller owns all memory. The library allocates nothing and keeps no
 *    reference after a call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). All
 *    work is enqueued on it asynchronously; no call synchronises with the host
 *    except nvfp4_init (and the first call on a device, which runs it).
 *  - Arguments are validated before anything is enqueued. On any error the call
 *    returns a non-zero nvfp4_status, enqueues nothing and writes nothing;
 *    nvfp4_last_error() then describes the failure (per host thread).
 *  - Integer sizes are element counts unless named *_bytes.
 *
 * Data formats (shared by producer output and GEMM input):
 *  - QDATA: E2M1 codes, bit 3 = sign, bits 2..0 = magnitude index into
 *    {0, 0.5, 1, 1.5, 2, 3, 4, 6}; two codes per byte, the even (first) element
 *    in the low nibble. Row-major [padded_rows, k/2] bytes, rows padded to a
 *    multiple of 16 with zero bytes.
 *  - Block scales: one UE4M3 byte per 16 consecutive elements of a row
 *    (value (1 + m/8) * 2^(E-7), or m * 2^-9 when E == 0; never above 0x7E),
 *    stored in 512-byte tiles of 128 rows x 4 scale columns: byte (r, c) sits at
 *      ((r >> 7) * (C / 4) + (c >> 2)) * 512 + (r & 31) * 16 + ((r >> 5) & 3) * 4 + (c & 3)
 *    with C = roundup(k/16, 4); the buffer holds roundup(padded_rows, 128) * C
 *    bytes and every byte outside real rows/columns is zero.
 *  - Global scale: one FP32 on the device; element value = e2m1 * v(S) * g.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID_ARG = 1,       /* null pointer, negative size, bad stride */
  NVFP4_ERR_UNSUPPORTED_SHAPE = 2, /* k % 64 != 0, n % 16 != 0, m_padded % 16 != 0, too large */
  NVFP4_ERR_MISALIGNED = 3,        /* a pointer or row stride breaks the 16-byte alignment rule */
  NVFP4_ERR_WORKSPACE = 4,         /* workspace pointer missing */
  NVFP4_ERR_NO_DEVICE = 5,         /* no HIP device, or the current device is not gfx950 */
  NVFP4_ERR_LAUNCH = 6             /* the HIP runtime refused the launch (see nvfp4_last_error) */
} nvfp4_status;

/* ---- sizes (pure functions; no device access) ------------------------------------- */

/* Rows after the producer's padding: roundup(rows, 16). 37,810 -> 37,824
 * ("FC2 NVFP4 Scheduling Results", "Canonical Operation"). Returns -1 if rows < 0. */
int64_t nvfp4_padded_rows(int64_t rows);

/* Rows of the block-scale buffer: roundup(nvfp4_padded_rows(rows), 128). The
 * component-2 summary's intermediate byte count (key
 * intermediate_materialization_bytes_across_four_projections) decomposes exactly
 * with scale buffers padded this way. */
int64_t nvfp4_scale_rows(int64_t rows);

/* Scale columns: roundup(k / 16, 4), whole 4-scale-column tiles (component-2
 * summary, key native_pack_validation.fix: the "128-row by 4-scale-column tiled"
 * scale offset). Returns -1 if k < 0. */
int64_t nvfp4_scale_cols(int64_t k);

/* QDATA bytes: nvfp4_padded_rows(rows) * k / 2, two E2M1 codes per byte over the
 * padded rows ("FC2 NVFP4 Scheduling Results", "Traffic Attribution": the
 * activation's one-pass footprint counts the 37,824 descriptor rows). Returns -1 if
 * rows < 0 or k < 0. */
int64_t nvfp4_qdata_bytes(int64_t rows, int64_t k);

/* Block-scale buffer bytes: nvfp4_scale_rows(rows) * nvfp4_scale_cols(k), one UE4M3
 * byte per 16 elements in whole 128 x 4 tiles (component-2 summary, keys
 * native_pack_validation.fix and
 * intermediate_materialization_bytes_across_four_projections). Returns -1 if
 * rows < 0 or k < 0. */
int64_t nvfp4_scale_bytes(int64_t rows, int64_t k);

/* Bytes of the two-pass producers' workspace (16,384): 64 absmax slots, 256 bytes
 * apart, into which the absmax launch folds its workgroups' maxima by atomic max
 * and which the quantize launch reduces to the tensor amax. The component-2
 * summary's "conclusion" names the global scale as the dependency that needs an
 * explicit synchronisation design; this buffer carries it across the launch
 * boundary. The caller allocates it on the device (16-byte aligned), owns it, and
 * fills it with zeros before its first use; the quantize launch clears the slots
 * after reading them, so every completed call leaves the workspace zero-filled
 * again. After a call that failed between its two launches (NVFP4_ERR_LAUNCH), zero
 * it again. Calls that may overlap in time (different streams) need distinct
 * workspaces. */
int64_t nvfp4_quantize_workspace_bytes(void);

/* ---- set-up -------------------------------------------------------------------------- */

/* One-time set-up of the current device: checks that it is gfx950, builds the
 * producer's correctly rounded bf16 silu table in device memory and sizes the
 * producer's persistent grid. "FC2 NVFP4 Scheduling Results", "Production
 * Integration": production start-up prepares the extension and caches its
 * compatibility result before inference; this is that step. Synchronous; safe to
 * call repeatedly and from several threads. Called implicitly by the first call on
 * a device (which therefore synchronises once); call it explicitly at start-up, and
 * before capturing calls into a HIP graph. Errors: NVFP4_ERR_NO_DEVICE (no device,
 * or not gfx950), NVFP4_ERR_LAUNCH (the silu table build failed). */
int nvfp4_init(void);

/* ---- stage P: producer ---------------------------------------------------------------- */

/*
 * Fused SwiGLU -> NVFP4 quantization of y = RN_bf16(silu_bf16(gate) * up), where
 * silu_bf16 is x / (1 + e^-x) correctly rounded to bf16 (the component-2 summary's
 * pre-fusion chain: a bf16 silu kernel, then a bf16 multiply kernel).
 *
 * gate_dev, up_dev : bf16 [m, k] row-major, row strides ld_gate, ld_up (elements,
 *                    multiples of 8, >= k); 16-byte aligned. Read only.
 * m, k             : logical rows (>= 0) and columns (k > 0, k % 64 == 0). With
 *                    m == 0 only the global scale (0) is written and the input,
 *                    qdata and scales pointers may be NULL.
 * qdata_dev        : out, nvfp4_qdata_bytes(m, k) bytes, 16-byte aligned.
 * scales_dev       : out, nvfp4_scale_bytes(m, k) bytes, 16-byte aligned.
 * global_scale_dev : out, one float: g = amax / 2688 rounded up to FP32 (2688 =
 *                    6 * 448), amax = max |y| over the m logical rows (0 if none).
 * workspace_dev    : nvfp4_quantize_workspace_bytes() bytes (see there).
 *
 * Every byte of qdata and scales is written, padding included. Block scale S is
 * the smallest UE4M3 byte with v(S) * 6 * g >= max |y| over its 16 elements; each
 * code is the E2M1 value nearest to |y| / (v(S) * g), ties to the even code, with
 * the sign of y (also on zero). Two ordinary launches on `stream`: the absmax pass
 * folds per-workgroup maxima into the workspace's slots, and the pack-and-swizzle
 * pass reduces them to the global scale (the launch boundary is the grid-wide
 * synchronisation) and clears them. The pack-and-swizzle pass takes its work from
 * run-time counters in static device memory (one set per launch, 64 sets per GPU
 * used in turn and left zero by each launch), so at most 64 producer launches may
 * be in flight on one GPU at a time. Inputs must be finite and keep every
 * |silu(gate) * up| below 2^128.
 */
int nvfp4_quantize_swiglu(const void* gate_dev, int64_t ld_gate, const void* up_dev, int64_t ld_up,
                          int64_t m, int64_t k, void* qdata_dev, void* scales_dev,
                          float* global_scale_dev, void* workspace_dev, void* stream);

/*
 * nvfp4_quantize_swiglu for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * same operation, arguments, layouts and outputs, without the workspace argument.
 * The absmax slots live in the library's own scratch, a fixed 16,384-byte device
 * array per GPU (one workspace, zero at load) held until the process ends; the call
 * allocates nothing and calls no allocating routine. Set-up allocates, so
 * nvfp4_init must have run on the current device first (otherwise
 * NVFP4_ERR_NO_DEVICE). Every call on a GPU shares that GPU's scratch: each call's
 * quantize launch clears the slots after reading them, so every call starts from
 * zero, but calls that overlap in time on one GPU (different streams) race and may
 * produce wrong global scales; serialise them, or use nvfp4_quantize_swiglu with
 * distinct workspaces.
 */
int nvfp4_quantize_swiglu_noalloc(const void* gate_dev, int64_t ld_gate, const void* up_dev, int64_t ld_up,
                                  int64_t m, int64_t k, void* qdata_dev, void* scales_dev,
                                  float* global_scale_dev, void* stream);

/* Plain NVFP4 quantization of x (y = x): the same contract as
 * nvfp4_quantize_swiglu with one bf16 [rows, k] input of row stride ld_x. The
 * component-2 summary lists this generic producer (absmax_partial, scale_finalize,
 * block_scale_zero, activation_pack) for the four NVFP4 projections of a block;
 * used here for the QKV / attention-output / FC1 activations and for weights. */
int nvfp4_quantize(const void* x_dev, int64_t ld_x, int64_t rows, int64_t k, void* qdata_dev,
                   void* scales_dev, float* global_scale_dev, void* workspace_dev, void* stream);

/*
 * Modulated plain quantization: NVFP4 of the adaLN-modulated activation
 *   y = RN_bf16(fma_fp32(x, RN_fp32(1 + scale[c]), shift[c]))
 * in one launch, for the QKV and FC1 inputs (the pages list a fused modulation at
 * those NVFP4 boundaries, next to the SwiGLU fusion of FC2). The modulation is
 * evaluated in fp32 (one correctly rounded fused multiply-add) and rounded once to
 * bf16, and y then goes through the nvfp4_quantize contract exactly.
 *
 * scale_dev, shift_dev : bf16 [k] (one sample's modulation vectors), 16-byte
 *                        aligned, finite. Read only.
 * Every other argument, layout and output as nvfp4_quantize; rows past the logical
 * rows are zero (padding), not the shift.
 */
int nvfp4_quantize_modulate(const void* x_dev, int64_t ld_x, int64_t rows, int64_t k, const void* scale_dev,
                            const void* shift_dev, void* qdata_dev, void* scales_dev, float* global_scale_dev,
                            void* workspace_dev, void* stream);

/*
 * Single-read producer: nvfp4_quantize_swiglu with the tensor amax supplied by the
 * caller, so every input byte is read once. The component-2 summary's conclusions
 * name the global scale as the dependency an exact fused producer must synchronize
 * on, and the boundary between two NVFP4 stages as the place where traffic is worth
 * removing; here the upstream stage that writes gate and up (e.g. the FC1 GEMM
 * epilogue) also produces max |y|.
 *
 * amax_dev : device float, read on the device: max |y| over the m logical rows
 *            (y as defined above), or any finite value above it; 4-byte aligned.
 *            g = amax / 2688 rounded up to FP32 is written to global_scale_dev;
 *            a NaN, zero or negative amax gives g = 0.
 * Every other argument, layout and output as nvfp4_quantize_swiglu; no workspace.
 * An amax below the true maximum is the caller's error; the result is still
 * defined: a block whose maximum exceeds v(126) * 6 * g gets scale byte 126 and
 * its codes saturate at +-6 (magnitude code 7). One ordinary launch, the two-pass
 * producer's pack-and-swizzle pass (with its run-time counters).
 */
int nvfp4_quantize_swiglu_amax(const void* gate_dev, int64_t ld_gate, const void* up_dev, int64_t ld_up,
                               int64_t m, int64_t k, const float* amax_dev, void* qdata_dev,
                               void* scales_dev, float* global_scale_dev, void* stream);

/* Single-read plain quantization (y = x) with the caller's amax: the contract of
 * nvfp4_quantize_swiglu_amax with one bf16 [rows, k] input of row stride ld_x. */
int nvfp4_quantize_amax(const void* x_dev, int64_t ld_x, int64_t rows, int64_t k, const float* amax_dev,
                        void* qdata_dev, void* scales_dev, float* global_scale_dev, void* stream);

/* ---- stage G: GEMM ---------------------------------------------------------------------- */

/*
 * D = RN_bf16(g_a * g_w * sum_b v(SA[m,b]) v(SW[n,b]) sum_{k in b} e2m1(A[m,k]) e2m1(W[n,k]))
 * for m < m_padded, n < n: the block-scaled NVFP4 GEMM with FP32 accumulation and
 * BF16 output ("FC2 NVFP4 Scheduling Results": split-K 1, zero workspace, no
 * global reduction, exactly one write of the padded BF16 output).
 *
 * a_qdata_dev, a_scales_dev : activation as written by the producer for
 *                             nvfp4_padded_rows(m) == m_padded rows.
 * a_global_dev, w_global_dev: device floats g_a, g_w (read on the device).
 * w_qdata_dev, w_scales_dev : weight [n, k] as written by nvfp4_quantize(rows = n).
 * d_dev                     : out, bf16 [m_padded, n] row-major, 16-byte aligned.
 * m_padded % 16 == 0, n % 16 == 0, k % 64 == 0. Rows of D whose activation rows
 * are zero padding come out +0. Takes no workspace from the caller.
 * Scheduling state: when the output has more 256 x 256 tiles than the device has
 * CUs, the workgroups take their tiles from run-time queues, so that faster XCDs
 * take more tiles. Here that means one persistent workgroup per CU; in the fused
 * entries below, one tile per workgroup. The library keeps 64 queue sets per
 * device (static device memory, 8 KiB) for all GEMM entries together. Launch i on
 * a device uses set i % 64, and the launch leaves its set cleared when it ends. So
 * up to 64 GEMM launches may be in flight at once on one device, from any streams.
 * A launch captured in a HIP graph keeps its set: replays of one captured launch
 * must not overlap each other.
 */
int nvfp4_gemm_bf16out(const void* a_qdata_dev, const void* a_scales_dev, const float* a_global_dev,
                       const void* w_qdata_dev, const void* w_scales_dev, const float* w_global_dev,
                       void* d_dev, int64_t m_padded, int64_t n, int64_t k, void* stream);

/*
 * The GEMM with its epilogue fusions. The FC2 kernel named on the pages carries a
 * bf16 bias in its epilogue, and the step profile of the pages keeps a
 * gate/residual add after the GEMM ("remaining_gate_add" among the production
 * components); both are folded into the store of D here:
 *
 *   D1[m, n] = RN_bf16(g_a * g_w * sum(...) + bias[n])   (bias_dev NULL: no bias)
 *   D[m, n]  = RN_bf16(residual[m, n] + gate[n] * D1[m, n]) with a residual
 *              (gate_dev NULL: gate 1), else D = D1.
 *
 * The chain is that of the unfused pipeline (a bf16 GEMM output, then a gated
 * residual add). Each step is an FP32 sum (the gate product exact) rounded to
 * bf16; the accumulation is FP32 as in nvfp4_gemm_bf16out.
 *
 * bias_dev     : bf16 [n] or NULL; 16-byte aligned; finite.
 * gate_dev     : bf16 [n] or NULL; needs residual_dev; 16-byte aligned.
 * residual_dev : bf16 [m_padded, n] row-major (row stride n) or NULL; 16-byte
 *                aligned; may be d_dev itself (in-place update of the residual
 *                stream): each element is read before the same thread writes it.
 * Every other argument as nvfp4_gemm_bf16out. Rows past the logical rows of the
 * activation come out RN_bf16(bias) (zero activation rows), combined with the
 * residual like any other row. No workspace; tile queues and errors as
 * nvfp4_gemm_bf16out, plus NVFP4_ERR_INVALID_ARG for a gate without a residual.
 */
int nvfp4_gemm_bf16out_fused(const void* a_qdata_dev, const void* a_scales_dev, const float* a_global_dev,
                             const void* w_qdata_dev, const void* w_scales_dev, const float* w_global_dev,
                             void* d_dev, int64_t m_padded, int64_t n, int64_t k, const void* bias_dev,
                             const void* gate_dev, const void* residual_dev, void* stream);

/*
 * The SwiGLU-pair GEMM: the FC1 projection that also produces the FC2 quantizer's
 * amax. The component-2 summary's conclusions put the global-scale dependency at
 * the FC2 producer and point at removing traffic where two NVFP4 stages meet; here
 * the stage that writes gate and up also reduces max |y| for
 * nvfp4_quantize_swiglu_amax, which then reads each input byte once.
 *
 * w_*              : the FC1 weight, 2 n_half rows, as written by nvfp4_quantize,
 *                    with gate and up rows interleaved in chunks of 8: rows
 *                    16c .. 16c+7 are gate channels 8c .. 8c+7 and rows
 *                    16c+8 .. 16c+15 the up channels 8c .. 8c+7.
 * gate_dev, up_dev : out, bf16 [m_padded, n_half] row-major each, 16-byte aligned:
 *                    D1 = RN_bf16(g_a g_w sum + bias) (as nvfp4_gemm_bf16out_fused)
 *                    split back into the gate and up channels.
 * bias_dev         : bf16 [2 n_half] in the interleaved order, or NULL.
 * amax_dev         : device float or NULL. The kernel folds
 *                    max |RN_bf16(silu_bf16(gate) * up)| over rows < amax_rows into
 *                    it with an atomic max, so the caller sets it (to 0, or to a
 *                    running maximum; a non-negative number) before the call;
 *                    4-byte aligned. Calls that fold into one amax may overlap.
 * amax_rows        : the logical rows, 0 <= amax_rows <= m_padded.
 * n_half           : a positive multiple of 8. Other arguments, the tile queues and
 *                    the errors as nvfp4_gemm_bf16out.
 */
int nvfp4_gemm_swiglu_pair(const void* a_qdata_dev, const void* a_scales_dev, const float* a_global_dev,
                           const void* w_qdata_dev, const void* w_scales_dev, const float* w_global_dev,
                           void* gate_dev, void* up_dev, int64_t m_padded, int64_t n_half, int64_t k,
                           const void* bias_dev, float* amax_dev, int64_t amax_rows, void* stream);

/* ---- self-test hook ---------------------------------------------------------------------- */

/* y[i] = silu_bf16(x[i]) for i < count, bf16 bit patterns, with the table the
 * producer uses (so the producer's activation can be checked on all 65,536
 * inputs). x_dev, y_dev: 2-byte aligned device arrays of count elements. */
int nvfp4_silu_bf16(const void* x_dev, void* y_dev, int64_t count, void* stream);

/* ---- measurement aid ---------------------------------------------------------------------- */

/* Not a step of the method: the dense fp16 matrix-core rate the device sustains and
 * its shader clock meanwhile, the ceiling beside which the GEMM's rate is read.
 * Launches `workgroups` workgroups of 4 waves; each wave issues iters x 4 independent
 * v_mfma_f32_32x32x16_f16 (32,768 FLOP each) and nothing else in its loop. For wave w
 * of workgroup b, out[(4 b + w) * 2] receives its shader-clock cycles and
 * out[(4 b + w) * 2 + 1] its 100 MHz real-time ticks over the loop (uint64 each).
 * workgroups in [1, 65536]; iters in [1, 2^24]; out_dev: 8-byte aligned device memory
 * of at least nvfp4_mfma_ceiling_out_bytes(workgroups) bytes, owned by the caller.
 * Time the call with events on `stream` for the rate. */
int64_t nvfp4_mfma_ceiling_out_bytes(int64_t workgroups);
int nvfp4_mfma_ceiling(int64_t workgroups, int64_t iters, void* out_dev, int64_t out_bytes, void* stream);

/* Not a step of the method: the HBM rate of a plain streaming kernel for a given mix of
 * reads and writes, the ceiling beside which the producer's two launches are read (the
 * absmax launch only reads; the quantize launch writes about 0.14 byte per byte read).
 * One workgroup per chunk of nvfp4_hbm_stream_chunk_bytes() bytes reads all read_bytes
 * of src (a one-shot grid dispatched in address order), and chunk c writes dst bytes
 * [c * w, (c + 1) * w) with w = 16 * floor(write_bytes / 16 / chunks), so
 * 16 * chunks * floor(write_bytes / (16 * chunks)) bytes are written in all.
 * src_dev: 16-byte aligned, read_bytes a positive multiple of the chunk size; dst_dev:
 * 16-byte aligned, at least max(write_bytes, 16) bytes (its first word may be
 * overwritten even when write_bytes is 0); write_bytes a multiple of 16, at most
 * read_bytes. Both owned by the caller. Time the call with events on `stream`. */
int64_t nvfp4_hbm_stream_chunk_bytes(void);
int nvfp4_hbm_stream_ceiling(const void* src_dev, int64_t read_bytes, void* dst_dev, int64_t write_bytes,
                             void* stream);

/* Not a step of the method: nvfp4_gemm_bf16out (same arguments, same kernel and
 * output) with shader-clock stamps, for the clock the GEMM runs at. Workgroup
 * b < slots writes its shader-clock cycles (s_memtime) from start to end to
 * clk_dev[2 b] and its 100 MHz real-time ticks (s_memrealtime) over the same span to
 * clk_dev[2 b + 1] (uint64 each); their ratio is the clock during its work.
 * clk_dev: 8-byte aligned device memory of 16 * slots bytes, owned by the caller;
 * slots in [1, 2^20] (the persistent grid has one workgroup per CU, plus the
 * quarter-tile tail). Errors as nvfp4_gemm_bf16out, plus NVFP4_ERR_INVALID_ARG /
 * NVFP4_ERR_MISALIGNED for the clock buffer. */
int nvfp4_gemm_bf16out_clock(const void* a_qdata_dev, const void* a_scales_dev, const float* a_global_dev,
                             const void* w_qdata_dev, const void* w_scales_dev, const float* w_global_dev,
                             void* d_dev, int64_t m_padded, int64_t n, int64_t k, void* clk_dev, int64_t slots,
                             void* stream);

/* ---- diagnostics -------------------------------------------------------------------------- */

/* Static text for a status code. The statuses are what a caller's guard tests
 * before falling back ("FC2 NVFP4 Scheduling Results", "Production Integration": a
 * load, check or execution failure falls back through the already produced NVFP4
 * bytes, which a failed call leaves untouched). Unknown codes give
 * "unknown status". */
const char* nvfp4_status_string(int status);

/* Detail of the last failing call on this host thread ("" after a successful
 * call): the failed check, or the HIP error of a refused launch (the failure
 * record the guards of "Production Integration" keep). The text lives in
 * thread-local storage until the thread's next call. */
const char* nvfp4_last_error(void);

/* Compile-time and run-time HIP versions, target architecture and the current
 * device's architecture once initialised, as one line of text ("FC2 NVFP4
 * Scheduling Results", "Production Integration": compile-time versions alone are
 * not runtime-ABI evidence, so both are recorded). The text lives in thread-local
 * storage until the thread's next call. */
const char* nvfp4_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
