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
// Epilogues (GemmEpilogue in common.hpp, one kernel instantiation each): the plain
// store; kind 1 adds a bf16 bias inside the fp32 multiply-add before the rounding
// and then a gated residual, res + gate[n] * D1; kind 2 is the SwiGLU pair of an
// FC1 whose gate and up rows are interleaved in chunks of 8 - it writes gate and up
// to separate tensors and folds max |silu(gate) * up| into the caller's amax.
//
// Tiling: a 256 x 256 output tile per workgroup of 4 waves (2 x 2), one wave per
// SIMD, each wave 128 x 128 (4 x 4 MFMA tiles of 32 x 32, accumulators in the 256
// AGPRs). A square wave tile needs the fewest dequantized fragments per MFMA: one
// K16 step converts 8 fragments for 16 MFMAs, i.e. two conversions and two packed
// multiplies per MFMA, which co-issue with the matrix pipe.
//
// Pipeline: K advances 128 per step. The packed operands (64 bytes per row) and
// two 512-byte scale tiles per 128 rows are moved global -> LDS by direct-to-LDS
// buffer loads (no VGPR staging) into a 3-stage ring, two K steps ahead; each
// wave's nine loads of a step are spread over its first K16 steps so that they
// issue between MFMAs. Rows of a stage are stored with an XOR swizzle of their
// four 16-byte chunks, so the fragment reads hit distinct LDS banks. Within a K
// step the lane's k-half h covers k in [64h, 64h + 64), eight consecutive k per
// MFMA, the same assignment for both operands. The K loop body is branch-free
// (the last two steps are peeled) so the scheduler can interleave the next K16
// step's conversions, the LDS reads and the loads with the MFMAs. Buffer range
// checks return zero past the end of A (rows >= m_padded) or W (rows >= n), and
// past K for the upper half of a final 64-wide K step.
//
// Traversal: tiles are numbered m-band-major in bands of 8 M-tiles, and workgroup
// ids (dispatched round-robin over the 8 XCDs) are remapped so that each XCD owns
// one contiguous range of tiles; its 32 concurrent workgroups then share A row
// bands and W panels in that XCD's L2. The plain kernel runs every tile with one
// persistent workgroup per CU. After its first tile, a workgroup takes the next
// tile of its XCD's range from a queue at run time, and once that range is used up
// it takes tiles from the back of the range of the XCD with the most left, then the
// quarters of the tail: the XCDs hold clocks a few per cent apart under this load,
// and a fixed split would leave the fast ones idle at the end. The first two K
// steps of the next tile are loaded while the current tile's epilogue runs, staged
// through an LDS area of its own. The fused kinds take their tiles from the same
// queues, one per workgroup, from a grid with a round of spare workgroups.
#include "common.hpp"

namespace nvfp4 {

// A workgroup of 4 waves (2 x 2, one per SIMD) computes a tile of
// (2 * FM * 32) x (2 * FN * 32); each wave owns FM x FN MFMA tiles of 32 x 32 with its
// accumulators in AGPRs. Full tiles are 256 x 256 (FM = FN = 4); when the last round
// of tiles would leave most CUs idle, its tiles are split into 128 x 128 quarters
// (FM = FN = 2), so that the tail is spread over four times as many CUs.
constexpr int WAVES_M = 2, WAVES_N = 2;
constexpr int kWaves = WAVES_M * WAVES_N;
constexpr int kGemmThreads = 64 * kWaves;
constexpr int kTK = 128;                         // K per step
constexpr int kStages = 3;                       // LDS stages (loads run two K steps ahead)
constexpr int kBandM = 8;                        // M-tiles per traversal band
constexpr int kTileBig = 256;                    // full tile edge
constexpr int kTileQuarter = 128;                // tail tile edge
constexpr int kCand = 1024;                      // SwiGLU-pair candidate list entries per wave (LDS)

template <int FM_, int FN_>
struct TileShape {
  static constexpr int TM = WAVES_M * FM_ * 32, TN = WAVES_N * FN_ * 32;
  static constexpr int CodesA = TM * 64, CodesW = TN * 64;         // 64 code bytes per row per K step
  static constexpr int ScaleA = TM / 128 * 1024, ScaleW = TN / 128 * 1024;  // two 512-B tiles per 128 rows
  static constexpr int StageBytes = CodesA + CodesW + ScaleA + ScaleW;
  // per wave and K step: code wave-loads of 1 KiB (16 rows) and scale loads
  static constexpr int LoadsA = CodesA / 1024 / kWaves, LoadsW = CodesW / 1024 / kWaves;
  static constexpr int ScalePerWave = (ScaleA + ScaleW) / kWaves;   // bytes
  static constexpr int ScaleLoadBytes = ScalePerWave >= 1024 ? 1024 : 256;  // dwordx4 or dword per lane
  static constexpr int LoadsS = ScalePerWave / ScaleLoadBytes;
  static constexpr int Loads = LoadsA + LoadsW + LoadsS;
  // VALU per MFMA of one K16 step: 8 per fragment (4 conversions, 4 multiplies) + a scale pair
  static constexpr int ValuPerMfma = ((FM_ + FN_) * 9 + FM_ * FN_ - 1) / (FM_ * FN_);
  static_assert(CodesA % (1024 * kWaves) == 0 && CodesW % (1024 * kWaves) == 0, "even code-load split");
  static_assert((ScaleA + ScaleW) % (ScaleLoadBytes * kWaves) == 0, "even scale-load split");
  static_assert(TM % 128 == 0 && TN % 128 == 0, "tiles cover whole 128-row scale tiles");
  static_assert(Loads <= 15, "vmcnt immediate");
};
using BigTile = TileShape<4, 4>;
using QuarterTile = TileShape<2, 2>;
static_assert(BigTile::TM == kTileBig && BigTile::TN == kTileBig, "full tile");
static_assert(QuarterTile::TM == kTileQuarter && QuarterTile::TN == kTileQuarter, "quarter tile");

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
  int tiles_m, tiles_n;                        // 256 x 256 tiles
  int big_tiles;                               // tiles [0, big_tiles) run whole; the rest as quarters
  int persist_wgs;                             // > 0: workgroups [0, persist_wgs) loop over the whole tiles
  int cgroups;                                 // scale column groups = C / 4
  int ksteps;
  int quarter_units;                           // 4 x (tiles past big_tiles): the quarter-tile tail
  uint64_t* sched;                             // the persistent grid's tile queues (TileQueues)
  GemmEpilogue ep;  // the epilogue's operands (kind 1 and 2 kernels)
};

// the value of the other lane of an even/odd lane pair (DPP quad permutation 1,0,3,2)
__device__ __forceinline__ uint32_t pair_swap(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

// two floats rounded to bf16 (ties to even), packed: lo in bits 0-15
__device__ __forceinline__ uint32_t cvt_pk_bf16_rn(float lo, float hi) {
  bf16x2_t c;
  c[0] = (__bf16)lo;
  c[1] = (__bf16)hi;
  uint32_t r;
  __builtin_memcpy(&r, &c, 4);
  return r;
}

typedef __attribute__((address_space(3))) void lds_void;

// Position of 16-byte chunk c of code row r inside that row's 64 LDS bytes. The
// XOR spreads the rows a fragment read touches (32 consecutive rows, one chunk
// each) over distinct banks for both 32- and 64-bank LDS.
__device__ __forceinline__ int chunk_pos(int r, int c) { return c ^ (((r >> 1) ^ (r >> 2)) & 3); }

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

// Dequantize the FM + FN fragments of one K16 step into (fa, fw). The half-rate
// conversions are issued in place, each multiply trails its conversion by four
// pairs, so no instruction waits on the one just before it.
template <int FM_, int FN_>
__device__ __forceinline__ void dequant_step(f16x8_t (&fa)[FM_], f16x8_t (&fw)[FN_], const uint32_t (&codes)[FM_ + FN_],
                                             const f16x2_t (&sv)[FM_ + FN_]) {
  constexpr int NP = (FM_ + FN_) * 4;  // pairs
  constexpr int LAG = 4;
#pragma unroll
  for (int q = 0; q < NP + LAG; ++q) {
    if (q < NP) {
      const int f = q / 4, e = q % 4;
      f16x2_t v;
      switch (e) {
        case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[f], 256.0f, 0); break;
        case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[f], 256.0f, 1); break;
        case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[f], 256.0f, 2); break;
        default: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[f], 256.0f, 3); break;
      }
      if (f < FM_) { fa[f][2 * e] = v[0]; fa[f][2 * e + 1] = v[1]; }
      else { fw[f - FM_][2 * e] = v[0]; fw[f - FM_][2 * e + 1] = v[1]; }
    }
    if (q >= LAG) {
      const int p = q - LAG, f = p / 4, e = p % 4;
      f16x2_t v;
      if (f < FM_) { v[0] = fa[f][2 * e]; v[1] = fa[f][2 * e + 1]; }
      else { v[0] = fw[f - FM_][2 * e]; v[1] = fw[f - FM_][2 * e + 1]; }
      v = v * sv[f];
      if (f < FM_) { fa[f][2 * e] = v[0]; fa[f][2 * e + 1] = v[1]; }
      else { fw[f - FM_][2 * e] = v[0]; fw[f - FM_][2 * e + 1] = v[1]; }
    }
  }
}

// fp16 pair (v(S) * 2^-8, v(S) * 2^-8) for scale byte b of a scale dword
__device__ __forceinline__ f16x2_t scale_pair(uint32_t sdw, int b) {
  // (S << 7) | (S << 23) == S * 0x800080 for S < 256: one byte-select multiply
  uint32_t u = ((sdw >> (8 * b)) & 0xFFu) * 0x800080u;
  f16x2_t r;
  __builtin_memcpy(&r, &u, 4);
  return r;
}

// Scheduling hints: in each K16 step, interleave each MFMA with its share of the
// VALU work (the next step's dequantization and scale pairs): five per MFMA for the
// full tile, nine for the quarter tile.
template <int NMFMA, int NVALU>
__device__ __forceinline__ void interleave_hint() {
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // 1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);  // its share of VALU
  }
}

// the same, with NDS LDS reads and NVM global loads placed two per MFMA from the start
template <int NMFMA, int NVALU, int NDS, int NVM>
__device__ __forceinline__ void interleave_hint_mem() {
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // 1 MFMA
    if (2 * i < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads, two at a time
    if (i < NVM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global loads
    __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);  // its share of VALU
  }
}

// Workgroup barrier for the LDS pipeline. Every wave has already waited for its
// own outstanding LDS reads and direct-to-LDS loads (explicit counters), so only
// the s_barrier is needed; the empty asm keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One output tile: the whole K loop and the epilogue for rows [m0, m0 + TM) and
// columns [n0, n0 + TN), by the workgroup's 4 waves.
// EPI is the GemmEpilogue kind: 0, D = RN_bf16(alpha * acc); 1, D1 = RN_bf16(alpha *
// acc + bias[n]) and, with a residual, D = RN_bf16(res + gate[n] * D1); 2, the SwiGLU
// pair (D1 split into gate and up outputs, and the amax of silu(gate) * up).
// The origin of whole tile t: tiles are numbered m-band-major (bands of kBandM M-tiles,
// M first within a band).
__device__ __forceinline__ void tile_origin(const GemmArgs& a, int t, int64_t& m0, int64_t& n0) {
  const int band = t / (kBandM * a.tiles_n);
  const int in_band = t - band * kBandM * a.tiles_n;
  const int band_m = (a.tiles_m - band * kBandM) < kBandM ? (a.tiles_m - band * kBandM) : kBandM;
  m0 = (int64_t)(band * kBandM + in_band % band_m) * kTileBig;
  n0 = (int64_t)(in_band / band_m) * kTileBig;
}

// ---- tile queues of the persistent grid ----
// The eight XCDs of the chip hold different clocks under this load (a few per cent
// apart), so a fixed split of the tiles leaves the fastest XCDs idle at the end. The
// whole tiles are split into one contiguous range per XCD as before (its 32
// workgroups then share A row bands and W panels in that XCD's L2), but beyond each
// workgroup's first tile they are taken at run time:
//   sched[x], x < 8: XCD x's queue. The low 32 bits count tiles taken from the front
//     of its range past the `slots` first tiles (which go one to each of its
//     workgroups), the high 32 bits tiles taken from the back by other XCDs' workgroups
//     once their own queue is empty. Both kinds of take add 1 to the same word, and a
//     take succeeds iff front + back before it is below the range's dynamic length, so
//     every tile is taken exactly once and the front and back never hand out the same
//     tile.
//   sched[8]: the next 128 x 128 quarter of the tail tiles, taken after every queue is
//     empty.
//   sched[9]: workgroups that have finished taking. The last one clears sched[0..9],
//     so the words are zero for the next launch that uses them. Relaxed order is
//     enough: a workgroup counts itself only after its last take has returned its
//     value, and the last one issues its clears only after its count has returned
//     gridDim.x - 1, so every take on a word is performed before the clear of it.
// All of them are agent-scope atomics (the XCDs' L2 caches are not coherent with each
// other); a take is one atomic with return, issued a K step before its result is used.
static_assert(kGemmQueueWords >= 10, "a queue set holds the 8 XCD queues, the quarter count and the exit count");

__device__ __forceinline__ void xcd_range(const GemmArgs& a, int x, int& start, int& len) {
  const int per = a.big_tiles / 8, rem = a.big_tiles % 8;
  start = x * per + (x < rem ? x : rem);
  len = per + (x < rem ? 1 : 0);
}

// the tile of a front take whose atomic returned `old`, or -1 when the queue was empty
__device__ __forceinline__ int front_tile(const GemmArgs& a, int x, int slots, uint64_t old) {
  int start, len;
  xcd_range(a, x, start, len);
  const int64_t dyn = len > slots ? len - slots : 0;
  const uint32_t f = (uint32_t)old, b = (uint32_t)(old >> 32);
  return (int64_t)f + b < dyn ? start + slots + (int)f : -1;
}

// Wave 0 of a persistent workgroup, all lanes: a tile from the back of the queue with
// the most tiles left, or -1 when every queue is empty. Lanes 0..7 read the eight
// queue words at once; lane 0 takes. A failed take means that queue emptied between
// the read and the take, and the counts only grow, so it reads as empty from then on:
// after at most 8 failures every queue is empty, and the loop bound is never reached.
__device__ __forceinline__ int steal_tile(const GemmArgs& a, int slots, int lane) {
  for (int round = 0; round < 9; ++round) {
    int left = 0;
    if (lane < 8) {
      const uint64_t v = __hip_atomic_load(a.sched + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int start, len;
      xcd_range(a, lane, start, len);
      const int64_t l = (int64_t)(len > slots ? len - slots : 0) - (int64_t)(uint32_t)v - (int64_t)(uint32_t)(v >> 32);
      left = l <= 0 ? 0 : (l < (1 << 24) ? (int)l : (1 << 24) - 1);
    }
    int key = left * 8 + (lane & 7);  // the most tiles left, then the highest XCD
#pragma unroll
    for (int off = 4; off >= 1; off >>= 1) {
      const int o = __shfl_xor(key, off, 64);
      key = key > o ? key : o;
    }
    key = __builtin_amdgcn_readfirstlane(key);
    if (key < 8) return -1;
    const int y = key & 7;
    int t = -1;
    if (lane == 0) {
      const uint64_t old = __hip_atomic_fetch_add(a.sched + y, (uint64_t)1 << 32, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      int start, len;
      xcd_range(a, y, start, len);
      const int64_t dyn = len > slots ? len - slots : 0;
      const uint32_t f = (uint32_t)old, b = (uint32_t)(old >> 32);
      if ((int64_t)f + b < dyn) t = start + len - 1 - (int)b;
    }
    t = __builtin_amdgcn_readfirstlane(t);
    if (t >= 0) return t;
  }
  return -1;
}

// LDS of the persistent workgroups: the stages, then per kind the plain kernel's
// epilogue staging or the SwiGLU pair's candidate lists, then one word that
// broadcasts a taken tile to the workgroup's waves
constexpr size_t kPersistStagingBytes = (size_t)kWaves * 32 * (BigTile::TN / WAVES_N * 2 + 16);
constexpr size_t kCandBytes = (size_t)kWaves * kCand * 4;
template <int EPI>
constexpr size_t sched_slot_offset() {
  return (size_t)kStages * BigTile::StageBytes + (EPI == 0 ? kPersistStagingBytes : EPI == 2 ? kCandBytes : 0);
}
constexpr size_t kSchedSlotOffset = sched_slot_offset<0>();

// PERSIST (plain epilogue, whole tiles): after tile (m0, n0) the workgroup goes on with
// the tiles it takes from the queues (front of XCD `xcd`'s queue, else the back of
// another's), until none is left. The take for the next tile is issued in the first K
// step of the current one. The first two K steps of the next tile are loaded while the
// current tile's epilogue runs; that epilogue stages through its own LDS area, past
// the pipeline stages.
template <int FM, int FN, int EPI, bool PERSIST = false>
__device__ __forceinline__ void run_tile(const GemmArgs& a, int64_t m0, int64_t n0, unsigned char* smem,
                                         int xcd = 0, int slots = 0) {
  using T = TileShape<FM, FN>;
  constexpr int kStageBytes = T::StageBytes, kCodesA = T::CodesA, kCodesW = T::CodesW, kScaleA = T::ScaleA;
  constexpr int kLoads = T::Loads;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lr = lane & 31, h = lane >> 5;

  __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)a.aq, 0, a.a_qbytes, 0x00020000);
  __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc((void*)a.wq, 0, a.w_qbytes, 0x00020000);
  __amdgpu_buffer_rsrc_t rSA = __builtin_amdgcn_make_buffer_rsrc((void*)a.as, 0, a.a_sbytes, 0x00020000);
  __amdgpu_buffer_rsrc_t rSW = __builtin_amdgcn_make_buffer_rsrc((void*)a.ws, 0, a.w_sbytes, 0x00020000);
  const int krow = (int)(a.k / 2);

  // ---- direct-to-LDS loads of one K step into a stage ----
  // Code wave-load j covers rows 16j .. 16j+15; lane L writes LDS bytes 16L..16L+15 of
  // that 1 KiB, i.e. row 16j + L/4 at chunk position L%4, which holds global chunk
  // chunk_pos(row, L%4) (the XOR is an involution). The scale part of a stage is one
  // 1 KiB block per 128 rows (A blocks, then W blocks), each the two 512-byte
  // column-group tiles of that row tile for the K step, contiguous in global memory;
  // each wave loads an equal share of it in pieces of ScaleLoadBytes.
  // Load idx (0..kLoads-1) of this wave's share of K step ks: code loads of A, then
  // of W, then scale pieces. Half K steps (K % 128 == 64) send the upper k-half past
  // the buffer range, where reads return zero.
  auto issue_one = [&](int ks, int stage, int idx) {
    const int oor = ((int64_t)(ks + 1) * kTK > a.k) ? 0x7FFFFFF0 : 0;  // wave-uniform
    unsigned char* st = smem + stage * kStageBytes;
    if (idx < T::LoadsA + T::LoadsW) {
      const int rsub = lane >> 2, p = lane & 3;
      const bool isA = idx < T::LoadsA;
      const int j = wave + (isA ? idx : idx - T::LoadsA) * kWaves;
      const int row = j * 16 + rsub;
      const int c = chunk_pos(row, p);
      const int off = ((int)(((isA ? m0 : n0) + row) * krow) + ks * 64 + c * 16) | (c >= 2 ? oor : 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isA ? rA : rW, (lds_void*)(st + (isA ? 0 : kCodesA) + j * 1024), 16, off,
                                               0, 0, 0);
    } else {
      // scale piece q of the stage's scale bytes
      constexpr int B = T::ScaleLoadBytes;
      const int q = wave * T::LoadsS + (idx - T::LoadsA - T::LoadsW);
      const int byte0 = q * B;                      // offset inside the scale part of the stage
      const bool isA = byte0 < kScaleA;
      const int rel = isA ? byte0 : byte0 - kScaleA;
      const int rt = rel >> 10, part = rel & 1023;  // row tile, offset inside its 1 KiB block
      const int64_t rt_g = (isA ? m0 : n0) / 128 + rt;
      const int lo = part + lane * (B / 64);        // this lane's bytes inside the block
      const int off = ((int)((rt_g * a.cgroups + (int64_t)ks * 2) * 512) + lo) | (lo >= 512 ? oor : 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isA ? rSA : rSW, (lds_void*)(st + kCodesA + kCodesW + byte0),
                                               TileShape<FM, FN>::ScaleLoadBytes / 64, off, 0, 0, 0);
    }
  };

  // ---- per-wave views of a stage ----
  const int rowA = wm * FM * 32 + lr, rowW = wn * FN * 32 + lr;
  auto read_codes = [&](int stage, int kq, u32x4_t (&ca)[FM], u32x4_t (&cw)[FN]) {
    const unsigned char* st = smem + stage * kStageBytes;
    const int c = h * 2 + kq;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = rowA + i * 32;
      ca[i] = *(const u32x4_t*)(st + r * 64 + chunk_pos(r, c) * 16);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = rowW + j * 32;
      cw[j] = *(const u32x4_t*)(st + kCodesA + r * 64 + chunk_pos(r, c) * 16);
    }
  };
  // scale dwords (the four blocks of this lane's k-half), one per fragment
  auto read_scales = [&](int stage, uint32_t (&sa)[FM], uint32_t (&sw)[FN]) {
    const unsigned char* ss = smem + stage * kStageBytes + kCodesA + kCodesW;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * FM * 32 + i * 32;
      sa[i] = *(const uint32_t*)(ss + ((r >> 7) * 2 + h) * 512 + lr * 16 + ((r >> 5) & 3) * 4);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = wn * FN * 32 + j * 32;
      sw[j] = *(const uint32_t*)(ss + kScaleA + ((r >> 7) * 2 + h) * 512 + lr * 16 + ((r >> 5) & 3) * 4);
    }
  };

  f32x16_t acc[FN][FM];

  // Software pipeline. K step ks lives in LDS stage ks % 3, loaded two K steps
  // ahead; the loads of step ks + 2 are spread over the first K16 steps of step ks
  // (two per K16 step) so that they issue between MFMAs. Within a K step, K16 step
  // kk (0..7) uses codes of half kk / 4, dword kk % 4, and scale block kk / 2. While
  // the MFMAs of step kk run, the fragments of step kk + 1 are dequantized into the
  // other register set. The second-half codes are read at kk = 1. At kk = 6 every
  // wave waits for its own loads of the next K step, the workgroup synchronises
  // (which also frees the stage read in the previous K step for the next loads),
  // and the next step's scales and first-half codes are read; they are dequantized
  // at kk = 7. The body is instantiated without branches: the last two K steps are
  // peeled.
  const int nks = a.ksteps;
  // g_a * g_w, read before any load of the pipeline so that waiting for it never
  // waits for those (the persistent epilogue overlaps the next tile's first loads)
  float alpha_p = 0.0f;
  if constexpr (PERSIST) alpha_p = (*a.ga) * (*a.gw);
  // the loads of the first two K steps of the current tile
  auto prologue = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int idx = 0; idx < kLoads; ++idx) issue_one(0, 0, idx);
    if (nks > 1) {
#pragma unroll
      for (int idx = 0; idx < kLoads; ++idx) issue_one(1, 1, idx);
    }
  };
  prologue();
  if (nks > 1) __builtin_amdgcn_s_waitcnt(0x0F70 | kLoads);  // vmcnt(kLoads): step 0 has landed
  else __builtin_amdgcn_s_waitcnt(0x0F70);                   // vmcnt(0)

  for (;;) {  // one pass without PERSIST
  stage_barrier();
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

  u32x4_t ca[2][FM], cw[2][FN];
  uint32_t sa[FM], sw[FN], nsa[FM], nsw[FN];
  f16x8_t fa[2][FM], fw[2][FN];
  // dequantize K16 step k (0..7) of the codes and scales in registers into set `set`
  auto dequant_k = [&](int k, int set) __attribute__((always_inline)) {
    uint32_t cd[FM + FN];
    f16x2_t sv[FM + FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) { cd[i] = ca[k >> 2][i][k & 3]; sv[i] = scale_pair(sa[i], k >> 1); }
#pragma unroll
    for (int j = 0; j < FN; ++j) { cd[FM + j] = cw[k >> 2][j][k & 3]; sv[FM + j] = scale_pair(sw[j], k >> 1); }
    dequant_step(fa[set], fw[set], cd, sv);
  };
  read_scales(0, sa, sw);
  read_codes(0, 0, ca[0], cw[0]);
  dequant_k(0, 0);

  // one K step; `loads`: issue the loads of step ks + 2; `next`: a step ks + 1 follows;
  // `take`: thread 0 takes the workgroup's next tile (the result is waited for with the
  // next K step's loads, a K step later)
  uint64_t qold = 0;
  auto kstep = [&](int ks, int stage, bool loads, bool next, bool take) __attribute__((always_inline)) {
    const int next_stage = stage == 2 ? 0 : stage + 1;
    const int far_stage = next_stage == 2 ? 0 : next_stage + 1;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int cur = kk & 1, nxt = cur ^ 1;
      if (loads) {
        if (2 * kk < kLoads) issue_one(ks + 2, far_stage, 2 * kk);
        if (2 * kk + 1 < kLoads) issue_one(ks + 2, far_stage, 2 * kk + 1);
      }
      if (kk == 1) read_codes(stage, 1, ca[1], cw[1]);  // second half, needed from step 4
      if (kk == 6 && next) {
        // the barrier stays in place; the reads after it (held below it by its memory
        // clobbers) are spread over this K16 step's first MFMAs and still lead their
        // use at kk = 7 by a whole MFMA group
        __builtin_amdgcn_sched_barrier(0);
        if (loads) __builtin_amdgcn_s_waitcnt(0x0F70 | kLoads);  // this step's batch may fly
        else __builtin_amdgcn_s_waitcnt(0x0F70);
        stage_barrier();
        read_scales(next_stage, nsa, nsw);
        read_codes(next_stage, 0, ca[0], cw[0]);
        if (take && tid == 0)
          qold = __hip_atomic_fetch_add(a.sched + xcd, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (kk < 7) {
        dequant_k(kk + 1, nxt);
      } else if (next) {
#pragma unroll
        for (int i = 0; i < FM; ++i) sa[i] = nsa[i];
#pragma unroll
        for (int j = 0; j < FN; ++j) sw[j] = nsw[j];
        dequant_k(0, nxt);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fw[cur][j], fa[cur][i], acc[j][i], 0, 0, 0);
      if (kk == 6 && next) {
        // the next step's LDS reads (after the barrier) spread over the first MFMAs
        interleave_hint_mem<FM * FN, T::ValuPerMfma, (FM + FN) + 2, 0>();
      } else {
        interleave_hint<FM * FN, T::ValuPerMfma>();
      }
    }
  };

  int stage = 0, ks = 0;
  bool took = false;
  if constexpr (PERSIST) {
    if (nks > 2) {
      kstep(0, 0, true, true, true);
      stage = 1;
      ks = 1;
      took = true;
    }
  }
  for (; ks + 2 < nks; ++ks) {
    kstep(ks, stage, true, true, false);
    stage = stage == 2 ? 0 : stage + 1;
  }
  if (ks + 1 < nks) {
    kstep(ks, stage, false, true, false);
    stage = stage == 2 ? 0 : stage + 1;
    ++ks;
  }
  kstep(ks, stage, false, false, false);

  // the epilogue's tile; PERSIST moves (m0, n0) on to the next tile and starts its loads
  const int64_t em0 = m0, en0 = n0;
  bool more = false;
  if constexpr (PERSIST) {
    // wave 0 resolves the next tile: its own queue's front (taken in the first K step,
    // or now for tiles of at most two K steps), else the back of another queue
    volatile int* slot = (volatile int*)(smem + kSchedSlotOffset);
    if (wave == 0) {
      if (!took && tid == 0)
        qold = __hip_atomic_fetch_add(a.sched + xcd, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int nt = -1;
      if (tid == 0) nt = front_tile(a, xcd, slots, qold);
      nt = __builtin_amdgcn_readfirstlane(nt);
      if (nt < 0) nt = steal_tile(a, slots, lane);
      if (tid == 0) *slot = nt;
    }
    stage_barrier();  // every wave has finished reading the last K step's stage; the slot is written
    const int nt = __builtin_amdgcn_readfirstlane(*slot);
    more = nt >= 0;
    if (more) {
      tile_origin(a, nt, m0, n0);
      prologue();
    }
  }
  if constexpr (EPI == 0 && PERSIST) {
    // ---- epilogue: D[m, n] = RN_bf16(alpha * acc), staged 32 rows at a time in the
    // wave's area past the stages (the next tile's loads are landing in the stages) ----
    const float alpha = alpha_p;
    constexpr int kWaveCols = FN * 32, kRowBytes = kWaveCols * 2 + 16;  // padded against bank conflicts
    constexpr int kChunksPerRow = kWaveCols / 8, kRowsPerStore = 64 / kChunksPerRow;
    unsigned char* stg = smem + kStages * BigTile::StageBytes + wave * (32 * kRowBytes);
    const int64_t wrow0 = em0 + wm * FM * 32, wcol0 = en0 + wn * FN * 32;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
          const u32x2_t v = {cvt_pk_bf16_rn(acc[j][i][q * 4 + 0] * alpha, acc[j][i][q * 4 + 1] * alpha),
                             cvt_pk_bf16_rn(acc[j][i][q * 4 + 2] * alpha, acc[j][i][q * 4 + 3] * alpha)};
          *(u32x2_t*)(stg + lr * kRowBytes + (j * 32 + q * 8 + h * 4) * 2) = v;
        }
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
      asm volatile("" ::: "memory");
      // LDS -> global: lane L takes 8 columns of one row
#pragma unroll
      for (int it = 0; it < 32 / kRowsPerStore; ++it) {
        const int r = it * kRowsPerStore + lane / kChunksPerRow, ch = lane % kChunksPerRow;
        const u32x4_t v = *(const u32x4_t*)(stg + r * kRowBytes + ch * 16);
        const int64_t m = wrow0 + i * 32 + r, n = wcol0 + ch * 8;
        if (m < a.m_pad && n < a.n) *(u32x4_t*)(a.d + m * a.n + n) = v;
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);  // the reads are done before the next fragment overwrites
      asm volatile("" ::: "memory");
    }
  } else if constexpr (EPI == 0) {
    // ---- epilogue: D[m, n] = RN_bf16(alpha * acc), alpha = g_a * g_w ----
    // Each wave stages its tile in its own quarter of the (now idle) LDS, 64 rows at a
    // time, then stores whole row segments: a store instruction writes 4 rows x 256 B
    // (full tile) or 8 rows x 128 B (quarter tile) instead of 16-byte pieces of 32 rows.
    const float alpha = (*a.ga) * (*a.gw);
    constexpr int kWaveCols = FN * 32, kRowBytes = kWaveCols * 2 + 16;  // padded against bank conflicts
    constexpr int kChunksPerRow = kWaveCols / 8, kRowsPerStore = 64 / kChunksPerRow;
    static_assert(64 * kRowBytes <= kStages * BigTile::StageBytes / kWaves, "staging fits the wave's LDS share");
    unsigned char* stg = smem + wave * (kStages * BigTile::StageBytes / kWaves);
    const int64_t wrow0 = em0 + wm * FM * 32, wcol0 = en0 + wn * FN * 32;
    stage_barrier();  // every wave has finished reading the last K step's stage
  #pragma unroll
    for (int half = 0; half < FM / 2; ++half) {
      // registers -> LDS: fragments i = 2 half, 2 half + 1 hold rows 64 half .. 64 half + 63
  #pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * half + ii;
  #pragma unroll
        for (int j = 0; j < FN; ++j) {
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            bf16x2_t lo, hi;
            lo[0] = (__bf16)(acc[j][i][q * 4 + 0] * alpha);
            lo[1] = (__bf16)(acc[j][i][q * 4 + 1] * alpha);
            hi[0] = (__bf16)(acc[j][i][q * 4 + 2] * alpha);
            hi[1] = (__bf16)(acc[j][i][q * 4 + 3] * alpha);
            uint32_t ul, uh;
            __builtin_memcpy(&ul, &lo, 4);
            __builtin_memcpy(&uh, &hi, 4);
            typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
            const u32x2_t v = {ul, uh};
            const int r = ii * 32 + lr, c = j * 32 + q * 8 + h * 4;
            *(u32x2_t*)(stg + r * kRowBytes + c * 2) = v;
          }
        }
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
      asm volatile("" ::: "memory");
      // LDS -> global: lane L takes 8 columns of one row
  #pragma unroll
      for (int it = 0; it < 64 / kRowsPerStore; ++it) {
        const int r = it * kRowsPerStore + lane / kChunksPerRow, ch = lane % kChunksPerRow;
        const u32x4_t v = *(const u32x4_t*)(stg + r * kRowBytes + ch * 16);
        const int64_t m = wrow0 + half * 64 + r, n = wcol0 + ch * 8;
        if (m < a.m_pad && n < a.n) *(u32x4_t*)(a.d + m * a.n + n) = v;
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);  // the reads are done before the next half overwrites
      asm volatile("" ::: "memory");
    }
  } else {
    // ---- fused epilogues (kind 1: bias + gated residual; kind 2: SwiGLU pair) ----
    // The staging is the plain one (bf16 through LDS, 64 rows at a time); the bias
    // enters the fp32 multiply-add that forms alpha * acc + bias before the one bf16
    // rounding, and the rest happens on the bf16 row segments of the store phase.
    typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
    const float alpha = (*a.ga) * (*a.gw);
    constexpr int kWaveCols = FN * 32, kRowBytes = kWaveCols * 2 + 16;  // padded against bank conflicts
    constexpr int kChunksPerRow = kWaveCols / 8, kRowsPerStore = 64 / kChunksPerRow;
    constexpr int kIts = 64 / kRowsPerStore;            // store iterations per 64-row half
    static_assert(64 * kRowBytes <= kStages * BigTile::StageBytes / kWaves, "staging fits the wave's LDS share");
    unsigned char* stg = smem + wave * (kStages * BigTile::StageBytes / kWaves);
    const int64_t wrow0 = em0 + wm * FM * 32, wcol0 = en0 + wn * FN * 32;
    const int ch = lane % kChunksPerRow, rl = lane / kChunksPerRow;
    const int64_t col = wcol0 + ch * 8;  // the 8 output columns of this lane in the store phase
    const bool col_ok = col < a.n;
    stage_barrier();  // every wave has finished reading the last K step's stage
    // bias of the lane's accumulator columns j*32 + q*8 + h*4 .. +3 (loaded after the
    // barrier so that nothing lives through the K loop); zero without a bias. Kept as
    // bf16 pairs and widened where used.
    u32x2_t bq[FN][4];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t c = wcol0 + j * 32 + q * 8 + h * 4;
        u32x2_t bv = {0u, 0u};
        if (a.ep.bias && c < a.n) bv = *(const u32x2_t*)(a.ep.bias + c);
        bq[j][q] = bv;
      }
    }
    // kind 1: the gate of the lane's 8 store-phase columns (1.0 without a gate)
    // (bf16 pairs, widened where used)
    u32x4_t gate8 = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    if (EPI == 1 && a.ep.gate && col_ok) gate8 = *(const u32x4_t*)(a.ep.gate + col);
    // kind 2: the SwiGLU pair. Even chunks of 8 columns are gate channels j0 .. j0+7,
    // odd chunks the same up channels (j0 = col / 16 * 8).
    const bool is_up = (ch & 1) != 0;
    const int64_t n_half = a.n >> 1, j0 = (col >> 4) << 3;
    // The amax only needs the largest |y|. The value already in *amax (the caller's
    // start, raised by tiles done so far) is a lower bound of the final one, and
    // |y| <= max(gate, 0.28125) |up| (1 + 2^-8) bounds an element, gate signed
    // (silu_bf16(x) <= x for x > 0, and |silu_bf16(x)| <= 0.2793 for x <= 0; one bf16
    // rounding of the product): elements whose bound is below the running maximum
    // cannot raise it and skip the silu lookup. With |gate| in place of the signed
    // gate the bound is loose without limit for negative gates, which then all become
    // candidates. ymax is the running maximum as an fp32 value of a bf16.
    float ymax = 0.0f;
    // Candidates are queued per wave in LDS (past the pipeline stages) as
    // gate | up << 16 and resolved together - their silu lookups in one batch - when
    // the list could fill and at the end of each scan. The count is wave-uniform.
    uint32_t* clist = (uint32_t*)(smem + kStages * BigTile::StageBytes) + wave * kCand;
    int ccount = 0;
    auto flush = [&]() __attribute__((always_inline)) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's list writes are done
      asm volatile("" ::: "memory");
      // rounds of 4 entries per lane, their silu lookups in flight together
#pragma nounroll
      for (int base = 0; base < ccount; base += 256) {
        uint32_t ent[4], sil[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ent[r] = (base + r * 64 + lane < ccount) ? clist[base + r * 64 + lane] : 0u;
#pragma unroll
        for (int r = 0; r < 4; ++r) sil[r] = (base + r * 64 + lane < ccount) ? a.ep.silu_table[ent[r] & 0xFFFFu] : 0u;
        // exact y = RN_bf16(silu(gate) * up): the product of two bf16 values is exact
        // in fp32 above 2^-126 (below, the fp64 product is)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (base + r * 64 + lane < ccount) {
            const float sv = bf16_bits_to_float(sil[r]), uv = bf16_bits_to_float(ent[r] >> 16);
            const float pr = fabsf(sv * uv);
            uint32_t y = cvt_pk_bf16_rn(pr, 0.0f) & 0x7FFFu;
            if (pr != 0.0f && pr < 0x1p-126f) y = rn_bf16_from_double(fabs((double)sv * (double)uv)) & 0x7FFFu;
            ymax = fmaxf(ymax, __uint_as_float(y << 16));
          }
        }
      }
      ccount = 0;
      // every lane continues from the wave's maximum (non-negative fp32 bits order as integers)
      uint32_t yb = __float_as_uint(ymax);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)yb, off, 64);
        yb = yb > o ? yb : o;
      }
      ymax = __uint_as_float(yb);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);  // the list reads are done before it is refilled
      asm volatile("" ::: "memory");
    };
    if (EPI == 2 && a.ep.amax)
      ymax = __uint_as_float(__hip_atomic_load((const uint32_t*)a.ep.amax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    // Kind 2 first screens each 64-row half in registers, on the fp32 values before
    // their bf16 rounding: for a gate g and up u of one channel, with G = max(g,
    // 0.28125), s = G |u| + G 2^-130 (one multiply, one fused multiply-add) satisfies
    // |silu_bf16(RN(g)) RN(u)| <= (1 + 2^-6) s for ymax >= 2^-100: (1 + 2^-8) per bf16
    // rounding, the fp32 roundings, and the subnormal-u term covered by G 2^-130. A half
    // whose largest s (rows below amax_rows) is at most T = ymax (1 - 2^-6) holds no
    // product above ymax, so it skips the exact scan. T is capped at 2^125 so that a
    // product that overflows bf16 is always scanned, and is 0 while ymax < 2^-100.
    auto threshold = [&]() -> float { return ymax < 0x1p-100f ? 0.0f : fminf(ymax * 0.984375f, 0x1p125f); };
    // the exact scan of the staged half: elements of rows < amax_rows whose bound on
    // the bf16 values reaches the running maximum go to the candidate list
    auto scan_half = [&](int half) __attribute__((always_inline)) {
      // seed: each lane's largest-bound element of the half is resolved first, so that
      // a half scanned while ymax is still low (the first tiles) queues few candidates
      float bbest = -1.0f;
      uint32_t best = 0;
#pragma nounroll
      for (int t = 0; t < kIts; ++t) {
        const int r = t * kRowsPerStore + rl;
        const int64_t m = wrow0 + half * 64 + r;
        const u32x4_t v = *(const u32x4_t*)(stg + r * kRowBytes + ch * 16);
        const uint32_t r0 = pair_swap(is_up ? v[0] : v[2]), r1 = pair_swap(is_up ? v[1] : v[3]);
        const uint32_t gpk[2] = {is_up ? r0 : v[0], is_up ? r1 : v[1]};
        const uint32_t upk[2] = {is_up ? v[2] : r0, is_up ? v[3] : r1};
        const bool ok = m < a.ep.amax_rows && col_ok;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t g16 = (gpk[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          const uint32_t u16 = (upk[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          const float bnd = fmaxf(bf16_bits_to_float(g16), 0.28125f) * fabsf(bf16_bits_to_float(u16));
          if (ok && bnd > bbest) {
            bbest = bnd;
            best = g16 | (u16 << 16);
          }
        }
      }
      // (the list is empty here: every scan ends with it flushed)
      {
        const bool has = bbest >= 0.0f;
        const uint64_t mask = __ballot(has);
        if (has) {
          const int off = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
          clist[ccount + off] = best;
        }
        ccount += __builtin_amdgcn_readfirstlane(__popcll(mask));
      }
      // Then every element whose bound reaches ymax. One flush site: the seeds first,
      // then whenever a row's 4 x 64 candidates might not fit, and once at the end. The
      // pair trades halves: the gate lane keeps (gate, up) of channels j0 .. j0+3, the
      // up lane those of j0+4 .. j0+7.
      bool pending = true;
      int t = 0;
#pragma nounroll
      for (;;) {
        if (pending || ccount + 256 > kCand) {
          flush();
          pending = false;
        }
        if (t == kIts) break;
        const int r = t * kRowsPerStore + rl;
        const int64_t m = wrow0 + half * 64 + r;
        const u32x4_t v = *(const u32x4_t*)(stg + r * kRowBytes + ch * 16);
        const uint32_t r0 = pair_swap(is_up ? v[0] : v[2]), r1 = pair_swap(is_up ? v[1] : v[3]);
        const uint32_t gpk[2] = {is_up ? r0 : v[0], is_up ? r1 : v[1]};
        const uint32_t upk[2] = {is_up ? v[2] : r0, is_up ? v[3] : r1};
        const bool ok = m < a.ep.amax_rows && col_ok;
#pragma nounroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t g16 = ((e >> 1) ? gpk[1] : gpk[0]) >> (16 * (e & 1)) & 0xFFFFu;
          const uint32_t u16 = ((e >> 1) ? upk[1] : upk[0]) >> (16 * (e & 1)) & 0xFFFFu;
          const float gb = fmaxf(bf16_bits_to_float(g16), 0.28125f);
          const float ub = fabsf(bf16_bits_to_float(u16));
          const bool cand = ok && gb * ub * (1.0f + 0x1p-7f) + 0x1p-140f >= ymax;  // margin covers fp32 rounding
          const uint64_t mask = __ballot(cand);
          const int nc = __builtin_amdgcn_readfirstlane(__popcll(mask));
          if (nc) {
            if (cand) {
              const int off = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
              clist[ccount + off] = g16 | (u16 << 16);
            }
            ccount += nc;
          }
        }
        ++t;
        if (t == kIts) pending = ccount != 0;
      }
    };
#pragma unroll
    for (int half = 0; half < FM / 2; ++half) {
      // kind 1: the residual row segments of this half, issued before its staging so
      // that their latency overlaps it
      u32x4_t rv[kIts];
      if constexpr (EPI == 1) {
        const int64_t m0r = wrow0 + half * 64 + rl;
        const uint16_t* rp = a.ep.res ? a.ep.res + m0r * a.n + col : nullptr;
        const int64_t rstride = (int64_t)kRowsPerStore * a.n;
#pragma unroll
        for (int t = 0; t < kIts; ++t) {
          const u32x4_t z = {0u, 0u, 0u, 0u};
          rv[t] = (a.ep.res && m0r + t * kRowsPerStore < a.m_pad && col_ok) ? *(const u32x4_t*)(rp + t * rstride) : z;
        }
      }
      // registers -> LDS: fragments i = 2 half, 2 half + 1 hold rows 64 half .. 64 half + 63
      float smax = 0.0f;  // kind 2: the half's largest screening bound s (rows < amax_rows)
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * half + ii;
        float smax_ii = 0.0f;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          float f[4][4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t bw = bq[j][q][e >> 1];
              const float b = (e & 1) ? __uint_as_float(bw & 0xFFFF0000u) : __uint_as_float(bw << 16);
              f[q][e] = __builtin_fmaf(acc[j][i][q * 4 + e], alpha, b);
            }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x2_t v = {cvt_pk_bf16_rn(f[q][0], f[q][1]), cvt_pk_bf16_rn(f[q][2], f[q][3])};
            const int r = ii * 32 + lr, c = j * 32 + q * 8 + h * 4;
            *(u32x2_t*)(stg + r * kRowBytes + c * 2) = v;
          }
          if constexpr (EPI == 2) {
            // accumulator chunks q = 0, 2 are gate channels, q = 1, 3 the same up channels
#pragma unroll
            for (int pq = 0; pq < 4; pq += 2)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float G = fmaxf(f[pq][e], 0.28125f);
                smax_ii = fmaxf(smax_ii, __builtin_fmaf(G, 0x1p-130f, G * fabsf(f[pq + 1][e])));
              }
          }
        }
        if constexpr (EPI == 2) {
          const int64_t m = wrow0 + half * 64 + ii * 32 + lr;
          smax = m < a.ep.amax_rows ? fmaxf(smax, smax_ii) : smax;
        }
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
      asm volatile("" ::: "memory");
      if constexpr (EPI == 1) {
        // LDS -> global: lane L takes 8 columns of one row
#pragma unroll
        for (int t = 0; t < kIts; ++t) {
          const int r = t * kRowsPerStore + rl;
          const int64_t m = wrow0 + half * 64 + r;
          u32x4_t v = *(const u32x4_t*)(stg + r * kRowBytes + ch * 16);
          if (a.ep.res) {
            // res + gate * D1 in fp32: the product of two bf16 values is exact, so
            // the fused multiply-add is that sum rounded once
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const float d0 = bf16_bits_to_float(v[w] & 0xFFFFu), d1 = __uint_as_float(v[w] & 0xFFFF0000u);
              const float r0 = bf16_bits_to_float(rv[t][w] & 0xFFFFu);
              const float r1 = __uint_as_float(rv[t][w] & 0xFFFF0000u);
              const float g0 = __uint_as_float(gate8[w] << 16), g1 = __uint_as_float(gate8[w] & 0xFFFF0000u);
              v[w] = cvt_pk_bf16_rn(__builtin_fmaf(g0, d0, r0), __builtin_fmaf(g1, d1, r1));
            }
          }
          if (m < a.m_pad && col_ok) *(u32x4_t*)(a.d + m * a.n + col) = v;
        }
      } else {
        // LDS -> global: gate and up row segments to their own tensors
#pragma unroll
        for (int t = 0; t < kIts; ++t) {
          const int r = t * kRowsPerStore + rl;
          const int64_t m = wrow0 + half * 64 + r;
          const u32x4_t v = *(const u32x4_t*)(stg + r * kRowBytes + ch * 16);
          if (m < a.m_pad && col_ok) *(u32x4_t*)((is_up ? a.ep.up_out : a.ep.gate_out) + m * n_half + j0) = v;
        }
        // (no amax pointer: nothing to fold, no scan)
        const float T = threshold();
        if (a.ep.amax && __ballot(smax > T) != 0) scan_half(half);
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);  // the reads are done before the next half overwrites
      asm volatile("" ::: "memory");
    }
    if constexpr (EPI == 2) {
      // (the candidate list is empty: each scan ends with it flushed)
      // one atomic max per wave (non-negative fp32 bits order as integers)
      uint32_t yb = __float_as_uint(ymax);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)yb, off, 64);
        yb = yb > o ? yb : o;
      }
      if (a.ep.amax && lane == 0)
        __hip_atomic_fetch_max((uint32_t*)a.ep.amax, yb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (!more) break;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next tile's first steps have landed
  }  // tiles
}

template <int EPI>
__device__ __forceinline__ void gemm_body(const GemmArgs& a, unsigned char* smem) {
  // Tiles (256 x 256) are numbered m-band-major: band = 8 M-tiles, within a band M
  // first. Workgroups [0, big_tiles) run tiles [0, big_tiles) whole, remapped so that
  // each XCD (workgroups are dispatched round-robin over the 8 XCDs) owns one
  // contiguous range of tiles. Workgroups past that run the remaining tiles as
  // 128 x 128 quarters; they are dispatched last and fill the CUs that free up.
  const int b = blockIdx.x;
  if constexpr (EPI == 0) {
    if (a.persist_wgs > 0) {
      // persistent (plain kernel): workgroup b (on XCD b % 8) starts with tile `slot`
      // of its XCD's range and then takes tiles from the queues inside run_tile; after
      // the whole tiles, the quarters of the tail tiles, one take each
      const int slots = a.persist_wgs / 8, xcd = b % 8, slot = b / 8;
      const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
      volatile int* qslot = (volatile int*)(smem + sched_slot_offset<EPI>());
      int start, len;
      xcd_range(a, xcd, start, len);
      if (slot < len) {
        int64_t m0, n0;
        tile_origin(a, start + slot, m0, n0);
        run_tile<4, 4, 0, true>(a, m0, n0, smem, xcd, slots);
      }
      for (;;) {
        stage_barrier();  // every wave has read the slot's previous value
        if (wave == 0 && tid == 0) {
          const uint64_t q = __hip_atomic_fetch_add(a.sched + 8, (uint64_t)1, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
          *qslot = q < (uint64_t)a.quarter_units ? (int)q : -1;
        }
        stage_barrier();
        const int q = __builtin_amdgcn_readfirstlane(*qslot);
        if (q < 0) break;
        int64_t m0, n0;
        tile_origin(a, a.big_tiles + q / 4, m0, n0);
        const int64_t qm0 = m0 + ((q % 4) >> 1) * kTileQuarter, qn0 = n0 + ((q % 4) & 1) * kTileQuarter;
        if (qm0 < a.m_pad && qn0 < a.n) run_tile<2, 2, EPI>(a, qm0, qn0, smem);  // else wholly past the output
      }
      // this workgroup takes nothing more; the last one to finish clears the queues
      if (tid == 0) {
        const uint64_t done = __hip_atomic_fetch_add(a.sched + 9, (uint64_t)1, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done == (uint64_t)gridDim.x - 1) {
#pragma unroll
          for (int i = 0; i < 10; ++i) __hip_atomic_store(a.sched + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      return;
    }
  }
  if constexpr (EPI != 0) {
    if (a.sched) {
      // fused kinds: a grid of one unit per workgroup plus a round of spare workgroups.
      // Each takes one unit: the front of its XCD's queue (every tile of the range is
      // taken at run time), else the back of the fullest other queue, else a quarter
      // of the tail; a workgroup that finds none exits. The spare workgroups of a fast
      // XCD take the tiles its slower neighbours have not reached.
      const int xcd = b % 8;
      const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
      volatile int* uslot = (volatile int*)(smem + sched_slot_offset<EPI>());
      if (wave == 0) {
        int u = -1;
        if (tid == 0)
          u = front_tile(a, xcd, 0,
                         __hip_atomic_fetch_add(a.sched + xcd, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        u = __builtin_amdgcn_readfirstlane(u);
        if (u < 0) u = steal_tile(a, 0, lane);
        if (u < 0 && tid == 0) {
          const uint64_t q = __hip_atomic_fetch_add(a.sched + 8, (uint64_t)1, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
          u = q < (uint64_t)a.quarter_units ? a.big_tiles + (int)q : -1;  // units past big_tiles are quarters
        }
        if (tid == 0) *uslot = u;
      }
      stage_barrier();
      const int u = __builtin_amdgcn_readfirstlane(*uslot);
      if (u >= a.big_tiles) {
        const int q = u - a.big_tiles;
        int64_t m0, n0;
        tile_origin(a, a.big_tiles + q / 4, m0, n0);
        const int64_t qm0 = m0 + ((q % 4) >> 1) * kTileQuarter, qn0 = n0 + ((q % 4) & 1) * kTileQuarter;
        if (qm0 < a.m_pad && qn0 < a.n) run_tile<2, 2, EPI>(a, qm0, qn0, smem);
      } else if (u >= 0) {
        int64_t m0, n0;
        tile_origin(a, u, m0, n0);
        run_tile<4, 4, EPI>(a, m0, n0, smem);
      }
      if (tid == 0) {
        const uint64_t done = __hip_atomic_fetch_add(a.sched + 9, (uint64_t)1, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done == (uint64_t)gridDim.x - 1) {
#pragma unroll
          for (int i = 0; i < 10; ++i) __hip_atomic_store(a.sched + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      return;
    }
  }
  int t, quarter = -1;
  if (b < a.big_tiles) {
    const int nb = a.big_tiles;
    const int per = nb / 8, rem = nb % 8;
    const int xcd = b % 8, idx = b / 8;
    t = xcd * per + (xcd < rem ? xcd : rem) + idx;
  } else {
    const int q = b - a.big_tiles;
    t = a.big_tiles + q / 4;
    quarter = q % 4;
  }
  const int ntiles = a.tiles_m * a.tiles_n;
  if (t >= ntiles) return;
  int64_t m0, n0;
  tile_origin(a, t, m0, n0);
  if (quarter < 0) {
    run_tile<4, 4, EPI>(a, m0, n0, smem);
  } else {
    const int64_t qm0 = m0 + (quarter >> 1) * kTileQuarter, qn0 = n0 + (quarter & 1) * kTileQuarter;
    if (qm0 >= a.m_pad || qn0 >= a.n) return;  // a quarter wholly past the padded output
    run_tile<2, 2, EPI>(a, qm0, qn0, smem);
  }
}

template <int EPI>
__global__ void __launch_bounds__(kGemmThreads, 1) gemm_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // clock stamps in the plain kernel only (the fused kernels have no registers to spare)
  const bool stamp = EPI == 0 && a.ep.clk != nullptr && (int)blockIdx.x < a.ep.clk_slots;
  uint64_t c0 = 0, t0 = 0;
  if (stamp) {
    c0 = __builtin_amdgcn_s_memtime();
    t0 = __builtin_amdgcn_s_memrealtime();
  }
  gemm_body<EPI>(a, smem);
  if (stamp) {
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), t1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
      a.ep.clk[2 * blockIdx.x] = c1 - c0;
      a.ep.clk[2 * blockIdx.x + 1] = t1 - t0;
    }
  }
}

// ---- host side -----------------------------------------------------------------------------

// the plain kernel's persistent workgroups stage their epilogue past the pipeline stages,
// followed by the word that broadcasts a taken tile
size_t gemm_smem_bytes(int kind) {
  return (kind == 2 ? sched_slot_offset<2>() : kind == 1 ? sched_slot_offset<1>() : sched_slot_offset<0>()) + 16;
}
const void* gemm_kernel_ptr(int kind) {
  return kind == 2 ? (const void*)gemm_kernel<2> : kind == 1 ? (const void*)gemm_kernel<1> : (const void*)gemm_kernel<0>;
}

hipError_t launch_gemm(const uint8_t* aq, const uint8_t* as, const float* ga, const uint8_t* wq,
                       const uint8_t* ws, const float* gw, uint16_t* d, int64_t m_pad, int64_t n, int64_t k,
                       const GemmEpilogue& ep, int cu_count, uint64_t* sched, hipStream_t stream) {
  GemmArgs args;
  args.ep = ep;
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
  args.tiles_m = (int)((m_pad + kTileBig - 1) / kTileBig);
  args.tiles_n = (int)((n + kTileBig - 1) / kTileBig);
  args.cgroups = (int)(cpad / 4);
  args.ksteps = (int)((k + kTK - 1) / kTK);
  const int ntiles = args.tiles_m * args.tiles_n;
  if (ntiles == 0) return hipSuccess;
  // One workgroup per CU at a time. When the last round of whole tiles would hold
  // at most a quarter of the CUs' worth, its tiles run as 128 x 128 quarters.
  const int tail = cu_count > 0 ? ntiles % cu_count : 0;
  args.big_tiles = (tail > 0 && ntiles > cu_count && 4 * tail <= cu_count) ? ntiles - tail : ntiles;
  // The plain kernel runs every tile with persistent workgroups, a multiple of 8 of
  // them (each XCD the same count), one per CU, when there are more whole tiles than
  // that: the next tile's first loads then overlap the current tile's epilogue, and
  // the tiles past each workgroup's first are taken from the queue set `sched` (zero
  // on entry, zero again when the launch ends). Taken at run time, the whole tiles end
  // up to one tile apart across the CUs whatever the count; when the last round is
  // more than a quarter full, half a round of tiles runs as quarters to even that out.
  const int persist = cu_count - cu_count % 8;
  const bool dynamic = sched && persist >= 8;
  if (dynamic && tail > 0 && 4 * tail > cu_count && ntiles - persist / 2 > persist)
    args.big_tiles = ntiles - persist / 2;
  args.quarter_units = 4 * (ntiles - args.big_tiles);
  args.persist_wgs = (dynamic && ep.kind == 0 && args.big_tiles > persist) ? persist : 0;
  // the fused kinds take one unit per workgroup at run time when there are more whole
  // tiles than CUs, with a round of spare workgroups; otherwise the grid is static
  const bool fused_dynamic = dynamic && ep.kind != 0 && args.big_tiles > persist;
  args.sched = (args.persist_wgs > 0 || fused_dynamic) ? sched : nullptr;
  const int grid = args.persist_wgs > 0 ? args.persist_wgs
                                        : args.big_tiles + args.quarter_units + (fused_dynamic ? persist : 0);
  if (ep.kind == 2)
    gemm_kernel<2><<<dim3(grid), dim3(kGemmThreads), gemm_smem_bytes(2), stream>>>(args);
  else if (ep.kind == 1)
    gemm_kernel<1><<<dim3(grid), dim3(kGemmThreads), gemm_smem_bytes(1), stream>>>(args);
  else
    gemm_kernel<0><<<dim3(grid), dim3(kGemmThreads), gemm_smem_bytes(0), stream>>>(args);
  return hipGetLastError();
}

}  // namespace nvfp4
