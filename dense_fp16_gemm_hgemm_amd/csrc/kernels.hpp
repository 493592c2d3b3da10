// HIP kernel templates of the TN half-precision GEMM for gfx950 (CDNA4).
//
// Pages this design follows (cited below by tag and section):
//   [P1] "H100 GEMM L2驻留优化：warp-specialized TMA异步拷贝与RL调优策略"
//        (blog.hotdry.top, 2025-12-05)
//   [P2] "RL驱动CUDA L2 GEMM内核自动调优：A100/H100 tile size与融合优化"
//        (blog.hotdry.top, 2025-12-05)
//   [P3] "B-08. Hopper TMA：从单线程 Bulk Copy 到吞吐墙" (lqnn.cn)
//
// What is computed: C[i][j] = fp16_rne(sum_k A[i][k] * B[j][k]) with the sum in
// fp32 on the matrix cores, A row-major, B column-major (stored as N rows of K
// halves, i.e. both operands K-contiguous), C row-major ([P2] 正文 paragraphs 1
// and 3).  The pages' dataflow (global -> shared -> registers -> tensor core ->
// global, [P2] 正文 paragraph 3) maps onto gfx950 as
//   global 16-byte loads -> XOR-swizzled LDS tile -> ds_read_b128 fragments ->
//   v_mfma_f32_{32x32x16,16x16x32}_f16 -> fp16 convert -> global store,
// with the next K tile's global loads in flight while the current tile's MFMAs
// run (the prefetch that [P3] §2 and §5 show is where the overlap gain comes
// from, and the multi-stage pipeline of [P1] 可落地参数清单 / [P2] 落地参数).
//
// MFMA operand layout used throughout (one wave of 64 lanes, instruction
// MF x MF x KI with MF in {32, 16} and KI = 512 / MF):
//   * lane l supplies row (l % MF) of the first source and column (l % MF) of
//     the second source, 8 consecutive reduction elements each, starting at
//     8 * (l / MF) within the instruction's KI;
//   * the result element (r, c) of the MF x MF block sits in lane
//     c + MF * ((r / 4) % (64 / MF)), register 4 * (r / (256 / MF)) + r % 4.
// Both sources are loaded with the same k placement, so the sum is the same
// dot product whatever order the hardware reduces in.  The first source is
// the B tile (rows = output columns j), the second the A tile (columns =
// output rows i), so each lane ends up owning 4 consecutive columns of one
// output row, which makes the C stores 8-byte vectors along N.
#pragma once

#include <type_traits>

#include "internal.h"
#include "ring_schedule.h"

namespace mihg {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int MF>
struct Mfma;

template <>
struct Mfma<32> {
  static constexpr int KI = 16;    // reduction depth per instruction
  static constexpr int NACC = 16;  // fp32 results per lane
  typedef f32x16 acc_t;
  __device__ static inline acc_t mma(h8 a, h8 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<16> {
  static constexpr int KI = 32;
  static constexpr int NACC = 4;
  typedef f32x4 acc_t;
  __device__ static inline acc_t mma(h8 a, h8 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

__device__ inline h8 zero_h8() {
  h8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (_Float16)0.0f;
  return z;
}

// Workgroup id -> output tile.  [P1] 正文 paragraph 2 and [P2] 正文
// paragraph 3 put the lever in keeping operand panels cache-resident; on
// MI355X each of the 8 XCDs has its own L2 and consecutive workgroup ids are
// dispatched round-robin over the XCDs.  With xcd_remap the id is first
// renumbered so that each XCD receives a contiguous range of logical ids; the
// logical id is then walked in groups of group_m tile rows, so the workgroups
// resident at one time share A row panels and B column panels.
__device__ inline void tile_coords(int pid, int tiles_m, int tiles_n, int group_m,
                                   int xcd_remap, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  if (xcd_remap) {
    const int q = total >> 3, r = total & 7;
    const int x = pid & 7, loc = pid >> 3;
    pid = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + loc;
  }
  const int width = group_m * tiles_n;
  const int group = pid / width;
  const int first_m = group * group_m;
  const int rows = min(tiles_m - first_m, group_m);
  const int in = pid - group * width;
  tm = first_m + in % rows;
  tn = in / rows;
}

// LDS tile rows hold 64 halves = 8 chunks of 16 bytes.  The chunk index is
// XORed with a function of the row: 16 consecutive rows read at one
// logical chunk then touch 16 distinct (row parity, chunk) pairs and 8
// consecutive rows 8 distinct chunks, so ds_read_b128 of an MFMA fragment and
// ds_write_b128 of a loaded row are free of bank conflicts whether the LDS
// serves 8 or 16 lanes of a b128 access per cycle.  [P3] §6.2 makes the point
// that the swizzle has to be designed against the read pattern; [P1]
// 可落地参数清单 uses the same 3-bit XOR (row bits into the 16-byte chunk index
// of a 128-byte row).
__device__ inline int swz(int row, int chunk) { return chunk ^ ((row ^ (row >> 3)) & 7); }

// Buffer resources.  A raw buffer descriptor bounds every access by its
// record count: loads past the end return 0 and stores past the end are
// dropped.  Each workgroup builds descriptors whose range ends at the last
// valid row of its tile, so rows beyond M or N need no code at all, and a
// chunk beyond K is given the offset kOOB, which is outside every range.  This
// is the zero-filled out-of-bounds behaviour [P3] §3.2 relies on for tile
// copies, and it keeps the K loop free of branches.  Offsets are 32-bit; the
// host only sends operands here whose tile rows span less than 2^31 bytes.
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9-family raw buffer, 32-bit data format
// Cache-policy operand of the buffer builtins: bit 4 is SC1, which on the
// gfx94x/gfx950 memory model gives an access device scope (coherent across
// the XCDs' L2 caches) without any cache-wide write-back or invalidate.
constexpr int kDeviceScope = 16;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}
__device__ inline h8 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ inline void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, h4 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 0);
}
__device__ inline void buf_store2(__amdgpu_buffer_rsrc_t r, uint32_t off, _Float16 v) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), r, off, 0, 0);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// gfx950's int8 MFMA: 16 x 16 outputs over a reduction of 64, each lane
// supplying 16 consecutive int8 values of its row (the same 16-byte fragment
// that holds 8 halves for v_mfma_f32_16x16x32_f16), int32 accumulation.
struct MfmaI8 {
  static constexpr int KI = 64;
  static constexpr int NACC = 4;
  typedef i32x4 acc_t;
  __device__ static inline acc_t mma(h8 a, h8 b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                                 __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
  }
};

// Element types of a GEMM variant.  Every variant moves operands as 16-byte
// lane fragments and LDS rows of 128 (or 256, 512) bytes, so copies, LDS
// layouts and schedules are shared, and each 64 bytes of a row are one MFMA
// K step; only the element width, the MFMA, the accumulator and the result
// conversion differ.
//   OpF16: binary16 operands, fp32 accumulation, binary16 result (RNE).
//   OpI8:  int8 operands, int32 accumulation, int32 result (exact).
struct OpF16 {
  static constexpr int kEB = 2;  // operand bytes per element
  static constexpr int kCB = 2;  // result bytes per element
  typedef _Float16 in_t;
  typedef _Float16 out_t;
  typedef f32x4 acc4_t;  // four accumulators of one output row
  template <int MF>
  using Mma = Mfma<MF>;
  // four consecutive results of one output row, at byte offset off
  __device__ static inline void store4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
    h4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (_Float16)v[e];
    buf_store8(r, off, o);
  }
  __device__ static inline void store1(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
    buf_store2(r, off, (_Float16)v);
  }
};

struct OpI8 {
  static constexpr int kEB = 1;
  static constexpr int kCB = 4;
  typedef int8_t in_t;
  typedef int32_t out_t;
  typedef i32x4 acc4_t;
  template <int MF>
  using Mma = MfmaI8;
  __device__ static inline void store4(__amdgpu_buffer_rsrc_t r, uint32_t off, i32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
  }
  __device__ static inline void store1(__amdgpu_buffer_rsrc_t r, uint32_t off, int v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, off, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// Tile family: BM x BN x 64 workgroup tiles, WGM x WGN waves, 2 LDS stages,
// operands in the 16-byte alignment class.
//
// LDS rows are padded from 128 to 144 bytes.  A 16-byte read of row r
// then starts at 4-byte bank 36*r mod 64: 16 consecutive rows read at one
// chunk start at 16 distinct multiples of 4, and 8 consecutive rows at 8
// distinct multiples of 4 mod 32, so the MFMA fragment reads (16 or 32 rows at
// one chunk) are free of bank conflicts whether the LDS serves 8 or 16 lanes
// of a ds_read_b128 per cycle.  [P3] §6.2 makes the point that the layout has
// to be designed against the read pattern; padding instead of an XOR keeps
// every fragment address a compile-time offset from one base register.
//
// Per K tile (one trip of the loop, a single basic block):
//   * 16-byte buffer loads of tile k+1 into registers are issued first, so
//     they are in flight during tile k's MFMAs.  The row of each load
//     slot and the K position are scalar offsets, so the loads cost no VALU;
//   * tile k's fragments are read from LDS one MFMA step ahead of use
//     (register double buffer), and the MFMAs run;
//   * tile k+1 is written to the other LDS stage and one barrier ends the
//     trip; the next tile's first fragments are read right after it, while
//     the last MFMAs are still in the pipe.
// The last trip loads a tile past K, which the descriptors turn into zeros.
// When K is not a multiple of 64 the same loop runs with per-chunk K masks.
constexpr int kLdsRow = 64 + 8;  // halves per padded LDS row

// Instruction order of one K trip, handed to the machine scheduler as groups
// (mask bits: 0x008 MFMA, 0x020 global read, 0x100 LDS read, 0x200 LDS write).
// Left alone the scheduler sinks the next tile's global loads down to the LDS
// writes that consume them and reads each fragment just before its MFMA; with
// one or two waves per SIMD both expose a full memory latency to the matrix
// pipe.  The order imposed here is, per MFMA step s:
//   LDS reads of step s+1's fragments, then step s's MFMAs;
// with the next tile's global loads spread over the first step's MFMAs and its
// LDS writes over the last step's, so every latency sits behind MFMA work.
template <int NM, int NR, int NG, int KSTEPS>
__device__ __forceinline__ void trip_schedule() {
  constexpr int PER = (NG + NM - 1) / NM;  // loads (or LDS writes) per MFMA
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    if (s + 1 < KSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (s == 0 && i * PER < NG) __builtin_amdgcn_sched_group_barrier(0x020, PER, 0);
      if (s == KSTEPS - 1 && i * PER < NG) __builtin_amdgcn_sched_group_barrier(0x200, PER, 0);
    }
  }
}

template <int BM, int BN, int WGM, int WGN, int MF, bool MASK_K>
__device__ __forceinline__ void tile_main_loop(
    const GemmArgs& p, _Float16 (*lds)[(BM + BN) * kLdsRow], __amdgpu_buffer_rsrc_t rsa,
    __amdgpu_buffer_rsrc_t rsb, typename Mfma<MF>::acc_t (&acc)[BM / WGM / MF][BN / WGN / MF]) {
  using MM = Mfma<MF>;
  constexpr int BK = 64, CPR = BK / 8;
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / MF, FN = WTN / MF;
  constexpr int KSTEPS = BK / MM::KI;
  constexpr int A_IT = BM * CPR / NT, B_IT = BN * CPR / NT;
  constexpr int ROWS_PER_IT = NT / CPR;
  static_assert(KSTEPS % 2 == 0, "fragment double buffer needs an even step count");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int K = p.K;
  const int c = tid % CPR, r0 = tid / CPR;
  // global: lane part of the offset in a VGPR, slot row and K position scalar
  const uint32_t a_voff = (uint32_t)(r0 * p.lda * 2 + c * 16);
  const uint32_t b_voff = (uint32_t)(r0 * p.ldb * 2 + c * 16);
  const uint32_t a_row_step = (uint32_t)(ROWS_PER_IT * p.lda * 2);
  const uint32_t b_row_step = (uint32_t)(ROWS_PER_IT * p.ldb * 2);
  // LDS: write slot and fragment bases (halves); everything else is immediate
  const int w_base = r0 * kLdsRow + c * 8;
  const int fa_base = (wm * WTM + lane % MF) * kLdsRow + (lane / MF) * 8;
  const int fb_base = BM * kLdsRow + (wn * WTN + lane % MF) * kLdsRow + (lane / MF) * 8;

  h8 ra[A_IT], rb[B_IT];
  auto gload = [&](int k0) {
    const uint32_t kb = (uint32_t)k0 * 2;
    bool kin = true;
    if constexpr (MASK_K) kin = k0 + c * 8 < K;
#pragma unroll
    for (int it = 0; it < A_IT; ++it) {
      const uint32_t voff = MASK_K ? (kin ? a_voff : kOOB) : a_voff;
      ra[it] = __builtin_bit_cast(
          h8, __builtin_amdgcn_raw_buffer_load_b128(rsa, voff, it * a_row_step + kb, 0));
    }
#pragma unroll
    for (int it = 0; it < B_IT; ++it) {
      const uint32_t voff = MASK_K ? (kin ? b_voff : kOOB) : b_voff;
      rb[it] = __builtin_bit_cast(
          h8, __builtin_amdgcn_raw_buffer_load_b128(rsb, voff, it * b_row_step + kb, 0));
    }
  };
  auto sstore = [&](int s) {
    _Float16* st = lds[s] + w_base;
#pragma unroll
    for (int it = 0; it < A_IT; ++it)
      *reinterpret_cast<h8*>(st + it * ROWS_PER_IT * kLdsRow) = ra[it];
#pragma unroll
    for (int it = 0; it < B_IT; ++it)
      *reinterpret_cast<h8*>(st + (BM + it * ROWS_PER_IT) * kLdsRow) = rb[it];
  };
  h8 fa[2][FM], fb[2][FN];
  auto fread = [&](int s, int step, int buf) {
    const _Float16* st = lds[s];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      fa[buf][fm] = *reinterpret_cast<const h8*>(st + fa_base + fm * MF * kLdsRow + step * MM::KI);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
      fb[buf][fn] = *reinterpret_cast<const h8*>(st + fb_base + fn * MF * kLdsRow + step * MM::KI);
  };

  const int nk = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  fread(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    gload((kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      if (s + 1 < KSTEPS) fread(cur, s + 1, (s + 1) & 1);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = MM::mma(fb[s & 1][fn], fa[s & 1][fm], acc[fm][fn]);
    }
    sstore(cur ^ 1);
    trip_schedule<FM * FN, FM + FN, A_IT + B_IT, KSTEPS>();
    __syncthreads();
    fread(cur ^ 1, 0, 0);
  }
}

template <int BM, int BN, int WGM, int WGN, int MF>
__global__ void __launch_bounds__(64 * WGM * WGN)
tile_kernel(GemmArgs p) {
  using MM = Mfma<MF>;
  constexpr int CPR = 8;
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / MF, FN = WTN / MF;
  static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must hold whole MFMA blocks");
  static_assert((BM * CPR) % NT == 0 && (BN * CPR) % NT == 0, "tile chunks must split evenly");

  __shared__ __attribute__((aligned(16))) _Float16 lds[2][(BM + BN) * kLdsRow];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int M = p.M, N = p.N, K = p.K;
  int tm, tn;
  tile_coords(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, p.group_m, p.xcd_remap, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t lda = p.lda, ldb = p.ldb, ldc = p.ldc;
  const auto rsa = make_rsrc(static_cast<const _Float16*>(p.A) + m0 * lda,
                             (uint32_t)(min(BM, M - m0) * lda * 2));
  const auto rsb = make_rsrc(static_cast<const _Float16*>(p.B) + n0 * ldb,
                             (uint32_t)(min(BN, N - n0) * ldb * 2));

  typename MM::acc_t acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int v = 0; v < MM::NACC; ++v) acc[fm][fn][v] = 0.0f;

  if ((K & 63) == 0)
    tile_main_loop<BM, BN, WGM, WGN, MF, false>(p, lds, rsa, rsb, acc);
  else
    tile_main_loop<BM, BN, WGM, WGN, MF, true>(p, lds, rsa, rsb, acc);

  // Epilogue: fp32 -> fp16 round-to-nearest-even, alpha = 1, beta = 0;
  // 8-byte stores along N, rows beyond M dropped by the descriptor.
  _Float16* Cw = static_cast<_Float16*>(p.C) + m0 * ldc;
  const auto rsc = make_rsrc(Cw, (uint32_t)(min(BM, M - m0) * ldc * 2));
  if ((N & 3) == 0) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int i = wm * WTM + fm * MF + lane % MF;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int g = 0; g < MM::NACC / 4; ++g) {
          const int j = n0 + wn * WTN + fn * MF + g * (256 / MF) + 4 * (lane / MF);
          h4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (_Float16)acc[fm][fn][4 * g + e];
          buf_store8(rsc, j < N ? (uint32_t)((i * ldc + j) * 2) : kOOB, o);
        }
    }
  } else {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int i = wm * WTM + fm * MF + lane % MF;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int g = 0; g < MM::NACC / 4; ++g) {
          const int j = n0 + wn * WTN + fn * MF + g * (256 / MF) + 4 * (lane / MF);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            buf_store2(rsc, j + e < N ? (uint32_t)((i * ldc + j + e) * 2) : kOOB,
                       (_Float16)acc[fm][fn][4 * g + e]);
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Direct-to-LDS tile family ("dtile"): BM x BN x 32 K tiles loaded by
// buffer_load_dwordx4 ... lds (global -> LDS without passing through VGPRs)
// into a ring of S LDS stages, one wave per SIMD, large wave tiles.
//
// LDS layout: row pairs.  A tile row holds 32 halves (64 bytes, 4 chunks of
// 16 bytes); LDS row R (128 bytes) holds tile rows 2R and 2R+1 as logical
// chunks c = 4*(row & 1) + k-chunk, stored at physical chunk c ^ (R & 7).
// (Plain 64-byte rows with the chunk XORed by (row >> 2) & 3 measured 4 bank
// conflict cycles per fragment read on gfx950; this layout measured none.)
// One DMA instruction of a wave fills a 1 KiB block = 8 LDS rows = 16 tile
// rows; lane l lands on LDS row l/8, physical chunk l%8, so it loads logical
// chunk (l%8) ^ (l/8) -- the same for every block, one offset register per
// operand.
//
// Pipeline (trip k): issue the DMA of tile k+S-1 into the stage tile k-1 used;
// read tile k+1's fragments (published one barrier ago) into the second
// register set; run tile k's MFMAs; wait until tile k+2's DMA has landed
// (this wave's part), and barrier.  The DMA of a tile therefore has S-2 trips
// to arrive, and the MFMAs of trip k+1 start right after the barrier.  Each
// stage is its own LDS object and trips are unrolled so stage and register
// indices are constants, which lets the compiler tell the in-flight DMA
// apart from the fragment reads instead of waiting for every DMA.
constexpr int kDRow = 32;  // halves per LDS row (no padding; XOR swizzle)

// Raw buffer descriptor as four dwords (base, base_hi | stride 0, records, word3).
__device__ inline u32x4 raw_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = (uint32_t)a;
  r[1] = (uint32_t)(a >> 32) & 0xffffu;
  r[2] = bytes;
  r[3] = (uint32_t)kRsrcWord3;
  return r;
}
// LDS byte address of a __shared__ object (the low half of its flat address).
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uint64_t>(p);
}
// One wave-wide 16-byte-per-lane copy global -> LDS: lane l's 16 bytes at
// voff + soff (bounded by the descriptor; out of range reads 0) land at LDS
// byte address lds + 16 * l.
__device__ inline void dma16(const u32x4& rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory", "m0");
}

// dma16 with the non-temporal cache policy: the lines are fetched for this
// copy and not kept for reuse.  For an operand that is streamed through once
// (B when the output has few tile rows) it leaves the L2 and MALL to the
// operand that is reused (A, read by every column of tiles).
__device__ inline void dma16_nt(const u32x4& rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory", "m0");
}

template <int BM, int BN>
struct DStages {
  static constexpr int kStage = (BM + BN) * kDRow;
  _Float16 s0[kStage], s1[kStage], s2[kStage], s3[kStage];
};

template <int I, int BM, int BN>
__device__ __forceinline__ _Float16* dstage(DStages<BM, BN>& d) {
  if constexpr (I == 0) return d.s0;
  else if constexpr (I == 1) return d.s1;
  else if constexpr (I == 2) return d.s2;
  else return d.s3;
}

// Spread the trip's ND copies and NR fragment reads evenly over its first
// three quarters of MFMAs: four waves issuing reads back to back ask the LDS
// for about twice its bandwidth, and a read issued near the end of the trip
// makes the wave wait for it at the barrier.  The last quarter is MFMA only.
template <int NM, int ND, int NR>
__device__ __forceinline__ void dtrip_schedule() {
  constexpr int SPAN = (NM * 3) / 4;
  constexpr int NX = ND + NR;
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    // memory slot x is placed after MFMA floor(x * SPAN / NX)
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      if (x * SPAN / NX == i) {
        // copies first (slots 0, 2, 4, ...), reads fill the rest
        const bool is_copy = (x % 2 == 0) && (x / 2 < ND);
        if (is_copy) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K fix-up shared by the tile families.  A workgroup is (tile, slice);
// after its K slice, every slice stores its fp32 partial tile in lane order
// (one contiguous 1 KiB per wave and store) and counts itself in; the slice
// that arrives last sums all partials in slice order 0..splitk-1 -- the same
// order whoever arrives last, so the result does not depend on timing -- and
// resets the counter for the next launch.  Returns false in every other
// slice, which then has nothing left to do; the last one returns true with
// acc holding the total.
//
// The workgroups of one tile run on different XCDs, whose L2 caches are not
// coherent with each other.  A device-scope fence would make that safe by
// writing back and invalidating the whole L2 of the XCD, once per workgroup,
// which costs the other workgroups their cached operand lines.  Instead only
// the workspace traffic is made device-coherent: partials are stored and
// loaded with device scope (cache policy SC1, which writes through and reads
// past the XCD's L2), every wave waits until its stores are acknowledged
// before the workgroup counts itself in, and the counter is a device-scope
// atomic.  The last slice reads the partials only after its atomic returned.
// VGMAX caps the 16-byte loads a lane keeps in flight while summing (its
// registers sit beside the accumulators).  REREAD: the last slice reads its
// own partial back like the others instead of keeping it in registers, so the
// accumulators are free while it sums (for register-bound instances).
template <int FM, int FN, int NT, int VGMAX = 16, bool REREAD = false, typename Acc>
__device__ __forceinline__ bool splitk_fixup(Acc (&acc)[FM][FN], const GemmArgs& p, int tile_id,
                                             int slice, int splitk, int tid, int* s_last) {
  typedef std::remove_cv_t<std::remove_reference_t<decltype(acc[0][0][0])>> E;  // float or int
  static_assert(sizeof(E) == 4, "32-bit accumulators");
  constexpr int NACC = sizeof(Acc) / sizeof(E);
  static_assert(NACC % 4 == 0, "accumulators come in groups of 4");
  constexpr int NV = FM * FN * (NACC / 4);  // 4-element values per lane
  typedef E f4 __attribute__((ext_vector_type(4)));
  const auto rsw = make_rsrc(reinterpret_cast<const f4*>(p.ws) + (int64_t)tile_id * splitk * (NV * NT),
                             (uint32_t)(splitk * NV * NT * 16));
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int g = 0; g < NACC / 4; ++g) {
        const int v = (fm * FN + fn) * (NACC / 4) + g;
        f4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[fm][fn][4 * g + e];
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rsw,
                                               (uint32_t)(((slice * NV + v) * NT + tid) * 16), 0,
                                               kDeviceScope);
      }
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xf << 8));  // vmcnt(0): partial stores acknowledged
  __syncthreads();
  if (tid == 0)
    *s_last = __hip_atomic_fetch_add(&p.cnt[tile_id], 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT) == splitk - 1;
  __syncthreads();
  if (!*s_last) return false;
  // running sum over slices 0..splitk-1 in order, VG float4 values per lane
  // at a time; a slice's VG loads are issued together before any is added
  constexpr int VG = NV < VGMAX ? NV : VGMAX;
  static_assert(NV % VG == 0, "whole groups");
#pragma unroll
  for (int v0 = 0; v0 < NV; v0 += VG) {
    f4 sum[VG];
#pragma unroll
    for (int u = 0; u < VG; ++u) sum[u] = f4{0, 0, 0, 0};
    for (int s2 = 0; s2 < splitk; ++s2) {
      if (!REREAD && s2 == slice) {
#pragma unroll
        for (int u = 0; u < VG; ++u) {
          const int v = v0 + u, fg = v / (NACC / 4), g = v % (NACC / 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) sum[u][e] += acc[fg / FN][fg % FN][4 * g + e];
        }
      } else {
        f4 x[VG];
#pragma unroll
        for (int u = 0; u < VG; ++u)
          x[u] = __builtin_bit_cast(
              f4, __builtin_amdgcn_raw_buffer_load_b128(
                      rsw, (uint32_t)(((s2 * NV + v0 + u) * NT + tid) * 16), 0, kDeviceScope));
#pragma unroll
        for (int u = 0; u < VG; ++u) sum[u] += x[u];
      }
    }
#pragma unroll
    for (int u = 0; u < VG; ++u) {
      const int v = v0 + u, fg = v / (NACC / 4), g = v % (NACC / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[fg / FN][fg % FN][4 * g + e] = sum[u][e];
    }
  }
  if (tid == 0)
    __hip_atomic_store(&p.cnt[tile_id], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Split-K is compiled into the direct-to-LDS instances of at most 256 x 128
// outputs: split-K pays only when output tiles are few, which larger tiles
// make worse, and the fix-up's registers would spill in the 256 x 256 ones.
template <int BM, int BN>
constexpr bool dtile_splits() { return BM * BN <= 256 * 128; }

template <int BM, int BN, int WGM, int WGN, int MF, int S>
__global__ void __launch_bounds__(64 * WGM * WGN)
dtile_kernel(GemmArgs p) {
  using MM = Mfma<MF>;
  constexpr int BK = 32;
  constexpr int NT = 64 * WGM * WGN, NW = NT / 64;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / MF, FN = WTN / MF;
  constexpr int KSTEPS = BK / MM::KI;
  constexpr int A_BLK = BM / 16 / NW, B_BLK = BN / 16 / NW;  // 1 KiB DMA blocks per wave
  constexpr int ND = A_BLK + B_BLK;
  constexpr int U = (S % 2 == 0) ? S : 2 * S;  // trips per unrolled loop body
  static_assert(S == 4, "four LDS stages");
  static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must hold whole MFMA blocks");
  static_assert(BM % (16 * NW) == 0 && BN % (16 * NW) == 0, "DMA blocks must split evenly");
  static_assert(FM % 4 == 0 || MF == 32 || true, "");

  __shared__ __attribute__((aligned(1024))) DStages<BM, BN> lds;
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int M = p.M, N = p.N, K = p.K;
  // split-K: workgroup id = tile * splitk + slice; slice s covers K range
  // [s * kchunk, min(K, (s + 1) * kchunk))
  const int splitk = dtile_splits<BM, BN>() ? p.splitk : 1;
  const int tile_id = blockIdx.x / splitk, slice = blockIdx.x - tile_id * splitk;
  const int k_begin = splitk > 1 ? slice * p.kchunk : 0;
  const int k_len = splitk > 1 ? min(p.kchunk, K - k_begin) : K;
  int tm, tn;
  tile_coords(tile_id, (M + BM - 1) / BM, (N + BN - 1) / BN, p.group_m, p.xcd_remap, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t lda = p.lda, ldb = p.ldb, ldc = p.ldc;
  // DMA: lane -> (row l/4 of a 16-row block, logical chunk (l%4)^(l/16)).
  // The copy is issued by inline asm: the compiler then does not treat it as
  // an LDS store, so the workgroup barrier's fence does not drain every copy
  // in flight; completion is tracked explicitly with vmcnt (wait_dma).
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int dlc = (lane & 7) ^ (lane >> 3);                 // logical chunk of LDS row l/8
  const int drow = 2 * (lane >> 3) + (dlc >> 2), dchunk = dlc & 3;  // tile row, k-chunk
  const uint32_t a_voff = (uint32_t)(drow * lda * 2 + dchunk * 16);
  const uint32_t b_voff = (uint32_t)(drow * ldb * 2 + dchunk * 16);
  const u32x4 rda = raw_rsrc(static_cast<const _Float16*>(p.A) + m0 * lda,
                             (uint32_t)(min(BM, M - m0) * lda * 2));
  const u32x4 rdb = raw_rsrc(static_cast<const _Float16*>(p.B) + n0 * ldb,
                             (uint32_t)(min(BN, N - n0) * ldb * 2));
  const bool mask_k = (K & 31) != 0;
  auto dma = [&](_Float16* stage, int k0) {
    const uint32_t kb = (uint32_t)k0 * 2;
    const bool kin = !mask_k || (k0 + dchunk * 8 < K);
    const uint32_t av = kin ? a_voff : kOOB, bv = kin ? b_voff : kOOB;
    const uint32_t sbase = lds_addr(stage);
#pragma unroll
    for (int i = 0; i < A_BLK; ++i) {
      const int blk = wave_u * A_BLK + i;
      dma16(rda, av, (uint32_t)(blk * 16 * lda * 2) + kb, sbase + blk * 16 * kDRow * 2);
    }
#pragma unroll
    for (int i = 0; i < B_BLK; ++i) {
      const int blk = wave_u * B_BLK + i;
      dma16(rdb, bv, (uint32_t)(blk * 16 * ldb * 2) + kb, sbase + (BM + blk * 16) * kDRow * 2);
    }
  };

  // copy number x of a trip: A blocks first, then B blocks
  auto dma_one = [&](_Float16* stage, int k0, int x) {
    const uint32_t kb = (uint32_t)k0 * 2;
    const bool kin = !mask_k || (k0 + dchunk * 8 < K);
    const uint32_t sbase = lds_addr(stage);
    if (x < A_BLK) {
      const int blk = wave_u * A_BLK + x;
      dma16(rda, kin ? a_voff : kOOB, (uint32_t)(blk * 16 * lda * 2) + kb,
            sbase + blk * 16 * kDRow * 2);
    } else {
      const int blk = wave_u * B_BLK + (x - A_BLK);
      dma16(rdb, kin ? b_voff : kOOB, (uint32_t)(blk * 16 * ldb * 2) + kb,
            sbase + (BM + blk * 16) * kDRow * 2);
    }
  };

  // fragment reads: LDS row of the lane's tile row + physical chunk; fm / fn /
  // step are immediates.  Fragment blocks start at multiples of 16 tile rows
  // (8 LDS rows), so the swizzle term of tile row frow is (frow / 2) & 7.
  const int frow = lane % MF, fq = lane / MF;
  int fa_off[KSTEPS], fb_off[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const int c = 4 * (frow & 1) + s * (MM::KI / 8) + fq;  // logical chunk in the LDS row
    const int in_row = (frow >> 1) * (2 * kDRow) + ((c ^ ((frow >> 1) & 7)) * 8);
    fa_off[s] = (wm * WTM) * kDRow + in_row;
    fb_off[s] = (BM + wn * WTN) * kDRow + in_row;
  }
  h8 fa[2][KSTEPS][FM], fb[2][KSTEPS][FN];
  auto fread = [&](const _Float16* stage, int buf) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        fa[buf][s][fm] = *reinterpret_cast<const h8*>(stage + fa_off[s] + fm * MF * kDRow);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        fb[buf][s][fn] = *reinterpret_cast<const h8*>(stage + fb_off[s] + fn * MF * kDRow);
    }
  };

  // fragment read number r of a tile: per step, the FM A fragments then the FN B fragments
  auto fread_one = [&](const _Float16* stage, int buf, int r) {
    const int s = r / (FM + FN), q = r % (FM + FN);
    if (q < FM)
      fa[buf][s][q] = *reinterpret_cast<const h8*>(stage + fa_off[s] + q * MF * kDRow);
    else
      fb[buf][s][q - FM] =
          *reinterpret_cast<const h8*>(stage + fb_off[s] + (q - FM) * MF * kDRow);
  };

  typename MM::acc_t acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int v = 0; v < MM::NACC; ++v) acc[fm][fn][v] = 0.0f;

  auto mfmas = [&](int buf) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = MM::mma(fb[buf][s][fn], fa[buf][s][fm], acc[fm][fn]);
  };
  // vmcnt(n) with the other counters left alone (gfx9 encoding)
  auto wait_dma = [&]() {
    constexpr int n = ND * (S - 3);
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
  };

  const int nk = (k_len + BK - 1) / BK;
  // prologue: tiles 0 .. S-2 in flight; tiles 0 and 1 published
  dma(dstage<0>(lds), k_begin);
  dma(dstage<1>(lds), k_begin + BK);
  if constexpr (S == 4) dma(dstage<2>(lds), k_begin + 2 * BK);
  wait_dma();
  __syncthreads();
  fread(dstage<0>(lds), 0);

  // trip J of the unrolled body handles tile kt + J: stage (J % S), buffers J & 1.
  // The trip is written out as an explicit order of slots: slot i issues MFMA
  // i, then possibly one copy or one fragment read of the next tile.  Copies
  // and reads are spread over the first three quarters of the trip (four
  // waves reading back to back would ask the LDS for twice its bandwidth);
  // the last quarter is MFMA only, so no wait is left for the barrier.  The
  // scheduler is not allowed to reorder slots: the copies are inline asm it
  // cannot place, and a block of them at the top of the trip idles the matrix
  // pipe.
  auto trip = [&](auto JC, int kt) {
    constexpr int J = decltype(JC)::value;
    constexpr int SN = (J + 1) % S, SW = (J + S - 1) % S;
    constexpr int BUF = J & 1, NB = BUF ^ 1;
    constexpr int NM = FM * FN * KSTEPS, NR = (FM + FN) * KSTEPS, NX = ND + NR;
    constexpr int SPAN = (NM * 3) / 4;
    _Float16* wst = dstage<SW>(lds);
    const _Float16* rst = dstage<SN>(lds);
    const int kw = k_begin + (kt + S - 1) * BK;
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int s = i / (FM * FN), fm = (i / FN) % FM, fn = i % FN;
      acc[fm][fn] = MM::mma(fb[BUF][s][fn], fa[BUF][s][fm], acc[fm][fn]);
#pragma unroll
      for (int x = 0; x < NX; ++x) {
        if (x * SPAN / NX != i) continue;
        // the first 2*ND slots alternate copy / read, the rest are reads
        if (x < 2 * ND) {
          if (x % 2 == 0) dma_one(wst, kw, x / 2);
          else fread_one(rst, NB, x / 2);
        } else {
          fread_one(rst, NB, x - ND);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_dma();
    __syncthreads();
  };
  for (int kt = 0; kt < nk; kt += U) {
    trip(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < nk) trip(std::integral_constant<int, 1>{}, kt + 1);
    if (kt + 2 < nk) trip(std::integral_constant<int, 2>{}, kt + 2);
    if constexpr (U > 3) {
      if (kt + 3 < nk) trip(std::integral_constant<int, 3>{}, kt + 3);
    }
    if constexpr (U > 4) {
      if (kt + 4 < nk) trip(std::integral_constant<int, 4>{}, kt + 4);
      if (kt + 5 < nk) trip(std::integral_constant<int, 5>{}, kt + 5);
    }
  }
  // drain the DMA still in flight before the workgroup exits
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xf << 8));

  if (dtile_splits<BM, BN>() && splitk > 1) {
    if (!splitk_fixup<FM, FN, NT>(acc, p, tile_id, slice, splitk, tid, &s_last)) return;
  }

  _Float16* Cw = static_cast<_Float16*>(p.C) + m0 * ldc;
  const auto rsc = make_rsrc(Cw, (uint32_t)(min(BM, M - m0) * ldc * 2));
  if ((N & 3) == 0) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int i = wm * WTM + fm * MF + lane % MF;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int g = 0; g < MM::NACC / 4; ++g) {
          const int j = n0 + wn * WTN + fn * MF + g * (256 / MF) + 4 * (lane / MF);
          h4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (_Float16)acc[fm][fn][4 * g + e];
          buf_store8(rsc, j < N ? (uint32_t)((i * ldc + j) * 2) : kOOB, o);
        }
    }
  } else {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int i = wm * WTM + fm * MF + lane % MF;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int g = 0; g < MM::NACC / 4; ++g) {
          const int j = n0 + wn * WTN + fn * MF + g * (256 / MF) + 4 * (lane / MF);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            buf_store2(rsc, j + e < N ? (uint32_t)((i * ldc + j + e) * 2) : kOOB,
                       (_Float16)acc[fm][fn][4 * g + e]);
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Two-stage direct-to-LDS family ("d2tile"): BM x BN x 64 K tiles, one wave
// per SIMD, the K tile split into two MFMA steps of 32 that are software
// pipelined across the barrier.
//
// A barrier costs the single wave on each SIMD its matrix pipe for the whole
// round trip, so the trip is made long: each one holds 2 x FM x FN MFMAs.
// Trip k (between two barriers):
//   first half : MFMAs of step 1 of tile k-1 (fragments read last trip), while
//                tile k+1 is copied into the other stage and the step-0
//                fragments of tile k (published by the barrier just passed)
//                are read;
//   second half: MFMAs of step 0 of tile k, while the step-1 fragments of tile
//                k are read;
//   then the wave waits for its copies of tile k+1 and the barrier publishes it.
// LDS rows are 128 bytes (64 halves, 8 chunks), chunk XORed with (row>>1)&7:
// 16 consecutive rows read at one logical chunk fall on 16 distinct (row
// parity, chunk) bank groups of a 64-bank LDS.  A copy instruction fills 8
// rows; its lanes need one of two global offsets (even or odd block).
//
// With one tile of copies in flight the global -> LDS copy path is bound by
// its latency, not its bandwidth (a 256 x 256 tile's copies alone run about
// 1.4x faster with two tiles in flight), but 160 KiB of LDS holds only 2.5
// stages of a 256 x 256 x 64 tile.  The SA = 3 form ("d2tile3") gives the
// spare half stage to A: A has three stages and is copied two trips ahead, B
// has two and is copied one trip ahead.  B's copies are issued first, so the
// wait at the end of a trip leaves exactly the A copies of this trip in
// flight (vmcnt counts this wave's copies in issue order).
constexpr int kD2Row = 64;  // halves per LDS row

// XS = false stores rows unswizzled (logical chunk = physical chunk): the
// tuner's "no swizzle" candidate, kept to measure what the XOR layout buys.
__device__ inline int ntiles_of(int tiles_m, int tiles_n) { return tiles_m * tiles_n; }

// PERSIST = true: one workgroup per CU walks the output tiles blockIdx.x,
// blockIdx.x + gridDim.x, ...; after a tile's last trip the next tile's first
// copies are issued before this tile's last MFMAs and C stores, so their
// latency hides behind that work instead of opening every tile.
// Staged C store (the "_sc" instances): one wave's FM x FN blocks of 16x16
// fp32 results go to binary16 through a private LDS scratch of 16 rows x WTN
// halves, one 16-row slice at a time, and are stored as 16-byte row chunks
// (whole row segments of the wave's columns) instead of 8-byte pieces of 16
// rows.  The scratch's 16-byte chunks are XORed with the row's low bits.  One
// wave's LDS writes and reads complete in order, so a slice needs no
// workgroup barrier; wave barriers between its write and read phases keep the
// compiler from reordering them.
// row0: the wave's first row within the tile; col0: its first column of C;
// rsc covers the tile's rows; columns at or past N are dropped (N % 8 == 0).
// (d2tile_body inlines the same steps: through this helper its 4-wave 256x256
// form, which uses every register, spilled one value.)
// nt: store with the non-temporal policy (short K: the launch is mostly C
// traffic, which then streams past the caches instead of evicting its own lines).
template <int FM, int FN, int WTN, typename Acc>
__device__ __forceinline__ void store_c_staged(const Acc (&acc)[FM][FN], _Float16* scr,
                                               __amdgpu_buffer_rsrc_t rsc, int row0, int col0,
                                               int N, int64_t ldc, int lane, bool nt = false) {
  constexpr int CPRW = WTN / 8;                  // 16-byte chunks per scratch row
  constexpr int SWM = CPRW >= 8 ? 7 : CPRW - 1;  // XOR mask of the chunk index
  static_assert(CPRW % 4 == 0 && (CPRW & (CPRW - 1)) == 0, "power-of-two rows of >= 4 chunks");
  const int srow = lane % 16, squad = lane / 16;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      h4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (_Float16)acc[fm][fn][e];
      const int col = fn * 16 + 4 * squad;  // in halves, within the wave's columns
      const int ch = (col >> 3) ^ (srow & SWM);
      *reinterpret_cast<h4*>(scr + srow * WTN + ch * 8 + (col & 7)) = o;
    }
    // the slice's writes stay before its reads, and (below) its reads before
    // the next slice's writes, whatever the compiler proves about aliasing
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int q = 0; q < 16 * CPRW / 64; ++q) {
      const int idx = q * 64 + lane, r = idx / CPRW, c = idx % CPRW;
      const h8 x = *reinterpret_cast<const h8*>(scr + r * WTN + ((c ^ (r & SWM)) * 8));
      const int i = row0 + fm * 16 + r;
      const int j = col0 + c * 8;
      const uint32_t off = j < N ? (uint32_t)((i * ldc + j) * 2) : kOOB;
      if (nt)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rsc, off, 0, 2);
      else
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rsc, off, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// SC = true stages each wave's C through LDS, 16 rows at a time, so that every
// store instruction writes whole 128-byte row segments (16 bytes a lane)
// instead of 32-byte pieces of 16 rows (8 bytes a lane from the MFMA layout).
template <typename Op, int BM, int BN, int WGM, int WGN, int SA, int MF = 16, bool XS = true,
          bool PERSIST = false, bool SC = false>
__device__ __forceinline__ void d2tile_body(const GemmArgs& p) {
  using MM = typename Op::template Mma<MF>;
  constexpr int EB = Op::kEB, CB = Op::kCB;
  constexpr int BK = 128 / EB;      // elements per 128-byte LDS row
  constexpr int EPC = 16 / EB;      // elements per 16-byte chunk
  constexpr int KSTEPS = BK / MM::KI;  // MFMA k-steps per K tile (2 for MF 16, 4 for MF 32)
  constexpr int SPH = KSTEPS / 2;      // k-steps per half trip
  constexpr int CPS = MM::KI / EPC;    // 16-byte chunks per k-step
  static_assert(MF == 16 || (MF == 32 && EB == 2), "32x32 MFMAs for binary16 only");
  constexpr int NT = 64 * WGM * WGN, NW = NT / 64;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / MF, FN = WTN / MF;
  constexpr int A_BLK = BM / 8 / NW, B_BLK = BN / 8 / NW;  // 1 KiB copies per wave
  constexpr int ND = A_BLK + B_BLK;
  constexpr int STAGE = (BM + BN) * kD2Row;
  // LDS: SA stages of A and 2 of B.  SA = 2: stage s holds A then B rows at
  // s * STAGE.  SA = 3: the A ring (3 x BM rows) and then the B ring (2 x BN
  // rows).
  constexpr int A_STRIDE = SA == 2 ? STAGE : BM * kD2Row;
  constexpr int B_OFF = SA == 2 ? BM * kD2Row : SA * BM * kD2Row;
  constexpr int B_STRIDE = SA == 2 ? STAGE : BN * kD2Row;
  constexpr int LDS_HALVES = SA == 2 ? 2 * STAGE : SA * BM * kD2Row + 2 * BN * kD2Row;
  static_assert(SA == 2 || SA == 3, "two or three A stages");
  static_assert(LDS_HALVES * 2 <= 160 * 1024, "LDS budget");
  static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must hold whole MFMA blocks");
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "copy blocks must split evenly");
  static_assert(A_BLK % 2 == 0 && B_BLK % 2 == 0, "blocks pair up by parity");

  __shared__ __attribute__((aligned(1024))) _Float16 lds[LDS_HALVES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int M = p.M, N = p.N, K = p.K;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tile = blockIdx.x, tm, tn;
  tile_coords(tile, tiles_m, tiles_n, p.group_m, p.xcd_remap, tm, tn);
  int m0 = tm * BM, n0 = tn * BN;
  const int64_t lda = p.lda, ldb = p.ldb, ldc = p.ldc;

  // copies: lane l -> row l/8 of an 8-row block, physical chunk l%8, which
  // holds logical chunk (l%8) ^ ((l>>4) ^ 4*(block&1))
  int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int drow = lane >> 3;
  const int dch0 = XS ? (lane & 7) ^ (lane >> 4) : lane & 7, dch1 = XS ? dch0 ^ 4 : dch0;
  u32x4 rda = raw_rsrc(static_cast<const char*>(p.A) + m0 * lda * EB,
                       (uint32_t)(min(BM, M - m0) * lda * EB));
  u32x4 rdb = raw_rsrc(static_cast<const char*>(p.B) + n0 * ldb * EB,
                       (uint32_t)(min(BN, N - n0) * ldb * EB));
  const uint32_t a_v0 = (uint32_t)(drow * lda * EB + dch0 * 16), a_v1 = (uint32_t)(drow * lda * EB + dch1 * 16);
  const uint32_t b_v0 = (uint32_t)(drow * ldb * EB + dch0 * 16), b_v1 = (uint32_t)(drow * ldb * EB + dch1 * 16);
  const bool mask_k = (K % BK) != 0;
  const uint32_t lds0 = lds_addr(lds);
  // copy x (0..ND-1): A block xa of tile ka into A stage ast, or B block xb of
  // tile kb into B stage bst.  SA = 2 issues A's blocks first, SA = 3 B's
  // (the B copies must land this trip, A's only the next).
  auto dma_a = [&](int ast, int k0, int xa) {
    const uint32_t kbytes = (uint32_t)k0 * EB;
    const int blk = wave_u * A_BLK + xa;
    const int ch = (xa & 1) ? dch1 : dch0;
    const bool kin = !mask_k || (k0 + ch * EPC < K);
    dma16(rda, kin ? ((xa & 1) ? a_v1 : a_v0) : kOOB, (uint32_t)(blk * 8 * lda * EB) + kbytes,
          lds0 + (uint32_t)((ast * A_STRIDE + blk * 8 * kD2Row) * 2));
  };
  auto dma_b = [&](int bst, int k0, int xb) {
    const uint32_t kbytes = (uint32_t)k0 * EB;
    const int blk = wave_u * B_BLK + xb;
    const int ch = (xb & 1) ? dch1 : dch0;
    const bool kin = !mask_k || (k0 + ch * EPC < K);
    dma16(rdb, kin ? ((xb & 1) ? b_v1 : b_v0) : kOOB, (uint32_t)(blk * 8 * ldb * EB) + kbytes,
          lds0 + (uint32_t)((B_OFF + bst * B_STRIDE + blk * 8 * kD2Row) * 2));
  };
  auto dma_one = [&](int ast, int bst, int ka, int kb, int x) {
    if constexpr (!ring::d2_b_first(SA)) {
      if (x < A_BLK) dma_a(ast, ka, x);
      else dma_b(bst, kb, x - A_BLK);
    } else {
      if (x < B_BLK) dma_b(bst, kb, x);
      else dma_a(ast, ka, x - B_BLK);
    }
  };

  // fragments of k-step t: row base + per-lane physical chunk of logical
  // chunk CPS*t + l/MF (rows are multiples of MF plus l % MF, so the swizzle
  // term is ((l % MF) >> 1) & 7; 16 lanes read 16 consecutive rows per pass)
  const int frow = lane % MF, fq = lane / MF, fsw = XS ? (frow >> 1) & 7 : 0;
  int fa_off[KSTEPS], fb_off[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const int phys = (CPS * s + fq) ^ fsw;
    fa_off[s] = (wm * WTM + frow) * kD2Row + phys * 8;
    fb_off[s] = (BM + wn * WTN + frow) * kD2Row + phys * 8;
  }
  h8 fa[2][SPH][FM], fb[2][SPH][FN];  // [half][k-step within the half]
  // read r of half h: k-step h*SPH + r / (FM + FN), A's fragments then B's
  auto fread_one = [&](int ast, int bst, int h, int r) {
    const int u = r / (FM + FN), q = r % (FM + FN), s = h * SPH + u;
    if (q < FM)
      fa[h][u][q] = *reinterpret_cast<const h8*>(lds + ast * A_STRIDE + fa_off[s] + q * MF * kD2Row);
    else
      fb[h][u][q - FM] = *reinterpret_cast<const h8*>(lds + B_OFF - BM * kD2Row + bst * B_STRIDE +
                                                      fb_off[s] + (q - FM) * MF * kD2Row);
  };

  typename MM::acc_t acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int v = 0; v < MM::NACC; ++v) acc[fm][fn][v] = 0;

  constexpr int NM = SPH * FM * FN, NR = SPH * (FM + FN);  // per half
  // One half trip: the NM MFMAs of step S_MFMA (when DO_MFMA), with the
  // copies of the next tile (when COPY) and the NR fragment reads of step
  // S_READ spread evenly over its MFMA slots; copies and reads alternate
  // while copies last.  (Spreading them over the whole half measured ~1.5%
  // faster on 8192^3 than packing them into its first three quarters, and
  // issuing every copy first was ~3% slower.)
  auto half = [&](auto DO_MFMA, auto COPY, auto S_MFMA, auto S_READ, int rast, int rbst, int ka,
                  int kb, int wast, int wbst) {
    constexpr int SPAN = NM;
    constexpr int nd = decltype(COPY)::value ? ND : 0;
    constexpr int nx = nd + NR;
    constexpr int npair = nd < NR ? nd : NR;  // alternate while both kinds remain
    constexpr int sm = decltype(S_MFMA)::value, sr = decltype(S_READ)::value;
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int u = i / (FM * FN), fm = (i % (FM * FN)) / FN, fn = i % FN;
      if constexpr (decltype(DO_MFMA)::value)
        acc[fm][fn] = MM::mma(fb[sm][u][fn], fa[sm][u][fm], acc[fm][fn]);
#pragma unroll
      for (int x = 0; x < nx; ++x) {
        if (x * SPAN / nx != i) continue;
        if (x < 2 * npair) {
          if (x % 2 == 0) dma_one(wast, wbst, ka, kb, x / 2);
          else fread_one(rast, rbst, sr, x / 2);
        } else if (nd > NR) {
          dma_one(wast, wbst, ka, kb, x - npair);
        } else {
          fread_one(rast, rbst, sr, x - npair);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using T = std::true_type;
  using F = std::false_type;
  (void)sizeof(F);
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto wait_all = [&]() { __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xf << 8)); };  // vmcnt(0)
  // at a trip's end (and after the prologue) all but this wave's last
  // ring::d2_in_flight copies have landed: with three A stages the A copies
  // of the tile two ahead may still fly
  auto wait_in_flight = [&]() {
    constexpr int n = ring::d2_in_flight(SA, A_BLK);
    static_assert(n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
  };

  const int nk = (K + BK - 1) / BK;
  // prologue: tile 0 in stage 0 (and, with SA = 3, A of tile 1 in A stage 1)
  auto prologue_copies = [&]() {
#pragma unroll
    for (int x = 0; x < A_BLK; ++x) dma_a(0, 0, x);
#pragma unroll
    for (int x = 0; x < B_BLK; ++x) dma_b(0, 0, x);
    if constexpr (SA == 3) {
#pragma unroll
      for (int x = 0; x < A_BLK; ++x) dma_a(1, BK, x);
    }
  };
  prologue_copies();
  for (bool first = true;; first = false) {
  // Persistent form: the copies' per-block addresses are recomputed for each
  // tile instead of being hoisted out of the tile loop and held (spilled)
  // across it; an empty asm makes the wave index opaque to that hoisting.
  if constexpr (PERSIST) asm volatile("" : "+s"(wave_u));
  if (first) {
    wait_in_flight();
  } else {
    wait_all();  // the previous tile's C stores count in vmcnt too
  }
  __syncthreads();
  if (!first) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int v = 0; v < MM::NACC; ++v) acc[fm][fn][v] = 0;
  }
  // Trip 0 runs the same body: its "step 1 of the previous tile" MFMAs use
  // zeroed fragments and add exactly 0.
#pragma unroll
  for (int u = 0; u < SPH; ++u) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) fa[1][u][fm] = zero_h8();
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) fb[1][u][fn] = zero_h8();
  }
  for (int kt = 0; kt < nk; ++kt) {
    // tile kt is in A stage tr.ra and B stage tr.rb; this trip copies B of
    // tile kt+1 and A of tile kt+SA-1 into the stages tile kt-1 left
    const ring::Trip tr = ring::d2_trip(kt, SA);
    // first half: step 1 of tile kt-1, the copies, step-0 fragments of tile kt
    half(T{}, T{}, I1{}, I0{}, tr.ra, tr.rb, tr.ta * BK, tr.tb * BK, tr.wa, tr.wb);
    // second half: step 0 of tile kt, step-1 fragments of tile kt
    half(T{}, F{}, I0{}, I1{}, tr.ra, tr.rb, 0, 0, 0, 0);
    wait_in_flight();  // tile kt+1 has landed; with SA = 3 A of kt+2 may fly
    __syncthreads();
  }
  // this output tile's origin (m0, n0 move on to the next tile below)
  const int em0 = m0, en0 = n0;
  bool more = false;
  if constexpr (PERSIST) {
    if (tile + (int)gridDim.x < ntiles_of(tiles_m, tiles_n)) {
      more = true;
      // every fragment read of this tile finished before the last barrier;
      // this wave's copies past the last K tile land before it refills its rows
      wait_all();
      tile += gridDim.x;
      tile_coords(tile, tiles_m, tiles_n, p.group_m, p.xcd_remap, tm, tn);
      m0 = tm * BM;
      n0 = tn * BN;
      rda = raw_rsrc(static_cast<const char*>(p.A) + m0 * lda * EB, (uint32_t)(min(BM, M - m0) * lda * EB));
      rdb = raw_rsrc(static_cast<const char*>(p.B) + n0 * ldb * EB, (uint32_t)(min(BN, N - n0) * ldb * EB));
      prologue_copies();
    }
  }
  // the last tile's step 1 (its fragments were read in the last trip)
#pragma unroll
  for (int u = 0; u < SPH; ++u)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = MM::mma(fb[1][u][fn], fa[1][u][fm], acc[fm][fn]);
  if constexpr (ring::d2_in_flight(SA, A_BLK) > 0) {
    if (!more) wait_all();  // A copies past the last tile drain before exit
  }

  // lane l holds, per MFMA block, output row l % MF and columns
  // g * (256 / MF) + 4 * (l / MF) + e for g < NACC / 4, e < 4
  char* Cw = static_cast<char*>(p.C) + em0 * ldc * CB;
  const auto rsc = make_rsrc(Cw, (uint32_t)(min(BM, M - em0) * ldc * CB));
  bool staged = false;
  if constexpr (SC) {
    static_assert(CB == 2 && MF == 16, "staged epilogue: binary16 C, 16x16 blocks");
    // Each wave owns a private scratch of 16 rows x WTN halves: in A stage 2
    // with three A stages (the next tile's first copies never target it),
    // else at the start of the ring.  16-byte chunks are XORed with row & 7.
    constexpr int SCR_OFF = SA == 3 ? 2 * A_STRIDE : 0;
    constexpr int SCR_HALVES = 16 * WTN;
    static_assert(NW * SCR_HALVES <= (SA == 3 ? A_STRIDE : LDS_HALVES), "staging scratch fits");
    constexpr int CPRW = WTN / 8;        // 16-byte chunks per scratch row
    constexpr int RPI = 64 / CPRW;       // scratch rows per 1 KiB read
    if ((N & 7) == 0) {
      staged = true;
      // every wave's copies past the last K tile have landed (one may target
      // the scratch rows) before any wave writes its scratch
      __syncthreads();
      _Float16* scr = lds + SCR_OFF + wave_u * SCR_HALVES;
      const int srow = lane % 16, squad = lane / 16;
      // With K this short the launch is mostly C traffic: store it non-temporally
      // so the output streams past the caches instead of evicting its own lines.
      const bool c_nt = K <= 128;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          h4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (_Float16)acc[fm][fn][e];
          const int col = fn * MF + 4 * squad;  // in halves, within the wave's columns
          const int ch = (col >> 3) ^ (srow & 7);
          *reinterpret_cast<h4*>(scr + srow * WTN + ch * 8 + (col & 7)) = o;
        }
        // one wave's LDS writes and reads complete in order: the reads below
        // see the writes above, and the next fm's writes follow these reads;
        // the wave barriers keep the compiler from moving either across
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = 0; q < 16 / RPI; ++q) {
          const int r = q * RPI + lane / CPRW, c = lane % CPRW;
          const h8 x = *reinterpret_cast<const h8*>(scr + r * WTN + ((c ^ (r & 7)) * 8));
          const int i = wm * WTM + fm * MF + r;
          const int j = en0 + wn * WTN + c * 8;
          const uint32_t off = j < N ? (uint32_t)((i * ldc + j) * CB) : kOOB;
          if (c_nt)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rsc, off, 0, 2);
          else
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rsc, off, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  if (staged) {
  } else if ((N & 3) == 0) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int i = wm * WTM + fm * MF + lane % MF;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int g = 0; g < MM::NACC / 4; ++g) {
          const int j = en0 + wn * WTN + fn * MF + g * (256 / MF) + 4 * (lane / MF);
          typename Op::acc4_t v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[fm][fn][4 * g + e];
          Op::store4(rsc, j < N ? (uint32_t)((i * ldc + j) * CB) : kOOB, v);
        }
    }
  } else {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int i = wm * WTM + fm * MF + lane % MF;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int g = 0; g < MM::NACC / 4; ++g) {
          const int j = en0 + wn * WTN + fn * MF + g * (256 / MF) + 4 * (lane / MF);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            Op::store1(rsc, j + e < N ? (uint32_t)((i * ldc + j + e) * CB) : kOOB,
                       acc[fm][fn][4 * g + e]);
        }
    }
  }
  if (!more) break;
  }
}
template <int BM, int BN, int WGM, int WGN>
__global__ void __launch_bounds__(64 * WGM * WGN) d2tile_kernel(GemmArgs p) {
  d2tile_body<OpF16, BM, BN, WGM, WGN, 2>(p);
}
template <int BM, int BN, int WGM, int WGN>
__global__ void __launch_bounds__(64 * WGM * WGN) i8_d2tile_kernel(GemmArgs p) {
  d2tile_body<OpI8, BM, BN, WGM, WGN, 2>(p);
}
// Three A stages: A's copies are issued two trips ahead, B's one.
template <int BM, int BN, int WGM, int WGN, int MF>
__global__ void __launch_bounds__(64 * WGM * WGN) d2tile3_kernel(GemmArgs p) {
  d2tile_body<OpF16, BM, BN, WGM, WGN, 3, MF>(p);
}
template <int BM, int BN, int WGM, int WGN>
__global__ void __launch_bounds__(64 * WGM * WGN) i8_d2tile3_kernel(GemmArgs p) {
  d2tile_body<OpI8, BM, BN, WGM, WGN, 3>(p);
}
// d2tile3 as a persistent grid of one workgroup per CU (launch_d2tile3p)
template <int BM, int BN, int WGM, int WGN, int MF>
__global__ void __launch_bounds__(64 * WGM * WGN) d2tile3p_kernel(GemmArgs p) {
  d2tile_body<OpF16, BM, BN, WGM, WGN, 3, MF, true, true>(p);
}
// C staged through LDS for whole-line stores (d2tile_body's SC)
template <int BM, int BN, int WGM, int WGN>
__global__ void __launch_bounds__(64 * WGM * WGN) d2tile3sc_kernel(GemmArgs p) {
  d2tile_body<OpF16, BM, BN, WGM, WGN, 3, 16, true, false, true>(p);
}
template <int BM, int BN, int WGM, int WGN>
__global__ void __launch_bounds__(64 * WGM * WGN) d2tilesc_kernel(GemmArgs p) {
  d2tile_body<OpF16, BM, BN, WGM, WGN, 2, 16, true, false, true>(p);
}


// ---------------------------------------------------------------------------
// Ping-pong family ("pptile"): BM x BN x 64 tiles, 8 waves in two groups of
// four that take turns at the matrix pipes.  Group g owns tile rows
// [g*BM/2, (g+1)*BM/2); its four waves hold (BM/4) x (BN/2) each.  Time is cut
// into slots, each ended by one workgroup barrier; in every slot one group
// runs the MFMAs of one 32-deep K step (at raised wave priority) while the
// other reads the next step's fragments from LDS into registers, so each
// SIMD has one wave feeding its matrix pipe and one doing memory work.  Each
// wave runs the same read / multiply / read / multiply loop, group 1 one
// slot behind group 0, so for K tile t (steps 0 and 1):
//   slot 4t+1: group 0 copies tile t+1 (global -> LDS), reads step 0 of t;
//              group 1 multiplies step 1 of tile t-1
//   slot 4t+2: group 0 multiplies step 0;  group 1 reads step 0
//   slot 4t+3: group 0 reads step 1;       group 1 multiplies step 0
//   slot 4t+4: group 0 multiplies step 1 and waits for its copies of t+1;
//              group 1 reads step 1
// Only group 0 copies; it overwrites a stage (slot 4t+1) only after group 1's
// last read of it (slot 4t), and its copies have landed (end of slot 4t+4)
// before anyone reads them (slot 4t+5).  One step's fragments (48 registers
// at 256 x 256) sit beside 128 accumulators within the 256 registers of a
// wave that shares its SIMD.  LDS layout and copies as in d2tile (128-byte
// rows, chunk XOR (row >> 1) & 7, two LDS stages).
template <int BM, int BN>
__global__ void __launch_bounds__(512)
pptile_kernel(GemmArgs p) {
  using MM = Mfma<16>;
  constexpr int MF = 16, BK = 64, KSTEPS = 2;
  constexpr int WTM = BM / 4, WTN = BN / 2;
  constexpr int FM = WTM / MF, FN = WTN / MF;
  constexpr int A_BLK = BM / 8 / 4, B_BLK = BN / 8 / 4;  // 1 KiB copies per group-0 wave
  constexpr int ND = A_BLK + B_BLK;
  constexpr int STAGE = (BM + BN) * kD2Row;
  static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must hold whole MFMA blocks");
  static_assert(BM % 64 == 0 && BN % 64 == 0, "copy blocks pair up by parity");

  __shared__ __attribute__((aligned(1024))) _Float16 lds[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);
  const int w4 = __builtin_amdgcn_readfirstlane(wave & 3);
  const int wm = w4 >> 1, wn = w4 & 1;
  const int M = p.M, N = p.N, K = p.K;
  int tm, tn;
  tile_coords(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, p.group_m, p.xcd_remap, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t lda = p.lda, ldb = p.ldb, ldc = p.ldc;

  // copies (group 0): lane l -> row l/8 of an 8-row block, physical chunk
  // l%8, which holds logical chunk (l%8) ^ ((l>>4) ^ 4*(block&1))
  const int drow = lane >> 3;
  const int dch0 = (lane & 7) ^ (lane >> 4), dch1 = dch0 ^ 4;
  const u32x4 rda = raw_rsrc(static_cast<const _Float16*>(p.A) + m0 * lda,
                             (uint32_t)(min(BM, M - m0) * lda * 2));
  const u32x4 rdb = raw_rsrc(static_cast<const _Float16*>(p.B) + n0 * ldb,
                             (uint32_t)(min(BN, N - n0) * ldb * 2));
  const uint32_t a_v0 = (uint32_t)(drow * lda * 2 + dch0 * 16), a_v1 = (uint32_t)(drow * lda * 2 + dch1 * 16);
  const uint32_t b_v0 = (uint32_t)(drow * ldb * 2 + dch0 * 16), b_v1 = (uint32_t)(drow * ldb * 2 + dch1 * 16);
  const bool mask_k = (K & 63) != 0;
  const uint32_t lds0 = lds_addr(lds);
  auto dma_one = [&](int st, int k0, int x) {
    const uint32_t kb = (uint32_t)k0 * 2;
    const uint32_t sbase = lds0 + (uint32_t)(st * STAGE * 2);
    if (x < A_BLK) {
      const int blk = w4 * A_BLK + x;
      const int ch = (x & 1) ? dch1 : dch0;
      const bool kin = !mask_k || (k0 + ch * 8 < K);
      dma16(rda, kin ? ((x & 1) ? a_v1 : a_v0) : kOOB, (uint32_t)(blk * 8 * lda * 2) + kb,
            sbase + blk * 8 * kD2Row * 2);
    } else {
      const int xb = x - A_BLK;
      const int blk = w4 * B_BLK + xb;
      const int ch = (xb & 1) ? dch1 : dch0;
      const bool kin = !mask_k || (k0 + ch * 8 < K);
      dma16(rdb, kin ? ((xb & 1) ? b_v1 : b_v0) : kOOB, (uint32_t)(blk * 8 * ldb * 2) + kb,
            sbase + (BM + blk * 8) * kD2Row * 2);
    }
  };

  // fragments: this wave's rows (group half, wave row) at logical chunk 4s + l/16
  const int frow = lane % MF, fq = lane / MF, fsw = (frow >> 1) & 7;
  int fa_off[KSTEPS], fb_off[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const int phys = (4 * s + fq) ^ fsw;
    fa_off[s] = (grp * (BM / 2) + wm * WTM + frow) * kD2Row + phys * 8;
    fb_off[s] = (BM + wn * WTN + frow) * kD2Row + phys * 8;
  }
  h8 fa[FM], fb[FN];  // one step's fragments
  auto fread_one = [&](int st, int s, int r) {  // read r of step s: A then B
    const _Float16* base = lds + st * STAGE;
    if (r < FM)
      fa[r] = *reinterpret_cast<const h8*>(base + fa_off[s] + r * MF * kD2Row);
    else
      fb[r - FM] = *reinterpret_cast<const h8*>(base + fb_off[s] + (r - FM) * MF * kD2Row);
  };

  typename MM::acc_t acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int v = 0; v < MM::NACC; ++v) acc[fm][fn][v] = 0.0f;

  constexpr int NR = FM + FN;
  constexpr int npair = ND < NR ? ND : NR;
  // memory slot: step s's NR fragment reads from stage rst, with (group 0,
  // step 0) the ND copies of the next tile into stage wst; copies and reads
  // alternate while both last
  auto mem = [&](auto S, bool copy, int rst, int kcopy, int wst) {
    constexpr int s = decltype(S)::value;
    if (copy) {
#pragma unroll
      for (int x = 0; x < NR + ND; ++x) {
        if (x < 2 * npair) {
          if (x % 2 == 0) dma_one(wst, kcopy, x / 2);
          else fread_one(rst, s, x / 2);
        } else if (ND > NR) {
          dma_one(wst, kcopy, x - npair);
        } else {
          fread_one(rst, s, x - npair);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < NR; ++r) fread_one(rst, s, r);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // MFMA slot: one step's MFMAs, at raised priority
  auto mfma = [&]() {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = MM::mma(fb[fn], fa[fm], acc[fm][fn]);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  auto wait_all = [&]() { __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xf << 8)); };  // vmcnt(0)

  const int nk = (K + BK - 1) / BK;
  // prologue: group 0 copies tile 0 into stage 0
  if (grp == 0) {
#pragma unroll
    for (int x = 0; x < ND; ++x) dma_one(0, 0, x);
    wait_all();
  }
  __syncthreads();
  // Both groups run the same four-slot loop; group 1 starts one barrier late,
  // which puts it one slot behind group 0 for the whole loop, and group 0
  // ends with one extra barrier so that both pass the same number.
  if (grp == 1) __builtin_amdgcn_s_barrier();
  const bool copier = grp == 0;
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    mem(S0{}, copier && kt + 1 < nk, st, (kt + 1) * BK, st ^ 1);
    __syncthreads();
    mfma();
    __syncthreads();
    mem(S1{}, false, st, 0, 0);
    __syncthreads();
    mfma();
    wait_all();  // group 0: its copies of tile kt+1 have landed
    __syncthreads();
  }
  if (grp == 0) __builtin_amdgcn_s_barrier();

  _Float16* Cw = static_cast<_Float16*>(p.C) + m0 * ldc;
  const auto rsc = make_rsrc(Cw, (uint32_t)(min(BM, M - m0) * ldc * 2));
  if ((N & 3) == 0) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int i = grp * (BM / 2) + wm * WTM + fm * MF + lane % MF;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int j = n0 + wn * WTN + fn * MF + 4 * (lane / MF);
        h4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (_Float16)acc[fm][fn][e];
        buf_store8(rsc, j < N ? (uint32_t)((i * ldc + j) * 2) : kOOB, o);
      }
    }
  } else {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int i = grp * (BM / 2) + wm * WTM + fm * MF + lane % MF;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int j = n0 + wn * WTN + fn * MF + 4 * (lane / MF);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          buf_store2(rsc, j + e < N ? (uint32_t)((i * ldc + j + e) * 2) : kOOB,
                     (_Float16)acc[fm][fn][e]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Full-tile ping-pong family ("pp2tile"): BM x BN tiles whose K tiles are one
// 128-byte row deep (64 binary16 or 128 int8 values), 8 waves in two groups
// of four; every SIMD holds one wave of each group.  Time is cut into
// phases by workgroup barriers.  In each phase one group multiplies a whole K
// tile -- all 2 x FM x FN MFMAs back to back from fragments already in its
// registers, at raised wave priority -- while the other group reads its
// fragments of its next K tile from LDS and issues copies, so each SIMD's
// matrix pipe is fed by one wave that never waits on memory.  ([P1] 正文
// paragraph 3 and 可落地参数清单: producer and consumer warp groups that take
// turns, here without a dedicated producer: each group is both in turn.)
//
// Group 0 owns output rows [0, BM/2), group 1 rows [BM/2, BM); wave w4 of a
// group owns columns [w4 * BN/4, (w4 + 1) * BN/4).  K tile kt is multiplied by
// group 0 in phase 2kt and by group 1 in phase 2kt+1, whose fragments the
// group read in its phase before.  LDS: d2tile3's ring (three A stages, two
// B stages, 128-byte rows, chunk XOR (row >> 1) & 7); A and B are both copied
// two tiles ahead, A by group 1 (in its memory phase 2kt, before its reads)
// and B by group 0 (in phase 2kt+1); ring::pp_trip gives the stages.  Group 1
// ends each memory phase with its previous A tile landed, group 0 each
// compute phase with its previous B tile landed, so tile kt+1 is complete
// before the barrier that opens its first reads (phase 2kt+1).
// SK: the instance splits K (GemmArgs::splitk slices, the shared fix-up);
// without it the slice bookkeeping compiles away.
// Op: the element types (OpF16, OpI8); a K tile is one 128-byte LDS row of
// each operand row (64 binary16 or 128 int8 elements).
template <typename Op, int BM, int BN, bool SC, int MF = 16, bool SK = false>
__device__ __forceinline__ void pp2_body(const GemmArgs& p) {
  using MM = typename Op::template Mma<MF>;
  constexpr int EB = Op::kEB, CB = Op::kCB;
  constexpr int BK = 128 / EB, EPC = 16 / EB;            // K elements per tile and per 16-byte chunk
  constexpr int KSTEPS = BK / MM::KI, CPS = MM::KI / EPC;  // CPS: 16-byte chunks per k-step
  static_assert(!SC || (MF == 16 && CB == 2), "the staged C store takes 16 x 16 binary16 blocks");
  constexpr int WTM = BM / 2, WTN = BN / 4;
  constexpr int FM = WTM / MF, FN = WTN / MF;
  constexpr int A_BLK = BM / 8 / 4, B_BLK = BN / 8 / 4;  // 1 KiB copies per wave of the copying group
  constexpr int A_STRIDE = BM * kD2Row, B_OFF = 3 * BM * kD2Row, B_STRIDE = BN * kD2Row;
  constexpr int LDS_HALVES = 3 * BM * kD2Row + 2 * BN * kD2Row;
  static_assert(LDS_HALVES * 2 <= 160 * 1024, "LDS budget");
  static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must hold whole MFMA blocks");
  static_assert(A_BLK % 2 == 0 && B_BLK % 2 == 0, "copy blocks pair up by parity");

  __shared__ __attribute__((aligned(1024))) _Float16 lds[LDS_HALVES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);
  const int w4 = __builtin_amdgcn_readfirstlane(wave & 3);
  const int M = p.M, N = p.N, K = p.K;
  // split-K: workgroup id = tile * splitk + slice; slice s covers K range
  // [s * kchunk, min(K, (s + 1) * kchunk)), kchunk a multiple of 64
  // (the division runs on the vector unit: its uniform results are moved back
  // to scalar registers, where everything derived from them stays)
  const int splitk = SK ? p.splitk : 1;
  const int tile_id = __builtin_amdgcn_readfirstlane(blockIdx.x / splitk);
  const int slice = __builtin_amdgcn_readfirstlane(blockIdx.x - tile_id * splitk);
  const int k_begin = splitk > 1 ? slice * p.kchunk : 0;
  const int KS = splitk > 1 ? min(p.kchunk, K - k_begin) : K;  // this slice's depth
  int tm, tn;
  tile_coords(tile_id, (M + BM - 1) / BM, (N + BN - 1) / BN, p.group_m, p.xcd_remap, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t lda = p.lda, ldb = p.ldb, ldc = p.ldc;

  // copies: lane l -> row l/8 of an 8-row block, physical chunk l%8, which
  // holds logical chunk (l%8) ^ ((l>>4) ^ 4*(block&1)).  The operand views
  // start at the slice's first k and end where the full rows end.
  const int drow = lane >> 3;
  const int dch0 = (lane & 7) ^ (lane >> 4), dch1 = dch0 ^ 4;
  const u32x4 rda = raw_rsrc(static_cast<const char*>(p.A) + (m0 * lda + k_begin) * EB,
                             (uint32_t)((min(BM, M - m0) * lda - k_begin) * EB));
  const u32x4 rdb = raw_rsrc(static_cast<const char*>(p.B) + (n0 * ldb + k_begin) * EB,
                             (uint32_t)((min(BN, N - n0) * ldb - k_begin) * EB));
  const int64_t ldx = grp == 1 ? lda : ldb;
  const uint32_t v0 = (uint32_t)(drow * ldx * EB + dch0 * 16), v1 = (uint32_t)(drow * ldx * EB + dch1 * 16);
  const bool mask_k = (KS % BK) != 0;
  const uint32_t lds0 = lds_addr(lds);
  // this wave's copies of K tile t: group 1 copies its quarter of A's rows into
  // A stage `st` (copy_a), group 0 its quarter of B's rows into B stage `st`
  // (copy_b); chunks at or past K read 0
  auto copy_a = [&](int st, int t) {
    const uint32_t kb = (uint32_t)(t * BK) * EB;
#pragma unroll
    for (int x = 0; x < A_BLK; ++x) {
      const int ch = (x & 1) ? dch1 : dch0;
      const bool kin = !mask_k || (t * BK + ch * EPC < KS);
      const int blk = w4 * A_BLK + x;
      dma16(rda, kin ? ((x & 1) ? v1 : v0) : kOOB, (uint32_t)(blk * 8 * lda * EB) + kb,
            lds0 + (uint32_t)((st * A_STRIDE + blk * 8 * kD2Row) * 2));
    }
  };
  auto copy_b = [&](int st, int t) {
    const uint32_t kb = (uint32_t)(t * BK) * EB;
#pragma unroll
    for (int x = 0; x < B_BLK; ++x) {
      const int ch = (x & 1) ? dch1 : dch0;
      const bool kin = !mask_k || (t * BK + ch * EPC < KS);
      const int blk = w4 * B_BLK + x;
      dma16(rdb, kin ? ((x & 1) ? v1 : v0) : kOOB, (uint32_t)(blk * 8 * ldb * EB) + kb,
            lds0 + (uint32_t)((B_OFF + st * B_STRIDE + blk * 8 * kD2Row) * 2));
    }
  };

  // fragments of k-step s: the lane's row at logical chunk 4s + l/16
  const int frow = lane % MF, fq = lane / MF, fsw = (frow >> 1) & 7;
  int fa_off[KSTEPS], fb_off[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const int phys = (CPS * s + fq) ^ fsw;
    fa_off[s] = (grp * WTM + frow) * kD2Row + phys * 8;
    fb_off[s] = (w4 * WTN + frow) * kD2Row + phys * 8;
  }
  h8 fa[KSTEPS][FM], fb[KSTEPS][FN];
  auto read_tile = [&](int ast, int bst) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
      for (int q = 0; q < FN; ++q)
        fb[s][q] = *reinterpret_cast<const h8*>(lds + B_OFF + bst * B_STRIDE + fb_off[s] + q * MF * kD2Row);
#pragma unroll
      for (int q = 0; q < FM; ++q)
        fa[s][q] = *reinterpret_cast<const h8*>(lds + ast * A_STRIDE + fa_off[s] + q * MF * kD2Row);
    }
  };

  typename MM::acc_t acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int v = 0; v < MM::NACC; ++v) acc[fm][fn][v] = 0.0f;
  auto multiply = [&]() {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = MM::mma(fb[s][fn], fa[s][fm], acc[fm][fn]);
    __builtin_amdgcn_s_setprio(0);
  };
  auto wait_vm = [&](auto NC) {
    constexpr int n = decltype(NC)::value;
    static_assert(n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
  };
  using InFlightA = std::integral_constant<int, ring::pp_in_flight_a(A_BLK)>;
  using InFlightB = std::integral_constant<int, ring::pp_in_flight_b(B_BLK)>;
  using CopiesA = std::integral_constant<int, A_BLK>;
  using None = std::integral_constant<int, 0>;

  const int nk = (KS + BK - 1) / BK;
  // prologue: group 1 copies A tiles 0 and 1, group 0 B tile 0; tile 0 landed
  if (grp == 1) {
    copy_a(0, 0);
    copy_a(1, 1);
    wait_vm(CopiesA{});
  } else {
    copy_b(0, 0);
    wait_vm(None{});
  }
  __syncthreads();
  // Phases ph = -1 .. 2nk-1, each ended by a barrier.  Group 0 multiplies K
  // tile ph / 2 in the even phases; in the odd ones it copies B tile
  // (ph - 1) / 2 + 2 and reads its fragments of tile (ph + 1) / 2.  Group 1
  // multiplies tile ph / 2 in the odd phases; in the even ones it copies A tile
  // ph / 2 + 2 and reads its fragments of tile ph / 2.  Each group runs its
  // own loop with one multiply and one read site, so that one set of fragment
  // registers is live beside the accumulators.
  if (grp == 0) {
    copy_b(1, 1);  // phase -1: B tile 1, fragments of tile 0
    read_tile(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      multiply();
      wait_vm(InFlightB{});  // B of tile kt+1 has landed
      __syncthreads();
      const ring::Trip tr = ring::pp_trip(kt);
      copy_b(tr.wb, tr.tb);
      if (kt + 1 < nk) {
        const ring::Trip nx = ring::pp_trip(kt + 1);
        read_tile(nx.ra, nx.rb);
      }
      __syncthreads();
    }
  } else {
    __syncthreads();  // phase -1
    for (int kt = 0; kt < nk; ++kt) {
      const ring::Trip tr = ring::pp_trip(kt);
      copy_a(tr.wa, tr.ta);
      read_tile(tr.ra, tr.rb);
      wait_vm(InFlightA{});  // A of tile kt+1 has landed (A of kt+2 may fly)
      __syncthreads();
      multiply();
      __syncthreads();
    }
  }
  wait_vm(None{});  // copies past the last tile drain before the scratch or the exit

  if constexpr (SK) {
    // the flag word reuses LDS word 0 (A stage 0): the fix-up writes it only
    // after a barrier that follows every wave's last fragment read and its
    // drained copies; the staged-C scratch below lies in A stage 2
    if (splitk > 1 && !splitk_fixup<FM, FN, 512, 16, true>(acc, p, tile_id, slice, splitk, tid,
                                                           reinterpret_cast<int*>(lds)))
      return;
  }

  char* Cw = static_cast<char*>(p.C) + m0 * ldc * CB;
  const auto rsc = make_rsrc(Cw, (uint32_t)(min(BM, M - m0) * ldc * CB));
  bool staged = false;
  if constexpr (SC) {
    constexpr int SCR_HALVES = 16 * WTN;
    static_assert(8 * SCR_HALVES <= A_STRIDE, "staging scratch fits in an A stage");
    if ((N & 7) == 0) {
      staged = true;
      __syncthreads();  // every wave's last copies have landed and its reads are done
      store_c_staged<FM, FN, WTN>(acc, lds + 2 * A_STRIDE + wave * SCR_HALVES, rsc, grp * WTM,
                                  n0 + w4 * WTN, N, ldc, lane, K <= 128);
    }
  }
  // lane l holds, per MFMA block, output row l % MF and columns
  // g * (256 / MF) + 4 * (l / MF) + e for g < NACC / 4, e < 4
  if (staged) {
  } else if ((N & 3) == 0) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int i = grp * WTM + fm * MF + lane % MF;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int g = 0; g < MM::NACC / 4; ++g) {
          const int j = n0 + w4 * WTN + fn * MF + g * (256 / MF) + 4 * (lane / MF);
          typename Op::acc4_t v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[fm][fn][4 * g + e];
          Op::store4(rsc, j < N ? (uint32_t)((i * ldc + j) * CB) : kOOB, v);
        }
    }
  } else {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int i = grp * WTM + fm * MF + lane % MF;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int g = 0; g < MM::NACC / 4; ++g) {
          const int j = n0 + w4 * WTN + fn * MF + g * (256 / MF) + 4 * (lane / MF);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            Op::store1(rsc, j + e < N ? (uint32_t)((i * ldc + j + e) * CB) : kOOB,
                       acc[fm][fn][4 * g + e]);
        }
    }
  }
}
template <int BM, int BN, int MF, bool SK = false>
__global__ void __launch_bounds__(512) pp2tile_kernel(GemmArgs p) {
  pp2_body<OpF16, BM, BN, false, MF, SK>(p);
}
template <int BM, int BN, bool SK = false>
__global__ void __launch_bounds__(512) pp2tilesc_kernel(GemmArgs p) {
  pp2_body<OpF16, BM, BN, true, 16, SK>(p);
}
template <int BM, int BN>
__global__ void __launch_bounds__(512) i8_pp2tile_kernel(GemmArgs p) {
  pp2_body<OpI8, BM, BN, false, 16, false>(p);
}

// ---------------------------------------------------------------------------
// Deep-K direct-to-LDS family ("ktile"): BM x BN output tiles with a K step of
// BK = 64*KB per trip (KB = 2 or 4), a ring of S LDS stages (S - 1 tiles of
// copies in flight) and one barrier per trip.  Small tiles stay latency-bound
// per trip, so a deep K step (few trips) is what makes them fast; the trip's
// KSTEPS = 2*KB MFMA steps are pipelined as in d2tile: part j runs the MFMAs
// of step j-1 while it reads the fragments of step j, and part 0 runs the last
// step of the previous tile while it issues the copies of tile k+S-1.
//
// LDS rows hold one tile row's BK halves (128*KB bytes, 8*KB chunks of 16
// bytes); logical chunk c of row r is stored at physical chunk c ^ (r & 15),
// which measured free of bank conflicts for 16x16x32 fragment reads from
// 256- and 512-byte rows.  A copy instruction fills a 1 KiB block of
// RPB = 8/KB rows; lane l lands on row l / (8*KB) of the block, physical
// chunk l % (8*KB), and so loads logical chunk (l % (8*KB)) ^ (row & 15).
// XS = false: unswizzled rows, the "no swizzle" candidate (as in d2tile_body)
template <typename Op, int BM, int BN, int WGM, int WGN, int KB, int S, int SB = S, bool B_NT = false,
          bool XS = true, bool SC = false>
__device__ __forceinline__ void ktile_body(const GemmArgs& p) {
  using MM = typename Op::template Mma<16>;
  constexpr int EB = Op::kEB, CB = Op::kCB;
  constexpr int MF = 16, KSTEPS = 2 * KB;
  constexpr int BK = 128 * KB / EB;        // K elements per trip (128 * KB bytes of a row)
  constexpr int EPC = 16 / EB;             // K elements per 16-byte chunk
  constexpr int ROWH = 64 * KB;            // halves per LDS row
  constexpr int CPR = 8 * KB;              // 16-byte chunks per LDS row
  constexpr int RPB = 1024 / (2 * ROWH);   // rows per 1 KiB copy block
  constexpr int NT = 64 * WGM * WGN, NW = NT / 64;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / MF, FN = WTN / MF;
  constexpr int A_BLK = BM / RPB / NW, B_BLK = BN / RPB / NW;  // copies per wave and trip
  constexpr int ND = A_BLK + B_BLK;
  constexpr int STAGE = (BM + BN) * ROWH;  // halves
  static_assert(KB == 2 || KB == 4, "K step of 128 or 256");
  static_assert(S == 2 || S == 3, "two or three LDS stages");
  static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must hold whole MFMA blocks");
  static_assert(BM % (RPB * NW) == 0 && BN % (RPB * NW) == 0, "copy blocks must split evenly");
  static_assert(BM % 16 == 0, "B's rows start at a multiple of 16 LDS rows");
  // LDS: S stages of A and SB of B.  SB = S: stage s holds A then B rows at
  // s * STAGE.  SB = S - 1: the A ring, then the B ring; A is copied one
  // trip further ahead than B (B's copies go first, see the trip-end wait).
  static_assert(SB == S || SB == S - 1, "B has as many stages as A, or one fewer");
  static_assert(SB >= 2, "at least two B stages");
  constexpr int A_STRIDE = SB == S ? STAGE : BM * ROWH;
  constexpr int B_OFF = SB == S ? BM * ROWH : S * BM * ROWH;
  constexpr int B_STRIDE = SB == S ? STAGE : BN * ROWH;
  constexpr int LDS_HALVES = SB == S ? S * STAGE : S * BM * ROWH + SB * BN * ROWH;
  static_assert(LDS_HALVES * 2 <= 160 * 1024, "LDS budget");
  static_assert(ND * (S - 2) < 64, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) _Float16 lds[LDS_HALVES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int M = p.M, N = p.N, K = p.K;
  // split-K: workgroup id = tile * splitk + slice; slice s covers K range
  // [s * kchunk, min(K, (s + 1) * kchunk)) (kchunk a multiple of 64)
  const int splitk = p.splitk;
  const int tile_id = blockIdx.x / splitk, slice = blockIdx.x - tile_id * splitk;
  const int k_begin = splitk > 1 ? slice * p.kchunk : 0;
  const int k_end = splitk > 1 ? min(K, k_begin + p.kchunk) : K;
  int tm, tn;
  tile_coords(tile_id, (M + BM - 1) / BM, (N + BN - 1) / BN, p.group_m, p.xcd_remap, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t lda = p.lda, ldb = p.ldb, ldc = p.ldc;

  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const u32x4 rda = raw_rsrc(static_cast<const char*>(p.A) + m0 * lda * EB,
                             (uint32_t)(min(BM, M - m0) * lda * EB));
  const u32x4 rdb = raw_rsrc(static_cast<const char*>(p.B) + n0 * ldb * EB,
                             (uint32_t)(min(BN, N - n0) * ldb * EB));
  // per copy x of a trip: this lane's source offset (row and chunk) and the
  // chunk's k offset within the trip
  uint32_t c_off[ND];
  int c_k[ND];
#pragma unroll
  for (int x = 0; x < ND; ++x) {
    const bool is_a = x < A_BLK;
    const int blk = is_a ? wave_u * A_BLK + x : wave_u * B_BLK + (x - A_BLK);
    const int row = blk * RPB + lane / CPR;
    const int c = XS ? (lane % CPR) ^ (row & 15) : lane % CPR;
    c_off[x] = (uint32_t)(row * (is_a ? lda : ldb) * EB + c * 16);
    c_k[x] = c * EPC;
  }
  const bool mask_k = ((k_end - k_begin) % BK) != 0;
  const uint32_t lds0 = lds_addr(lds);
  // k0: the trip's first k (absolute); chunks at or past the slice's end read 0
  // copy xa of A (tile at k0) into A stage ast, copy xb of B into B stage bst
  auto dma_a = [&](int ast, int k0, int xa) {
    const bool kin = !mask_k || (k0 + c_k[xa] < k_end);
    const int blk = wave_u * A_BLK + xa;
    dma16(rda, kin ? c_off[xa] : kOOB, (uint32_t)k0 * EB,
          lds0 + (uint32_t)(ast * A_STRIDE * 2 + blk * 1024));
  };
  auto dma_b = [&](int bst, int k0, int xb) {
    const bool kin = !mask_k || (k0 + c_k[A_BLK + xb] < k_end);
    const int blk = wave_u * B_BLK + xb;
    const uint32_t boff = kin ? c_off[A_BLK + xb] : kOOB;
    const uint32_t blds = lds0 + (uint32_t)((B_OFF + bst * B_STRIDE) * 2 + blk * 1024);
    if constexpr (B_NT) dma16_nt(rdb, boff, (uint32_t)k0 * EB, blds);
    else dma16(rdb, boff, (uint32_t)k0 * EB, blds);
  };
  // copy x of a trip: A's then B's (SB = S), or B's then A's (SB = S - 1)
  auto dma_one = [&](int ast, int bst, int ka, int kb, int x) {
    if constexpr (!ring::k_b_first(S, SB)) {
      if (x < A_BLK) dma_a(ast, ka, x);
      else dma_b(bst, kb, x - A_BLK);
    } else {
      if (x < B_BLK) dma_b(bst, kb, x);
      else dma_a(ast, ka, x - B_BLK);
    }
  };

  // fragments of step s: the lane's row (a multiple of 16 plus lane % 16, so
  // the swizzle term is lane % 16) at logical chunk 4*s + lane / 16
  const int frow = lane % MF, fq = lane / MF;
  int fa_off[KSTEPS], fb_off[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const int phys = XS ? (4 * s + fq) ^ frow : 4 * s + fq;
    fa_off[s] = (wm * WTM + frow) * ROWH + phys * 8;
    fb_off[s] = (BM + wn * WTN + frow) * ROWH + phys * 8;
  }
  h8 fa[2][FM], fb[2][FN];  // [step & 1]
  auto fread_one = [&](int ast, int bst, int s, int r) {
    if (r < FM)
      fa[s & 1][r] = *reinterpret_cast<const h8*>(lds + ast * A_STRIDE + fa_off[s] + r * MF * ROWH);
    else
      fb[s & 1][r - FM] = *reinterpret_cast<const h8*>(lds + B_OFF - BM * ROWH + bst * B_STRIDE +
                                                       fb_off[s] + (r - FM) * MF * ROWH);
  };

  typename MM::acc_t acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int v = 0; v < MM::NACC; ++v) acc[fm][fn][v] = 0;

  constexpr int NM = FM * FN, NR = FM + FN;
  // Part J of a trip: the NM MFMAs of step (J - 1) mod KSTEPS, with the NR
  // fragment reads of step J -- and, in part 0, the copies of the tile S - 1
  // ahead -- spread evenly over the MFMA slots (copies and reads alternate
  // while copies last).
  auto part = [&](auto JC, int rast, int rbst, int ka, int kb, int wast, int wbst) {
    constexpr int J = decltype(JC)::value;
    constexpr int sm = (J + KSTEPS - 1) % KSTEPS;
    constexpr int nd = J == 0 ? ND : 0;
    constexpr int nx = nd + NR;
    constexpr int npair = nd < NR ? nd : NR;  // alternate while both kinds remain
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int fm = i / FN, fn = i % FN;
      acc[fm][fn] = MM::mma(fb[sm & 1][fn], fa[sm & 1][fm], acc[fm][fn]);
#pragma unroll
      for (int x = 0; x < nx; ++x) {
        if (x * NM / nx != i) continue;
        if (x < 2 * npair) {
          if (x % 2 == 0) dma_one(wast, wbst, ka, kb, x / 2);
          else fread_one(rast, rbst, J, x / 2);
        } else if (nd > NR) {
          dma_one(wast, wbst, ka, kb, x - npair);
        } else {
          fread_one(rast, rbst, J, x - npair);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // vmcnt(n) with the other counters left alone (gfx9 encoding)
  auto wait_vm = [&](auto NC) {
    constexpr int n = decltype(NC)::value;
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
  };
  // at a trip's end the copies issued after the next tile's may stay in flight
  using WaitInFlight = std::integral_constant<int, ring::k_in_flight(S, SB, A_BLK, B_BLK)>;
  using WaitAll = std::integral_constant<int, 0>;

  const int nk = (k_end - k_begin + BK - 1) / BK;
  // prologue: A tiles 0 .. S-2 and B tiles 0 .. SB-2 into their stages, tile 0 published
#pragma unroll
  for (int t0 = 0; t0 < S - 1; ++t0) {
#pragma unroll
    for (int x = 0; x < A_BLK; ++x) dma_a(t0, k_begin + t0 * BK, x);
    if (t0 < SB - 1) {
#pragma unroll
      for (int x = 0; x < B_BLK; ++x) dma_b(t0, k_begin + t0 * BK, x);
    }
  }
  wait_vm(WaitInFlight{});
  __syncthreads();
  // trip 0's part 0 runs "the last step of tile -1" on zeroed fragments (adds 0)
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) fa[1][fm] = zero_h8();
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) fb[1][fn] = zero_h8();
  for (int kt = 0; kt < nk; ++kt) {
    const ring::Trip tr = ring::k_trip(kt, S, SB);
    const int ast = tr.ra, bst = tr.rb;
    const int ka = k_begin + tr.ta * BK, kb = k_begin + tr.tb * BK;
    part(std::integral_constant<int, 0>{}, ast, bst, ka, kb, tr.wa, tr.wb);
    part(std::integral_constant<int, 1>{}, ast, bst, 0, 0, 0, 0);
    part(std::integral_constant<int, 2>{}, ast, bst, 0, 0, 0, 0);
    part(std::integral_constant<int, 3>{}, ast, bst, 0, 0, 0, 0);
    if constexpr (KSTEPS == 8) {
      part(std::integral_constant<int, 4>{}, ast, bst, 0, 0, 0, 0);
      part(std::integral_constant<int, 5>{}, ast, bst, 0, 0, 0, 0);
      part(std::integral_constant<int, 6>{}, ast, bst, 0, 0, 0, 0);
      part(std::integral_constant<int, 7>{}, ast, bst, 0, 0, 0, 0);
    }
    wait_vm(WaitInFlight{});  // tile kt+1 has landed (later tiles may still be in flight)
    __syncthreads();
  }
  // the last tile's last step (its fragments were read in the last trip)
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = MM::mma(fb[1][fn], fa[1][fm], acc[fm][fn]);
  wait_vm(WaitAll{});  // copies of tiles past the end are drained before the workgroup exits
  if (splitk > 1) {
    // the fix-up's flag word reuses the first LDS word: the fix-up's first
    // barrier comes after every wave's last fragment read and drained copy
    if (!splitk_fixup<FM, FN, NT>(acc, p, tile_id, slice, splitk, tid, reinterpret_cast<int*>(lds)))
      return;
  }

  char* Cw = static_cast<char*>(p.C) + m0 * ldc * CB;
  const auto rsc = make_rsrc(Cw, (uint32_t)(min(BM, M - m0) * ldc * CB));
  bool staged = false;
  if constexpr (SC) {
    static_assert(CB == 2, "staged epilogue: binary16 C");
    static_assert(NW * 16 * WTN <= LDS_HALVES, "staging scratch fits");
    if ((N & 7) == 0) {
      staged = true;
      // every wave is done with the ring (and with the split-K flag word)
      __syncthreads();
      store_c_staged<FM, FN, WTN>(acc, lds + wave_u * (16 * WTN), rsc, wm * WTM, n0 + wn * WTN, N,
                                  ldc, lane);
    }
  }
  if (staged) {
  } else if ((N & 3) == 0) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int i = wm * WTM + fm * MF + lane % MF;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int j = n0 + wn * WTN + fn * MF + 4 * (lane / MF);
        Op::store4(rsc, j < N ? (uint32_t)((i * ldc + j) * CB) : kOOB, acc[fm][fn]);
      }
    }
  } else {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int i = wm * WTM + fm * MF + lane % MF;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int j = n0 + wn * WTN + fn * MF + 4 * (lane / MF);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Op::store1(rsc, j + e < N ? (uint32_t)((i * ldc + j + e) * CB) : kOOB, acc[fm][fn][e]);
      }
    }
  }
}

template <int BM, int BN, int WGM, int WGN, int KB, int S, int SB>
__global__ void __launch_bounds__(64 * WGM * WGN) ktile_kernel(GemmArgs p) {
  ktile_body<OpF16, BM, BN, WGM, WGN, KB, S, SB>(p);
}
template <int BM, int BN, int WGM, int WGN, int KB, int S, int SB>
__global__ void __launch_bounds__(64 * WGM * WGN) i8_ktile_kernel(GemmArgs p) {
  ktile_body<OpI8, BM, BN, WGM, WGN, KB, S, SB>(p);
}
// unswizzled LDS rows (tuner candidates that measure the XOR layout's worth)
template <int BM, int BN, int WGM, int WGN, int MF>
__global__ void __launch_bounds__(64 * WGM * WGN) d2tile3_ns_kernel(GemmArgs p) {
  d2tile_body<OpF16, BM, BN, WGM, WGN, 3, MF, false>(p);
}
template <int BM, int BN, int WGM, int WGN, int KB, int S, int SB>
__global__ void __launch_bounds__(64 * WGM * WGN) ktile_ns_kernel(GemmArgs p) {
  ktile_body<OpF16, BM, BN, WGM, WGN, KB, S, SB, false, false>(p);
}
// C staged through LDS for whole row-segment stores
template <int BM, int BN, int WGM, int WGN, int KB, int S, int SB>
__global__ void __launch_bounds__(64 * WGM * WGN) ktilesc_kernel(GemmArgs p) {
  ktile_body<OpF16, BM, BN, WGM, WGN, KB, S, SB, false, true, true>(p);
}
// B copied with the non-temporal policy (a tuner candidate for few tile rows)
template <int BM, int BN, int WGM, int WGN, int KB, int S>
__global__ void __launch_bounds__(64 * WGM * WGN) ktile_nt_kernel(GemmArgs p) {
  ktile_body<OpF16, BM, BN, WGM, WGN, KB, S, S, true>(p);
}
template <int BM, int BN, int WGM, int WGN, int KB, int S>
__global__ void __launch_bounds__(64 * WGM * WGN) i8_ktile_nt_kernel(GemmArgs p) {
  ktile_body<OpI8, BM, BN, WGM, WGN, KB, S, S, true>(p);
}

// ---------------------------------------------------------------------------
// Element-wise instance: any alignment, any leading dimensions.  Same
// tiling and arithmetic as the tile family, but every global access is a
// 2-byte access with its own bounds check; it exists for operands outside the
// 16-byte class and as the tuner's reference.
template <typename Op, int BM, int BN, int WGM, int WGN, int MF>
__device__ __forceinline__ void generic_body(const GemmArgs& p) {
  using MM = typename Op::template Mma<MF>;
  using In = typename Op::in_t;
  using Out = typename Op::out_t;
  constexpr int EPC = 16 / Op::kEB;      // elements per 16-byte chunk
  constexpr int BK = 8 * EPC, CPR = 8;   // 128-byte rows of 8 chunks
  constexpr int RH = 64;                 // halves per LDS row
  constexpr int CPS = MM::KI / EPC;      // chunks per MFMA K step
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / MF, FN = WTN / MF;
  constexpr int KSTEPS = BK / MM::KI;
  constexpr int A_IT = BM * CPR / NT, B_IT = BN * CPR / NT;
  static_assert((BM * CPR) % NT == 0 && (BN * CPR) % NT == 0, "tile chunks must split evenly");

  __shared__ __attribute__((aligned(16))) _Float16 lds[(BM + BN) * RH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int M = p.M, N = p.N, K = p.K;
  int tm, tn;
  tile_coords(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, p.group_m, p.xcd_remap, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const In* __restrict__ A = static_cast<const In*>(p.A);
  const In* __restrict__ B = static_cast<const In*>(p.B);
  Out* __restrict__ C = static_cast<Out*>(p.C);
  const int64_t lda = p.lda, ldb = p.ldb, ldc = p.ldc;

  typename MM::acc_t acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int v = 0; v < MM::NACC; ++v) acc[fm][fn][v] = 0;

  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int it = 0; it < A_IT; ++it) {
      const int idx = tid + it * NT, row = idx / CPR, c = idx % CPR;
      const int gm = m0 + row, gk = k0 + c * EPC;
      In v[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) v[e] = (gm < M && gk + e < K) ? A[gm * lda + gk + e] : (In)0;
      *reinterpret_cast<h8*>(lds + row * RH + swz(row, c) * 8) = __builtin_bit_cast(h8, v);
    }
#pragma unroll
    for (int it = 0; it < B_IT; ++it) {
      const int idx = tid + it * NT, row = idx / CPR, c = idx % CPR;
      const int gn = n0 + row, gk = k0 + c * EPC;
      In v[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) v[e] = (gn < N && gk + e < K) ? B[gn * ldb + gk + e] : (In)0;
      *reinterpret_cast<h8*>(lds + BM * RH + row * RH + swz(row, c) * 8) = __builtin_bit_cast(h8, v);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int c = ks * CPS + lane / MF;
      h8 af[FM], bf[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int row = wm * WTM + fm * MF + lane % MF;
        af[fm] = *reinterpret_cast<const h8*>(lds + row * RH + swz(row, c) * 8);
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int row = wn * WTN + fn * MF + lane % MF;
        bf[fn] = *reinterpret_cast<const h8*>(lds + BM * RH + row * RH + swz(row, c) * 8);
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = MM::mma(bf[fn], af[fm], acc[fm][fn]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int i = m0 + wm * WTM + fm * MF + lane % MF;
    if (i >= M) continue;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int g = 0; g < MM::NACC / 4; ++g) {
        const int j = n0 + wn * WTN + fn * MF + g * (256 / MF) + 4 * (lane / MF);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j + e < N) C[i * ldc + j + e] = (Out)acc[fm][fn][4 * g + e];
      }
  }
}

template <int BM, int BN, int WGM, int WGN, int MF>
__global__ void __launch_bounds__(64 * WGM * WGN) generic_kernel(GemmArgs p) {
  generic_body<OpF16, BM, BN, WGM, WGN, MF>(p);
}
template <int BM, int BN, int WGM, int WGN, int MF>
__global__ void __launch_bounds__(64 * WGM * WGN) i8_generic_kernel(GemmArgs p) {
  static_assert(MF == 16, "the int8 MFMA is 16 x 16 x 64");
  generic_body<OpI8, BM, BN, WGM, WGN, MF>(p);
}

// ---------------------------------------------------------------------------
// Skinny family (small M): no LDS staging of operands.  Each workgroup owns a
// (16*FM) x (16*FN) output tile; its WAVES waves take turns over groups of
// UNROLL k-steps and stream A and B fragments straight from global memory
// into registers in the 16x16x32 MFMA layout, one group per load,
// with the next group's loads issued before the current group's MFMAs.  The
// per-wave fp32 partial tiles are summed through LDS in wave order (so the
// result does not depend on timing) and converted once.  B, the large operand
// for these shapes, is read exactly once; A is re-read from L2 by every column
// tile, so wide column tiles split over K (workgroup = tile x slice, the same
// device-coherent fix-up as the direct-to-LDS family, slices summed in order)
// fill the device while cutting that re-read.
// Requires the 16-byte alignment class.
template <int FM, int FN, int WAVES, int UNROLL, int DEPTH = 2>
__global__ void __launch_bounds__(64 * WAVES)
skinny_kernel(GemmArgs p) {
  using MM = Mfma<16>;
  constexpr int BM = 16 * FM, BN = 16 * FN;
  __shared__ __attribute__((aligned(16))) float red[WAVES][BM * BN];

  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = p.M, N = p.N, K = p.K;
  const int tiles_m = (M + BM - 1) / BM;
  // split-K: workgroup id = tile * splitk + slice; slice s covers K range
  // [s * kchunk, min(K, (s + 1) * kchunk)), kchunk a multiple of 64
  const int splitk = p.splitk;
  const int tile_id = blockIdx.x / splitk, slice = blockIdx.x - tile_id * splitk;
  const int tm = tile_id % tiles_m, tn = tile_id / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const _Float16* A = static_cast<const _Float16*>(p.A);
  const _Float16* B = static_cast<const _Float16*>(p.B);
  _Float16* C = static_cast<_Float16*>(p.C);

  const int r = lane & 15, q = lane >> 4;
  // rows beyond M / N fall outside the descriptors' ranges and read as 0
  const auto rsa = make_rsrc(A + m0 * p.lda, (uint32_t)(min(BM, M - m0) * p.lda * 2));
  const auto rsb = make_rsrc(B + n0 * p.ldb, (uint32_t)(min(BN, N - n0) * p.ldb * 2));
  uint32_t a_off[FM], b_off[FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) a_off[fm] = (uint32_t)((fm * 16 + r) * p.lda * 2 + q * 16);
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) b_off[fn] = (uint32_t)((fn * 16 + r) * p.ldb * 2 + q * 16);

  // The slice's k-steps form groups of UNROLL; wave w takes groups w,
  // w + WAVES, ...  so the waves of a workgroup stream neighbouring stretches
  // of the same B rows at the same time.
  const int steps = (K + MM::KI - 1) / MM::KI;
  const int sl_lo = splitk > 1 ? slice * (p.kchunk / MM::KI) : 0;
  const int sl_hi = splitk > 1 ? min(steps, (slice + 1) * (p.kchunk / MM::KI)) : steps;
  const int ngroups = (sl_hi - sl_lo + UNROLL - 1) / UNROLL;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[fm][fn][v] = 0.0f;

  static_assert(DEPTH >= 2 && DEPTH <= 4, "2 to 4 register load groups");
  h8 af[DEPTH][UNROLL][FM], bf[DEPTH][UNROLL][FN];
  auto load = [&](int buf, int s0) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int s = s0 + u;
      const int k = s * MM::KI;
      const bool kin = s < sl_hi && k + q * 8 < K;
      const uint32_t kb = (uint32_t)k * 2;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) af[buf][u][fm] = buf_load16(rsa, kin ? a_off[fm] + kb : kOOB);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) bf[buf][u][fn] = buf_load16(rsb, kin ? b_off[fn] + kb : kOOB);
    }
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = MM::mma(bf[buf][u][fn], af[buf][u][fm], acc[fm][fn]);
  };

  // DEPTH register groups: DEPTH - 1 groups of loads stay in flight while
  // one is computed.  This wave's groups are j = 0, 1, ... (group index
  // wave + j * WAVES); the count is rounded up to a multiple of DEPTH, and
  // groups past the slice read as 0 and add nothing.
  const int mine = wave < ngroups ? (ngroups - wave + WAVES - 1) / WAVES : 0;
  auto grp = [&](int j) { return sl_lo + (wave + j * WAVES) * UNROLL; };
  if (mine > 0) {
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d) load(d, grp(d));
    for (int j = 0; j < mine; j += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        load((d + DEPTH - 1) % DEPTH, grp(j + d + DEPTH - 1));
        compute(d);
      }
    }
  }

  // partial tiles -> LDS, summed in wave order
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        red[wave][(fm * 16 + r) * BN + fn * 16 + 4 * q + v] = acc[fm][fn][v];
  __syncthreads();
  constexpr int NT = 64 * WAVES, NE = BM * BN / 4, EPT = (NE + NT - 1) / NT;
  f32x4 sum[EPT];
#pragma unroll
  for (int t = 0; t < EPT; ++t) {
    const int e = tid + t * NT;
    if (e < NE) {
      const int ii = (e * 4) / BN, jj = (e * 4) % BN;
      f32x4 s = *reinterpret_cast<const f32x4*>(&red[0][ii * BN + jj]);
#pragma unroll
      for (int w = 1; w < WAVES; ++w) s += *reinterpret_cast<const f32x4*>(&red[w][ii * BN + jj]);
      sum[t] = s;
    }
  }
  if (splitk > 1) {
    // Fix-up as in the direct-to-LDS family: partials stored and read with
    // device scope (SC1), the counter a relaxed device-scope atomic taken
    // after every wave's stores are acknowledged; the last slice sums the
    // slices in order 0..splitk-1, writes C and resets the counter.
    const auto rsw = make_rsrc(reinterpret_cast<const f32x4*>(p.ws) + (int64_t)tile_id * splitk * NE,
                               (uint32_t)(splitk * NE * 16));
#pragma unroll
    for (int t = 0; t < EPT; ++t) {
      const int e = tid + t * NT;
      if (e < NE)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sum[t]), rsw,
                                               (uint32_t)((slice * NE + e) * 16), 0, kDeviceScope);
    }
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xf << 8));  // vmcnt(0): partial stores acknowledged
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(&p.cnt[tile_id], 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == splitk - 1;
    __syncthreads();
    if (!s_last) return;
#pragma unroll
    for (int t = 0; t < EPT; ++t) {
      const int e = tid + t * NT;
      if (e < NE) {
        f32x4 total = {0.f, 0.f, 0.f, 0.f};
        for (int s2 = 0; s2 < splitk; ++s2)
          total += s2 == slice
                       ? sum[t]
                       : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rsw, (uint32_t)((s2 * NE + e) * 16), 0,
                                                       kDeviceScope));
        sum[t] = total;
      }
    }
    if (tid == 0)
      __hip_atomic_store(&p.cnt[tile_id], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  _Float16* Cw = C + m0 * p.ldc;
  const auto rsc = make_rsrc(Cw, (uint32_t)(min(BM, M - m0) * p.ldc * 2));
  const bool n_quads = (N & 3) == 0;
#pragma unroll
  for (int t = 0; t < EPT; ++t) {
    const int e = tid + t * NT;
    if (e >= NE) continue;
    const int ii = (e * 4) / BN, jj = (e * 4) % BN;
    const int j = n0 + jj;
    h4 o;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) o[q4] = (_Float16)sum[t][q4];
    const uint32_t off = (uint32_t)((ii * p.ldc + j) * 2);
    if (n_quads) {
      buf_store8(rsc, j < N ? off : kOOB, o);
    } else {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) buf_store2(rsc, j + q4 < N ? off + 2 * q4 : kOOB, o[q4]);
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
template <int BM, int BN, int WGM, int WGN, int MF>
hipError_t launch_tile(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((tile_kernel<BM, BN, WGM, WGN, MF>), dim3((unsigned)g), dim3(64 * WGM * WGN),
                     0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int MF, int S>
hipError_t launch_dtile(const GemmArgs& a, hipStream_t s) {
  const int sk = dtile_splits<BM, BN>() ? a.splitk : 1;
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * sk;
  hipLaunchKernelGGL((dtile_kernel<BM, BN, WGM, WGN, MF, S>), dim3((unsigned)g),
                     dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN>
hipError_t launch_pptile(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((pptile_kernel<BM, BN>), dim3((unsigned)g), dim3(512), 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int MF, bool SK = false>
hipError_t launch_pp2tile(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * (SK ? a.splitk : 1);
  hipLaunchKernelGGL((pp2tile_kernel<BM, BN, MF, SK>), dim3((unsigned)g), dim3(512), 0, s, a);
  return hipGetLastError();
}
template <int BM, int BN>
hipError_t launch_i8_pp2tile(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((i8_pp2tile_kernel<BM, BN>), dim3((unsigned)g), dim3(512), 0, s, a);
  return hipGetLastError();
}
template <int BM, int BN, bool SK = false>
hipError_t launch_pp2tilesc(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * (SK ? a.splitk : 1);
  hipLaunchKernelGGL((pp2tilesc_kernel<BM, BN, SK>), dim3((unsigned)g), dim3(512), 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int KB, int S, int SB>
hipError_t launch_ktile(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * a.splitk;
  hipLaunchKernelGGL((ktile_kernel<BM, BN, WGM, WGN, KB, S, SB>), dim3((unsigned)g),
                     dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}
// Compute units of the current device, read once per process (the persistent
// grids launch one workgroup per CU).
inline int device_cu_count() {
  static const int cus = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    return v;
  }();
  return cus;
}
template <int BM, int BN, int WGM, int WGN, int MF>
hipError_t launch_d2tile3p(const GemmArgs& a, hipStream_t s) {
  const int64_t tiles = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const int64_t g = tiles < device_cu_count() ? tiles : device_cu_count();
  hipLaunchKernelGGL((d2tile3p_kernel<BM, BN, WGM, WGN, MF>), dim3((unsigned)g), dim3(64 * WGM * WGN),
                     0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int KB, int S, int SB>
hipError_t launch_ktilesc(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * a.splitk;
  hipLaunchKernelGGL((ktilesc_kernel<BM, BN, WGM, WGN, KB, S, SB>), dim3((unsigned)g),
                     dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}
template <int BM, int BN, int WGM, int WGN>
hipError_t launch_d2tile3sc(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((d2tile3sc_kernel<BM, BN, WGM, WGN>), dim3((unsigned)g), dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}
template <int BM, int BN, int WGM, int WGN>
hipError_t launch_d2tilesc(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((d2tilesc_kernel<BM, BN, WGM, WGN>), dim3((unsigned)g), dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}
template <int BM, int BN, int WGM, int WGN, int KB, int S, int SB>
hipError_t launch_ktile_ns(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * a.splitk;
  hipLaunchKernelGGL((ktile_ns_kernel<BM, BN, WGM, WGN, KB, S, SB>), dim3((unsigned)g),
                     dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}
template <int BM, int BN, int WGM, int WGN, int MF>
hipError_t launch_d2tile3_ns(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((d2tile3_ns_kernel<BM, BN, WGM, WGN, MF>), dim3((unsigned)g),
                     dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}
template <int BM, int BN, int WGM, int WGN, int KB, int S>
hipError_t launch_ktile_nt(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * a.splitk;
  hipLaunchKernelGGL((ktile_nt_kernel<BM, BN, WGM, WGN, KB, S>), dim3((unsigned)g),
                     dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}
template <int BM, int BN, int WGM, int WGN, int KB, int S>
hipError_t launch_i8_ktile_nt(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * a.splitk;
  hipLaunchKernelGGL((i8_ktile_nt_kernel<BM, BN, WGM, WGN, KB, S>), dim3((unsigned)g),
                     dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN>
hipError_t launch_d2tile(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((d2tile_kernel<BM, BN, WGM, WGN>), dim3((unsigned)g), dim3(64 * WGM * WGN), 0,
                     s, a);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int MF>
hipError_t launch_generic(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((generic_kernel<BM, BN, WGM, WGN, MF>), dim3((unsigned)g),
                     dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int MF>
hipError_t launch_d2tile3(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((d2tile3_kernel<BM, BN, WGM, WGN, MF>), dim3((unsigned)g), dim3(64 * WGM * WGN),
                     0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN>
hipError_t launch_i8_d2tile3(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((i8_d2tile3_kernel<BM, BN, WGM, WGN>), dim3((unsigned)g),
                     dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int KB, int S, int SB>
hipError_t launch_i8_ktile(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * a.splitk;
  hipLaunchKernelGGL((i8_ktile_kernel<BM, BN, WGM, WGN, KB, S, SB>), dim3((unsigned)g),
                     dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN>
hipError_t launch_i8_d2tile(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((i8_d2tile_kernel<BM, BN, WGM, WGN>), dim3((unsigned)g),
                     dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int MF>
hipError_t launch_i8_generic(const GemmArgs& a, hipStream_t s) {
  const int64_t g = (int64_t)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((i8_generic_kernel<BM, BN, WGM, WGN, MF>), dim3((unsigned)g),
                     dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN>
int64_t grid_tile(int32_t M, int32_t N) {
  return (int64_t)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
}

template <int FM, int FN, int WAVES, int UNROLL, int DEPTH = 2>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t s) {
  const int64_t g =
      (int64_t)((a.M + 16 * FM - 1) / (16 * FM)) * ((a.N + 16 * FN - 1) / (16 * FN)) * a.splitk;
  hipLaunchKernelGGL((skinny_kernel<FM, FN, WAVES, UNROLL, DEPTH>), dim3((unsigned)g), dim3(64 * WAVES),
                     0, s, a);
  return hipGetLastError();
}

}  // namespace mihg
