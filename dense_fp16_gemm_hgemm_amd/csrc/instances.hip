// Compiled kernel instances of the TN half-precision GEMM and their registry.
//
// The instance set spans the tuner's search space: workgroup tiles from
// 16 to 256 in M and N, 4 or 8 waves, both gfx950 fp16 MFMA shapes, and the
// skinny direct-to-register family for small M.  Tile sizes start from the
// menus of "H100 GEMM L2驻留优化：warp-specialized TMA异步拷贝与RL调优策略"
// (blog.hotdry.top), 可落地参数清单 (M 64/128, N 64/128 and the 32..512 log-spaced
// search range) and "RL驱动CUDA L2 GEMM内核自动调优：A100/H100 tile size与融合优化"
// (blog.hotdry.top), 正文 paragraph 3 and 落地参数与监控要点 (128x64 and 128x128
// blocks, 4 warps), extended to 256 where the 160 KiB LDS of a gfx950 CU allows.
#include "kernels.hpp"

namespace mihg {

// X-macro lists of the compiled instances.  Each list is expanded twice: into
// explicit instantiations of the kernel templates (both compilation passes, so
// the device code object holds every kernel) and into the registry (host pass).
//   TILE:   X(BM, BN, WGM, WGN, MF)
//   SKINNY: X(FM, FN, WAVES, UNROLL)
// (256 x 256 register-staged tiles with 16x16 MFMAs, or with 4 waves, spill;
// the direct-to-LDS families cover that size.)
#define MIHG_TILE_INSTANCES(X) \
  X(256, 256, 2, 4, 32)          \
  X(128, 128, 2, 2, 16)          \
  X(256, 128, 2, 2, 32)          \
  X(128, 256, 2, 2, 32)          \
  X(256, 128, 4, 2, 32)          \
  X(128, 128, 2, 2, 32)          \
  X(128, 64, 2, 2, 32)           \
  X(64, 128, 2, 2, 32)           \
  X(64, 64, 2, 2, 32)            \
  X(64, 64, 2, 2, 16)            \
  X(32, 64, 1, 4, 16)            \
  X(64, 32, 4, 1, 16)            \
  X(32, 32, 2, 2, 16)            \
  X(16, 64, 1, 2, 16)

#define MIHG_DTILE_INSTANCES(X) \
  X(256, 256, 2, 2, 16, 4)        \
  X(256, 256, 2, 4, 16, 4)        \
  X(256, 128, 2, 2, 16, 4)        \
  X(128, 256, 2, 2, 16, 4)        \
  X(128, 128, 2, 2, 16, 4)

#define MIHG_D2TILE_INSTANCES(X) \
  X(256, 256, 2, 4)               \
  X(256, 256, 2, 2)               \
  X(256, 128, 2, 2)               \
  X(128, 128, 2, 2)               \
  X(128, 64, 2, 2)                \
  X(64, 128, 2, 2)                \
  X(64, 64, 2, 2)

// D2TILE3: X(BM, BN, WGM, WGN, MF): d2tile with three A stages (A copied two
// trips ahead), MFMA 16x16x32 or 32x32x16
#define MIHG_D2TILE3_INSTANCES(X) \
  X(256, 192, 2, 2, 16)           \
  X(256, 256, 2, 4, 16)           \
  X(256, 256, 2, 2, 16)           \
  X(256, 256, 2, 4, 32)           \
  X(256, 256, 2, 2, 32)

// PPTILE: X(BM, BN): eight waves in two ping-pong groups
#define MIHG_PPTILE_INSTANCES(X) \
  X(256, 256)                    \
  X(256, 128)
// PP2TILE: X(BM, BN): two groups taking turns, one whole K tile per turn;
// PP2TILESC: the same with C staged through LDS (wave tiles of 32 or 64 columns)
#define MIHG_PP2TILE_INSTANCES(X) \
  X(256, 256)                     \
  X(256, 192)                     \
  X(256, 128)                     \
  X(128, 256)
#define MIHG_PP2TILESC_INSTANCES(X) \
  X(256, 256)                       \
  X(256, 128)                       \
  X(128, 256)
// PP2TILESK: X(BM, BN): PP2TILESC splitting K (few output tiles, long K)
#define MIHG_PP2TILESK_INSTANCES(X) \
  X(256, 256)                       \
  X(256, 128)

// Int8 variant (int8 operands, int32 results).  I8_D2TILE: X(BM, BN, WGM, WGN),
// K step 128; I8_KTILE: X(BM, BN, WGM, WGN, BK, S), K step BK of 256 or 512.
#define MIHG_I8_D2TILE_INSTANCES(X) \
  X(256, 256, 2, 4)                 \
  X(256, 128, 2, 2)                 \
  X(128, 128, 2, 2)

#define MIHG_I8_D2TILE3_INSTANCES(X) \
  X(256, 256, 2, 4)

// I8_PP2TILE: X(BM, BN): the ping-pong tile on int8 operands (K tile of 128)
#define MIHG_I8_PP2TILE_INSTANCES(X) \
  X(256, 256)                        \
  X(256, 128)

#define MIHG_I8_KTILE_INSTANCES(X) \
  X(128, 128, 2, 4, 256, 2)        \
  X(128, 128, 2, 2, 256, 2)        \
  X(128, 64, 2, 2, 256, 3)         \
  X(64, 128, 2, 2, 256, 3)         \
  X(64, 64, 2, 2, 256, 3)          \
  X(64, 64, 2, 2, 512, 2)          \
  X(32, 64, 2, 2, 256, 3)          \
  X(16, 64, 1, 4, 256, 3)          \
  X(16, 64, 1, 4, 512, 3)

// KTILE_NT: X(BM, BN, WGM, WGN, BK, S) as KTILE, B copied non-temporally; the
// tiles that serve outputs of at most 64 rows, where B is streamed once
#define MIHG_KTILE_NT_INSTANCES(X) \
  X(64, 64, 2, 2, 128, 3)          \
  X(64, 64, 2, 4, 128, 3)          \
  X(32, 64, 2, 4, 128, 3)          \
  X(64, 128, 2, 2, 128, 3)         \
  X(32, 64, 2, 2, 128, 3)          \
  X(16, 64, 1, 4, 256, 3)          \
  X(16, 64, 1, 4, 128, 3)          \
  X(16, 128, 1, 4, 128, 3)         \
  X(16, 16, 1, 1, 256, 3)          \
  X(16, 32, 1, 2, 256, 3)

#define MIHG_I8_KTILE_NT_INSTANCES(X) \
  X(64, 64, 2, 2, 256, 3)             \
  X(32, 64, 2, 2, 256, 3)             \
  X(16, 64, 1, 4, 256, 3)             \
  X(16, 64, 1, 4, 512, 3)

// Unswizzled twins of the large tiles (logical chunk = physical chunk in
// every LDS row): tuner candidates that show what the XOR layout is worth
#define MIHG_D2TILE3_NS_INSTANCES(X) \
  X(256, 256, 2, 2, 16)              \
  X(256, 256, 2, 4, 16)
// Persistent d2tile3 (one workgroup per CU walks the tiles).  Only the 8-wave
// form: the 4-wave one already uses every register, and the tile loop's state
// spills it.
#define MIHG_D2TILE3P_INSTANCES(X) \
  X(256, 256, 2, 4, 16)
// C staged through LDS for whole-line stores (the "_sc" instances)
#define MIHG_D2TILE3SC_INSTANCES(X) \
  X(256, 256, 2, 4)                 \
  X(256, 256, 2, 2)
// (8-wave forms of the small tiles: a CU's global -> LDS copy rate rises
// with the number of waves issuing copies, ~54 GB/s with 4 and ~64 GB/s with
// 8 on L2-resident data, and these tiles are bound by that rate; the
// two-stage 64 x 64 forms fit two workgroups in a CU's LDS.  The staged C
// store needs wave tiles at least 32 columns wide.)
#define MIHG_KTILESC_INSTANCES(X) \
  X(128, 128, 2, 4, 128, 3, 2)     \
  X(128, 128, 2, 2, 128, 3, 2)     \
  X(64, 64, 2, 2, 128, 3, 3)       \
  X(32, 64, 2, 2, 128, 3, 3)       \
  X(64, 64, 4, 2, 128, 3, 3)       \
  X(128, 64, 4, 2, 128, 3, 3)      \
  X(64, 128, 2, 4, 128, 3, 3)      \
  X(64, 64, 2, 2, 128, 2, 2)       \
  X(64, 64, 4, 2, 128, 2, 2)
#define MIHG_D2TILESC_INSTANCES(X) \
  X(128, 128, 2, 2)
#define MIHG_KTILE_NS_B_INSTANCES(X) \
  X(128, 128, 2, 4, 128, 3, 2)

// KTILE_B: X(BM, BN, WGM, WGN, BK, S, SB): S stages of A, SB = S - 1 of B
#define MIHG_KTILE_B_INSTANCES(X) \
  X(128, 128, 2, 2, 128, 3, 2)     \
  X(128, 128, 2, 4, 128, 3, 2)

#define MIHG_I8_KTILE_B_INSTANCES(X) \
  X(128, 128, 2, 2, 256, 3, 2)        \
  X(128, 128, 2, 4, 256, 3, 2)

// KTILE: X(BM, BN, WGM, WGN, BK, S): K step BK (128 or 256), S LDS stages
#define MIHG_KTILE_INSTANCES(X) \
  X(64, 64, 2, 2, 128, 2)        \
  X(64, 64, 2, 2, 128, 3)        \
  X(64, 64, 2, 2, 256, 2)        \
  X(128, 64, 2, 2, 128, 2)       \
  X(64, 128, 2, 2, 128, 2)       \
  X(128, 128, 2, 2, 128, 2)      \
  X(32, 64, 2, 2, 256, 2)        \
  X(16, 64, 1, 4, 256, 2)        \
  X(16, 64, 1, 4, 256, 3)        \
  X(16, 64, 1, 4, 128, 3)        \
  X(16, 128, 1, 4, 128, 3)       \
  X(16, 16, 1, 1, 256, 3)        \
  X(16, 32, 1, 2, 256, 3)        \
  X(32, 64, 2, 2, 128, 3)        \
  X(128, 64, 2, 2, 128, 3)       \
  X(64, 128, 2, 2, 128, 3)       \
  X(128, 128, 2, 4, 128, 2)

#define MIHG_SKINNY_INSTANCES(X) \
  X(1, 1, 4, 4)                  \
  X(1, 1, 8, 4)                  \
  X(1, 2, 4, 4)                  \
  X(1, 2, 8, 4)                  \
  X(1, 4, 4, 2)                  \
  X(2, 1, 8, 4)                  \
  X(2, 2, 4, 4)                  \
  X(4, 1, 4, 4)                  \
  X(4, 1, 8, 2)                  \
  X(4, 2, 4, 2)


#define INSTANTIATE_TILE(BM, BN, WGM, WGN, MF) \
  template __global__ void tile_kernel<BM, BN, WGM, WGN, MF>(GemmArgs);
#define INSTANTIATE_DTILE(BM, BN, WGM, WGN, MF, S) \
  template __global__ void dtile_kernel<BM, BN, WGM, WGN, MF, S>(GemmArgs);
#define INSTANTIATE_D2TILE(BM, BN, WGM, WGN) \
  template __global__ void d2tile_kernel<BM, BN, WGM, WGN>(GemmArgs);
#define INSTANTIATE_D2TILE3(BM, BN, WGM, WGN, MF) \
  template __global__ void d2tile3_kernel<BM, BN, WGM, WGN, MF>(GemmArgs);
#define INSTANTIATE_I8_D2TILE3(BM, BN, WGM, WGN) \
  template __global__ void i8_d2tile3_kernel<BM, BN, WGM, WGN>(GemmArgs);
#define INSTANTIATE_PPTILE(BM, BN) template __global__ void pptile_kernel<BM, BN>(GemmArgs);
#define INSTANTIATE_I8_PP2TILE(BM, BN) template __global__ void i8_pp2tile_kernel<BM, BN>(GemmArgs);
#define INSTANTIATE_PP2TILE(BM, BN) template __global__ void pp2tile_kernel<BM, BN, 16>(GemmArgs);
#define INSTANTIATE_PP2TILESC(BM, BN) template __global__ void pp2tilesc_kernel<BM, BN>(GemmArgs);
#define INSTANTIATE_PP2TILESK(BM, BN) template __global__ void pp2tilesc_kernel<BM, BN, true>(GemmArgs);
#define INSTANTIATE_KTILE(BM, BN, WGM, WGN, BK, S) \
  template __global__ void ktile_kernel<BM, BN, WGM, WGN, BK / 64, S, S>(GemmArgs);
#define INSTANTIATE_KTILE_B(BM, BN, WGM, WGN, BK, S, SB) \
  template __global__ void ktile_kernel<BM, BN, WGM, WGN, BK / 64, S, SB>(GemmArgs);
#define INSTANTIATE_KTILE_NT(BM, BN, WGM, WGN, BK, S) \
  template __global__ void ktile_nt_kernel<BM, BN, WGM, WGN, BK / 64, S>(GemmArgs);
#define INSTANTIATE_I8_KTILE_NT(BM, BN, WGM, WGN, BK, S) \
  template __global__ void i8_ktile_nt_kernel<BM, BN, WGM, WGN, BK / 128, S>(GemmArgs);
#define INSTANTIATE_D2TILE3_NS(BM, BN, WGM, WGN, MF) \
  template __global__ void d2tile3_ns_kernel<BM, BN, WGM, WGN, MF>(GemmArgs);
#define INSTANTIATE_D2TILE3P(BM, BN, WGM, WGN, MF) \
  template __global__ void d2tile3p_kernel<BM, BN, WGM, WGN, MF>(GemmArgs);
#define INSTANTIATE_D2TILE3SC(BM, BN, WGM, WGN) \
  template __global__ void d2tile3sc_kernel<BM, BN, WGM, WGN>(GemmArgs);
#define INSTANTIATE_KTILESC(BM, BN, WGM, WGN, BK, S, SB) \
  template __global__ void ktilesc_kernel<BM, BN, WGM, WGN, BK / 64, S, SB>(GemmArgs);
#define INSTANTIATE_D2TILESC(BM, BN, WGM, WGN) \
  template __global__ void d2tilesc_kernel<BM, BN, WGM, WGN>(GemmArgs);
#define INSTANTIATE_KTILE_NS_B(BM, BN, WGM, WGN, BK, S, SB) \
  template __global__ void ktile_ns_kernel<BM, BN, WGM, WGN, BK / 64, S, SB>(GemmArgs);
#define INSTANTIATE_I8_D2TILE(BM, BN, WGM, WGN) \
  template __global__ void i8_d2tile_kernel<BM, BN, WGM, WGN>(GemmArgs);
#define INSTANTIATE_I8_KTILE(BM, BN, WGM, WGN, BK, S) \
  template __global__ void i8_ktile_kernel<BM, BN, WGM, WGN, BK / 128, S, S>(GemmArgs);
#define INSTANTIATE_I8_KTILE_B(BM, BN, WGM, WGN, BK, S, SB) \
  template __global__ void i8_ktile_kernel<BM, BN, WGM, WGN, BK / 128, S, SB>(GemmArgs);
#define INSTANTIATE_SKINNY(FM, FN, W, U) \
  template __global__ void skinny_kernel<FM, FN, W, U, 2>(GemmArgs);
template __global__ void generic_kernel<64, 64, 2, 2, 32>(GemmArgs);
MIHG_TILE_INSTANCES(INSTANTIATE_TILE)
MIHG_DTILE_INSTANCES(INSTANTIATE_DTILE)
MIHG_D2TILE_INSTANCES(INSTANTIATE_D2TILE)
MIHG_D2TILE3_INSTANCES(INSTANTIATE_D2TILE3)
MIHG_PPTILE_INSTANCES(INSTANTIATE_PPTILE)
MIHG_PP2TILE_INSTANCES(INSTANTIATE_PP2TILE)
MIHG_PP2TILESC_INSTANCES(INSTANTIATE_PP2TILESC)
MIHG_PP2TILESK_INSTANCES(INSTANTIATE_PP2TILESK)
MIHG_KTILE_INSTANCES(INSTANTIATE_KTILE)
MIHG_KTILE_B_INSTANCES(INSTANTIATE_KTILE_B)
MIHG_KTILE_NT_INSTANCES(INSTANTIATE_KTILE_NT)
MIHG_D2TILE3_NS_INSTANCES(INSTANTIATE_D2TILE3_NS)
MIHG_D2TILE3P_INSTANCES(INSTANTIATE_D2TILE3P)
MIHG_D2TILE3SC_INSTANCES(INSTANTIATE_D2TILE3SC)
MIHG_D2TILESC_INSTANCES(INSTANTIATE_D2TILESC)
MIHG_KTILESC_INSTANCES(INSTANTIATE_KTILESC)
MIHG_KTILE_NS_B_INSTANCES(INSTANTIATE_KTILE_NS_B)
MIHG_SKINNY_INSTANCES(INSTANTIATE_SKINNY)
template __global__ void i8_generic_kernel<64, 64, 2, 2, 16>(GemmArgs);
MIHG_I8_D2TILE_INSTANCES(INSTANTIATE_I8_D2TILE)
MIHG_I8_D2TILE3_INSTANCES(INSTANTIATE_I8_D2TILE3)
MIHG_I8_PP2TILE_INSTANCES(INSTANTIATE_I8_PP2TILE)
MIHG_I8_KTILE_INSTANCES(INSTANTIATE_I8_KTILE)
MIHG_I8_KTILE_B_INSTANCES(INSTANTIATE_I8_KTILE_B)
MIHG_I8_KTILE_NT_INSTANCES(INSTANTIATE_I8_KTILE_NT)

// The registry holds host launch functions, so it exists only in the host pass.
#if !defined(__HIP_DEVICE_COMPILE__)
#define TILE_DESC(BM, BN, WGM, WGN, MF)                                                     \
  {"tile_" #BM "x" #BN "_w" #WGM "x" #WGN "_m" #MF, FAMILY_TILE, BM, BN, 64, WGM * WGN, MF, 1, 1, \
   2 * (BM + BN) * kLdsRow * 2, 0, &launch_tile<BM, BN, WGM, WGN, MF>, &grid_tile<BM, BN>},
#define DTILE_DESC(BM, BN, WGM, WGN, MF, S)                                             \
  {"dtile_" #BM "x" #BN "_w" #WGM "x" #WGN "_m" #MF "_s" #S, FAMILY_TILE, BM, BN, 32,       \
   WGM * WGN, MF, 1, 1, 4 * (BM + BN) * kDRow * 2, dtile_splits<BM, BN>() ? 1 : 0,          \
   &launch_dtile<BM, BN, WGM, WGN, MF, S>,                                                   \
   &grid_tile<BM, BN>},
#define D2TILE_DESC(BM, BN, WGM, WGN)                                                     \
  {"d2tile_" #BM "x" #BN "_w" #WGM "x" #WGN "_m16", FAMILY_TILE, BM, BN, 64, WGM * WGN, 16, 1, \
   1, 2 * (BM + BN) * kD2Row * 2, 0, &launch_d2tile<BM, BN, WGM, WGN>, &grid_tile<BM, BN>},
#define D2TILE3_DESC(BM, BN, WGM, WGN, MF)                                                  \
  {"d2tile3_" #BM "x" #BN "_w" #WGM "x" #WGN "_m" #MF, FAMILY_TILE, BM, BN, 64, WGM * WGN, MF, \
   1, 1, (3 * BM + 2 * BN) * kD2Row * 2, 0, &launch_d2tile3<BM, BN, WGM, WGN, MF>,              \
   &grid_tile<BM, BN>},
#define I8_D2TILE3_DESC(BM, BN, WGM, WGN)                                                    \
  {"i8_d2tile3_" #BM "x" #BN "_w" #WGM "x" #WGN "_m16", FAMILY_TILE, BM, BN, 128, WGM * WGN,   \
   16, 1, 1, (3 * BM + 2 * BN) * kD2Row * 2, 0, &launch_i8_d2tile3<BM, BN, WGM, WGN>,          \
   &grid_tile<BM, BN>, DTYPE_I8},
#define I8_PP2TILE_DESC(BM, BN)                                                            \
  {"i8_pp2tile_" #BM "x" #BN "_w8_m16", FAMILY_TILE, BM, BN, 128, 8, 16, 1, 1,                \
   (3 * BM + 2 * BN) * kD2Row * 2, 0, &launch_i8_pp2tile<BM, BN>, &grid_tile<BM, BN>,         \
   DTYPE_I8},
#define PPTILE_DESC(BM, BN)                                                                \
  {"pptile_" #BM "x" #BN "_w8_m16", FAMILY_TILE, BM, BN, 64, 8, 16, 1, 1,                     \
   2 * (BM + BN) * kD2Row * 2, 0, &launch_pptile<BM, BN>, &grid_tile<BM, BN>},
#define PP2TILE_DESC(BM, BN)                                                               \
  {"pp2tile_" #BM "x" #BN "_w8_m16", FAMILY_TILE, BM, BN, 64, 8, 16, 1, 1,                    \
   (3 * BM + 2 * BN) * kD2Row * 2, 0, &launch_pp2tile<BM, BN, 16>, &grid_tile<BM, BN>},
#define PP2TILESC_DESC(BM, BN)                                                             \
  {"pp2tile_" #BM "x" #BN "_w8_m16_sc", FAMILY_TILE, BM, BN, 64, 8, 16, 1, 1,                 \
   (3 * BM + 2 * BN) * kD2Row * 2, 0, &launch_pp2tilesc<BM, BN>, &grid_tile<BM, BN>},
#define PP2TILESK_DESC(BM, BN)                                                             \
  {"pp2tile_" #BM "x" #BN "_w8_m16_sc_sk", FAMILY_TILE, BM, BN, 64, 8, 16, 1, 1,              \
   (3 * BM + 2 * BN) * kD2Row * 2, 1, &launch_pp2tilesc<BM, BN, true>, &grid_tile<BM, BN>,   \
   DTYPE_F16, 1},
#define KTILE_DESC(BM, BN, WGM, WGN, BK, S)                                                 \
  {"ktile_" #BM "x" #BN "_w" #WGM "x" #WGN "_k" #BK "_s" #S, FAMILY_TILE, BM, BN, BK,          \
   WGM * WGN, 16, 1, 1, S * (BM + BN) * BK * 2, 1,                                             \
   &launch_ktile<BM, BN, WGM, WGN, BK / 64, S, S>, &grid_tile<BM, BN>},
#define KTILE_B_DESC(BM, BN, WGM, WGN, BK, S, SB)                                             \
  {"ktile_" #BM "x" #BN "_w" #WGM "x" #WGN "_k" #BK "_s" #S "b" #SB, FAMILY_TILE, BM, BN, BK,   \
   WGM * WGN, 16, 1, 1, (S * BM + SB * BN) * BK * 2, 1,                                        \
   &launch_ktile<BM, BN, WGM, WGN, BK / 64, S, SB>, &grid_tile<BM, BN>},
#define KTILE_NT_DESC(BM, BN, WGM, WGN, BK, S)                                              \
  {"ktile_" #BM "x" #BN "_w" #WGM "x" #WGN "_k" #BK "_s" #S "_nt", FAMILY_TILE, BM, BN, BK,     \
   WGM * WGN, 16, 1, 1, S * (BM + BN) * BK * 2, 1,                                             \
   &launch_ktile_nt<BM, BN, WGM, WGN, BK / 64, S>, &grid_tile<BM, BN>},
#define I8_KTILE_NT_DESC(BM, BN, WGM, WGN, BK, S)                                           \
  {"i8_ktile_" #BM "x" #BN "_w" #WGM "x" #WGN "_k" #BK "_s" #S "_nt", FAMILY_TILE, BM, BN, BK, \
   WGM * WGN, 16, 1, 1, S * (BM + BN) * BK, 1,                                                 \
   &launch_i8_ktile_nt<BM, BN, WGM, WGN, BK / 128, S>, &grid_tile<BM, BN>, DTYPE_I8},
#define D2TILE3_NS_DESC(BM, BN, WGM, WGN, MF)                                               \
  {"d2tile3_" #BM "x" #BN "_w" #WGM "x" #WGN "_m" #MF "_noxor", FAMILY_TILE, BM, BN, 64,       \
   WGM * WGN, MF, 1, 1, (3 * BM + 2 * BN) * kD2Row * 2, 0,                                     \
   &launch_d2tile3_ns<BM, BN, WGM, WGN, MF>, &grid_tile<BM, BN>},
#define D2TILE3P_DESC(BM, BN, WGM, WGN, MF)                                                 \
  {"d2tile3p_" #BM "x" #BN "_w" #WGM "x" #WGN "_m" #MF, FAMILY_TILE, BM, BN, 64, WGM * WGN, MF, \
   1, 1, (3 * BM + 2 * BN) * kD2Row * 2, 0, &launch_d2tile3p<BM, BN, WGM, WGN, MF>,             \
   &grid_tile<BM, BN>},
#define D2TILE3SC_DESC(BM, BN, WGM, WGN)                                                    \
  {"d2tile3_" #BM "x" #BN "_w" #WGM "x" #WGN "_m16_sc", FAMILY_TILE, BM, BN, 64, WGM * WGN, 16,  \
   1, 1, (3 * BM + 2 * BN) * kD2Row * 2, 0, &launch_d2tile3sc<BM, BN, WGM, WGN>,              \
   &grid_tile<BM, BN>},
#define KTILESC_DESC(BM, BN, WGM, WGN, BK, S, SB)                                              \
  {"ktile_" #BM "x" #BN "_w" #WGM "x" #WGN "_k" #BK "_s" #S "b" #SB "_sc", FAMILY_TILE, BM, BN,  \
   BK, WGM * WGN, 16, 1, 1, (S * BM + SB * BN) * BK * 2, 1,                                     \
   &launch_ktilesc<BM, BN, WGM, WGN, BK / 64, S, SB>, &grid_tile<BM, BN>},
#define D2TILESC_DESC(BM, BN, WGM, WGN)                                                     \
  {"d2tile_" #BM "x" #BN "_w" #WGM "x" #WGN "_m16_sc", FAMILY_TILE, BM, BN, 64, WGM * WGN, 16,   \
   1, 1, 2 * (BM + BN) * kD2Row * 2, 0, &launch_d2tilesc<BM, BN, WGM, WGN>, &grid_tile<BM, BN>},
#define KTILE_NS_B_DESC(BM, BN, WGM, WGN, BK, S, SB)                                          \
  {"ktile_" #BM "x" #BN "_w" #WGM "x" #WGN "_k" #BK "_s" #S "b" #SB "_noxor", FAMILY_TILE, BM, \
   BN, BK, WGM * WGN, 16, 1, 1, (S * BM + SB * BN) * BK * 2, 1,                                 \
   &launch_ktile_ns<BM, BN, WGM, WGN, BK / 64, S, SB>, &grid_tile<BM, BN>},
#define I8_D2TILE_DESC(BM, BN, WGM, WGN)                                                    \
  {"i8_d2tile_" #BM "x" #BN "_w" #WGM "x" #WGN "_m16", FAMILY_TILE, BM, BN, 128, WGM * WGN, 16, \
   1, 1, 2 * (BM + BN) * kD2Row * 2, 0, &launch_i8_d2tile<BM, BN, WGM, WGN>,                   \
   &grid_tile<BM, BN>, DTYPE_I8},
#define I8_KTILE_DESC(BM, BN, WGM, WGN, BK, S)                                                 \
  {"i8_ktile_" #BM "x" #BN "_w" #WGM "x" #WGN "_k" #BK "_s" #S, FAMILY_TILE, BM, BN, BK,        \
   WGM * WGN, 16, 1, 1, S * (BM + BN) * BK, 1,                                                 \
   &launch_i8_ktile<BM, BN, WGM, WGN, BK / 128, S, S>, &grid_tile<BM, BN>, DTYPE_I8},
#define I8_KTILE_B_DESC(BM, BN, WGM, WGN, BK, S, SB)                                           \
  {"i8_ktile_" #BM "x" #BN "_w" #WGM "x" #WGN "_k" #BK "_s" #S "b" #SB, FAMILY_TILE, BM, BN,   \
   BK, WGM * WGN, 16, 1, 1, (S * BM + SB * BN) * BK, 1,                                        \
   &launch_i8_ktile<BM, BN, WGM, WGN, BK / 128, S, SB>, &grid_tile<BM, BN>, DTYPE_I8},
#define SKINNY_DESC(FM, FN, W, U)                                                          \
  {"skinny_" #FM "x" #FN "_w" #W "_u" #U, FAMILY_SKINNY, 16 * FM, 16 * FN, 32, W, 16, 1, U, \
   W * 16 * FM * 16 * FN * 4, 1, &launch_skinny<FM, FN, W, U, 2>, &grid_tile<16 * FM, 16 * FN>},

const KernelDesc kKernels[] = {
    // element-wise instance: any alignment, any leading dimensions (must stay first)
    {"generic_64x64_w2x2_m32", FAMILY_TILE, 64, 64, 64, 4, 32, 0, 1, 128 * 64 * 2, 0,
     &launch_generic<64, 64, 2, 2, 32>, &grid_tile<64, 64>},
    MIHG_TILE_INSTANCES(TILE_DESC)
    MIHG_DTILE_INSTANCES(DTILE_DESC)
    MIHG_D2TILE_INSTANCES(D2TILE_DESC)
    MIHG_D2TILE3_INSTANCES(D2TILE3_DESC)
    MIHG_PPTILE_INSTANCES(PPTILE_DESC)
    MIHG_PP2TILE_INSTANCES(PP2TILE_DESC)
    MIHG_PP2TILESC_INSTANCES(PP2TILESC_DESC)
    MIHG_PP2TILESK_INSTANCES(PP2TILESK_DESC)
    MIHG_KTILE_INSTANCES(KTILE_DESC)
    MIHG_KTILE_B_INSTANCES(KTILE_B_DESC)
    MIHG_KTILE_NT_INSTANCES(KTILE_NT_DESC)
    MIHG_D2TILE3_NS_INSTANCES(D2TILE3_NS_DESC)
    MIHG_D2TILE3P_INSTANCES(D2TILE3P_DESC)
    MIHG_D2TILE3SC_INSTANCES(D2TILE3SC_DESC)
    MIHG_D2TILESC_INSTANCES(D2TILESC_DESC)
    MIHG_KTILESC_INSTANCES(KTILESC_DESC)
    MIHG_KTILE_NS_B_INSTANCES(KTILE_NS_B_DESC)
    MIHG_SKINNY_INSTANCES(SKINNY_DESC)
    // int8 variant: element-wise instance first, then the vector-load tiles
    {"i8_generic_64x64_w2x2_m16", FAMILY_TILE, 64, 64, 128, 4, 16, 0, 1, 128 * 64 * 2, 0,
     &launch_i8_generic<64, 64, 2, 2, 16>, &grid_tile<64, 64>, DTYPE_I8},
    MIHG_I8_D2TILE_INSTANCES(I8_D2TILE_DESC)
    MIHG_I8_D2TILE3_INSTANCES(I8_D2TILE3_DESC)
    MIHG_I8_PP2TILE_INSTANCES(I8_PP2TILE_DESC)
    MIHG_I8_KTILE_INSTANCES(I8_KTILE_DESC)
    MIHG_I8_KTILE_B_INSTANCES(I8_KTILE_B_DESC)
    MIHG_I8_KTILE_NT_INSTANCES(I8_KTILE_NT_DESC)
};

const int kNumKernels = (int)(sizeof(kKernels) / sizeof(kKernels[0]));
#endif

// ---------------------------------------------------------------------------
__global__ void zero_fill_kernel(_Float16* C, int64_t ldc, int32_t M, int32_t N) {
  const int64_t total = (int64_t)M * N;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = t / N, j = t - i * N;
    C[i * ldc + j] = (_Float16)0.0f;
  }
}

hipError_t launch_zero_fill(void* C, int64_t ldc, int32_t M, int32_t N, hipStream_t s) {
  const int64_t total = (int64_t)M * N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<_Float16*>(C), ldc, M, N);
  return hipGetLastError();
}

__device__ inline uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

__global__ void fill_small_int_kernel(_Float16* X, int64_t n, uint32_t seed) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n;
       t += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t h = mix32((uint32_t)t ^ mix32(seed ^ (uint32_t)(t >> 32)));
    X[t] = (_Float16)(float)((int)(h % 9u) - 4);
  }
}

hipError_t launch_fill_small_int(void* X, int64_t n, uint32_t seed, hipStream_t s) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_small_int_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<_Float16*>(X), n, seed);
  return hipGetLastError();
}

// Values uniform in (-scale, scale) with full random mantissas: timing
// operands whose switching activity (and so power draw and clock) matches
// real data, unlike the small integers used for the exactness check.
__global__ void fill_uniform_kernel(_Float16* X, int64_t n, uint32_t seed, float scale) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n;
       t += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t h = mix32((uint32_t)t ^ mix32(seed ^ (uint32_t)(t >> 32)));
    X[t] = (_Float16)(scale * ((float)(h >> 8) * (2.0f / 16777216.0f) - 1.0f));
  }
}

hipError_t launch_fill_uniform(void* X, int64_t n, uint32_t seed, float scale, hipStream_t s) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_uniform_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<_Float16*>(X), n, seed, scale);
  return hipGetLastError();
}

// Int8 operands with every byte value equally likely: both the exactness check
// and the timing data of the int8 variant (integer products are exact).
__global__ void fill_i8_kernel(int8_t* X, int64_t n, uint32_t seed) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n;
       t += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t h = mix32((uint32_t)t ^ mix32(seed ^ (uint32_t)(t >> 32)));
    X[t] = (int8_t)(h >> 24);
  }
}

hipError_t launch_fill_i8(void* X, int64_t n, uint32_t seed, hipStream_t s) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_i8_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<int8_t*>(X), n, seed);
  return hipGetLastError();
}

__global__ void count_mismatch32_kernel(const uint32_t* X, const uint32_t* Y, int32_t M,
                                        int32_t N, int64_t ld, int* count) {
  const int64_t total = (int64_t)M * N;
  int bad = 0;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = t / N, j = t - i * N;
    bad += X[i * ld + j] != Y[i * ld + j];
  }
  if (bad) atomicAdd(count, bad);
}

hipError_t launch_count_mismatch32(const void* X, const void* Y, int32_t M, int32_t N, int64_t ld,
                                   int* d_count, hipStream_t s) {
  hipError_t e = hipMemsetAsync(d_count, 0, sizeof(int), s);
  if (e != hipSuccess) return e;
  const int64_t total = (int64_t)M * N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(count_mismatch32_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const uint32_t*>(X), static_cast<const uint32_t*>(Y), M, N, ld,
                     d_count);
  return hipGetLastError();
}

__global__ void count_mismatch_kernel(const uint16_t* X, const uint16_t* Y, int32_t M, int32_t N,
                                      int64_t ld, int* count) {
  const int64_t total = (int64_t)M * N;
  int bad = 0;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = t / N, j = t - i * N;
    const uint16_t x = X[i * ld + j], y = Y[i * ld + j];
    bad += (x != y) && (((x | y) & 0x7fff) != 0);
  }
  if (bad) atomicAdd(count, bad);
}

hipError_t launch_count_mismatch(const void* X, const void* Y, int32_t M, int32_t N, int64_t ld,
                                 int* d_count, hipStream_t s) {
  hipError_t e = hipMemsetAsync(d_count, 0, sizeof(int), s);
  if (e != hipSuccess) return e;
  const int64_t total = (int64_t)M * N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(count_mismatch_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(Y), M, N, ld,
                     d_count);
  return hipGetLastError();
}

}  // namespace mihg
