/*
 * mi_overlap.h -- C ABI of libmi_overlap, a load/compute overlap
 * micro-benchmark for AMD Instinct MI355X (gfx950).
 *
 * It measures what the GEMM kernels' copy pipeline buys: how much of the
 * global -> LDS copy time is hidden behind arithmetic, as a function of the
 * arithmetic per loaded element.  This is the copy-versus-compute experiment
 * of "B-08. Hopper TMA：从单线程 Bulk Copy 到吞吐墙" (lqnn.cn), §5 (modes sync,
 * immediate-wait engine copies and a 2-stage prefetch, swept over an
 * arithmetic-intensity knob) and §5.1 (expected shape: the prefetch wins at
 * low intensity and every mode tends to the same time at high intensity),
 * re-designed for gfx950's three ways of filling LDS.
 *
 * The operation (identical in every mode).  The input x of n floats is cut
 * into tiles of 1024 floats (4 KiB); workgroup g of 256 threads owns tiles
 * [g * tiles_per_block, (g + 1) * tiles_per_block).  Each tile is staged
 * through LDS; thread t computes the 4 floats of 16-byte chunk
 * c = (t + 64) mod 256 of its tile (a chunk another wave loaded, so every
 * mode needs the barrier), and for every element
 *
 *     y = x[i];  repeat fma_iters times: y = fmaf(y, alpha, beta);  out[i] = y
 *
 * with fmaf the correctly rounded binary32 fused multiply-add.  So out is
 * a function of x alone, bit-exact across modes.
 *
 * Modes (how a tile reaches LDS):
 *   MI_OVERLAP_SYNC   each thread loads its chunk into VGPRs, writes it to
 *                     LDS, barrier, compute: no overlap (the baseline);
 *   MI_OVERLAP_DIRECT buffer_load ... lds (global -> LDS without VGPRs), wait
 *                     for it at once, barrier, compute: a copy engine path
 *                     with an immediate wait;
 *   MI_OVERLAP_PIPE2  direct-to-LDS copies into a 2-stage ring: tile t+1 is
 *                     in flight while tile t is computed (the GEMM kernels'
 *                     d2tile/ktile pipeline);
 *   MI_OVERLAP_REG2   VGPR-staged prefetch: tile t+1 is loaded into VGPRs
 *                     while tile t is computed, then written to LDS (the
 *                     register-staged tile family's pipeline).
 *
 * Conventions: x and out are DEVICE pointers (caller-owned, 16-byte aligned,
 * not overlapping); n counts floats and must be a positive multiple of
 * 1024 * tiles_per_block; stream is a hipStream_t as void* (NULL: the null
 * stream); the call enqueues one kernel and returns without synchronising.
 */
#ifndef MI_OVERLAP_H
#define MI_OVERLAP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MI_OVERLAP_SYNC = 0,
  MI_OVERLAP_DIRECT = 1,
  MI_OVERLAP_PIPE2 = 2,
  MI_OVERLAP_REG2 = 3
} mi_overlap_mode_t;

/* Returns 0 on success; 1 for invalid arguments (unknown mode, NULL pointers,
 * misaligned pointers, n not a positive multiple of 1024 * tiles_per_block,
 * tiles_per_block < 1, fma_iters < 0, n * 4 bytes beyond 4 GiB); 2 when the
 * kernel launch failed (the hipError_t is then in *hip_error when non-NULL). */
int mi_overlap_run(int mode, const float* x, float* out, int64_t n, int32_t tiles_per_block,
                   int32_t fma_iters, float alpha, float beta, void* stream, int* hip_error);

/* Floats per tile (1024) and threads per workgroup (256). */
int mi_overlap_tile_floats(void);
int mi_overlap_block_threads(void);

#ifdef __cplusplus
}
#endif

#endif /* MI_OVERLAP_H */
