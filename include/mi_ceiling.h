/*
 * mi_ceiling.h -- C ABI of libmi_ceiling: practical ceilings of one MI355X
 * (gfx950), measured by kernels that do only one kind of work.
 *
 * The GEMM's roofline divides by the published peaks (2516.6 TFLOP/s dense
 * fp16 MFMA, 8 TB/s HBM).  These probes measure what the chip delivers for
 * each kind of work alone, under its own clock and power limits, so that a
 * kernel's time can be set against both:
 *   - mi_ceiling_mfma: back-to-back v_mfma_f32_16x16x32_f16 on operands held
 *     in registers, nothing else; it also counts the shader clock, so the
 *     clock under that load is measured too;
 *   - mi_ceiling_copy_lds: global -> LDS copies (buffer_load_dwordx4 ... lds,
 *     the GEMM tiles' copy instruction) of a contiguous buffer through a
 *     two-stage LDS ring, nothing else;
 *   - mi_ceiling_copy_lds_cycle: the same copies, with the workgroups
 *     cycling through a buffer small enough to stay in L2: the rate at which
 *     one CU can pull operand rows from L2 into its LDS;
 *   - mi_ceiling_read: 16-byte global loads into registers, nothing else (the
 *     streaming read rate of HBM when the buffer exceeds the 256 MiB MALL).
 * "H100 GEMM L2驻留优化：warp-specialized TMA异步拷贝与RL调优策略"
 * (blog.hotdry.top), 回滚策略 / monitoring, watches the tensor-core issue
 * rate and the copy engine's utilisation against targets; these are the
 * gfx950 denominators for the same two quantities.
 *
 * Each probe's result is exact, so a test can check it:
 *   - mfma: workgroup g's wave w (4 waves of 64 lanes per workgroup) holds
 *     NACC = 8 fragment pairs; fragment pair j is read from
 *       frags[((s * 8 + j) * 2 + 0) * 512 + lane * 8 + e]  (the first source)
 *       frags[((s * 8 + j) * 2 + 1) * 512 + lane * 8 + e]  (the second source)
 *     for lane 0..63, e 0..7, with s = (4 g + w) mod 64 (frags holds
 *     64 * 8 * 2 * 512 halves).  It runs `iters` rounds of one MFMA per pair,
 *     accumulating into 8 fp32 accumulators of 4 values per lane, which it
 *     stores at out[(((4 g + w) * 8 + j) * 64 + lane) * 4 + v].  With
 *     integer-valued operands whose block products stay below 2^24 / iters in
 *     magnitude, every value is exactly iters times the 16 x 16 block product
 *     of the operands (in the MFMA operand layout).
 *   - copy_lds, read: out[g] is the XOR of every 32-bit word of workgroup g's
 *     contiguous share of src (bytes / workgroups bytes).
 *   - copy_lds_cycle: with T = bytes / 65536 trips of 64 KiB in src, workgroup
 *     g copies trips (g + t) mod T for t = 0 .. trips-1, and out[g] is the XOR
 *     of every 32-bit word of those trips (a trip copied twice cancels).
 *
 * Conventions: pointers are DEVICE pointers, 16-byte aligned, caller-owned;
 * stream is a hipStream_t as void* (NULL: the null stream); each call
 * enqueues one kernel and returns without synchronising.  Returns 0 on
 * success, 1 for invalid arguments, 2 when the launch failed (the hipError_t
 * is then in *hip_error when non-NULL).
 */
#ifndef MI_CEILING_H
#define MI_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* workgroups >= 1 (256 threads each), iters >= 1.  clocks (device, may be
 * NULL): receives 4 uint64 -- the shader-clock counter and the constant
 * 100 MHz real-time counter, both read by workgroup 0's first wave at its
 * start and at its end (s_memtime, s_memrealtime) -- from which the clock
 * under MFMA load is (c1 - c0) / ((r1 - r0) / 1e8) Hz. */
int mi_ceiling_mfma(const void* frags, int32_t workgroups, int32_t iters, float* out,
                    uint64_t* clocks, void* stream, int* hip_error);

/* bytes a positive multiple of workgroups * 65536, at most 2^40; each
 * workgroup copies its share in 64 KiB trips through a two-stage LDS ring. */
int mi_ceiling_copy_lds(const void* src, int64_t bytes, int32_t workgroups, uint32_t* out,
                        void* stream, int* hip_error);

/* bytes a positive multiple of 65536, at most 2^40; trips >= 1 64 KiB trips
 * per workgroup through the same two-stage LDS ring. */
int mi_ceiling_copy_lds_cycle(const void* src, int64_t bytes, int32_t workgroups, int32_t trips,
                              uint32_t* out, void* stream, int* hip_error);

/* bytes a positive multiple of workgroups * 4096, at most 2^40. */
int mi_ceiling_read(const void* src, int64_t bytes, int32_t workgroups, uint32_t* out,
                    void* stream, int* hip_error);

#ifdef __cplusplus
}
#endif

#endif /* MI_CEILING_H */
