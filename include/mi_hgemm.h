/*
 * mi_hgemm.h -- C ABI of libmi_hgemm, a half-precision GEMM for AMD Instinct
 * MI355X (gfx950).
 *
 * The operation.  For 0 <= i < M and 0 <= j < N:
 *
 *     C[i*ldc + j] = fp16_rne( sum_{k=0}^{K-1} A[i*lda + k] * B[j*ldb + k] )
 *
 * A is an M x K row-major matrix, B a K x N column-major matrix (stored as N
 * columns of K contiguous halves), C an M x N row-major matrix; all three hold
 * IEEE binary16.  Products are accumulated in binary32 on the matrix cores and
 * the sum is rounded once to binary16, round-to-nearest-even, overflow to
 * infinity.  alpha = 1 and beta = 0: C is only written.  This is the TN
 * half-precision GEMM of "RL驱动CUDA L2 GEMM内核自动调优：A100/H100 tile
 * size与融合优化" (blog.hotdry.top, 2025-12-05), 正文 paragraph 1 (HGEMM) and
 * paragraph 3 (row-major A, column-major B, the kernel family named ...TN), and
 * of the per-shape tile/pipeline/swizzle search of "H100 GEMM L2驻留优化：
 * warp-specialized TMA异步拷贝与RL调优策略" (blog.hotdry.top), 正文 paragraph 4
 * and 可落地参数清单, which here is mi_hgemm_tune.  In torch terms C = A @ Bt.T
 * where Bt is the [N, K] storage of B (the nn.Linear weight layout).
 *
 * Conventions for every function:
 *   - Pointers named A, B, C are DEVICE pointers on the handle's device; the
 *     caller owns them.  Sizes and leading dimensions count elements.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued on it and the call returns without synchronising; a device
 *     fault surfaces at the caller's next synchronisation.
 *   - Nothing is allocated per call by mi_hgemm_run.  No exception crosses the
 *     ABI; every failure is a status code.
 *   - A handle may be shared by threads calling mi_hgemm_run / mi_hgemm_plan
 *     concurrently, provided their launches are ordered on one stream: a
 *     handle owns one split-K workspace (below), so launches of one handle
 *     that may run at the same time on different streams must use separate
 *     handles.  mi_hgemm_tune and mi_hgemm_destroy need exclusive use.
 *   - Split-K: a handle created on a device allocates, once, a 64 MiB device
 *     workspace for fp32 partial tiles and a table of per-tile counters.  For
 *     shapes whose output tiles alone cannot occupy the device, the dispatcher
 *     may split K into slices; the last slice to finish sums the partial
 *     tiles in slice order (deterministic) and writes C.
 */
#ifndef MI_HGEMM_H
#define MI_HGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MI_HGEMM_VERSION_MAJOR 0
#define MI_HGEMM_VERSION_MINOR 2

typedef struct mi_hgemm_ctx* mi_hgemm_handle_t;

/* Only the TN layout (A row-major, B column-major) is provided. */
typedef enum { MI_HGEMM_LAYOUT_TN = 0 } mi_hgemm_layout_t;

typedef enum {
  MI_HGEMM_OK = 0,
  MI_HGEMM_ERR_INVALID_ARG = 1,   /* null handle/pointer, negative size, ld too small, C overlapping A or B */
  MI_HGEMM_ERR_UNSUPPORTED = 2,   /* layout other than TN, a size above INT32_MAX, no instance for the shape */
  MI_HGEMM_ERR_NO_DEVICE = 3,     /* no gfx950 device (or an inspection-only handle asked to launch) */
  MI_HGEMM_ERR_HIP = 4,           /* a HIP call failed; see mi_hgemm_last_hip_error */
  MI_HGEMM_ERR_IO = 5,            /* a table file could not be written */
  MI_HGEMM_WARN_TABLE_DEFAULTS = 6 /* handle created, but the named table was missing or had bad lines */
} mi_hgemm_status_t;

/* Flags of mi_hgemm_create_ex. */
#define MI_HGEMM_CREATE_NO_DEVICE 1u  /* inspection handle: tables and dispatch only, no launches */

/* Flags of mi_hgemm_tune. */
#define MI_HGEMM_TUNE_EXHAUSTIVE 1u   /* every compiled instance x raster setting (default) */
#define MI_HGEMM_TUNE_HEURISTIC 2u    /* a pruned candidate list around the built-in choice */
#define MI_HGEMM_TUNE_PERSIST 4u      /* append the winner to the handle's table file */
#define MI_HGEMM_TUNE_INT8 8u         /* tune the int8 variant (mi_hgemm_run_i8) for the shape */

/*
 * Create a handle on the current HIP device.
 *   table_path: shape->config table to load.  NULL: the path in the
 *     MI_HGEMM_TABLE environment variable, else the table shipped next to the
 *     library (tables/gfx950.tsv), else built-in heuristics only.
 * Returns OK, WARN_TABLE_DEFAULTS (a named table is missing or has malformed
 * lines: valid lines are kept, heuristics cover the rest), NO_DEVICE (the
 * current device is not gfx950 or there is none), or INVALID_ARG (out NULL).
 * On OK and WARN_TABLE_DEFAULTS *out holds a handle to release with
 * mi_hgemm_destroy; otherwise *out is NULL.
 */
mi_hgemm_status_t mi_hgemm_create(mi_hgemm_handle_t* out, const char* table_path);

/* As mi_hgemm_create; with MI_HGEMM_CREATE_NO_DEVICE no device is needed and
 * the handle supports mi_hgemm_plan and the table functions only. */
mi_hgemm_status_t mi_hgemm_create_ex(mi_hgemm_handle_t* out, const char* table_path,
                                     uint32_t flags);

/* Release a handle (NULL is a no-op).  Waits for nothing: the caller must not
 * destroy a handle whose launches may still read its scratch memory. */
mi_hgemm_status_t mi_hgemm_destroy(mi_hgemm_handle_t h);

/*
 * C = A * B as defined at the top of this file, enqueued on `stream`.
 *   M, N, K >= 0.  M == 0 or N == 0: OK, nothing is done.  K == 0: C is set
 *   to +0 (beta = 0), by a fill kernel on the stream.
 *   lda >= max(K,1), ldb >= max(K,1), ldc >= max(N,1).
 *   A, B, C must be non-NULL when their extent is non-empty, and C's extent
 *   must not overlap A's or B's (INVALID_ARG).
 * Alignment: operands in the 16-byte class (A, B, C 16-byte aligned; lda, ldb,
 * ldc multiples of 8 and at most 2^21; K a multiple of 8) run the vector-load
 * kernels; anything else runs the element-wise instance with the same
 * arithmetic.  Misalignment is never an error.
 * Returns OK, INVALID_ARG, UNSUPPORTED, NO_DEVICE or ERR_HIP (launch failed).
 */
mi_hgemm_status_t mi_hgemm_run(mi_hgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                               const void* A, int64_t lda, const void* B, int64_t ldb,
                               void* C, int64_t ldc, mi_hgemm_layout_t layout, void* stream);

/*
 * The int8 variant: for 0 <= i < M and 0 <= j < N,
 *
 *     C[i*ldc + j] = sum_{k=0}^{K-1} A[i*lda + k] * B[j*ldb + k]
 *
 * with A (M x K, row-major) and B (K x N, column-major) of int8_t and C
 * (M x N, row-major) of int32_t; the sum is exact.  This is the INT8 mode of
 * the pages' multi-precision scheduling ("RL驱动CUDA L2 GEMM内核自动调优：
 * A100/H100 tile size与融合优化" (blog.hotdry.top, 2025-12-05), 正文
 * paragraph 3: FP16/INT8 switching, with the K tile doubled under INT8 to
 * use the higher peak).  The pages leave the result type open; int32 is
 * taken, so that the result is exact (v_mfma_i32_16x16x64_i8 accumulates in
 * int32).  The K step of every int8 instance is twice its fp16 sibling's in
 * elements (the same bytes per LDS row).
 *   Arguments, sizes, leading dimensions (in elements), the empty-output and
 *   overlap rules and the return codes are those of mi_hgemm_run; K == 0
 *   writes 0.  K > 131071 returns UNSUPPORTED (beyond it the int32 sum of
 *   (-128)*(-128) products can overflow).
 * Alignment: the 16-byte class is A, B, C 16-byte aligned, K, lda, ldb
 * multiples of 16, ldc a multiple of 4, every ld at most 2^21; anything else
 * runs the element-wise int8 instance.  Misalignment is never an error.
 * Split-K partial tiles are int32, summed in slice order (exact in any order).
 */
mi_hgemm_status_t mi_hgemm_run_i8(mi_hgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                  const void* A, int64_t lda, const void* B, int64_t ldb,
                                  void* C, int64_t ldc, mi_hgemm_layout_t layout, void* stream);

/*
 * Search the compiled instances, raster settings and K splits for the shape
 * (M, N, K) in the 16-byte alignment class.  Each candidate is first run on
 * library-owned small-integer operands, on which every correct candidate gives
 * C bit-identical to the element-wise instance's (a candidate that differs is
 * discarded); it is then timed on operands with random mantissas scaled by
 * 1/sqrt(K) (the clock under load depends on the data), as the median of 5
 * replays of a captured graph of repeated launches on a private stream; the
 * three fastest are then re-timed in three interleaved rounds and the lowest
 * median over each one's 15 replays wins.  The
 * launches rotate over enough copies of the operands and of the output to
 * overflow the 256 MiB MALL (at most 64 copies and 4 GiB), so each reads its
 * operands from HBM and writes its C past the MALL, as in real use.  The fastest correct one becomes the handle's entry for the shape.
 * With MI_HGEMM_TUNE_PERSIST the entry is appended to the handle's table file.
 * With MI_HGEMM_TUNE_INT8 the int8 instances are searched instead (K a
 * multiple of 16 and at most 131071); their check and timing operands are
 * uniform random int8 and the reference is the element-wise int8 instance.
 * Synchronises `stream`.  Allocates scratch (the operand sets and two
 * outputs, freed before returning).  With the environment variable
 * MI_HGEMM_TUNE_LOG set (and not "0"), every timed candidate is printed to
 * stderr as one line: M N K kernel g<group_m> x<xcd_remap> s<split> µs, and
 * each finalist as "final M N K kernel g x s median .. min .. max ..".
 * Returns OK, INVALID_ARG, UNSUPPORTED, NO_DEVICE, ERR_HIP or ERR_IO.
 */
mi_hgemm_status_t mi_hgemm_tune(mi_hgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                mi_hgemm_layout_t layout, void* stream, uint32_t flags);

/* Human-readable name of a status. Never NULL. */
const char* mi_hgemm_status_string(mi_hgemm_status_t s);

/* The hipError_t of the handle's last failed HIP call (0 if none). */
int mi_hgemm_last_hip_error(mi_hgemm_handle_t h);

/* Number of compiled kernel instances, and the name of instance `index`
 * (NULL when out of range).  Instance 0 is the element-wise (any alignment) one. */
int mi_hgemm_kernel_count(void);
const char* mi_hgemm_kernel_name(int index);

/*
 * What mi_hgemm_run would launch for these arguments, without launching:
 * validates exactly as mi_hgemm_run and writes the instance index, raster
 * group height, XCD remap flag and requested K split (any output pointer may
 * be NULL).  *kernel_index is -1 when no kernel would run (empty C, K == 0).
 * Works on inspection handles; device pointers are only compared, never read.
 */
mi_hgemm_status_t mi_hgemm_plan(mi_hgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                const void* A, int64_t lda, const void* B, int64_t ldb,
                                const void* C, int64_t ldc, mi_hgemm_layout_t layout,
                                int32_t* kernel_index, int32_t* group_m, int32_t* xcd_remap,
                                int32_t* split_k);

/* mi_hgemm_plan for mi_hgemm_run_i8's arguments. */
mi_hgemm_status_t mi_hgemm_plan_i8(mi_hgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                   const void* A, int64_t lda, const void* B, int64_t ldb,
                                   const void* C, int64_t ldc, mi_hgemm_layout_t layout,
                                   int32_t* kernel_index, int32_t* group_m, int32_t* xcd_remap,
                                   int32_t* split_k);

/*
 * mi_hgemm_run with a forced instance, raster setting and K split (tests,
 * benchmarks, external tuners).  Validation as mi_hgemm_run, plus
 * UNSUPPORTED when the instance needs the 16-byte class and the operands are
 * not in it, kernel_index is out of range, split_k > 1 is asked of an
 * instance without split-K, or the partial tiles exceed the workspace.
 * group_m >= 1; xcd_remap 0 or 1; 1 <= split_k <= 64 (the effective split may
 * be smaller: slices are whole multiples of 64 in K).  Instances whose name
 * starts with "i8_" are int8 instances: their operands, result and checks are
 * those of mi_hgemm_run_i8.
 */
mi_hgemm_status_t mi_hgemm_run_kernel(mi_hgemm_handle_t h, int32_t kernel_index,
                                      int32_t group_m, int32_t xcd_remap, int32_t split_k,
                                      int64_t M, int64_t N, int64_t K,
                                      const void* A, int64_t lda, const void* B, int64_t ldb,
                                      void* C, int64_t ldc, mi_hgemm_layout_t layout,
                                      void* stream);

/*
 * mi_hgemm_run for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, validation, dispatch, alignment rules and return codes are those
 * of mi_hgemm_run, and the call allocates nothing (device or host).  The one
 * difference is where a split-K launch keeps its fp32 partial tiles and its
 * per-tile arrival counters: not in the handle's workspace but in a static
 * device array of the library, MI_HGEMM_NOALLOC_PARTIAL_BYTES of partials and
 * MI_HGEMM_NOALLOC_TILE_COUNTERS counters.  Each device holds its own copy of
 * the array until the process ends; its address is resolved and its counters
 * cleared when the first handle is created on that device (ERR_HIP here if
 * that failed; mi_hgemm_last_hip_error says why).
 *   - A planned K split whose partial tiles do not fit the array is halved
 *     until they do (split 1 needs no scratch), so no shape is refused for
 *     lack of scratch, and no launch is issued with more partials or counters
 *     than the array holds (UNSUPPORTED if one would be).  With a different
 *     split the sum is the same; for non-integer operands its rounding may
 *     differ from mi_hgemm_run's within the tolerance of the operation.
 *   - Every call on a device shares that device's array, which keeps the last
 *     call's partials; the counters are back at zero after every launch.
 *     Calls on one device that may overlap in time (different streams, or
 *     threads without ordering) race on the array: order them on one stream.
 */
#define MI_HGEMM_NOALLOC_PARTIAL_BYTES (16u << 20)
#define MI_HGEMM_NOALLOC_TILE_COUNTERS 4096
mi_hgemm_status_t mi_hgemm_run_noalloc(mi_hgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                       const void* A, int64_t lda, const void* B, int64_t ldb,
                                       void* C, int64_t ldc, mi_hgemm_layout_t layout,
                                       void* stream);

/* Number of (shape -> config) entries the handle holds. */
int mi_hgemm_table_size(mi_hgemm_handle_t h);

/* Write the handle's entries to `path` in the table format (ERR_IO on failure). */
mi_hgemm_status_t mi_hgemm_table_save(mi_hgemm_handle_t h, const char* path);

#ifdef __cplusplus
}
#endif

#endif /* MI_HGEMM_H */
