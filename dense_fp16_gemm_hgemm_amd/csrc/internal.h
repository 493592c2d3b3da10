// Internal declarations shared by the kernel translation units and the host
// dispatcher of libmi_hgemm.  Nothing here crosses the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mihg {

// Arguments of one launch.  A is M x K row-major (lda >= K), B is the K x N
// column-major operand stored as N rows of K halves (ldb >= K), C is M x N
// row-major (ldc >= N).  Element pointers are IEEE binary16 (int8 operands
// and int32 results for the int8 instances).
struct GemmArgs {
  const void* A;
  const void* B;
  void* C;
  int64_t lda, ldb, ldc;
  int32_t M, N, K;
  int32_t group_m;    // tile rows per raster group (>= 1)
  int32_t xcd_remap;  // 1: undo the round-robin workgroup -> XCD dispatch
  int32_t splitk;     // K slices per output tile (1: no split)
  int32_t kchunk;     // K elements per slice (a multiple of 64) when splitk > 1
  float* ws;          // split-K partial tiles (splitk > 1)
  int* cnt;           // split-K arrival counters, one per output tile, zero between launches
};

enum Dtype : int32_t {
  DTYPE_F16 = 0,  // binary16 operands and result, fp32 accumulation
  DTYPE_I8 = 1,   // int8 operands, int32 accumulation and result
};

enum Family : int32_t {
  FAMILY_TILE = 0,    // LDS-staged MFMA tiles, double-buffered over K
  FAMILY_SKINNY = 1,  // direct-to-register MFMA, K split across waves
};

// One compiled kernel instance.
struct KernelDesc {
  const char* name;
  int32_t family;
  int32_t bm, bn, bk;  // workgroup tile (skinny: bk = k per MFMA step)
  int32_t waves;       // wavefronts per workgroup
  int32_t mfma;        // 32: v_mfma_f32_32x32x16_f16, 16: v_mfma_f32_16x16x32_f16
  int32_t aligned;     // 1: requires the 16-byte alignment class
  int32_t unroll;      // skinny: MFMA k-steps per load group
  int32_t lds_bytes;
  int32_t splitk_ok;   // 1: honours GemmArgs::splitk > 1
  hipError_t (*launch)(const GemmArgs&, hipStream_t);
  int64_t (*grid)(int32_t M, int32_t N);  // workgroups for an M x N output
  int32_t dtype = DTYPE_F16;
  int32_t split_only = 0;  // 1: a split-K twin of another instance; the tuner times it split only
};

extern const KernelDesc kKernels[];
extern const int kNumKernels;

// Writes +0 to the M x N block of C (K == 0 with beta = 0).
hipError_t launch_zero_fill(void* C, int64_t ldc, int32_t M, int32_t N, hipStream_t s);
// Fills an n-element binary16 buffer with integers in [-4, 4] from a hash of
// (seed, index); used for the tuner's scratch operands.
hipError_t launch_fill_small_int(void* X, int64_t n, uint32_t seed, hipStream_t s);
hipError_t launch_fill_uniform(void* X, int64_t n, uint32_t seed, float scale, hipStream_t s);
// Fills n bytes with int8 values, every byte value equally likely.
hipError_t launch_fill_i8(void* X, int64_t n, uint32_t seed, hipStream_t s);

// Counts the elements of the M x N blocks (leading dimension ld) of two binary16
// arrays whose bit patterns differ, +0 and -0 counted equal; the count is
// written to *d_count (device memory, cleared first on the stream).
hipError_t launch_count_mismatch(const void* X, const void* Y, int32_t M, int32_t N, int64_t ld,
                                 int* d_count, hipStream_t s);
// The same for arrays of 32-bit words, compared bit for bit.
hipError_t launch_count_mismatch32(const void* X, const void* Y, int32_t M, int32_t N, int64_t ld,
                                   int* d_count, hipStream_t s);

}  // namespace mihg
