// Load/compute overlap micro-benchmark for gfx950 (the C ABI and the
// operation are specified in include/mi_overlap.h).
//
// "B-08. Hopper TMA：从单线程 Bulk Copy 到吞吐墙" (lqnn.cn) §5 compares a
// cooperative synchronous tile load, engine copies waited on at once, and a
// 2-stage prefetch, over a sweep of FMA iterations per element.  On gfx950
// the three ways of filling LDS are: VGPR-staged (global_load, ds_write),
// direct-to-LDS (buffer_load ... lds, completion tracked by vmcnt) and the
// prefetching forms of both.  Each mode here is one of them, with the same
// tile (1024 floats, 4 KiB), the same arithmetic and the same output.
#include <hip/hip_runtime.h>

#include "../../include/mi_overlap.h"

namespace {

constexpr int kTile = 1024;     // floats per tile
constexpr int kThreads = 256;   // 4 waves; one 16-byte chunk per thread per tile
constexpr int kRsrcWord3 = 0x00020000;

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ inline u32x4 raw_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = (uint32_t)a;
  r[1] = (uint32_t)(a >> 32) & 0xffffu;
  r[2] = bytes;
  r[3] = (uint32_t)kRsrcWord3;
  return r;
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

// one wave-wide copy: lane l's 16 bytes at voff + soff land at LDS byte lds + 16 l
__device__ inline void dma16(const u32x4& rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory", "m0");
}

__device__ inline void wait_vm0() { __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xf << 8)); }

__device__ inline f4 chain(f4 v, int iters, float alpha, float beta) {
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(v[e], alpha, beta);
  }
  return v;
}

template <int MODE>
__global__ void __launch_bounds__(kThreads) overlap_kernel(const float* x, float* out, int tpb,
                                                           int iters, float alpha, float beta,
                                                           uint32_t nbytes) {
  __shared__ __attribute__((aligned(16))) float lds[2][kTile];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int rc = (tid + 64) & (kThreads - 1);  // the chunk this thread computes
  const int64_t first = (int64_t)blockIdx.x * tpb;
  const auto rin = make_rsrc(x, nbytes);
  const auto rout = make_rsrc(out, nbytes);
  const u32x4 rdma = raw_rsrc(x, nbytes);
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uint64_t>(&lds[0][0]);
  auto tile_byte = [&](int t) { return (uint32_t)((first + t) * kTile * 4); };
  auto load_vgpr = [&](int t) {
    return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(
                                      rin, tile_byte(t) + (uint32_t)tid * 16, 0, 0));
  };
  // wave w copies chunks 64w .. 64w+63 of tile t into stage st
  auto load_direct = [&](int t, int st) {
    dma16(rdma, (uint32_t)tid * 16, tile_byte(t),
          lds0 + (uint32_t)(st * kTile * 4 + wave * 1024));
  };
  auto compute_store = [&](int t, int st) {
    const f4 v = *reinterpret_cast<const f4*>(&lds[st][rc * 4]);
    const f4 y = chain(v, iters, alpha, beta);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, y), rout,
                                           tile_byte(t) + (uint32_t)rc * 16, 0, 0);
  };

  if constexpr (MODE == MI_OVERLAP_SYNC) {
    for (int t = 0; t < tpb; ++t) {
      const f4 v = load_vgpr(t);
      *reinterpret_cast<f4*>(&lds[0][tid * 4]) = v;
      __syncthreads();
      compute_store(t, 0);
      __syncthreads();
    }
  } else if constexpr (MODE == MI_OVERLAP_DIRECT) {
    for (int t = 0; t < tpb; ++t) {
      load_direct(t, 0);
      wait_vm0();
      __syncthreads();
      compute_store(t, 0);
      __syncthreads();
    }
  } else if constexpr (MODE == MI_OVERLAP_PIPE2) {
    // Iteration t: wait for every earlier copy and store (tile t landed),
    // barrier (every wave has finished reading tile t-1, whose stage the next
    // copy reuses), issue tile t+1's copy, then compute tile t while it flies.
    load_direct(0, 0);
    for (int t = 0; t < tpb; ++t) {
      wait_vm0();
      __syncthreads();
      if (t + 1 < tpb) load_direct(t + 1, (t + 1) & 1);
      compute_store(t, t & 1);
    }
    wait_vm0();
  } else {  // MI_OVERLAP_REG2
    f4 next = load_vgpr(0);
    for (int t = 0; t < tpb; ++t) {
      const int st = t & 1;
      *reinterpret_cast<f4*>(&lds[st][tid * 4]) = next;
      __syncthreads();
      if (t + 1 < tpb) next = load_vgpr(t + 1);  // in flight during the compute
      compute_store(t, st);
    }
  }
}

template <int MODE>
hipError_t launch(const float* x, float* out, int64_t n, int tpb, int iters, float a, float b,
                  hipStream_t s) {
  const int64_t blocks = n / ((int64_t)kTile * tpb);
  hipLaunchKernelGGL(overlap_kernel<MODE>, dim3((unsigned)blocks), dim3(kThreads), 0, s, x, out,
                     tpb, iters, a, b, (uint32_t)(n * 4));
  return hipGetLastError();
}

}  // namespace

extern "C" int mi_overlap_run(int mode, const float* x, float* out, int64_t n,
                              int32_t tiles_per_block, int32_t fma_iters, float alpha,
                              float beta, void* stream, int* hip_error) {
  if (hip_error) *hip_error = 0;
  if (mode < MI_OVERLAP_SYNC || mode > MI_OVERLAP_REG2 || !x || !out || tiles_per_block < 1 ||
      fma_iters < 0 || n <= 0 || n % ((int64_t)kTile * tiles_per_block) != 0 ||
      n * 4 > (int64_t)UINT32_MAX || (reinterpret_cast<uintptr_t>(x) & 15) ||
      (reinterpret_cast<uintptr_t>(out) & 15))
    return 1;
  const uintptr_t x0 = reinterpret_cast<uintptr_t>(x), o0 = reinterpret_cast<uintptr_t>(out);
  if (x0 < o0 + (uintptr_t)n * 4 && o0 < x0 + (uintptr_t)n * 4) return 1;
  if (n / ((int64_t)kTile * tiles_per_block) > INT32_MAX) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (mode) {
    case MI_OVERLAP_SYNC: e = launch<MI_OVERLAP_SYNC>(x, out, n, tiles_per_block, fma_iters, alpha, beta, s); break;
    case MI_OVERLAP_DIRECT: e = launch<MI_OVERLAP_DIRECT>(x, out, n, tiles_per_block, fma_iters, alpha, beta, s); break;
    case MI_OVERLAP_PIPE2: e = launch<MI_OVERLAP_PIPE2>(x, out, n, tiles_per_block, fma_iters, alpha, beta, s); break;
    default: e = launch<MI_OVERLAP_REG2>(x, out, n, tiles_per_block, fma_iters, alpha, beta, s); break;
  }
  if (e != hipSuccess) {
    if (hip_error) *hip_error = (int)e;
    return 2;
  }
  return 0;
}

extern "C" int mi_overlap_tile_floats(void) { return kTile; }
extern "C" int mi_overlap_block_threads(void) { return kThreads; }
