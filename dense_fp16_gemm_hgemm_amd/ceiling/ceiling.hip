// Practical ceilings of gfx950: kernels that do one kind of work only (the C
// ABI and the exact results are specified in include/mi_ceiling.h).
//
// The GEMM kernels do three things at once: MFMAs, global -> LDS copies and
// LDS -> register fragment reads.  Each probe here does one of them at the
// fastest rate the hardware sustains under its clock and power limits, so that
// a kernel's time can be compared with what its dominant unit delivers alone,
// beside the published peaks.
#include <hip/hip_runtime.h>

#include "../../include/mi_ceiling.h"

namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kNacc = 8;       // independent accumulators (MFMA chains) per wave
constexpr int kSets = 64;      // distinct operand sets, one per wave modulo 64
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kTrip = 65536;   // bytes per workgroup and copy trip

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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

// lane l's 16 bytes at voff + soff land at LDS byte address lds + 16 l
__device__ inline void dma16(const u32x4& rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory", "m0");
}

__device__ inline uint32_t wave_xor(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v ^= __shfl_xor(v, o);
  return v;
}

// kNacc MFMA chains per wave, `iters` rounds of one MFMA per chain.
__global__ void __launch_bounds__(kThreads) mfma_kernel(const _Float16* frags, int iters,
                                                        float* out, uint64_t* clocks) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int set = gw % kSets;
  h8 a[kNacc], b[kNacc];
  f32x4 acc[kNacc];
#pragma unroll
  for (int j = 0; j < kNacc; ++j) {
    const _Float16* p = frags + ((set * kNacc + j) * 2) * 512 + lane * 8;
    a[j] = *reinterpret_cast<const h8*>(p);
    b[j] = *reinterpret_cast<const h8*>(p + 512);
    acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bool timer = clocks != nullptr && blockIdx.x == 0 && threadIdx.x == 0;
  uint64_t c0 = 0, r0 = 0;
  if (timer) {
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  // 16 rounds per loop trip (the rest one round at a time)
  int it = 0;
  for (; it + 16 <= iters; it += 16) {
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
      for (int j = 0; j < kNacc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j], b[j], acc[j], 0, 0, 0);
  }
  for (; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kNacc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j], b[j], acc[j], 0, 0, 0);
  }
  if (timer) {
    // the last MFMAs' results are needed before the clocks are read again
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kNacc; ++j) s += acc[j][0];
    asm volatile("" ::"v"(s));
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    clocks[0] = c0;
    clocks[1] = r0;
    clocks[2] = c1;
    clocks[3] = r1;
  }
#pragma unroll
  for (int j = 0; j < kNacc; ++j)
    *reinterpret_cast<f32x4*>(out + (((int64_t)gw * kNacc + j) * 64 + lane) * 4) = acc[j];
}

// Workgroup g copies `trips` 64 KiB trips into a two-stage LDS ring: trip t
// is trip (g * first_stride + t) mod ntrips of src.  Trip t+1 is in flight
// while trip t is read back and folded into a running XOR.  Wave w copies
// 16 KiB of each trip: 1 KiB blocks 16w .. 16w+15.  With first_stride = trips
// every workgroup streams its own contiguous share once; with a small src and
// first_stride = 1 the workgroups cycle through a buffer that stays in L2.
__global__ void __launch_bounds__(kThreads) copy_lds_kernel(const char* src, int64_t ntrips,
                                                            int64_t first_stride, int trips,
                                                            uint32_t* out) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * kTrip];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int64_t first = (int64_t)blockIdx.x * first_stride;
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uint64_t>(&lds[0]);
  auto issue = [&](int t) {
    // one descriptor per trip keeps every offset below 2^32 whatever the buffer
    const u32x4 r = raw_rsrc(src + ((first + t) % ntrips) * kTrip, (uint32_t)kTrip);
    const int st = t & 1;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int blk = wave * 16 + x;
      dma16(r, (uint32_t)((tid & 63) * 16), (uint32_t)(blk * 1024),
            lds0 + (uint32_t)(st * kTrip + blk * 1024));
    }
  };
  uint32_t acc = 0;
  issue(0);
  for (int t = 0; t < trips; ++t) {
    if (t + 1 < trips) {
      issue(t + 1);
      // vmcnt(16) (gfx9 encoding: count bits 3:0 and 15:14): trip t has landed
      __builtin_amdgcn_s_waitcnt((16 & 15) | ((16 >> 4) << 14) | (0x7 << 4) | (0xf << 8));
    } else {
      __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xf << 8));  // vmcnt(0)
    }
    __syncthreads();
    // every lane folds the 16-byte pieces it copied itself
    const char* st = lds + (t & 1) * kTrip;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(st + (wave * 16 + x) * 1024 + (tid & 63) * 16);
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    __syncthreads();  // trip t's stage is refilled by trip t+2 only after every wave read it
  }
  acc = wave_xor(acc);
  if ((tid & 63) == 0) atomicXor(out + blockIdx.x, acc);
}

// Workgroup g reads its `share` bytes with 16-byte loads (4 loads in flight per
// lane per step) and folds them into a running XOR.
__global__ void __launch_bounds__(kThreads) read_kernel(const char* src, int64_t share,
                                                        uint32_t* out) {
  const int tid = threadIdx.x;
  const char* base = src + (int64_t)blockIdx.x * share;
  constexpr int kStep = kThreads * 16 * 4;  // bytes per workgroup and step
  uint32_t acc = 0;
  for (int64_t off = 0; off < share; off += kStep) {
    const int64_t chunk = share - off < kStep ? share - off : kStep;
    const auto r = make_rsrc(base + off, (uint32_t)chunk);
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           r, (uint32_t)((u * kThreads + tid) * 16), 0, 0));
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  acc = wave_xor(acc);
  if ((tid & 63) == 0) atomicXor(out + blockIdx.x, acc);
}

__global__ void zero_kernel(uint32_t* out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launched(int* hip_error) {
  const hipError_t e = hipGetLastError();
  if (hip_error) *hip_error = (int)e;
  return e == hipSuccess ? 0 : 2;
}

}  // namespace

extern "C" {

int mi_ceiling_mfma(const void* frags, int32_t workgroups, int32_t iters, float* out,
                    uint64_t* clocks, void* stream, int* hip_error) {
  if (hip_error) *hip_error = 0;
  if (!frags || !out || workgroups < 1 || iters < 1 || !aligned16(frags) || !aligned16(out) ||
      (clocks && (reinterpret_cast<uintptr_t>(clocks) & 7u)))
    return 1;
  hipLaunchKernelGGL(mfma_kernel, dim3((unsigned)workgroups), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const _Float16*>(frags), iters,
                     out, clocks);
  return launched(hip_error);
}

int mi_ceiling_copy_lds(const void* src, int64_t bytes, int32_t workgroups, uint32_t* out,
                        void* stream, int* hip_error) {
  if (hip_error) *hip_error = 0;
  if (!src || !out || workgroups < 1 || bytes < 1 || bytes > (int64_t(1) << 40) ||
      bytes % ((int64_t)workgroups * kTrip) != 0 || !aligned16(src))
    return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((workgroups + 255) / 256)), dim3(256), 0, s, out,
                     workgroups);
  if (launched(hip_error)) return 2;
  const int64_t per_wg = bytes / workgroups / kTrip;
  if (per_wg > INT32_MAX) return 1;
  hipLaunchKernelGGL(copy_lds_kernel, dim3((unsigned)workgroups), dim3(kThreads), 0, s,
                     static_cast<const char*>(src), bytes / kTrip, per_wg, (int)per_wg, out);
  return launched(hip_error);
}

int mi_ceiling_copy_lds_cycle(const void* src, int64_t bytes, int32_t workgroups, int32_t trips,
                              uint32_t* out, void* stream, int* hip_error) {
  if (hip_error) *hip_error = 0;
  if (!src || !out || workgroups < 1 || trips < 1 || bytes < kTrip || bytes > (int64_t(1) << 40) ||
      bytes % kTrip != 0 || !aligned16(src))
    return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((workgroups + 255) / 256)), dim3(256), 0, s, out,
                     workgroups);
  if (launched(hip_error)) return 2;
  hipLaunchKernelGGL(copy_lds_kernel, dim3((unsigned)workgroups), dim3(kThreads), 0, s,
                     static_cast<const char*>(src), bytes / kTrip, (int64_t)1, (int)trips, out);
  return launched(hip_error);
}

int mi_ceiling_read(const void* src, int64_t bytes, int32_t workgroups, uint32_t* out,
                    void* stream, int* hip_error) {
  if (hip_error) *hip_error = 0;
  if (!src || !out || workgroups < 1 || bytes < 1 || bytes > (int64_t(1) << 40) ||
      bytes % ((int64_t)workgroups * 4096) != 0 || !aligned16(src))
    return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((workgroups + 255) / 256)), dim3(256), 0, s, out,
                     workgroups);
  if (launched(hip_error)) return 2;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)workgroups), dim3(kThreads), 0, s,
                     static_cast<const char*>(src), bytes / workgroups, out);
  return launched(hip_error);
}

}  // extern "C"
