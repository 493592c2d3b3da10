// Server-mode load generator for libmi_hgemm: GEMM requests arrive as a
// Poisson process at a target rate (or back to back with a bounded number in
// flight) and are served one after another on one HIP stream, as an inference
// server's GPU queue would serve them.  Reports the achieved request rate and
// the arrival-to-completion latency of every request.
//
// This is the server mode of "RL驱动CUDA L2 GEMM内核自动调优：A100/H100 tile
// size与融合优化" (blog.hotdry.top, 2025-12-05), 集成步骤: the evaluation runs
// offline (back to back) or as a server at a target QPS (100 in the page's
// example) on the (64, 4096, 64) problem, and compares the QPS reached with the
// vendor library's.  The page gives no more detail; the readings taken are:
//   * a request is one GEMM call whose operands are already on the device;
//     requests rotate over `sets` operand copies (independent requests);
//   * arrivals are Poisson at the target rate (exponential gaps from a seeded
//     std::mt19937_64); latency = completion - planned arrival, so a late
//     issue counts against the server;
//   * "closed" mode issues the next request as soon as fewer than `depth` are
//     in flight: the highest rate the server sustains.
//
// Backends: the library's own dispatch (mi_hgemm_run), or rocBLAS's
// rocblas_gemm_ex (fp16 in and out, fp32 compute) on the same operands, for
// the vendor comparison, or "launch": one empty kernel per request, the floor
// that a HIP launch and its event set for any backend in this harness.  The
// record also reports the host time each request's issue call took.
//
//   mi_hgemm_serve --mnk M_N_K [--mode poisson|closed] [--qps Q] [--requests N]
//                  [--depth D] [--sets S] [--seed X] [--backend mi_hgemm|rocblas|launch]
//                  [--dump DIR]
// prints one JSON line.  --dump writes set 0's A, B (binary16, row-major, K
// contiguous) and its C after the run as raw files A.bin, B.bin, C.bin.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <numeric>
#include <random>
#include <string>
#include <thread>
#include <vector>

#include "../../include/mi_hgemm.h"

namespace {

using Clock = std::chrono::steady_clock;

double now_us() {
  return std::chrono::duration<double, std::micro>(Clock::now().time_since_epoch()).count();
}

[[noreturn]] void die(const char* what, const char* detail) {
  std::fprintf(stderr, "mi_hgemm_serve: %s: %s\n", what, detail);
  std::exit(2);
}

void check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) die(what, hipGetErrorString(e));
}

__device__ inline uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

__global__ void empty_kernel() {}

// operand values uniform in (-scale, scale), from a hash of (seed, index)
__global__ void fill_kernel(_Float16* x, int64_t n, uint32_t seed, float scale) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n;
       t += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t h = mix32((uint32_t)t ^ mix32(seed ^ (uint32_t)(t >> 32)));
    x[t] = (_Float16)(scale * ((float)(h >> 8) * (2.0f / 16777216.0f) - 1.0f));
  }
}

struct Options {
  int64_t M = 64, N = 4096, K = 64;
  std::string mode = "poisson";
  double qps = 100.0;
  int requests = 1000;
  int depth = 8;
  int sets = 64;
  uint64_t seed = 1;
  std::string backend = "mi_hgemm";
  std::string dump;
};

Options parse(int argc, char** argv) {
  Options o;
  for (int i = 1; i < argc; ++i) {
    std::string a = argv[i];
    auto val = [&]() -> std::string {
      if (i + 1 >= argc) die("missing value for", a.c_str());
      return argv[++i];
    };
    if (a == "--mnk") {
      long long m, n, k;
      if (std::sscanf(val().c_str(), "%lld_%lld_%lld", &m, &n, &k) != 3) die("bad --mnk", "");
      o.M = m, o.N = n, o.K = k;
    } else if (a == "--mode") o.mode = val();
    else if (a == "--qps") o.qps = std::atof(val().c_str());
    else if (a == "--requests") o.requests = std::atoi(val().c_str());
    else if (a == "--depth") o.depth = std::atoi(val().c_str());
    else if (a == "--sets") o.sets = std::atoi(val().c_str());
    else if (a == "--seed") o.seed = std::strtoull(val().c_str(), nullptr, 10);
    else if (a == "--backend") o.backend = val();
    else if (a == "--dump") o.dump = val();
    else die("unknown option", a.c_str());
  }
  if (o.M < 1 || o.N < 1 || o.K < 1 || o.requests < 1 || o.depth < 1 || o.sets < 1 ||
      o.qps <= 0.0 || (o.mode != "poisson" && o.mode != "closed") ||
      (o.backend != "mi_hgemm" && o.backend != "rocblas" && o.backend != "launch"))
    die("bad arguments", "see the usage in the source header");
  return o;
}

double pct(std::vector<double> v, double q) {
  std::sort(v.begin(), v.end());
  const size_t i = std::min(v.size() - 1, (size_t)std::floor(q * (v.size() - 1) + 0.5));
  return v[i];
}

void write_file(const std::string& path, const void* p, size_t n) {
  FILE* f = std::fopen(path.c_str(), "wb");
  if (!f || std::fwrite(p, 1, n, f) != n) die("cannot write", path.c_str());
  std::fclose(f);
}

}  // namespace

int main(int argc, char** argv) {
  const Options o = parse(argc, argv);
  check_hip(hipSetDevice(0), "hipSetDevice");
  const int64_t M = o.M, N = o.N, K = o.K;
  const size_t a_n = (size_t)M * K, b_n = (size_t)N * K, c_n = (size_t)M * N;

  std::vector<_Float16*> A(o.sets), B(o.sets), C(o.sets);
  for (int s = 0; s < o.sets; ++s) {
    check_hip(hipMalloc(&A[s], a_n * 2), "hipMalloc A");
    check_hip(hipMalloc(&B[s], b_n * 2), "hipMalloc B");
    check_hip(hipMalloc(&C[s], c_n * 2), "hipMalloc C");
    const float scale = 1.0f / std::sqrt((float)K);
    hipLaunchKernelGGL(fill_kernel, dim3(1024), dim3(256), 0, nullptr, A[s], (int64_t)a_n,
                       (uint32_t)(o.seed * 7919 + 2 * s), scale);
    hipLaunchKernelGGL(fill_kernel, dim3(1024), dim3(256), 0, nullptr, B[s], (int64_t)b_n,
                       (uint32_t)(o.seed * 7919 + 2 * s + 1), scale);
  }
  check_hip(hipDeviceSynchronize(), "fill");

  hipStream_t stream;
  check_hip(hipStreamCreateWithFlags(&stream, hipStreamNonBlocking), "hipStreamCreate");
  mi_hgemm_handle_t h = nullptr;
  rocblas_handle rb = nullptr;
  if (o.backend == "mi_hgemm") {
    const mi_hgemm_status_t st = mi_hgemm_create(&h, nullptr);
    if (st != MI_HGEMM_OK && st != MI_HGEMM_WARN_TABLE_DEFAULTS)
      die("mi_hgemm_create", mi_hgemm_status_string(st));
  } else if (o.backend == "rocblas") {
    if (rocblas_create_handle(&rb) != rocblas_status_success) die("rocblas", "create_handle");
    if (rocblas_set_stream(rb, stream) != rocblas_status_success) die("rocblas", "set_stream");
  }
  const float alpha = 1.0f, beta = 0.0f;
  auto issue = [&](int s) {
    if (h) {
      const mi_hgemm_status_t st = mi_hgemm_run(h, M, N, K, A[s], K, B[s], K, C[s], N,
                                                MI_HGEMM_LAYOUT_TN, stream);
      if (st != MI_HGEMM_OK) die("mi_hgemm_run", mi_hgemm_status_string(st));
    } else if (!rb) {
      hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
      check_hip(hipGetLastError(), "empty_kernel");
    } else {
      // row-major C = A Bt^T is column-major C^T (N x M) = Bt (as K x N, transposed) * A^T
      const rocblas_status st = rocblas_gemm_ex(
          rb, rocblas_operation_transpose, rocblas_operation_none, (rocblas_int)N, (rocblas_int)M,
          (rocblas_int)K, &alpha, B[s], rocblas_datatype_f16_r, (rocblas_int)K, A[s],
          rocblas_datatype_f16_r, (rocblas_int)K, &beta, C[s], rocblas_datatype_f16_r,
          (rocblas_int)N, C[s], rocblas_datatype_f16_r, (rocblas_int)N, rocblas_datatype_f32_r,
          rocblas_gemm_algo_standard, 0, 0);
      if (st != rocblas_status_success) die("rocblas_gemm_ex", rocblas_status_to_string(st));
    }
  };
  // warm-up: every set once, so first-touch and code loading stay out of the run
  for (int s = 0; s < o.sets; ++s) issue(s);
  check_hip(hipStreamSynchronize(stream), "warm-up");

  const int n = o.requests;
  std::vector<hipEvent_t> ev(n);
  for (int i = 0; i < n; ++i)
    check_hip(hipEventCreateWithFlags(&ev[i], hipEventDisableTiming), "hipEventCreate");
  std::vector<double> arrive(n, 0.0), done(n, 0.0), issue_us(n, 0.0);
  std::atomic<int> issued{0}, completed{0};

  // completion side: requests finish in order on the one stream
  std::thread waiter([&]() {
    for (int i = 0; i < n; ++i) {
      while (issued.load(std::memory_order_acquire) <= i) std::this_thread::yield();
      check_hip(hipEventSynchronize(ev[i]), "hipEventSynchronize");
      done[i] = now_us();
      completed.store(i + 1, std::memory_order_release);
    }
  });

  std::mt19937_64 rng(o.seed);
  std::exponential_distribution<double> gap(o.qps / 1e6);  // per microsecond
  const double t0 = now_us() + 1000.0;
  double next = t0;
  for (int i = 0; i < n; ++i) {
    if (o.mode == "poisson") {
      next += (i == 0) ? 0.0 : gap(rng);
      // sleep through long gaps, spin the last 200 us for a precise issue
      for (;;) {
        const double d = next - now_us();
        if (d <= 0.0) break;
        if (d > 300.0) std::this_thread::sleep_for(std::chrono::microseconds((int64_t)(d - 200.0)));
      }
      arrive[i] = next;
    } else {
      while (i - completed.load(std::memory_order_acquire) >= o.depth) {
      }
      arrive[i] = now_us();
    }
    const double ti = now_us();
    issue(i % o.sets);
    issue_us[i] = now_us() - ti;
    check_hip(hipEventRecord(ev[i], stream), "hipEventRecord");
    issued.store(i + 1, std::memory_order_release);
  }
  waiter.join();

  std::vector<double> lat(n);
  double sum = 0.0;
  for (int i = 0; i < n; ++i) {
    lat[i] = done[i] - arrive[i];
    sum += lat[i];
  }
  const double span = done[n - 1] - arrive[0];
  const double offered = o.mode == "poisson" ? (n - 1) / ((arrive[n - 1] - arrive[0]) * 1e-6) : 0.0;

  if (!o.dump.empty()) {
    std::vector<_Float16> ha(a_n), hb(b_n), hc(c_n);
    check_hip(hipMemcpy(ha.data(), A[0], a_n * 2, hipMemcpyDeviceToHost), "copy A");
    check_hip(hipMemcpy(hb.data(), B[0], b_n * 2, hipMemcpyDeviceToHost), "copy B");
    check_hip(hipMemcpy(hc.data(), C[0], c_n * 2, hipMemcpyDeviceToHost), "copy C");
    write_file(o.dump + "/A.bin", ha.data(), a_n * 2);
    write_file(o.dump + "/B.bin", hb.data(), b_n * 2);
    write_file(o.dump + "/C.bin", hc.data(), c_n * 2);
  }

  std::printf(
      "{\"backend\": \"%s\", \"mode\": \"%s\", \"M\": %lld, \"N\": %lld, \"K\": %lld, "
      "\"requests\": %d, \"target_qps\": %s, \"offered_qps\": %.3f, \"achieved_qps\": %.3f, "
      "\"depth\": %d, \"sets\": %d, \"seed\": %llu, \"latency_us\": {\"mean\": %.3f, "
      "\"p50\": %.3f, \"p90\": %.3f, \"p99\": %.3f, \"max\": %.3f}, "
      "\"issue_us\": {\"mean\": %.3f, \"p50\": %.3f, \"p99\": %.3f}}\n",
      o.backend.c_str(), o.mode.c_str(), (long long)M, (long long)N, (long long)K, n,
      o.mode == "poisson" ? std::to_string(o.qps).c_str() : "null", offered,
      n / (span * 1e-6), o.depth, o.sets, (unsigned long long)o.seed, sum / n, pct(lat, 0.5),
      pct(lat, 0.9), pct(lat, 0.99), pct(lat, 1.0),
      std::accumulate(issue_us.begin(), issue_us.end(), 0.0) / n, pct(issue_us, 0.5),
      pct(issue_us, 0.99));

  for (int i = 0; i < n; ++i) (void)hipEventDestroy(ev[i]);
  if (h) mi_hgemm_destroy(h);
  if (rb) rocblas_destroy_handle(rb);
  (void)hipStreamDestroy(stream);
  for (int s = 0; s < o.sets; ++s) {
    (void)hipFree(A[s]);
    (void)hipFree(B[s]);
    (void)hipFree(C[s]);
  }
  return 0;
}
