// Host side of libmi_hgemm: the C ABI declared in include/mi_hgemm.h.
//
// Pages this follows:
//   [P1] "H100 GEMM L2驻留优化：warp-specialized TMA异步拷贝与RL调优策略" (blog.hotdry.top)
//   [P2] "RL驱动CUDA L2 GEMM内核自动调优：A100/H100 tile size与融合优化" (blog.hotdry.top)
//   [P3] "B-08. Hopper TMA：从单线程 Bulk Copy 到吞吐墙" (lqnn.cn)
//
// Responsibilities:
//   * argument validation and status codes (the alignment rules of [P3] §3.1
//     and §6.1: misaligned vector copies are undefined, so alignment is decided
//     on the host and misaligned operands take the element-wise instance);
//   * dispatch: (M, N, K, alignment class) -> table entry, else the nearest
//     tuned shape, else built-in heuristics -> one launch on the caller's
//     stream, with nothing rebuilt or allocated per call ([P3] §8 lists
//     per-launch rebuilding as a classic mistake);
//   * the shape -> config table file and the tuner, which replaces the
//     pages' RL agent ([P1] 正文 paragraph 4, [P2] 正文 paragraph 2) with an
//     exhaustive or pruned timed sweep over the compiled instances and raster
//     settings, checked for correctness before it may win.
#include <dlfcn.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "../../include/mi_hgemm.h"
#include "internal.h"

namespace {

using mihg::GemmArgs;
using mihg::KernelDesc;
using mihg::kKernels;
using mihg::kNumKernels;

constexpr int kGenericKernel = 0;   // element-wise instance, any alignment
constexpr const char* kArch = "gfx950";

struct Config {
  int32_t kernel = kGenericKernel;
  int32_t group_m = 1;
  int32_t xcd = 0;
  int32_t splitk = 1;  // K slices per output tile (instances with splitk_ok only)
  double us = 0.0;     // measured time when tuned; 0 for heuristic picks
};

// Split-K workspace the handle owns: fp32 partial tiles and per-tile counters.
constexpr size_t kWsBytes = size_t(64) << 20;
constexpr int kMaxTiles = 1 << 16;

// Dispatch class of a call: element type x alignment class.  Table entries and
// the nearest-shape search never cross classes.
enum Cls : int32_t { CLS_F16_ANY = 0, CLS_F16_A16 = 1, CLS_I8_ANY = 2, CLS_I8_A16 = 3 };
constexpr const char* kClsName[4] = {"any", "a16", "i8any", "i8a16"};

int32_t make_cls(int32_t dtype, bool aligned) { return 2 * dtype + (aligned ? 1 : 0); }
int32_t cls_dtype(int32_t cls) { return cls / 2; }
bool cls_aligned(int32_t cls) { return (cls & 1) != 0; }

struct Key {
  int64_t M, N, K;
  int32_t cls;
  bool operator<(const Key& o) const {
    return std::tie(M, N, K, cls) < std::tie(o.M, o.N, o.K, o.cls);
  }
  bool operator==(const Key& o) const {
    return M == o.M && N == o.N && K == o.K && cls == o.cls;
  }
};

struct KeyHash {
  size_t operator()(const Key& k) const noexcept {
    uint64_t h = (uint64_t)k.M * 0x9E3779B97F4A7C15ull;
    h = (h ^ (uint64_t)k.N) * 0xBF58476D1CE4E5B9ull;
    h = (h ^ (uint64_t)k.K) * 0x94D049BB133111EBull;
    return (size_t)(h ^ (uint64_t)k.cls ^ (h >> 31));
  }
};

// Resolved configs kept per handle (table hits, nearest-shape picks and
// heuristic picks alike), so a repeated shape costs one hash lookup.  Cleared
// when the table changes (tune) and when it reaches this many entries.
constexpr size_t kMemoMax = 4096;

// Where a launch's split-K partial tiles and per-tile arrival counters live,
// and how much of each there is.
struct Workspace {
  float* ws = nullptr;
  int* cnt = nullptr;
  size_t ws_bytes = 0;
  int64_t max_tiles = 0;
};

}  // namespace

struct mi_hgemm_ctx {
  int device = -1;
  bool no_device = false;
  float* ws = nullptr;  // kWsBytes of split-K partials
  int* cnt = nullptr;   // kMaxTiles split-K counters, zero between launches
  int last_hip_error = 0;
  std::string table_path;  // resolved path (may be empty)
  std::map<Key, Config> table;
  std::mutex mu;           // guards table updates (tune) and last_hip_error
  std::unordered_map<Key, Config, KeyHash> memo;  // resolved dispatch, see kMemoMax
  std::mutex memo_mu;      // guards memo (run/plan may be called from several threads)
};

// ------------------------------------------------------ static scratch --
// The split-K scratch of mi_hgemm_run_noalloc: partial tiles, then one arrival
// counter per output tile.  Each device that loads the library holds its own
// copy until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its address on a device is resolved once per
// device (static_scratch_init) and only that address is ever used.
namespace {
constexpr size_t kStaticPartialBytes = size_t(MI_HGEMM_NOALLOC_PARTIAL_BYTES);
constexpr int64_t kStaticCounters = MI_HGEMM_NOALLOC_TILE_COUNTERS;
constexpr size_t kStaticBytes = kStaticPartialBytes + size_t(kStaticCounters) * sizeof(int);
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticBytes];

namespace {

struct StaticScratch {
  std::mutex mu;
  void* ptr[kMaxDevices] = {};      // device address of `scratch` per device, once resolved
  hipError_t err[kMaxDevices] = {};  // why resolving failed, if it did
};
StaticScratch& static_scratch() {
  static StaticScratch s;
  return s;
}

// With device `dev` current: resolve the array's address on it and clear its
// counters (they must start at zero; every split launch leaves them at zero).
// Runs once per device, at handle creation (no stream is being captured then).
void static_scratch_init(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return;
  StaticScratch& st = static_scratch();
  std::lock_guard<std::mutex> lk(st.mu);
  if (st.ptr[dev]) return;
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e == hipSuccess && ptr == nullptr) e = hipErrorInvalidSymbol;
  if (e == hipSuccess)
    e = hipMemset(static_cast<char*>(ptr) + kStaticPartialBytes, 0, kStaticCounters * sizeof(int));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipGetLastError();
    st.err[dev] = e;
    return;
  }
  st.ptr[dev] = ptr;
  st.err[dev] = hipSuccess;
}

// The resolved scratch of device `dev` as a workspace (ws == nullptr if it
// could not be resolved; *err then says why).
Workspace static_ws(int dev, hipError_t* err) {
  Workspace w;
  *err = hipErrorInvalidDevice;
  if (dev < 0 || dev >= kMaxDevices) return w;
  StaticScratch& st = static_scratch();
  std::lock_guard<std::mutex> lk(st.mu);
  *err = st.ptr[dev] ? hipSuccess : (st.err[dev] != hipSuccess ? st.err[dev] : hipErrorNotInitialized);
  if (!st.ptr[dev]) return w;
  char* base = static_cast<char*>(st.ptr[dev]);
  w.ws = reinterpret_cast<float*>(base);
  w.cnt = reinterpret_cast<int*>(base + kStaticPartialBytes);
  w.ws_bytes = kStaticPartialBytes;
  w.max_tiles = kStaticCounters;
  return w;
}

bool is_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int find_kernel(const char* name) {
  for (int i = 0; i < kNumKernels; ++i)
    if (std::strcmp(kKernels[i].name, name) == 0) return i;
  return -1;
}

// The int8 variant's int32 sums stay exact while K * 128 * 128 < 2^31.
constexpr int64_t kMaxKInt8 = 131071;

// Element bytes of operands and result.
int operand_bytes(int32_t dtype) { return dtype == mihg::DTYPE_I8 ? 1 : 2; }
int result_bytes(int32_t dtype) { return dtype == mihg::DTYPE_I8 ? 4 : 2; }

// Instance 0 is the fp16 element-wise instance; the int8 one is found by name.
int generic_kernel(int32_t dtype) {
  if (dtype == mihg::DTYPE_F16) return kGenericKernel;
  static const int i8 = find_kernel("i8_generic_64x64_w2x2_m16");
  return i8;
}

// Shared argument checks of run, plan and run_kernel, for element type dtype.
mi_hgemm_status_t validate(int32_t dtype, int64_t M, int64_t N, int64_t K, const void* A,
                           int64_t lda, const void* B, int64_t ldb, const void* C, int64_t ldc,
                           mi_hgemm_layout_t layout) {
  if (layout != MI_HGEMM_LAYOUT_TN) return MI_HGEMM_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0) return MI_HGEMM_ERR_INVALID_ARG;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return MI_HGEMM_ERR_UNSUPPORTED;
  if (dtype == mihg::DTYPE_I8 && K > kMaxKInt8) return MI_HGEMM_ERR_UNSUPPORTED;
  if (lda < std::max<int64_t>(K, 1) || ldb < std::max<int64_t>(K, 1) ||
      ldc < std::max<int64_t>(N, 1))
    return MI_HGEMM_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return MI_HGEMM_OK;
  if (C == nullptr) return MI_HGEMM_ERR_INVALID_ARG;
  if (K > 0 && (A == nullptr || B == nullptr)) return MI_HGEMM_ERR_INVALID_ARG;
  // C must not overlap the operands it is computed from.
  const uintptr_t eb = (uintptr_t)operand_bytes(dtype), cb = (uintptr_t)result_bytes(dtype);
  const uintptr_t c0 = reinterpret_cast<uintptr_t>(C);
  const uintptr_t c1 = c0 + cb * (uintptr_t)((M - 1) * ldc + N);
  auto overlaps = [&](const void* X, int64_t rows, int64_t ld, int64_t cols) {
    if (rows == 0 || cols == 0) return false;
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(X);
    const uintptr_t x1 = x0 + eb * (uintptr_t)((rows - 1) * ld + cols);
    return x0 < c1 && c0 < x1;
  };
  if (K > 0 && (overlaps(A, M, lda, K) || overlaps(B, N, ldb, K))) return MI_HGEMM_ERR_INVALID_ARG;
  return MI_HGEMM_OK;
}

// The vector-load kernels address a tile through 32-bit buffer offsets, so
// their leading dimensions are capped at kMaxVectorLd elements (a 256-row tile
// then spans at most 2^30 bytes).
constexpr int64_t kMaxVectorLd = int64_t(1) << 21;

// The 16-byte class: rows of A, B and C start on 16-byte boundaries and K is
// a whole number of 16-byte chunks (8 halves, or 16 int8 values).
bool aligned_class(int32_t dtype, int64_t K, const void* A, int64_t lda, const void* B,
                   int64_t ldb, const void* C, int64_t ldc) {
  const int64_t ek = 16 / operand_bytes(dtype), ec = 16 / result_bytes(dtype);
  return (K % ek) == 0 && (lda % ek) == 0 && (ldb % ek) == 0 && (ldc % ec) == 0 &&
         lda <= kMaxVectorLd && ldb <= kMaxVectorLd && ldc <= kMaxVectorLd &&
         is_aligned16(A) && is_aligned16(B) && is_aligned16(C);
}

// The K split a launch of `kd` would use for a requested split: slices are
// whole multiples of 64 K elements and empty trailing slices are dropped, so
// the result may be smaller than asked (1 = no split).  -1 when the instance
// cannot split or the partial tiles would not fit the workspace.
int64_t effective_split(const KernelDesc& kd, int64_t M, int64_t N, int64_t K, int requested,
                        int64_t* chunk_out, size_t ws_bytes = kWsBytes, int64_t max_tiles = kMaxTiles) {
  if (requested <= 1) {
    *chunk_out = K;
    return 1;
  }
  if (!kd.splitk_ok) return -1;
  const int64_t chunk = ((K + requested - 1) / requested + 63) / 64 * 64;
  const int64_t sk = (K + chunk - 1) / chunk;
  *chunk_out = sk > 1 ? chunk : K;
  if (sk <= 1) return 1;
  const int64_t tiles = kd.grid((int32_t)M, (int32_t)N);
  if (tiles > max_tiles || tiles * sk > INT32_MAX ||
      (size_t)tiles * sk * kd.bm * kd.bn * sizeof(float) > ws_bytes)
    return -1;
  return sk;
}

// Built-in choice when the table has nothing close: the largest tile that
// still fills a good part of the machine ([P2] 正文 paragraph 3: large tiles
// raise reuse and lower occupancy), else a K split.  The thresholds come from
// timing every instance over the LLM projection and square shapes on MI355X:
//  - the binary16 picks stage C through LDS ("_sc"): whole row-segment stores
//    make short-K shapes up to 1.2-1.3x faster and cost nothing at long K;
//  - one partial wave of 256x256 tiles beats more waves of smaller tiles (the
//    chip is power-bound: idle CUs buy clock for the busy ones); in its
//    ping-pong form (pp2tile, binary16 and int8) down to five eighths of a
//    wave;
//  - below that, two or more full waves of 128x128 direct-to-LDS tiles win, at
//    every K (14-33% ahead of a half wave of 256x256 tiles on the shape sweep);
//  - below that, the deep-K tiles (K step 128) win: 128x128, then 64x64, then
//    32x64 / 16x64 for the smallest M; small tiles are latency-bound per K
//    step, so a deep step beats more parallel tiles;
//  - when even those leave half the CUs idle and K is long, K is split.
Config heuristic(int64_t M, int64_t N, int64_t K, int32_t cls) {
  Config c;
  const int32_t dtype = cls_dtype(cls);
  c.kernel = generic_kernel(dtype);
  if (!cls_aligned(cls)) return c;
  auto tiles = [&](int k) { return k >= 0 ? kKernels[k].grid((int32_t)M, (int32_t)N) : 0; };
  // as many K slices of kernel k as keep every slice >= 1024 deep and the
  // grid <= 256 workgroups (1 = no split)
  auto split_for = [&](int k) {
    if (k < 0 || !kKernels[k].splitk_ok) return 1;
    const int64_t t = tiles(k);
    int s = 1;
    while (s < 8 && t * s * 2 <= 256 && K / (s * 2) >= 1024) s *= 2;
    int64_t chunk = K;
    return (s > 1 && effective_split(kKernels[k], M, N, K, s, &chunk) > 1) ? s : 1;
  };
  auto pick = [&](int k, int g, int x, int s) {
    c.kernel = k;
    c.group_m = g;
    c.xcd = x;
    c.splitk = s;
  };
  // the int8 instances with the same tiles and a K step of the same bytes
  const bool i8 = dtype == mihg::DTYPE_I8;
  const int k128 = find_kernel(i8 ? "i8_ktile_128x128_w2x4_k256_s3b2" : "ktile_128x128_w2x4_k128_s3b2_sc");
  // When the output is one row of tiles B is streamed through once: those
  // tiles copy it with the non-temporal policy ("_nt"), which
  // leaves the caches to A (measured 1-10% faster on the 16- and 64-row
  // projection shapes).
  const bool one_row = M <= 64;
  const int k64 = find_kernel(i8 ? (one_row ? "i8_ktile_64x64_w2x2_k256_s3_nt" : "i8_ktile_64x64_w2x2_k256_s3")
                                 : (one_row ? "ktile_64x64_w2x2_k128_s3_nt" : "ktile_64x64_w2x2_k128_s3b3_sc"));
  const int k32 = find_kernel(i8 ? (M <= 32 ? "i8_ktile_32x64_w2x2_k256_s3_nt" : "i8_ktile_32x64_w2x2_k256_s3")
                                 : (M <= 32 ? "ktile_32x64_w2x2_k128_s3_nt" : "ktile_32x64_w2x2_k128_s3b3_sc"));
  const int k16 = find_kernel(i8 ? "i8_ktile_16x64_w1x4_k256_s3_nt" : "ktile_16x64_w1x4_k128_s3_nt");
  const int k128d = find_kernel(i8 ? "i8_d2tile_128x128_w2x2_m16" : "d2tile_128x128_w2x2_m16_sc");
  // five eighths of a wave of 256x256 tiles or more: the ping-pong tile (two
  // wave groups taking turns at the matrix pipes) measured 4-14% ahead of
  // d2tile3 from 172 tiles up (1024x11008x4096 .. 8192^3) in binary16, 5-9%
  // in int8
  // Its raster: up to one wave of tiles (256 or fewer) the XCD-local groups of
  // 8 tile rows (g8 x1) measured 0-20% ahead of row-major order over
  // 4096x4096, 8192x2048 and 2048x8192 at K = 128..2048 (e.g. 8192x2048x1024:
  // 32.7 against 37.7 us); from four waves up row-major order (g1 x0) was
  // 2-26% ahead on 8192x8192 at K = 64..2048 (e.g. 8192x8192x256: 52.8
  // against 60.6 us), and at two waves the two were within 3% at K >= 256.
  const int kpp = find_kernel(i8 ? "i8_pp2tile_256x256_w8_m16" : "pp2tile_256x256_w8_m16_sc");
  // binary16 with 96 to 159 tiles of 256x128 over a K of 8192 or more and an
  // N of 2048 or more: the ping-pong 256x128 tile, K split in two
  // (1024x4096x11008 cold: 99.8 against 108.2 us for the deep-K 128x128
  // tile; 512x8192x8192: 81.0 against 84.6 us; at N = 512 it lost, 99.6
  // against 82.0 us on 8192x512x8192)
  const int kppsk = i8 ? -1 : find_kernel("pp2tile_256x128_w8_m16_sc_sk");
  int64_t chunk2 = K;
  if (M > 64 && kpp >= 0 && tiles(kpp) >= 160) {
    if (tiles(kpp) <= 256)
      pick(kpp, 8, 1, 1);
    else
      pick(kpp, 1, 0, 1);
  } else if (M > 64 && N >= 2048 && kppsk >= 0 && K >= 8192 && tiles(kppsk) >= 96 && tiles(kppsk) < 160 &&
             effective_split(kKernels[kppsk], M, N, K, 2, &chunk2) == 2) {
    pick(kppsk, 1, 0, 2);
  } else if (M > 64 && k128d >= 0 && tiles(k128d) >= 512) {
    pick(k128d, 8, 1, 1);
  } else if (M > 64 && k128 >= 0 && tiles(k128) >= 128) {
    pick(k128, 8, 1, split_for(k128));
  } else if (M > 32 && k64 >= 0 && (tiles(k64) >= 128 || K >= 8192)) {
    const int s = split_for(k64);
    pick(k64, s > 1 ? 1 : 8, s > 1 ? 0 : 1, s);
  } else if (M > 16 && k32 >= 0) {
    pick(k32, 1, 0, split_for(k32));
  } else if (k16 >= 0 && (i8 || tiles(k16) >= 128 || K >= 8192)) {
    pick(k16, 1, 0, split_for(k16));
  } else {
    // 16 rows or fewer over a short K: B streamed straight into registers
    const int ks = find_kernel("skinny_1x1_w4_u4");
    pick(ks >= 0 ? ks : kGenericKernel, 1, 0, 1);
  }
  if (c.kernel < 0) c.kernel = generic_kernel(dtype);
  return c;
}

// A table entry's split may not suit the shape it is applied to (a nearest
// entry, or an edited table): such a split is dropped rather than failing.
Config checked(Config c, int64_t M, int64_t N, int64_t K) {
  int64_t chunk = K;
  if (c.splitk > 1 && effective_split(kKernels[c.kernel], M, N, K, c.splitk, &chunk) < 1)
    c.splitk = 1;
  return c;
}

Config select_uncached(mi_hgemm_ctx* h, int64_t M, int64_t N, int64_t K, int32_t cls) {
  const Key key{M, N, K, cls};
  auto it = h->table.find(key);
  if (it != h->table.end()) return checked(it->second, M, N, K);
  // nearest tuned shape in log2(M, N, K), within a factor of two overall
  double best = 1.0 + 1e-9;
  const Config* pick = nullptr;
  // (within a factor of two overall means within a factor of two in each of
  // M, N and K: integer tests skip the logarithms for every other entry)
  auto near = [](int64_t x, int64_t t) { return t <= 2 * x && x <= 2 * t; };
  for (const auto& kv : h->table) {
    if (kv.first.cls != key.cls || !near(M, kv.first.M) || !near(N, kv.first.N) ||
        !near(K, kv.first.K))
      continue;
    const double d = std::fabs(std::log2((double)M / kv.first.M)) +
                     std::fabs(std::log2((double)N / kv.first.N)) +
                     std::fabs(std::log2((double)K / kv.first.K));
    if (d <= best) {
      best = d;
      pick = &kv.second;
    }
  }
  if (pick) return checked(*pick, M, N, K);
  return heuristic(M, N, K, cls);
}

// Dispatch: the exact table entry, else the nearest tuned shape, else the
// heuristic -- resolved once per (M, N, K, class) and then looked up.
// remember = false resolves a miss without storing it (no host allocation).
Config select(mi_hgemm_ctx* h, int64_t M, int64_t N, int64_t K, int32_t cls,
              bool remember = true) {
  const Key key{M, N, K, cls};
  {
    std::lock_guard<std::mutex> lk(h->memo_mu);
    auto it = h->memo.find(key);
    if (it != h->memo.end()) return it->second;
  }
  const Config c = select_uncached(h, M, N, K, cls);
  if (!remember) return c;
  std::lock_guard<std::mutex> lk(h->memo_mu);
  if (h->memo.size() >= kMemoMax) h->memo.clear();
  h->memo.emplace(key, c);
  return c;
}

void forget_resolved(mi_hgemm_ctx* h) {
  std::lock_guard<std::mutex> lk(h->memo_mu);
  h->memo.clear();
}

// Table file: one entry per line,
//   <arch> <M> <N> <K> <layout> <class> <kernel name> <group_m> <xcd_remap> <microseconds> [<split_k>]
// with class a16 / any (fp16 in / outside the 16-byte class) or i8a16 / i8any
// (the int8 variant).
// '#' starts a comment.  Lines for another arch or layout are skipped; lines
// that do not parse, or name an unknown kernel, mark the table as damaged.
bool load_table(mi_hgemm_ctx* h, const std::string& path, bool* file_missing) {
  *file_missing = false;
  FILE* f = std::fopen(path.c_str(), "r");
  if (!f) {
    *file_missing = true;
    return false;
  }
  bool clean = true;
  char line[512];
  while (std::fgets(line, sizeof line, f)) {
    char* p = line;
    while (*p == ' ' || *p == '\t') ++p;
    if (*p == '#' || *p == '\n' || *p == '\r' || *p == '\0') continue;
    char arch[64], layout[16], align[16], kname[128];
    long long M, N, K;
    int gm, xcd, sk = 1;
    double us;
    const int got = std::sscanf(p, "%63s %lld %lld %lld %15s %15s %127s %d %d %lf %d", arch, &M,
                                &N, &K, layout, align, kname, &gm, &xcd, &us, &sk);
    if ((got != 10 && got != 11) || M < 1 || N < 1 || K < 1 || gm < 1 || (xcd != 0 && xcd != 1) ||
        sk < 1 || sk > 64) {
      clean = false;
      continue;
    }
    if (std::strcmp(arch, kArch) != 0 || std::strcmp(layout, "TN") != 0) continue;
    const int k = find_kernel(kname);
    int cls = -1;
    for (int i = 0; i < 4; ++i)
      if (std::strcmp(align, kClsName[i]) == 0) cls = i;
    if (k < 0 || cls < 0 || kKernels[k].dtype != cls_dtype(cls) ||
        (!cls_aligned(cls) && kKernels[k].aligned) || (sk > 1 && !kKernels[k].splitk_ok)) {
      clean = false;
      continue;
    }
    Config c;
    c.kernel = k;
    c.group_m = gm;
    c.xcd = xcd;
    c.splitk = sk;
    c.us = us;
    h->table[Key{M, N, K, cls}] = c;
  }
  std::fclose(f);
  return clean;
}

bool write_entry(FILE* f, const Key& k, const Config& c) {
  return std::fprintf(f, "%s %lld %lld %lld TN %s %s %d %d %.3f %d\n", kArch, (long long)k.M,
                      (long long)k.N, (long long)k.K, kClsName[k.cls],
                      kKernels[c.kernel].name, c.group_m, c.xcd, c.us, c.splitk) > 0;
}

std::string default_table_path() {
  Dl_info info;
  if (dladdr(reinterpret_cast<void*>(&default_table_path), &info) && info.dli_fname) {
    std::string so = info.dli_fname;
    const size_t slash = so.rfind('/');
    const std::string dir = slash == std::string::npos ? "." : so.substr(0, slash);
    return dir + "/tables/gfx950.tsv";
  }
  return std::string();
}

mi_hgemm_status_t hip_fail(mi_hgemm_ctx* h, hipError_t e) {
  if (h) {
    std::lock_guard<std::mutex> lk(h->mu);
    h->last_hip_error = (int)e;
  }
  return MI_HGEMM_ERR_HIP;
}

// Makes the handle's device current for the scope of a call.
struct DeviceGuard {
  int prev = -1;
  bool switched = false;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int dev) {
    err = hipGetDevice(&prev);
    if (err == hipSuccess && prev != dev) {
      err = hipSetDevice(dev);
      switched = err == hipSuccess;
    }
  }
  ~DeviceGuard() {
    if (switched) (void)hipSetDevice(prev);
  }
};

// The handle's own split-K workspace.
Workspace handle_ws(const mi_hgemm_ctx* h) {
  Workspace w;
  w.ws = h->ws;
  w.cnt = h->cnt;
  w.ws_bytes = h->ws ? kWsBytes : 0;
  w.max_tiles = h->cnt ? kMaxTiles : 0;
  return w;
}

mi_hgemm_status_t launch(mi_hgemm_ctx* h, const Config& c, int64_t M, int64_t N, int64_t K,
                         const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                         int64_t ldc, hipStream_t stream, const Workspace& w) {
  const KernelDesc& kd = kKernels[c.kernel];
  if (kd.grid((int32_t)M, (int32_t)N) > INT32_MAX) return MI_HGEMM_ERR_UNSUPPORTED;
  GemmArgs a;
  a.A = A;
  a.B = B;
  a.C = C;
  a.lda = lda;
  a.ldb = ldb;
  a.ldc = ldc;
  a.M = (int32_t)M;
  a.N = (int32_t)N;
  a.K = (int32_t)K;
  a.group_m = std::max(1, c.group_m);
  a.xcd_remap = c.xcd ? 1 : 0;
  a.splitk = 1;
  a.kchunk = (int32_t)K;
  a.ws = w.ws;
  a.cnt = w.cnt;
  if (c.splitk > 1) {
    if (!w.ws || !w.cnt) return MI_HGEMM_ERR_UNSUPPORTED;
    int64_t chunk = K;
    // never more partial tiles or counters than the workspace holds
    const int64_t sk = effective_split(kd, M, N, K, c.splitk, &chunk, w.ws_bytes, w.max_tiles);
    if (sk < 1) return MI_HGEMM_ERR_UNSUPPORTED;
    a.splitk = (int32_t)sk;
    a.kchunk = (int32_t)chunk;
  }
  const hipError_t e = kd.launch(a, stream);
  if (e != hipSuccess) return hip_fail(h, e);
  return MI_HGEMM_OK;
}

mi_hgemm_status_t run_config(mi_hgemm_ctx* h, int32_t dtype, const Config& c, int64_t M,
                             int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                             int64_t ldb, void* C, int64_t ldc, void* stream,
                             const Workspace& w) {
  if (M == 0 || N == 0) return MI_HGEMM_OK;
  if (h->no_device) return MI_HGEMM_ERR_NO_DEVICE;
  DeviceGuard g(h->device);
  if (g.err != hipSuccess) return hip_fail(h, g.err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (K == 0) {
    // +0 in binary16 and 0 in int32 are all-zero bits: an int32 row is cleared
    // as twice as many halves
    const int64_t w = result_bytes(dtype) / 2;
    if (N * w > INT32_MAX) return MI_HGEMM_ERR_UNSUPPORTED;
    const hipError_t e = mihg::launch_zero_fill(C, ldc * w, (int32_t)M, (int32_t)(N * w), s);
    return e == hipSuccess ? MI_HGEMM_OK : hip_fail(h, e);
  }
  return launch(h, c, M, N, K, A, lda, B, ldb, C, ldc, s, w);
}

mi_hgemm_status_t plan_impl(mi_hgemm_ctx* h, int32_t dtype, int64_t M, int64_t N, int64_t K,
                            const void* A, int64_t lda, const void* B, int64_t ldb,
                            const void* C, int64_t ldc, mi_hgemm_layout_t layout,
                            int32_t* kernel_index, int32_t* group_m, int32_t* xcd_remap,
                            int32_t* split_k) {
  if (!h) return MI_HGEMM_ERR_INVALID_ARG;
  const mi_hgemm_status_t st = validate(dtype, M, N, K, A, lda, B, ldb, C, ldc, layout);
  if (st != MI_HGEMM_OK) return st;
  Config c;
  c.kernel = -1;
  if (M > 0 && N > 0 && K > 0)
    c = select(h, M, N, K, make_cls(dtype, aligned_class(dtype, K, A, lda, B, ldb, C, ldc)));
  if (kernel_index) *kernel_index = c.kernel;
  if (group_m) *group_m = c.group_m;
  if (xcd_remap) *xcd_remap = c.xcd;
  if (split_k) *split_k = c.kernel >= 0 ? c.splitk : 1;
  return MI_HGEMM_OK;
}

mi_hgemm_status_t run_impl(mi_hgemm_ctx* h, int32_t dtype, int64_t M, int64_t N, int64_t K,
                           const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                           int64_t ldc, mi_hgemm_layout_t layout, void* stream) {
  if (!h) return MI_HGEMM_ERR_INVALID_ARG;
  const mi_hgemm_status_t st = validate(dtype, M, N, K, A, lda, B, ldb, C, ldc, layout);
  if (st != MI_HGEMM_OK) return st;
  if (M == 0 || N == 0) return MI_HGEMM_OK;
  Config c;
  c.kernel = generic_kernel(dtype);
  if (K > 0)
    c = select(h, M, N, K, make_cls(dtype, aligned_class(dtype, K, A, lda, B, ldb, C, ldc)));
  if (c.kernel < 0) return MI_HGEMM_ERR_UNSUPPORTED;
  return run_config(h, dtype, c, M, N, K, A, lda, B, ldb, C, ldc, stream, handle_ws(h));
}

}  // namespace

// ----------------------------------------------------------------- C ABI ---
extern "C" {

const char* mi_hgemm_status_string(mi_hgemm_status_t s) {
  switch (s) {
    case MI_HGEMM_OK: return "MI_HGEMM_OK";
    case MI_HGEMM_ERR_INVALID_ARG: return "MI_HGEMM_ERR_INVALID_ARG";
    case MI_HGEMM_ERR_UNSUPPORTED: return "MI_HGEMM_ERR_UNSUPPORTED";
    case MI_HGEMM_ERR_NO_DEVICE: return "MI_HGEMM_ERR_NO_DEVICE";
    case MI_HGEMM_ERR_HIP: return "MI_HGEMM_ERR_HIP";
    case MI_HGEMM_ERR_IO: return "MI_HGEMM_ERR_IO";
    case MI_HGEMM_WARN_TABLE_DEFAULTS: return "MI_HGEMM_WARN_TABLE_DEFAULTS";
  }
  return "MI_HGEMM_UNKNOWN_STATUS";
}

mi_hgemm_status_t mi_hgemm_create_ex(mi_hgemm_handle_t* out, const char* table_path,
                                     uint32_t flags) {
  if (!out) return MI_HGEMM_ERR_INVALID_ARG;
  *out = nullptr;
  mi_hgemm_ctx* h = new (std::nothrow) mi_hgemm_ctx();
  if (!h) return MI_HGEMM_ERR_INVALID_ARG;
  if (flags & MI_HGEMM_CREATE_NO_DEVICE) {
    h->no_device = true;
  } else {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count < 1 || hipGetDevice(&h->device) != hipSuccess) {
      delete h;
      return MI_HGEMM_ERR_NO_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, h->device) != hipSuccess ||
        std::strncmp(prop.gcnArchName, kArch, std::strlen(kArch)) != 0) {
      delete h;
      return MI_HGEMM_ERR_NO_DEVICE;
    }
    // split-K workspace: allocated once here, never per call
    void* ws = nullptr;
    void* cnt = nullptr;
    if (hipMalloc(&ws, kWsBytes) == hipSuccess && hipMalloc(&cnt, kMaxTiles * sizeof(int)) == hipSuccess &&
        hipMemset(cnt, 0, kMaxTiles * sizeof(int)) == hipSuccess && hipDeviceSynchronize() == hipSuccess) {
      h->ws = static_cast<float*>(ws);
      h->cnt = static_cast<int*>(cnt);
    } else {
      if (ws) (void)hipFree(ws);
      if (cnt) (void)hipFree(cnt);
      (void)hipGetLastError();
    }
    // the no-allocation entry point's scratch on this device (once per device)
    static_scratch_init(h->device);
  }
  bool named = false;
  if (table_path && *table_path) {
    h->table_path = table_path;
    named = true;
  } else if (const char* env = std::getenv("MI_HGEMM_TABLE"); env && *env) {
    h->table_path = env;
    named = true;
  } else {
    h->table_path = default_table_path();
  }
  mi_hgemm_status_t st = MI_HGEMM_OK;
  if (!h->table_path.empty()) {
    bool missing = false;
    const bool clean = load_table(h, h->table_path, &missing);
    if ((missing && named) || (!missing && !clean)) st = MI_HGEMM_WARN_TABLE_DEFAULTS;
  }
  *out = h;
  return st;
}

mi_hgemm_status_t mi_hgemm_create(mi_hgemm_handle_t* out, const char* table_path) {
  return mi_hgemm_create_ex(out, table_path, 0u);
}

mi_hgemm_status_t mi_hgemm_destroy(mi_hgemm_handle_t h) {
  if (!h) return MI_HGEMM_OK;
  if (h->ws || h->cnt) {
    DeviceGuard g(h->device);
    if (h->ws) (void)hipFree(h->ws);
    if (h->cnt) (void)hipFree(h->cnt);
  }
  delete h;
  return MI_HGEMM_OK;
}

int mi_hgemm_last_hip_error(mi_hgemm_handle_t h) {
  if (!h) return 0;
  std::lock_guard<std::mutex> lk(h->mu);
  return h->last_hip_error;
}

int mi_hgemm_kernel_count(void) { return kNumKernels; }

const char* mi_hgemm_kernel_name(int index) {
  return (index >= 0 && index < kNumKernels) ? kKernels[index].name : nullptr;
}

mi_hgemm_status_t mi_hgemm_plan(mi_hgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                const void* A, int64_t lda, const void* B, int64_t ldb,
                                const void* C, int64_t ldc, mi_hgemm_layout_t layout,
                                int32_t* kernel_index, int32_t* group_m, int32_t* xcd_remap,
                                int32_t* split_k) {
  return plan_impl(h, mihg::DTYPE_F16, M, N, K, A, lda, B, ldb, C, ldc, layout, kernel_index,
                   group_m, xcd_remap, split_k);
}

mi_hgemm_status_t mi_hgemm_plan_i8(mi_hgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                   const void* A, int64_t lda, const void* B, int64_t ldb,
                                   const void* C, int64_t ldc, mi_hgemm_layout_t layout,
                                   int32_t* kernel_index, int32_t* group_m, int32_t* xcd_remap,
                                   int32_t* split_k) {
  return plan_impl(h, mihg::DTYPE_I8, M, N, K, A, lda, B, ldb, C, ldc, layout, kernel_index,
                   group_m, xcd_remap, split_k);
}

mi_hgemm_status_t mi_hgemm_run(mi_hgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                               const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                               int64_t ldc, mi_hgemm_layout_t layout, void* stream) {
  return run_impl(h, mihg::DTYPE_F16, M, N, K, A, lda, B, ldb, C, ldc, layout, stream);
}

mi_hgemm_status_t mi_hgemm_run_i8(mi_hgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                  const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                                  int64_t ldc, mi_hgemm_layout_t layout, void* stream) {
  return run_impl(h, mihg::DTYPE_I8, M, N, K, A, lda, B, ldb, C, ldc, layout, stream);
}

mi_hgemm_status_t mi_hgemm_run_noalloc(mi_hgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                       const void* A, int64_t lda, const void* B, int64_t ldb,
                                       void* C, int64_t ldc, mi_hgemm_layout_t layout,
                                       void* stream) {
  if (!h) return MI_HGEMM_ERR_INVALID_ARG;
  const mi_hgemm_status_t st = validate(mihg::DTYPE_F16, M, N, K, A, lda, B, ldb, C, ldc, layout);
  if (st != MI_HGEMM_OK) return st;
  if (M == 0 || N == 0) return MI_HGEMM_OK;
  if (h->no_device) return MI_HGEMM_ERR_NO_DEVICE;
  hipError_t err = hipSuccess;
  const Workspace w = static_ws(h->device, &err);
  if (!w.ws) return hip_fail(h, err);
  Config c;
  c.kernel = kGenericKernel;
  if (K > 0) {
    c = select(h, M, N, K, make_cls(mihg::DTYPE_F16, aligned_class(mihg::DTYPE_F16, K, A, lda, B, ldb, C, ldc)),
               false);
    // The array holds fewer partial tiles than a handle's workspace: a planned
    // split that does not fit is halved until it does (split 1 needs none).
    // launch() still refuses any split beyond the array (UNSUPPORTED).
    while (c.splitk > 1) {
      int64_t chunk = K;
      if (effective_split(kKernels[c.kernel], M, N, K, c.splitk, &chunk, w.ws_bytes, w.max_tiles) >= 1)
        break;
      c.splitk /= 2;
    }
  }
  return run_config(h, mihg::DTYPE_F16, c, M, N, K, A, lda, B, ldb, C, ldc, stream, w);
}

mi_hgemm_status_t mi_hgemm_run_kernel(mi_hgemm_handle_t h, int32_t kernel_index, int32_t group_m,
                                      int32_t xcd_remap, int32_t split_k, int64_t M, int64_t N,
                                      int64_t K,
                                      const void* A, int64_t lda, const void* B, int64_t ldb,
                                      void* C, int64_t ldc, mi_hgemm_layout_t layout,
                                      void* stream) {
  if (!h) return MI_HGEMM_ERR_INVALID_ARG;
  if (kernel_index < 0 || kernel_index >= kNumKernels) return MI_HGEMM_ERR_UNSUPPORTED;
  if (group_m < 1 || (xcd_remap != 0 && xcd_remap != 1) || split_k < 1 || split_k > 64)
    return MI_HGEMM_ERR_INVALID_ARG;
  if (split_k > 1 && !kKernels[kernel_index].splitk_ok) return MI_HGEMM_ERR_UNSUPPORTED;
  const int32_t dtype = kKernels[kernel_index].dtype;
  const mi_hgemm_status_t st = validate(dtype, M, N, K, A, lda, B, ldb, C, ldc, layout);
  if (st != MI_HGEMM_OK) return st;
  if (kKernels[kernel_index].aligned && !aligned_class(dtype, K, A, lda, B, ldb, C, ldc))
    return MI_HGEMM_ERR_UNSUPPORTED;
  Config c;
  c.kernel = kernel_index;
  c.group_m = group_m;
  c.xcd = xcd_remap;
  c.splitk = split_k;
  return run_config(h, dtype, c, M, N, K, A, lda, B, ldb, C, ldc, stream, handle_ws(h));
}

int mi_hgemm_table_size(mi_hgemm_handle_t h) {
  if (!h) return 0;
  std::lock_guard<std::mutex> lk(h->mu);
  return (int)h->table.size();
}

mi_hgemm_status_t mi_hgemm_table_save(mi_hgemm_handle_t h, const char* path) {
  if (!h || !path) return MI_HGEMM_ERR_INVALID_ARG;
  FILE* f = std::fopen(path, "w");
  if (!f) return MI_HGEMM_ERR_IO;
  bool ok = std::fprintf(f, "# arch M N K layout align kernel group_m xcd_remap us split_k\n") > 0;
  {
    std::lock_guard<std::mutex> lk(h->mu);
    for (const auto& kv : h->table) ok = ok && write_entry(f, kv.first, kv.second);
  }
  ok = (std::fclose(f) == 0) && ok;
  return ok ? MI_HGEMM_OK : MI_HGEMM_ERR_IO;
}

}  // extern "C"

// ------------------------------------------------------------------ tuner --
namespace {

struct Scratch {
  void* p = nullptr;
  ~Scratch() {
    if (p) (void)hipFree(p);
  }
};

double median(std::vector<double> v) {
  std::sort(v.begin(), v.end());
  return v.empty() ? 0.0 : v[v.size() / 2];
}

struct TimingStream {
  hipStream_t s = nullptr;
  ~TimingStream() {
    if (s) (void)hipStreamDestroy(s);
  }
};

// Capture `reps` launches of one candidate on stream `ts` into a graph and
// time 5 replays; appends microseconds per launch to `trials`.
// The timing operands: nsets copies of (A, B) back to back, set i at
// base + i * (M + N) * K elements of eb bytes (A first), and nsets outputs C,
// output i at cbase + i * cstride bytes.
struct TimingSets {
  char* base = nullptr;
  char* cbase = nullptr;
  int64_t cstride = 0;
  int nsets = 1;
  int eb = 2;
  void* C(int i) const { return cbase + (int64_t)i * cstride; }
  const void* A(int64_t M, int64_t N, int64_t K, int i) const {
    return base + ((int64_t)i * (M + N) * K) * eb;
  }
  const void* B(int64_t M, int64_t N, int64_t K, int i) const {
    return base + ((int64_t)i * (M + N) * K + M * K) * eb;
  }
};

// Capture `reps` launches of one candidate on stream `ts` into a graph (launch r
// reads timing set r mod nsets and writes its output, so that together they
// overflow the MALL and each launch reads its operands from HBM and writes C
// past the MALL, as in real use) and time 5 replays;
// appends microseconds per launch to `trials`.
hipError_t time_replays(mi_hgemm_ctx* h, const Config& cand, int64_t M, int64_t N, int64_t K,
                        const TimingSets& sets, int64_t ldc, int reps,
                        hipStream_t ts, hipEvent_t ev0, hipEvent_t ev1,
                        std::vector<double>& trials) {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipError_t e = hipStreamBeginCapture(ts, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return e;
  mi_hgemm_status_t st = MI_HGEMM_OK;
  for (int r = 0; r < reps && st == MI_HGEMM_OK; ++r)
    st = launch(h, cand, M, N, K, sets.A(M, N, K, r % sets.nsets), K, sets.B(M, N, K, r % sets.nsets),
                K, sets.C(r % sets.nsets), ldc, ts, handle_ws(h));
  e = hipStreamEndCapture(ts, &graph);
  if (e == hipSuccess && st != MI_HGEMM_OK) e = hipErrorLaunchFailure;
  if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e == hipSuccess) e = hipGraphLaunch(exec, ts);  // warm-up replay
  for (int t = 0; t < 5 && e == hipSuccess; ++t) {
    float ms = 0.f;
    if ((e = hipEventRecord(ev0, ts)) != hipSuccess) break;
    if ((e = hipGraphLaunch(exec, ts)) != hipSuccess) break;
    if ((e = hipEventRecord(ev1, ts)) != hipSuccess) break;
    if ((e = hipEventSynchronize(ev1)) != hipSuccess) break;
    if ((e = hipEventElapsedTime(&ms, ev0, ev1)) != hipSuccess) break;
    trials.push_back(1000.0 * ms / reps);
  }
  if (exec) (void)hipGraphExecDestroy(exec);
  if (graph) (void)hipGraphDestroy(graph);
  return e;
}

}  // namespace

extern "C" mi_hgemm_status_t mi_hgemm_tune(mi_hgemm_handle_t h, int64_t M, int64_t N, int64_t K,
                                           mi_hgemm_layout_t layout, void* stream,
                                           uint32_t flags) {
  if (!h) return MI_HGEMM_ERR_INVALID_ARG;
  if (layout != MI_HGEMM_LAYOUT_TN) return MI_HGEMM_ERR_UNSUPPORTED;
  if (M < 1 || N < 1 || K < 1) return MI_HGEMM_ERR_INVALID_ARG;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return MI_HGEMM_ERR_UNSUPPORTED;
  const int32_t dtype = (flags & MI_HGEMM_TUNE_INT8) ? mihg::DTYPE_I8 : mihg::DTYPE_F16;
  const int eb = operand_bytes(dtype), cb = result_bytes(dtype);
  // Only the 16-byte class has a choice to make; K and N must allow it.
  if (K % (16 / eb) != 0 || K > kMaxVectorLd || N > kMaxVectorLd) return MI_HGEMM_ERR_UNSUPPORTED;
  // fp16: integer scratch operands stay exact in fp32 only while 16*K < 2^24;
  // int8: the int32 sums stay exact.
  if (dtype == mihg::DTYPE_F16 ? K >= (1 << 20) : K > kMaxKInt8) return MI_HGEMM_ERR_UNSUPPORTED;
  if (h->no_device) return MI_HGEMM_ERR_NO_DEVICE;
  DeviceGuard g(h->device);
  if (g.err != hipSuccess) return hip_fail(h, g.err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t ldc = (N + 16 / cb - 1) / (16 / cb) * (16 / cb);

  // a, b: small integers (fp16) or uniform int8, for the bit-exact check.
  // Timing sets: random mantissas scaled by 1/sqrt(K) (the clock depends on the
  // data), or uniform int8, each with its own output, in as many copies as make
  // 2.2x the 256 MiB MALL (at most 64 copies and 4 GiB), so that the timed
  // launches read their operands from HBM and write C as in real use (one
  // output shared by every launch would stay in the MALL and flatter the
  // store-heavy candidates).
  Scratch a, b, tsets, tcs, c, cref, cnt;
  hipError_t e;
  const double set_bytes = (double)(M + N) * K * eb + (double)M * ldc * cb;
  TimingSets sets;
  sets.eb = eb;
  sets.nsets = (int)std::max(1.0, std::min({64.0, std::ceil(2.2 * 256.0 * 1048576.0 / set_bytes),
                                            std::floor(4.0 * 1073741824.0 / set_bytes)}));
  if ((e = hipMalloc(&a.p, (size_t)M * K * eb)) != hipSuccess) return hip_fail(h, e);
  if ((e = hipMalloc(&b.p, (size_t)N * K * eb)) != hipSuccess) return hip_fail(h, e);
  if ((e = hipMalloc(&tsets.p, (size_t)sets.nsets * (M + N) * K * eb)) != hipSuccess)
    return hip_fail(h, e);
  sets.base = static_cast<char*>(tsets.p);
  sets.cstride = M * ldc * cb;
  if ((e = hipMalloc(&tcs.p, (size_t)sets.nsets * sets.cstride)) != hipSuccess) return hip_fail(h, e);
  sets.cbase = static_cast<char*>(tcs.p);
  if ((e = hipMalloc(&c.p, (size_t)M * ldc * cb)) != hipSuccess) return hip_fail(h, e);
  if ((e = hipMalloc(&cref.p, (size_t)M * ldc * cb)) != hipSuccess) return hip_fail(h, e);
  if ((e = hipMalloc(&cnt.p, sizeof(int))) != hipSuccess) return hip_fail(h, e);
  const int64_t nset_elems = (int64_t)sets.nsets * (M + N) * K;
  if (dtype == mihg::DTYPE_F16) {
    if ((e = mihg::launch_fill_small_int(a.p, M * K, 0x1234u, s)) != hipSuccess) return hip_fail(h, e);
    if ((e = mihg::launch_fill_small_int(b.p, N * K, 0x5678u, s)) != hipSuccess) return hip_fail(h, e);
    const float tscale = 1.0f / std::sqrt((float)K);
    if ((e = mihg::launch_fill_uniform(tsets.p, nset_elems, 0x9abcu, tscale, s)) != hipSuccess)
      return hip_fail(h, e);
  } else {
    if ((e = mihg::launch_fill_i8(a.p, M * K, 0x1234u, s)) != hipSuccess) return hip_fail(h, e);
    if ((e = mihg::launch_fill_i8(b.p, N * K, 0x5678u, s)) != hipSuccess) return hip_fail(h, e);
    if ((e = mihg::launch_fill_i8(tsets.p, nset_elems, 0x9abcu, s)) != hipSuccess)
      return hip_fail(h, e);
  }

  // Reference result: the element-wise instance.
  Config ref;
  ref.kernel = generic_kernel(dtype);
  if (ref.kernel < 0) return MI_HGEMM_ERR_UNSUPPORTED;
  mi_hgemm_status_t st = launch(h, ref, M, N, K, a.p, K, b.p, K, cref.p, ldc, s, handle_ws(h));
  if (st != MI_HGEMM_OK) return st;

  hipEvent_t ev0, ev1;
  if ((e = hipEventCreate(&ev0)) != hipSuccess) return hip_fail(h, e);
  if ((e = hipEventCreate(&ev1)) != hipSuccess) {
    (void)hipEventDestroy(ev0);
    return hip_fail(h, e);
  }

  TimingStream ts;
  if ((e = hipStreamCreateWithFlags(&ts.s, hipStreamNonBlocking)) != hipSuccess) {
    (void)hipEventDestroy(ev0);
    (void)hipEventDestroy(ev1);
    return hip_fail(h, e);
  }
  const bool heuristic_only = (flags & MI_HGEMM_TUNE_HEURISTIC) != 0;
  const Config start = heuristic(M, N, K, make_cls(dtype, true));
  std::vector<Config> cands;
  // split K when the output tiles alone leave CUs idle
  auto add_splits = [&](int k) {
    const KernelDesc& kd = kKernels[k];
    const int64_t tiles = kd.grid((int32_t)M, (int32_t)N);
    // up to two workgroups per CU: a split can also pay where the tiles just
    // fill the CUs once (two small-LDS workgroups share a CU's copy bandwidth)
    if (!kd.splitk_ok || !h->ws || tiles >= 512) return;
    // the slices of a tile are adjacent workgroups, so the XCD remap (which
    // assumes one tile per workgroup) stays off; the raster height still
    // decides which tiles share an XCD's L2
    for (int s = 2; s <= 16; s *= 2) {
      int64_t chunk = K;
      if (K / s < 256 || tiles * s > 1024 || effective_split(kd, M, N, K, s, &chunk) < s) break;
      for (int g : {1, 4, 8}) {
        if (heuristic_only && g != 1) continue;
        Config c;
        c.kernel = k;
        c.splitk = s;
        c.group_m = g;
        cands.push_back(c);
      }
    }
  };
  for (int k = 0; k < kNumKernels; ++k) {
    const KernelDesc& kd = kKernels[k];
    if (!kd.aligned || kd.dtype != dtype) continue;
    if (kd.grid((int32_t)M, (int32_t)N) > INT32_MAX) continue;
    if (kd.split_only) {
      // unsplit, it is the same kernel as its twin plus unused bookkeeping
      add_splits(k);
    } else if (kd.family == mihg::FAMILY_TILE) {
      static const int rasters[][2] = {{1, 0}, {4, 0}, {8, 0}, {16, 0}, {1, 1}, {4, 1}, {8, 1}, {16, 1}};
      for (const auto& r : rasters) {
        if (heuristic_only && !((r[0] == 8 && r[1] == 1) || (r[0] == 1 && r[1] == 0))) continue;
        Config c;
        c.kernel = k;
        c.group_m = r[0];
        c.xcd = r[1];
        cands.push_back(c);
      }
      add_splits(k);
    } else {
      if (heuristic_only && M > 128) continue;
      Config c;
      c.kernel = k;
      cands.push_back(c);
      add_splits(k);
    }
  }
  if (std::find_if(cands.begin(), cands.end(), [&](const Config& c) {
        return c.kernel == start.kernel && c.group_m == start.group_m && c.xcd == start.xcd &&
               c.splitk == start.splitk;
      }) == cands.end())
    cands.push_back(start);

  // MI_HGEMM_TUNE_LOG=1 prints every timed candidate to stderr
  const char* log_env = std::getenv("MI_HGEMM_TUNE_LOG");
  const bool log_search = log_env && *log_env && std::strcmp(log_env, "0") != 0;
  Config best;
  best.kernel = -1;
  double best_us = 1e300;
  mi_hgemm_status_t result = MI_HGEMM_OK;
  std::vector<std::pair<double, Config>> timed;  // every correct candidate's median
  for (const Config& cand : cands) {
    // correctness first: bit-identical to the reference on exact integer data
    st = launch(h, cand, M, N, K, a.p, K, b.p, K, c.p, ldc, s, handle_ws(h));
    if (st != MI_HGEMM_OK) {
      result = st;
      break;
    }
    e = dtype == mihg::DTYPE_F16
            ? mihg::launch_count_mismatch(c.p, cref.p, (int32_t)M, (int32_t)N, ldc,
                                          static_cast<int*>(cnt.p), s)
            : mihg::launch_count_mismatch32(c.p, cref.p, (int32_t)M, (int32_t)N, ldc,
                                            static_cast<int*>(cnt.p), s);
    if (e != hipSuccess) {
      result = hip_fail(h, e);
      break;
    }
    int bad = -1;
    if ((e = hipMemcpyAsync(&bad, cnt.p, sizeof(int), hipMemcpyDeviceToHost, s)) != hipSuccess ||
        (e = hipStreamSynchronize(s)) != hipSuccess) {
      result = hip_fail(h, e);
      break;
    }
    if (bad != 0) continue;  // a wrong candidate never wins
    // time: `reps` launches (about 1 ms of work) captured in one graph on a
    // private stream and replayed, so that the figure is device time rather
    // than host launch cost; the median of 5 replays is kept
    float ms = 0.f;
    (void)hipEventRecord(ev0, s);
    (void)launch(h, cand, M, N, K, sets.A(M, N, K, 0), K, sets.B(M, N, K, 0), K, c.p, ldc, s,
                 handle_ws(h));
    (void)hipEventRecord(ev1, s);
    if ((e = hipEventSynchronize(ev1)) != hipSuccess) {
      result = hip_fail(h, e);
      break;
    }
    (void)hipEventElapsedTime(&ms, ev0, ev1);
    // about 1 ms of launches, and every timing set at least once
    const int reps = (int)std::max((double)sets.nsets,
                                   std::min(200.0, std::ceil(1.0 / std::max(1e-4, (double)ms))));
    std::vector<double> trials;
    e = time_replays(h, cand, M, N, K, sets, ldc, reps, ts.s, ev0, ev1, trials);
    if (e != hipSuccess) {
      result = hip_fail(h, e);
      break;
    }
    const double us = median(trials);
    if (log_search)
      std::fprintf(stderr, "mi_hgemm_tune %lld %lld %lld %s g%d x%d s%d %.3f us\n", (long long)M,
                   (long long)N, (long long)K, kKernels[cand.kernel].name, cand.group_m,
                   cand.xcd, cand.splitk, us);
    timed.emplace_back(us, cand);
    if (us < best_us) {
      best_us = us;
      best = cand;
      best.us = us;
    }
  }
  // Finalists: the three fastest are often within a few percent of each other,
  // about as far apart as one replay is from the next while the clock drifts
  // with power and temperature.  They are re-timed in three interleaved
  // rounds (A B C A B C A B C, 5 replays each) and the lowest median of all
  // of a finalist's 15 replays wins.
  if (result == MI_HGEMM_OK && timed.size() > 1) {
    std::sort(timed.begin(), timed.end(),
              [](const std::pair<double, Config>& x, const std::pair<double, Config>& y) {
                return x.first < y.first;
              });
    const size_t nf = std::min<size_t>(3, timed.size());
    std::vector<std::vector<double>> samples(nf);
    for (int round = 0; round < 3 && result == MI_HGEMM_OK; ++round)
      for (size_t f = 0; f < nf && result == MI_HGEMM_OK; ++f) {
        float ms = 0.f;
        const Config& cand = timed[f].second;
        (void)hipEventRecord(ev0, s);
        (void)launch(h, cand, M, N, K, sets.A(M, N, K, 0), K, sets.B(M, N, K, 0), K, c.p, ldc, s,
                     handle_ws(h));
        (void)hipEventRecord(ev1, s);
        if ((e = hipEventSynchronize(ev1)) != hipSuccess) {
          result = hip_fail(h, e);
          break;
        }
        (void)hipEventElapsedTime(&ms, ev0, ev1);
        const int reps = (int)std::max((double)sets.nsets,
                                       std::min(200.0, std::ceil(1.0 / std::max(1e-4, (double)ms))));
        e = time_replays(h, cand, M, N, K, sets, ldc, reps, ts.s, ev0, ev1, samples[f]);
        if (e != hipSuccess) result = hip_fail(h, e);
      }
    if (result == MI_HGEMM_OK) {
      best_us = 1e300;
      for (size_t f = 0; f < nf; ++f) {
        const double us = median(samples[f]);
        if (log_search) {
          const Config& cand = timed[f].second;
          const auto mm = std::minmax_element(samples[f].begin(), samples[f].end());
          std::fprintf(stderr,
                       "mi_hgemm_tune final %lld %lld %lld %s g%d x%d s%d median %.3f us min %.3f "
                       "max %.3f over %zu replays\n",
                       (long long)M, (long long)N, (long long)K, kKernels[cand.kernel].name,
                       cand.group_m, cand.xcd, cand.splitk, us, *mm.first, *mm.second,
                       samples[f].size());
        }
        if (us < best_us) {
          best_us = us;
          best = timed[f].second;
          best.us = us;
        }
      }
    }
  }
  (void)hipEventDestroy(ev0);
  (void)hipEventDestroy(ev1);
  if (result != MI_HGEMM_OK) return result;
  if (best.kernel < 0) return MI_HGEMM_ERR_UNSUPPORTED;

  const Key key{M, N, K, make_cls(dtype, true)};
  {
    std::lock_guard<std::mutex> lk(h->mu);
    h->table[key] = best;
  }
  forget_resolved(h);
  if (flags & MI_HGEMM_TUNE_PERSIST) {
    if (h->table_path.empty()) return MI_HGEMM_ERR_IO;
    FILE* f = std::fopen(h->table_path.c_str(), "a");
    if (!f) return MI_HGEMM_ERR_IO;
    const bool ok = write_entry(f, key, best);
    if (std::fclose(f) != 0 || !ok) return MI_HGEMM_ERR_IO;
  }
  return MI_HGEMM_OK;
}
