"""Host cost of one dispatch decision, measured in C (no Python in the loop).

mi_hgemm_run's host work per call is: validate, decide the alignment class,
resolve (M, N, K, class) -> config, then launch.  The resolution is done once
per shape and remembered in the handle, so a repeated shape -- a table hit or
a miss that fell to the nearest tuned shape or the heuristic -- costs one hash
lookup.  This test times mi_hgemm_plan, which does exactly that work without
the launch, on an inspection handle (no GPU), and prints nanoseconds per call
for a table hit, for the first and for repeated calls of a table miss.
"""
import os
import re
import shutil
import subprocess

import pytest

import dense_fp16_gemm_hgemm_amd as mh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.dirname(mh.LIB_PATH)

SOURCE = r"""
#include <stdio.h>
#include <time.h>
#include "mi_hgemm.h"

static double now_ns(void) {
  struct timespec t;
  clock_gettime(CLOCK_MONOTONIC, &t);
  return t.tv_sec * 1e9 + t.tv_nsec;
}

/* fake 256-byte aligned device addresses: an inspection handle only compares them */
#define A0 ((const void*)0x7F0000000000ull)
#define B0 ((const void*)0x7F1000000000ull)
#define C0 ((const void*)0x7F2000000000ull)

static double per_call(mi_hgemm_handle_t h, long long M, long long N, long long K, int reps,
                       int* kernel) {
  int32_t k = -2, g, x, s;
  double t0 = now_ns();
  for (int r = 0; r < reps; ++r)
    mi_hgemm_plan(h, M, N, K, A0, K, B0, K, C0, N, MI_HGEMM_LAYOUT_TN, &k, &g, &x, &s);
  *kernel = k;
  return (now_ns() - t0) / reps;
}

int main(void) {
  mi_hgemm_handle_t h;
  if (mi_hgemm_create_ex(&h, NULL, MI_HGEMM_CREATE_NO_DEVICE) != MI_HGEMM_OK) return 1;
  int k1, k2, k3;
  double hit = (per_call(h, 8192, 8192, 8192, 1, &k1), per_call(h, 8192, 8192, 8192, 200000, &k1));
  double miss_first = per_call(h, 1000, 3000, 520, 1, &k2);
  double miss_again = per_call(h, 1000, 3000, 520, 200000, &k3);
  printf("table_hit_ns %.1f\nmiss_first_ns %.1f\nmiss_repeat_ns %.1f\nkernels %d %d %d\n", hit,
         miss_first, miss_again, k1, k2, k3);
  mi_hgemm_destroy(h);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_repeated_dispatch_is_a_lookup(tmp_path, monkeypatch):
    monkeypatch.delenv("MI_HGEMM_TABLE", raising=False)
    src = tmp_path / "plan_cost.c"
    exe = tmp_path / "plan_cost"
    src.write_text(SOURCE)
    subprocess.run(["gcc", "-O2", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    "-L", PKG, "-lmi_hgemm", f"-Wl,-rpath,{PKG}"], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    print(out)
    vals = dict(re.findall(r"(\w+_ns) ([\d.]+)", out))
    kernels = [int(x) for x in re.search(r"kernels (.*)", out).group(1).split()]
    assert kernels[1] == kernels[2] >= 0, "the remembered config differs from the first"
    # a hash lookup plus validation: far below a kernel launch (microseconds)
    assert float(vals["table_hit_ns"]) < 2000
    assert float(vals["miss_repeat_ns"]) < 2000
