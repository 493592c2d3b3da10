"""CPU replay of the LDS rings of the direct-to-LDS tile kernels (no GPU).

tests/ring_model.cpp replays the stage functions the kernels use
(dense_fp16_gemm_hgemm_amd/csrc/ring_schedule.h) over whole K loops of the
d2tile (two A stages), d2tile3 (three A stages), persistent d2tile3, ktile
and pp2tile (two groups of waves in turn) rings, with the staged-C scratch and
the split-K flag word, and reports every read of a stage before its copies
have landed, every refill of a stage while
it is still read, two copies into one stage in flight together, and scratch
written over LDS still in use.  The shipped functions must replay with no
hazard; copies of them with one planted mistake each (a stage index one off,
a copy one tile short or long, a wait that leaves one copy too many in flight,
A's and B's copies issued in the wrong order) must each be caught.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_fp16_gemm_hgemm_amd", "csrc")
MODEL = os.path.join(ROOT, "tests", "ring_model.cpp")
HEADER = os.path.join(CSRC, "ring_schedule.h")

MUTANTS = {
    "d2_refill_the_next_tiles_stage": (
        "t.wa = SA == 2 ? (ra ^ 1) : (ra == 0 ? 2 : ra - 1);",
        "t.wa = SA == 2 ? (ra ^ 1) : (ra == 2 ? 0 : ra + 1);"),
    "d2_a_copy_one_tile_short": ("t.ta = kt + SA - 1;", "t.ta = kt + SA - 2;"),
    "d2_b_copy_one_tile_long": ("t.tb = kt + 1;", "t.tb = kt + 2;"),
    "d2_wait_leaves_one_copy_more": ("return SA == 3 ? a_blk : 0;", "return SA == 3 ? a_blk + 1 : 0;"),
    "d2_a_copies_issued_first": ("MIHG_RING_FN bool d2_b_first(int SA) { return SA == 3; }",
                                 "MIHG_RING_FN bool d2_b_first(int SA) { return SA != SA; }"),
    "k_read_stage_one_off": ("t.ra = kt % S;", "t.ra = (kt + 1) % S;"),
    "k_refill_the_stage_being_read": ("t.wa = (kt + S - 1) % S;", "t.wa = (kt + S) % S;"),
    "k_b_copy_one_tile_long": ("t.tb = kt + SB - 1;", "t.tb = kt + SB;"),
    "k_wait_leaves_a_trip_more": ("return a_blk * (S - 2) + b_blk * (SB - 2);",
                                  "return a_blk * (S - 1) + b_blk * (SB - 2);"),
    "pp_a_refills_the_stage_being_read": ("t.wa = (kt + 2) % 3;", "t.wa = (kt + 1) % 3;"),
    "pp_b_refills_the_next_tiles_stage": ("t.wb = kt & 1;", "t.wb = (kt + 1) & 1;"),
    "pp_a_wait_one_tile_short": ("MIHG_RING_FN int pp_in_flight_a(int a_blk) { return a_blk; }",
                                 "MIHG_RING_FN int pp_in_flight_a(int a_blk) { return 2 * a_blk; }"),
    "pp_b_wait_leaves_a_copy": ("MIHG_RING_FN int pp_in_flight_b(int) { return 0; }",
                                "MIHG_RING_FN int pp_in_flight_b(int) { return 1; }"),
    "k_a_copies_issued_first": ("MIHG_RING_FN bool k_b_first(int S, int SB) { return SB != S; }",
                                "MIHG_RING_FN bool k_b_first(int S, int SB) { return S != S + SB - SB; }"),
}

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def build_and_run(tmp_path, header_text=None):
    inc = os.path.dirname(HEADER)
    if header_text is not None:
        inc = str(tmp_path / "inc")
        os.makedirs(inc, exist_ok=True)
        with open(os.path.join(inc, "ring_schedule.h"), "w") as f:
            f.write(header_text)
    exe = tmp_path / "ring_model"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", inc, MODEL, "-o", str(exe)], check=True)
    return subprocess.run([str(exe)], capture_output=True, text=True)


def test_shipped_rings_have_no_hazard(tmp_path):
    r = build_and_run(tmp_path)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-3000:]
    assert "0 with hazards" in r.stdout


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(HEADER, encoding="utf-8").read()
    assert text.count(old) == 1, f"mutation site of {name} not found once"
    r = build_and_run(tmp_path, text.replace(old, new))
    assert r.returncode == 1 and "HAZARD" in r.stdout, f"{name} was not caught:\n{r.stdout[-1500:]}"
