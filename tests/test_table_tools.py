"""The tuned table's tooling on the host: the shape grid that make_table
tunes, the evidence file kept across runs, and what the shipped table holds
(no GPU: make_table's tuning itself needs one and is not run here)."""
import os

import dense_fp16_gemm_hgemm_amd as mh
from dense_fp16_gemm_hgemm_amd import make_table, provenance

TABLE = os.path.join(os.path.dirname(mh.LIB_PATH), "tables", "gfx950.tsv")


def table_rows():
    with open(TABLE, encoding="utf-8") as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_grid_is_the_power_of_two_cube_less_the_named_shapes():
    grid = make_table.grid_shapes()
    named = set(make_table.default_shapes(False))
    powers = {1 << e for e in range(6, 14)}
    assert len(set(grid)) == len(grid) == 8 ** 3 - len(named & {(m, n, k) for m in powers
                                                                 for n in powers for k in powers})
    assert all(m in powers and n in powers and k in powers for m, n, k in grid)
    assert not named & set(grid)
    # the parts partition the grid
    parts = [grid[i::3] for i in range(3)]
    assert sorted(sum(parts, [])) == sorted(grid)


def test_shipped_table_covers_the_named_shapes_and_the_grid():
    rows = table_rows()
    f16 = {(int(r[1]), int(r[2]), int(r[3])) for r in rows if r[5] == "a16"}
    i8 = {(int(r[1]), int(r[2]), int(r[3])) for r in rows if r[5] == "i8a16"}
    assert set(make_table.default_shapes(False)) <= f16
    assert set(make_table.default_shapes(True)) <= i8
    assert set(make_table.grid_shapes()) <= f16
    assert len(rows) == len(f16) + len(i8)       # one entry per (shape, class)


def test_shipped_table_header_names_digest_and_commands():
    with open(TABLE, encoding="utf-8") as f:
        head = [ln for ln in f if ln.startswith("#")]
    assert f"device-source digest {provenance.source_digest()}" in head[0]
    cmds = [ln for ln in head if ln.startswith("# written") or ln.startswith("#   then")]
    assert cmds[0].startswith("# written") and "--fresh --all" in cmds[0]
    assert any("--grid --part 1/2" in c for c in cmds) and any("--grid --part 2/2" in c for c in cmds)


def test_evidence_of_a_run_keeps_the_sections_it_did_not_retune(tmp_path):
    old = tmp_path / "old_evidence.md"
    old.write_text("# old header\n\n## 64x64x64\n\nWinner: stale\n\n## int8 16x4096x4096\n\n"
                   "Winner: kept\n", encoding="utf-8")
    finals = [("64", "64", "64", "k1", "1", "0", "1", "2.0", "1.9", "2.1", "15"),
              ("64", "64", "64", "k2", "8", "1", "1", "2.2", "2.1", "2.3", "15")]
    ev = [((64, 64, 64), False, ("k1", 1, 0, 1), [0] * 3, finals, 1.5, True),
          ((128, 64, 64), False, ("k3", 1, 0, 1), [0], [], 1.0, False)]
    out = tmp_path / "new_evidence.md"
    make_table.write_evidence(str(out), ev, "gpu", keep_from=str(old))
    text = out.read_text(encoding="utf-8")
    titles = [ln for ln in text.splitlines() if ln.startswith("## ")]
    assert titles == ["## 64x64x64", "## int8 16x4096x4096", "## 128x64x64"]
    assert "stale" not in text and "Winner: kept" in text
    assert "`k1` group_m 1 xcd_remap 0 split 1; 3 candidates timed in 1.5 s (pruned list)" in text
    assert "Runner-up gap: 10.00%" in text
    assert "`k3` group_m 1 xcd_remap 0 split 1; 1 candidates timed in 1.0 s." in text
    # from nothing: only this run's sections
    fresh = tmp_path / "fresh_evidence.md"
    make_table.write_evidence(str(fresh), ev, "gpu")
    assert [ln for ln in fresh.read_text(encoding="utf-8").splitlines()
            if ln.startswith("## ")] == ["## 64x64x64", "## 128x64x64"]


def test_off_grid_shapes_take_the_nearest_grid_entry(tmp_path):
    """Between grid points the dispatcher serves a shape with the tuned entry
    nearest in log2(M) + log2(N) + log2(K) if that sum is at most 1, else with
    the built-in rules; checked against that rule worked out here over the
    shipped table's binary16 rows.  The shapes have one nearest entry (no tie)
    and N and K multiples of 8, so that the operands are in the 16-byte class."""
    import math

    rows = [r for r in table_rows() if r[5] == "a16"]
    entries = {(int(r[1]), int(r[2]), int(r[3])): (r[6], int(r[7]), int(r[8])) for r in rows}
    st, h = mh.mi_hgemm_create_ex(TABLE, mh.MI_HGEMM_CREATE_NO_DEVICE)
    assert st == mh.MI_HGEMM_OK
    st, rules = mh.mi_hgemm_create_ex(str(tmp_path / "absent.tsv"), mh.MI_HGEMM_CREATE_NO_DEVICE)
    assert st == mh.MI_HGEMM_WARN_TABLE_DEFAULTS
    names = mh.kernel_names()
    base = 0x7F0000000000

    def plan(handle, M, N, K):
        r = mh.mi_hgemm_plan(handle, M, N, K, base, K, base + (1 << 36), K, base + (2 << 36), N)
        assert r[0] == mh.MI_HGEMM_OK
        return names[r[1]], r[2], r[3]

    near = far = 0
    try:
        for M, N, K in [(1000, 3000, 520), (100, 7000, 4104), (5000, 304, 3000), (70, 9000, 1504),
                        (600, 600, 6000), (3000, 3000, 200), (3000, 200, 3000), (48, 11000, 700)]:
            dist = sorted((sum(abs(math.log2(a / b)) for a, b in zip((M, N, K), key)), key)
                          for key in entries)
            assert dist[1][0] - dist[0][0] > 1e-6, (M, N, K, dist[:2])
            if dist[0][0] <= 1:
                assert plan(h, M, N, K) == entries[dist[0][1]], (M, N, K, dist[0][1])
                near += 1
            else:
                assert plan(h, M, N, K) == plan(rules, M, N, K), (M, N, K)
                far += 1
        assert near >= 5 and far >= 2
    finally:
        mh.mi_hgemm_destroy(h)
        mh.mi_hgemm_destroy(rules)
