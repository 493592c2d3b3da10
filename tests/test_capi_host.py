"""Host-side checks of the C ABI (no GPU, no kernel launches).

The library must load and export every function include/mi_hgemm.h declares;
argument validation, the alignment-class decision, table parsing and dispatch
are checked through an inspection handle (MI_HGEMM_CREATE_NO_DEVICE), with
fake device addresses that the library only compares, never dereferences.
"""
import os
import re

import pytest
import torch

import dense_fp16_gemm_hgemm_amd as mh

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "mi_hgemm.h")
BASE = 0x7F0000000000  # fake, 256-byte aligned device addresses
A0, B0, C0 = BASE, BASE + (1 << 36), BASE + (2 << 36)


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mi_hgemm_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("mi_hgemm_create", "mi_hgemm_run", "mi_hgemm_tune", "mi_hgemm_destroy",
                 "mi_hgemm_status_string"):
        assert must in names


def test_library_exports_every_declared_symbol():
    import ctypes
    lib = ctypes.CDLL(mh.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings():
    for st in range(7):
        assert mh.mi_hgemm_status_string(st).startswith("MI_HGEMM_")
    assert mh.mi_hgemm_status_string(99) == "MI_HGEMM_UNKNOWN_STATUS"


def test_kernel_registry():
    names = mh.kernel_names()
    assert len(names) == mh.mi_hgemm_kernel_count() > 10
    assert names[0] == "generic_64x64_w2x2_m32"
    assert len(set(names)) == len(names)
    assert mh.mi_hgemm_kernel_name(-1) is None
    assert mh.mi_hgemm_kernel_name(len(names)) is None


@pytest.mark.skipif(torch.cuda.is_available(), reason="a GPU is visible")
def test_create_without_device_reports_no_device():
    st, h = mh.mi_hgemm_create()
    assert st == mh.MI_HGEMM_ERR_NO_DEVICE and h is None


@pytest.fixture
def inspect_handle(tmp_path, monkeypatch):
    monkeypatch.delenv("MI_HGEMM_TABLE", raising=False)
    st, h = mh.mi_hgemm_create_ex(str(tmp_path / "absent.tsv"), mh.MI_HGEMM_CREATE_NO_DEVICE)
    assert st == mh.MI_HGEMM_WARN_TABLE_DEFAULTS  # a named table that is missing
    yield h
    mh.mi_hgemm_destroy(h)


def plan(h, M, N, K, lda=None, ldb=None, ldc=None, A=A0, B=B0, C=C0, layout=0):
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return mh.mi_hgemm_plan(h, M, N, K, A, lda, B, ldb, C, ldc, layout)


def test_validation_status_codes(inspect_handle):
    h = inspect_handle
    ok, bad, uns = mh.MI_HGEMM_OK, mh.MI_HGEMM_ERR_INVALID_ARG, mh.MI_HGEMM_ERR_UNSUPPORTED
    assert plan(h, 64, 64, 64)[0] == ok
    assert plan(h, -1, 64, 64)[0] == bad
    assert plan(h, 64, -1, 64)[0] == bad
    assert plan(h, 64, 64, -1)[0] == bad
    assert plan(h, 64, 64, 64, lda=63)[0] == bad
    assert plan(h, 64, 64, 64, ldb=63)[0] == bad
    assert plan(h, 64, 64, 64, ldc=63)[0] == bad
    assert plan(h, 64, 64, 64, layout=1)[0] == uns
    assert plan(h, 2 ** 31, 64, 64, lda=64)[0] == uns
    assert plan(h, 64, 64, 64, A=0)[0] == bad
    assert plan(h, 64, 64, 64, B=0)[0] == bad
    assert plan(h, 64, 64, 64, C=0)[0] == bad
    # C overlapping an operand
    assert plan(h, 64, 64, 64, C=A0 + 128)[0] == bad
    assert plan(h, 64, 64, 64, C=B0 + 2 * 64 * 64 - 2)[0] == bad
    assert plan(h, 64, 64, 64, C=B0 + 2 * 64 * 64)[0] == ok   # adjacent, not overlapping
    assert mh.mi_hgemm_plan(None, 1, 1, 1, A0, 1, B0, 1, C0, 1)[0] == bad


def test_empty_and_k_zero_launch_nothing(inspect_handle):
    h = inspect_handle
    assert plan(h, 0, 64, 64, A=0, B=0, C=0) == (mh.MI_HGEMM_OK, -1, 1, 0, 1)
    assert plan(h, 64, 0, 64, A=0, B=0, C=0, ldc=1)[:2] == (mh.MI_HGEMM_OK, -1)
    assert plan(h, 64, 0, 64, A=0, B=0, C=0, ldc=0)[0] == mh.MI_HGEMM_ERR_INVALID_ARG
    assert plan(h, 64, 64, 0, lda=1, ldb=1, A=0, B=0)[:2] == (mh.MI_HGEMM_OK, -1)  # K == 0: fill only


def test_inspection_handle_does_not_launch(inspect_handle):
    h = inspect_handle
    st = mh.mi_hgemm_run(h, 64, 64, 64, A0, 64, B0, 64, C0, 64)
    assert st == mh.MI_HGEMM_ERR_NO_DEVICE
    assert mh.mi_hgemm_run(h, 0, 64, 64, 0, 64, 0, 64, 0, 64) == mh.MI_HGEMM_OK
    assert mh.mi_hgemm_tune(h, 64, 64, 64) == mh.MI_HGEMM_ERR_NO_DEVICE
    assert mh.mi_hgemm_run_kernel(h, 0, 1, 0, 1, 64, 64, 64, A0, 64, B0, 64, C0, 64) == \
        mh.MI_HGEMM_ERR_NO_DEVICE
    assert mh.mi_hgemm_run_kernel(h, 999, 1, 0, 1, 64, 64, 64, A0, 64, B0, 64, C0, 64) == \
        mh.MI_HGEMM_ERR_UNSUPPORTED
    assert mh.mi_hgemm_run_kernel(h, 0, 0, 0, 1, 64, 64, 64, A0, 64, B0, 64, C0, 64) == \
        mh.MI_HGEMM_ERR_INVALID_ARG
    assert mh.mi_hgemm_run_kernel(h, 0, 1, 0, 0, 64, 64, 64, A0, 64, B0, 64, C0, 64) == \
        mh.MI_HGEMM_ERR_INVALID_ARG
    assert mh.mi_hgemm_run_kernel(h, 0, 1, 0, 2, 64, 64, 64, A0, 64, B0, 64, C0, 64) == \
        mh.MI_HGEMM_ERR_UNSUPPORTED   # the element-wise instance has no split-K


def test_misalignment_selects_the_elementwise_instance(inspect_handle):
    h = inspect_handle
    generic = 0
    assert plan(h, 256, 256, 256)[1] != generic
    assert plan(h, 256, 256, 256, A=A0 + 2)[1] == generic      # A not 16-byte aligned
    assert plan(h, 256, 256, 256, C=C0 + 8)[1] == generic      # C not 16-byte aligned
    assert plan(h, 256, 256, 250)[1] == generic                # K not a multiple of 8
    assert plan(h, 256, 256, 256, lda=260)[1] == generic       # lda not a multiple of 8
    assert plan(h, 256, 256, 256, ldb=264)[1] != generic       # padded but aligned
    assert plan(h, 256, 256, 256, ldb=(1 << 21) + 8)[1] == generic  # beyond 32-bit tile offsets
    aligned_only = mh.mi_hgemm_run_kernel(h, 1, 1, 0, 1, 256, 256, 250, A0, 256, B0, 256, C0, 256)
    assert aligned_only == mh.MI_HGEMM_ERR_UNSUPPORTED


def test_heuristic_picks_by_shape(inspect_handle):
    h = inspect_handle
    names = mh.kernel_names()

    def choice(M, N, K):
        r = plan(h, M, N, K)
        assert r[0] == mh.MI_HGEMM_OK
        return names[r[1]], r[4]

    # five eighths of a wave or more of 256x256 tiles keeps the large tile, in
    # its ping-pong form (binary16 picks stage C through LDS for whole-line stores)
    assert choice(8192, 8192, 8192) == ("pp2tile_256x256_w8_m16_sc", 1)
    assert choice(8192, 8192, 64) == ("pp2tile_256x256_w8_m16_sc", 1)
    assert choice(4096, 4096, 4096) == ("pp2tile_256x256_w8_m16_sc", 1)
    assert choice(1024, 14336, 4096) == ("pp2tile_256x256_w8_m16_sc", 1)
    assert choice(1024, 11008, 4096) == ("pp2tile_256x256_w8_m16_sc", 1)
    # its raster: XCD-local groups of 8 tile rows up to one wave, row-major above
    assert plan(h, 4096, 4096, 1024)[2:4] == (8, 1)
    assert plan(h, 1024, 14336, 4096)[2:4] == (8, 1)
    assert plan(h, 8192, 4096, 1024)[2:4] == (1, 0)
    assert plan(h, 8192, 8192, 8192)[2:4] == (1, 0)
    # 96..159 tiles of 256x128 over a long K: the same tile split in two along K
    assert choice(1024, 4096, 11008) == ("pp2tile_256x128_w8_m16_sc_sk", 2)
    assert choice(8192, 512, 8192)[0] != "pp2tile_256x128_w8_m16_sc_sk"   # narrow N
    # below that, two waves or more of 128x128 direct-to-LDS tiles, at any K
    assert choice(2048, 4096, 64) == ("d2tile_128x128_w2x2_m16_sc", 1)
    assert choice(2048, 4096, 4096) == ("d2tile_128x128_w2x2_m16_sc", 1)
    assert choice(4096, 2048, 8192) == ("d2tile_128x128_w2x2_m16_sc", 1)
    # then deep-K 128x128 tiles while there are 128 of them
    assert choice(1024, 4096, 4096) == ("ktile_128x128_w2x4_k128_s3b2_sc", 1)
    assert choice(256, 11008, 4096) == ("ktile_128x128_w2x4_k128_s3b2_sc", 1)
    # then 64x64, split over K when the tiles are few and K is long; when the
    # output is one row of tiles B is streamed once and copied non-temporally
    assert choice(256, 4096, 4096) == ("ktile_64x64_w2x2_k128_s3b3_sc", 1)
    assert choice(64, 11008, 4096) == ("ktile_64x64_w2x2_k128_s3_nt", 1)
    assert choice(64, 4096, 11008) == ("ktile_64x64_w2x2_k128_s3_nt", 4)
    # M <= 64 over a short K: 32x64 tiles, split to fill the device (two rows
    # of tiles read B twice: the cached copy)
    assert choice(64, 4096, 4096) == ("ktile_32x64_w2x2_k128_s3b3_sc", 2)
    assert choice(32, 4096, 4096) == ("ktile_32x64_w2x2_k128_s3_nt", 4)
    # 16 rows: 16x64 deep-K tiles for wide or deep shapes, skinny otherwise
    assert choice(16, 14336, 4096) == ("ktile_16x64_w1x4_k128_s3_nt", 1)
    assert choice(16, 4096, 11008) == ("ktile_16x64_w1x4_k128_s3_nt", 4)
    assert choice(16, 4096, 4096) == ("skinny_1x1_w4_u4", 1)
    # a short K is never split
    assert choice(256, 4096, 1024)[1] == 1


def test_nearest_table_entry_drops_a_split_that_does_not_fit(tmp_path, monkeypatch):
    """A nearest-shape entry's K split is checked against the shape it serves:
    partial tiles beyond the workspace fall back to no split, not an error."""
    monkeypatch.delenv("MI_HGEMM_TABLE", raising=False)
    p = tmp_path / "t.tsv"
    # 256x128 tiles: 32 x 112 tiles x 8 slices x 128 KiB = 3.5 GiB >> 64 MiB workspace
    p.write_text("gfx950 8192 14336 4096 TN a16 dtile_256x128_w2x2_m16_s4 1 0 1.0 8\n")
    st, h = mh.mi_hgemm_create_ex(str(p), mh.MI_HGEMM_CREATE_NO_DEVICE)
    assert st == mh.MI_HGEMM_OK
    try:
        names = mh.kernel_names()
        r = plan(h, 8192, 14336, 4096)
        assert names[r[1]] == "dtile_256x128_w2x2_m16_s4" and r[4] == 1
        r = plan(h, 8192, 14336, 6144)                # nearest entry, same result
        assert names[r[1]] == "dtile_256x128_w2x2_m16_s4" and r[4] == 1
    finally:
        mh.mi_hgemm_destroy(h)


def test_table_split_k_column(tmp_path, monkeypatch):
    monkeypatch.delenv("MI_HGEMM_TABLE", raising=False)
    names = mh.kernel_names()
    p = tmp_path / "sk.tsv"
    write_table(p, ["gfx950 256 4096 4096 TN a16 dtile_128x128_w2x2_m16_s4 1 0 9.0 4",
                    "gfx950 128 128 128 TN a16 tile_64x64_w2x2_m16 1 0 1.0 4"])  # no split-K
    st, h = mh.mi_hgemm_create_ex(str(p), mh.MI_HGEMM_CREATE_NO_DEVICE)
    assert st == mh.MI_HGEMM_WARN_TABLE_DEFAULTS and mh.mi_hgemm_table_size(h) == 1
    r = plan(h, 256, 4096, 4096)
    assert names[r[1]] == "dtile_128x128_w2x2_m16_s4" and r[4] == 4
    mh.mi_hgemm_destroy(h)


def write_table(path, lines):
    with open(path, "w") as f:
        f.write("# arch M N K layout align kernel group_m xcd_remap us\n")
        for ln in lines:
            f.write(ln + "\n")


def test_table_exact_and_nearest_shape(tmp_path, monkeypatch):
    monkeypatch.delenv("MI_HGEMM_TABLE", raising=False)
    names = mh.kernel_names()
    p = tmp_path / "t.tsv"
    write_table(p, ["gfx950 1000 2000 3000 TN a16 tile_64x64_w2x2_m16 4 1 12.5",
                    "gfx942 1000 2000 3000 TN a16 tile_32x32_w2x2_m16 1 0 1.0",  # other arch: skipped
                    "gfx950 512 512 512 TN any generic_64x64_w2x2_m32 2 0 3.0"])
    st, h = mh.mi_hgemm_create_ex(str(p), mh.MI_HGEMM_CREATE_NO_DEVICE)
    assert st == mh.MI_HGEMM_OK
    try:
        assert mh.mi_hgemm_table_size(h) == 2
        r = plan(h, 1000, 2000, 3000)
        assert names[r[1]] == "tile_64x64_w2x2_m16" and r[2:] == (4, 1, 1)
        r = plan(h, 1000, 2000, 3000 * 2)                  # one factor of 2 away: nearest entry
        assert names[r[1]] == "tile_64x64_w2x2_m16"
        r = plan(h, 1000 * 4, 2000, 3000)                  # too far: heuristics
        assert names[r[1]] != "tile_64x64_w2x2_m16"
        r = plan(h, 512, 512, 512, lda=516)                # unaligned class entry
        assert r[1:] == (0, 2, 0, 1)
        out = tmp_path / "saved.tsv"
        assert mh.mi_hgemm_table_save(h, str(out)) == mh.MI_HGEMM_OK
        st2, h2 = mh.mi_hgemm_create_ex(str(out), mh.MI_HGEMM_CREATE_NO_DEVICE)
        assert st2 == mh.MI_HGEMM_OK and mh.mi_hgemm_table_size(h2) == 2
        mh.mi_hgemm_destroy(h2)
        assert mh.mi_hgemm_table_save(h, str(tmp_path / "no" / "dir.tsv")) == mh.MI_HGEMM_ERR_IO
    finally:
        mh.mi_hgemm_destroy(h)


def test_corrupt_table_warns_and_keeps_good_lines(tmp_path, monkeypatch):
    monkeypatch.delenv("MI_HGEMM_TABLE", raising=False)
    p = tmp_path / "bad.tsv"
    write_table(p, ["gfx950 1000 2000 3000 TN a16 tile_64x64_w2x2_m16 4 1 12.5",
                    "gfx950 not a number",
                    "gfx950 64 64 64 TN a16 no_such_kernel 1 0 1.0",
                    "gfx950 64 64 64 TN any tile_128x128_w2x2_m32 1 0 1.0",  # aligned kernel in 'any'
                    "gfx950 64 64 64 TN a16 tile_32x32_w2x2_m16 0 0 1.0"])   # group_m < 1
    st, h = mh.mi_hgemm_create_ex(str(p), mh.MI_HGEMM_CREATE_NO_DEVICE)
    assert st == mh.MI_HGEMM_WARN_TABLE_DEFAULTS
    assert mh.mi_hgemm_table_size(h) == 1
    mh.mi_hgemm_destroy(h)


def test_table_from_environment(tmp_path, monkeypatch):
    p = tmp_path / "env.tsv"
    write_table(p, ["gfx950 64 64 64 TN a16 tile_32x32_w2x2_m16 1 0 1.0"])
    monkeypatch.setenv("MI_HGEMM_TABLE", str(p))
    st, h = mh.mi_hgemm_create_ex(None, mh.MI_HGEMM_CREATE_NO_DEVICE)
    assert st == mh.MI_HGEMM_OK and mh.mi_hgemm_table_size(h) == 1
    mh.mi_hgemm_destroy(h)


def test_create_rejects_null_out():
    import ctypes
    lib = ctypes.CDLL(mh.LIB_PATH)
    lib.mi_hgemm_create.restype = ctypes.c_int
    lib.mi_hgemm_create.argtypes = [ctypes.c_void_p, ctypes.c_char_p]
    assert lib.mi_hgemm_create(None, None) == mh.MI_HGEMM_ERR_INVALID_ARG


# ------------------------------------------------------------ int8 variant --

def plan_i8(h, M, N, K, lda=None, ldb=None, ldc=None, A=A0, B=B0, C=C0, layout=0):
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return mh.mi_hgemm_plan_i8(h, M, N, K, A, lda, B, ldb, C, ldc, layout)


def test_int8_registry_and_validation(inspect_handle):
    h = inspect_handle
    names = mh.kernel_names()
    i8 = [n for n in names if n.startswith("i8_")]
    assert "i8_generic_64x64_w2x2_m16" in i8 and len(i8) >= 8
    ok, bad, uns = mh.MI_HGEMM_OK, mh.MI_HGEMM_ERR_INVALID_ARG, mh.MI_HGEMM_ERR_UNSUPPORTED
    assert plan_i8(h, 64, 64, 64)[0] == ok
    assert plan_i8(h, 64, 64, 64, lda=63)[0] == bad
    assert plan_i8(h, 64, 64, 64, layout=1)[0] == uns
    # the int32 sum is exact up to K = 131071
    assert plan_i8(h, 4, 4, 131071)[0] == ok
    assert plan_i8(h, 4, 4, 131072)[0] == uns
    assert plan(h, 4, 4, 131072)[0] == ok                  # the fp16 path has no such limit
    # overlap is measured in the variant's element sizes: int8 operands, int32 C
    assert plan_i8(h, 64, 64, 64, C=B0 + 64 * 64 - 1)[0] == bad
    assert plan_i8(h, 64, 64, 64, C=B0 + 64 * 64)[0] == ok
    assert plan_i8(h, 64, 64, 64, A=C0 + 4 * 64 * 64 - 4, C=C0)[0] == bad
    assert plan_i8(h, 64, 64, 64, A=C0 + 4 * 64 * 64, C=C0)[0] == ok
    # K == 0 launches only the fill
    assert plan_i8(h, 64, 64, 0, lda=1, ldb=1, A=0, B=0)[:2] == (ok, -1)


def test_int8_alignment_class_and_heuristic(inspect_handle):
    h = inspect_handle
    names = mh.kernel_names()
    generic = names.index("i8_generic_64x64_w2x2_m16")

    def choice(M, N, K, **kw):
        r = plan_i8(h, M, N, K, **kw)
        assert r[0] == mh.MI_HGEMM_OK
        return names[r[1]], r[4]

    for M, N, K in ((8192, 8192, 8192), (1024, 4096, 4096), (64, 4096, 11008), (16, 4096, 4096)):
        n, _ = choice(M, N, K)
        assert n.startswith("i8_") and n != names[generic], (M, N, K, n)
    assert choice(8192, 8192, 8192)[0] == "i8_pp2tile_256x256_w8_m16"
    assert choice(1024, 11008, 4096)[0] == "i8_pp2tile_256x256_w8_m16"
    assert choice(1024, 4096, 4096)[0] == "i8_ktile_128x128_w2x4_k256_s3b2"
    assert choice(16, 4096, 4096)[0] == "i8_ktile_16x64_w1x4_k256_s3_nt"
    # the 16-byte class in int8 elements: K, lda, ldb multiples of 16, ldc of 4
    assert plan_i8(h, 256, 256, 264)[1] == generic              # K = 8 mod 16
    assert plan_i8(h, 256, 256, 256, lda=264)[1] == generic
    assert plan_i8(h, 256, 256, 256, ldb=272)[1] != generic
    assert plan_i8(h, 256, 256, 256, ldc=260)[1] != generic     # 4 int32 = 16 bytes
    assert plan_i8(h, 256, 256, 256, ldc=258)[1] == generic
    assert plan_i8(h, 256, 256, 256, A=A0 + 8)[1] == generic


def test_int8_instances_refuse_fp16_class_and_vice_versa(inspect_handle):
    """run_kernel validates with the instance's own element type: an int8
    instance checks int8 alignment rules, and fp16 rules stay with fp16."""
    h = inspect_handle
    names = mh.kernel_names()
    k = names.index("i8_ktile_64x64_w2x2_k256_s3")
    # K = 40 is in the fp16 16-byte class but not the int8 one
    assert mh.mi_hgemm_run_kernel(h, k, 1, 0, 1, 64, 64, 40, A0, 64, B0, 64, C0, 64) == \
        mh.MI_HGEMM_ERR_UNSUPPORTED
    assert mh.mi_hgemm_run_kernel(h, k, 1, 0, 1, 64, 64, 48, A0, 64, B0, 64, C0, 64) == \
        mh.MI_HGEMM_ERR_NO_DEVICE
    assert mh.mi_hgemm_run_kernel(h, k, 1, 0, 1, 64, 64, 131072, A0, 131072, B0, 131072, C0,
                                  64) == mh.MI_HGEMM_ERR_UNSUPPORTED


def test_int8_table_classes(tmp_path, monkeypatch):
    monkeypatch.delenv("MI_HGEMM_TABLE", raising=False)
    names = mh.kernel_names()
    p = tmp_path / "i8.tsv"
    write_table(p, ["gfx950 1024 4096 4096 TN i8a16 i8_ktile_64x128_w2x2_k256_s3 4 1 30.0 2",
                    "gfx950 1024 4096 4096 TN a16 ktile_64x64_w2x2_k128_s3 8 0 40.0 1",
                    "gfx950 77 77 77 TN i8any i8_generic_64x64_w2x2_m16 1 0 2.0"])
    st, h = mh.mi_hgemm_create_ex(str(p), mh.MI_HGEMM_CREATE_NO_DEVICE)
    assert st == mh.MI_HGEMM_OK and mh.mi_hgemm_table_size(h) == 3
    try:
        r = plan_i8(h, 1024, 4096, 4096)
        assert names[r[1]] == "i8_ktile_64x128_w2x2_k256_s3" and r[2:] == (4, 1, 2)
        r = plan(h, 1024, 4096, 4096)                 # same shape, fp16 entry
        assert names[r[1]] == "ktile_64x64_w2x2_k128_s3" and r[2:] == (8, 0, 1)
        out = tmp_path / "saved.tsv"
        assert mh.mi_hgemm_table_save(h, str(out)) == mh.MI_HGEMM_OK
        text = out.read_text()
        assert " i8a16 i8_ktile_64x128_w2x2_k256_s3 " in text and " i8any " in text
    finally:
        mh.mi_hgemm_destroy(h)
    # an entry whose kernel does not match its class marks the table as damaged
    write_table(p, ["gfx950 64 64 64 TN i8a16 ktile_64x64_w2x2_k128_s3 1 0 1.0",
                    "gfx950 64 64 64 TN a16 i8_ktile_64x64_w2x2_k256_s3 1 0 1.0",
                    "gfx950 64 64 64 TN i8any i8_ktile_64x64_w2x2_k256_s3 1 0 1.0"])
    st, h = mh.mi_hgemm_create_ex(str(p), mh.MI_HGEMM_CREATE_NO_DEVICE)
    assert st == mh.MI_HGEMM_WARN_TABLE_DEFAULTS and mh.mi_hgemm_table_size(h) == 0
    mh.mi_hgemm_destroy(h)


def test_run_kernel_rejects_operands_of_the_other_type():
    """The binding refuses to pair an instance with tensors of the other element
    type, before anything reaches the C ABI (it needs no GPU)."""
    h = mh.Hgemm(inspect_only=True)
    try:
        a = torch.zeros((4, 16), dtype=torch.float16)
        with pytest.raises(TypeError):
            h.run_kernel("i8_ktile_64x64_w2x2_k256_s3", a, a)
        b = torch.zeros((4, 16), dtype=torch.int8)
        with pytest.raises(TypeError):
            h.run_kernel("ktile_64x64_w2x2_k128_s3", b, b)
    finally:
        h.close()


def test_shipped_table_loads_whole_and_dispatches_its_entries(monkeypatch):
    """Every line of the shipped table names a compiled instance of the right
    class with a valid raster, and is what dispatch picks for its shape."""
    monkeypatch.delenv("MI_HGEMM_TABLE", raising=False)
    path = os.path.join(os.path.dirname(mh.LIB_PATH), "tables", "gfx950.tsv")
    rows = [ln.split() for ln in open(path, encoding="utf-8")
            if ln.strip() and not ln.lstrip().startswith("#")]
    st, h = mh.mi_hgemm_create_ex(path, mh.MI_HGEMM_CREATE_NO_DEVICE)
    assert st == mh.MI_HGEMM_OK
    try:
        assert mh.mi_hgemm_table_size(h) == len(rows)
        names = mh.kernel_names()
        for r in rows:
            M, N, K = int(r[1]), int(r[2]), int(r[3])
            kernel, gm, xcd = r[6], int(r[7]), int(r[8])
            split = int(r[10]) if len(r) > 10 else 1
            assert r[0] == "gfx950" and r[4] == "TN"
            fn = plan_i8 if r[5].startswith("i8") else plan
            got = fn(h, M, N, K)
            assert got[0] == mh.MI_HGEMM_OK, r
            assert (names[got[1]], got[2], got[3]) == (kernel, gm, xcd), r
            assert got[4] <= split, r
    finally:
        mh.mi_hgemm_destroy(h)
