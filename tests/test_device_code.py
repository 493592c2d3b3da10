"""Every registered kernel instance has device code for gfx950 in libmi_hgemm.so.

Host-only check: the .hip_fatbin section of the library is unbundled with the
ROCm clang-offload-bundler and its symbol table read with llvm-readelf.  A
registry entry whose kernel template was never instantiated in the device pass
would otherwise only show up as a launch failure on the GPU.
"""
import os
import re
import shutil
import subprocess

import pytest

import dense_fp16_gemm_hgemm_amd as mh

LLVM = "/opt/rocm/lib/llvm/bin"


def mangled(name):
    if name.startswith("i8_"):
        return mangled_i8(name[3:])
    m = re.fullmatch(r"(tile|generic)_(\d+)x(\d+)_w(\d+)x(\d+)_m(\d+)", name)
    if m:
        kind, bm, bn, wm, wn, mf = m.groups()
        tmpl = f"{len(kind) + 7}{kind}_kernel"
        return f"_ZN4mihg{tmpl}ILi{bm}ELi{bn}ELi{wm}ELi{wn}ELi{mf}EEEvNS_8GemmArgsE"
    m = re.fullmatch(r"d2tile_(\d+)x(\d+)_w(\d+)x(\d+)_m16", name)
    if m:
        bm, bn, wm, wn = m.groups()
        return f"_ZN4mihg13d2tile_kernelILi{bm}ELi{bn}ELi{wm}ELi{wn}EEEvNS_8GemmArgsE"
    m = re.fullmatch(r"d2tile3_(\d+)x(\d+)_w(\d+)x(\d+)_m(\d+)", name)
    if m:
        bm, bn, wm, wn, mf = m.groups()
        return f"_ZN4mihg14d2tile3_kernelILi{bm}ELi{bn}ELi{wm}ELi{wn}ELi{mf}EEEvNS_8GemmArgsE"
    m = re.fullmatch(r"pp2tile_(\d+)x(\d+)_w8_m(\d+)(_sc)?(_sk)?", name)
    if m:
        bm, bn, mf, sc, sk = m.groups()
        b = 1 if sk else 0
        if sc:
            return f"_ZN4mihg16pp2tilesc_kernelILi{bm}ELi{bn}ELb{b}EEEvNS_8GemmArgsE"
        return f"_ZN4mihg14pp2tile_kernelILi{bm}ELi{bn}ELi{mf}ELb{b}EEEvNS_8GemmArgsE"
    m = re.fullmatch(r"pptile_(\d+)x(\d+)_w8_m16", name)
    if m:
        bm, bn = m.groups()
        return f"_ZN4mihg13pptile_kernelILi{bm}ELi{bn}EEEvNS_8GemmArgsE"
    m = re.fullmatch(r"(dtile)_(\d+)x(\d+)_w(\d+)x(\d+)_m(\d+)_(?:la|s)(\d+)", name)
    if m:
        kind, bm, bn, wm, wn, mf, x = m.groups()
        return (f"_ZN4mihg12{kind}_kernelILi{bm}ELi{bn}ELi{wm}ELi{wn}ELi{mf}ELi{x}"
                "EEEvNS_8GemmArgsE")
    m = re.fullmatch(r"ktile_(\d+)x(\d+)_w(\d+)x(\d+)_k(\d+)_s(\d+)(?:b(\d+))?", name)
    if m:
        bm, bn, wm, wn, bk, s, sb = m.groups()
        return (f"_ZN4mihg12ktile_kernelILi{bm}ELi{bn}ELi{wm}ELi{wn}ELi{int(bk) // 64}ELi{s}"
                f"ELi{sb or s}EEEvNS_8GemmArgsE")
    m = re.fullmatch(r"ktile_(\d+)x(\d+)_w(\d+)x(\d+)_k(\d+)_s(\d+)_nt", name)
    if m:
        bm, bn, wm, wn, bk, s = m.groups()
        return (f"_ZN4mihg15ktile_nt_kernelILi{bm}ELi{bn}ELi{wm}ELi{wn}ELi{int(bk) // 64}ELi{s}"
                "EEEvNS_8GemmArgsE")
    m = re.fullmatch(r"ktile_(\d+)x(\d+)_w(\d+)x(\d+)_k(\d+)_s(\d+)b(\d+)_noxor", name)
    if m:
        bm, bn, wm, wn, bk, s, sb = m.groups()
        return (f"_ZN4mihg15ktile_ns_kernelILi{bm}ELi{bn}ELi{wm}ELi{wn}ELi{int(bk) // 64}ELi{s}"
                f"ELi{sb}EEEvNS_8GemmArgsE")
    m = re.fullmatch(r"ktile_(\d+)x(\d+)_w(\d+)x(\d+)_k(\d+)_s(\d+)b(\d+)_sc", name)
    if m:
        bm, bn, wm, wn, bk, s, sb = m.groups()
        return (f"_ZN4mihg14ktilesc_kernelILi{bm}ELi{bn}ELi{wm}ELi{wn}ELi{int(bk) // 64}ELi{s}"
                f"ELi{sb}EEEvNS_8GemmArgsE")
    m = re.fullmatch(r"(d2tile3p|d2tile3|d2tile)_(\d+)x(\d+)_w(\d+)x(\d+)_m16_sc", name)
    if m:
        kind, bm, bn, wm, wn = m.groups()
        kname = {"d2tile3p": "d2tile3psc", "d2tile3": "d2tile3sc", "d2tile": "d2tilesc"}[kind]
        return f"_ZN4mihg{len(kname) + 7}{kname}_kernelILi{bm}ELi{bn}ELi{wm}ELi{wn}EEEvNS_8GemmArgsE"
    m = re.fullmatch(r"d2tile3p_(\d+)x(\d+)_w(\d+)x(\d+)_m(\d+)", name)
    if m:
        bm, bn, wm, wn, mf = m.groups()
        return f"_ZN4mihg15d2tile3p_kernelILi{bm}ELi{bn}ELi{wm}ELi{wn}ELi{mf}EEEvNS_8GemmArgsE"
    m = re.fullmatch(r"d2tile3_(\d+)x(\d+)_w(\d+)x(\d+)_m(\d+)_noxor", name)
    if m:
        bm, bn, wm, wn, mf = m.groups()
        return f"_ZN4mihg17d2tile3_ns_kernelILi{bm}ELi{bn}ELi{wm}ELi{wn}ELi{mf}EEEvNS_8GemmArgsE"
    m = re.fullmatch(r"skinny_(\d+)x(\d+)_w(\d+)_u(\d+)(?:_d(\d+))?", name)
    if m:
        fm, fn, w, u, d = m.groups()
        return (f"_ZN4mihg13skinny_kernelILi{fm}ELi{fn}ELi{w}ELi{u}ELi{d or 2}"
                "EEEvNS_8GemmArgsE")
    raise AssertionError(f"unrecognised kernel name {name}")


def mangled_i8(name):
    """Int8 instances: the same tile templates with an i8_ kernel name; the name's
    K step counts int8 elements (128 per 128-byte LDS row)."""
    m = re.fullmatch(r"generic_(\d+)x(\d+)_w(\d+)x(\d+)_m(\d+)", name)
    if m:
        bm, bn, wm, wn, mf = m.groups()
        return f"_ZN4mihg17i8_generic_kernelILi{bm}ELi{bn}ELi{wm}ELi{wn}ELi{mf}EEEvNS_8GemmArgsE"
    m = re.fullmatch(r"d2tile_(\d+)x(\d+)_w(\d+)x(\d+)_m16", name)
    if m:
        bm, bn, wm, wn = m.groups()
        return f"_ZN4mihg16i8_d2tile_kernelILi{bm}ELi{bn}ELi{wm}ELi{wn}EEEvNS_8GemmArgsE"
    m = re.fullmatch(r"(d2tile3)_(\d+)x(\d+)_w(\d+)x(\d+)_m16", name)
    if m:
        kind, bm, bn, wm, wn = m.groups()
        return (f"_ZN4mihg{len(kind) + 10}i8_{kind}_kernelILi{bm}ELi{bn}ELi{wm}ELi{wn}"
                "EEEvNS_8GemmArgsE")
    m = re.fullmatch(r"pp2tile_(\d+)x(\d+)_w8_m16", name)
    if m:
        bm, bn = m.groups()
        return f"_ZN4mihg17i8_pp2tile_kernelILi{bm}ELi{bn}EEEvNS_8GemmArgsE"
    m = re.fullmatch(r"ktile_(\d+)x(\d+)_w(\d+)x(\d+)_k(\d+)_s(\d+)(?:b(\d+))?", name)
    if m:
        bm, bn, wm, wn, bk, s, sb = m.groups()
        return (f"_ZN4mihg15i8_ktile_kernelILi{bm}ELi{bn}ELi{wm}ELi{wn}ELi{int(bk) // 128}"
                f"ELi{s}ELi{sb or s}EEEvNS_8GemmArgsE")
    m = re.fullmatch(r"ktile_(\d+)x(\d+)_w(\d+)x(\d+)_k(\d+)_s(\d+)_nt", name)
    if m:
        bm, bn, wm, wn, bk, s = m.groups()
        return (f"_ZN4mihg18i8_ktile_nt_kernelILi{bm}ELi{bn}ELi{wm}ELi{wn}ELi{int(bk) // 128}"
                f"ELi{s}EEEvNS_8GemmArgsE")
    raise AssertionError(f"unrecognised int8 kernel name {name}")


@pytest.mark.skipif(not (shutil.which("objcopy") and os.path.exists(LLVM + "/llvm-readelf")),
                    reason="binutils / ROCm llvm tools not available")
def test_every_registered_kernel_has_gfx950_code(tmp_path):
    fat = tmp_path / "fat.bin"
    subprocess.run(["objcopy", "--dump-section", f".hip_fatbin={fat}", mh.LIB_PATH,
                    str(tmp_path / "copy.so")], check=True)
    targets = subprocess.run([LLVM + "/clang-offload-bundler", "--list", "--type=o",
                              f"--input={fat}"], check=True, capture_output=True,
                             text=True).stdout.split()
    gfx = [t for t in targets if t.endswith("gfx950")]
    assert gfx, f"no gfx950 code object in the library: {targets}"
    co = tmp_path / "dev.co"
    subprocess.run([LLVM + "/clang-offload-bundler", "--unbundle", "--type=o", f"--input={fat}",
                    f"--targets={gfx[0]}", f"--output={co}"], check=True)
    syms = subprocess.run([LLVM + "/llvm-readelf", "-s", "-W", str(co)], check=True,
                          capture_output=True, text=True).stdout
    have = set(re.findall(r"(_ZN4mihg\S+)", syms))
    missing = [n for n in mh.kernel_names() if mangled(n) not in have]
    assert not missing, f"kernels without device code: {missing}"


@pytest.mark.skipif(not (shutil.which("objcopy") and os.path.exists(LLVM + "/llvm-readelf")),
                    reason="binutils / ROCm llvm tools not available")
def test_no_registered_kernel_spills_to_scratch(tmp_path):
    """Register spills go to per-lane scratch memory and wreck a tile's schedule."""
    fat = tmp_path / "fat.bin"
    subprocess.run(["objcopy", "--dump-section", f".hip_fatbin={fat}", mh.LIB_PATH,
                    str(tmp_path / "copy.so")], check=True)
    targets = subprocess.run([LLVM + "/clang-offload-bundler", "--list", "--type=o",
                              f"--input={fat}"], check=True, capture_output=True,
                             text=True).stdout.split()
    gfx = [t for t in targets if t.endswith("gfx950")]
    co = tmp_path / "dev.co"
    subprocess.run([LLVM + "/clang-offload-bundler", "--unbundle", "--type=o", f"--input={fat}",
                    f"--targets={gfx[0]}", f"--output={co}"], check=True)
    notes = subprocess.run([LLVM + "/llvm-readelf", "--notes", "-W", str(co)], check=True,
                           capture_output=True, text=True).stdout
    info = {}
    for block in re.split(r"\n\s*- \.", notes):
        name = re.search(r"\.name:\s+(\S+)", "." + block)
        if not name:
            continue
        spill = re.search(r"\.vgpr_spill_count:\s+(\d+)", block)
        priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", block)
        info[name.group(1)] = (int(spill.group(1)) if spill else 0,
                               int(priv.group(1)) if priv else 0)
    wanted = {mangled(n): n for n in mh.kernel_names()}
    assert set(wanted) <= set(info), "metadata missing for some kernels"
    bad = {wanted[m]: info[m] for m in wanted if info[m] != (0, 0)}
    assert not bad, f"kernels with spills or private segment (spills, bytes): {bad}"
