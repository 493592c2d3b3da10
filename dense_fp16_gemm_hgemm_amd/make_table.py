"""Tune the shape -> config table that ships beside the library.

    python -m dense_fp16_gemm_hgemm_amd.make_table [--out PATH] [--fresh] [--all] [--grid]
                                                   [--heuristic] [--shapes M_N_K ...]
                                                   [--int8] [--evidence PATH] [--log PATH]

For every shape, ``mi_hgemm_tune`` times each compiled instance, raster setting
and K split on the current GPU (exhaustive unless ``--heuristic``), re-times
the three fastest in interleaved rounds, keeps the fastest one whose result is
bit-identical to the element-wise instance, and stores it in the handle; the
handle's table is then written to PATH (default: ``tables/gfx950.tsv`` beside
the library, which new handles load), headed by the library version, the
digest of the device sources and the GPU it was tuned on.  Without
``--shapes`` the shapes are the named benchmark problems: the LLM projection
shapes, the two small cases and the large square.  ``--int8`` tunes the int8
variant instead (entries of class i8a16; default shapes: the LLM projection
shapes and the large square); ``--all`` tunes both, so that

    python -m dense_fp16_gemm_hgemm_amd.make_table --fresh --all

writes the named shapes' entries from nothing.  ``--grid`` adds the binary16
shapes of the power-of-two grid M, N, K in {64, 128, ..., 8192} (the grid the
shape sweep draws from) that are not named shapes, tuned over the pruned
candidate list (every instance at rasters g1 x0 and g8 x1, K splits at g1:
about 1-3 s a shape instead of 3-30 s); the shipped table is

    python -m dense_fp16_gemm_hgemm_amd.make_table --fresh --all
    python -m dense_fp16_gemm_hgemm_amd.make_table --grid

(the second run loads the first one's table and adds to it; ``--part I/N``
tunes every N-th grid shape only, so that the grid can be tuned in N runs,
each loading the table the previous one wrote through MI_HGEMM_TABLE).  The evidence of
each choice (the finalists' medians and spreads, how many candidates were
timed, the runner-up) goes to ``tables/gfx950_evidence.md`` (or
``--evidence``); without ``--fresh`` the sections of shapes not tuned in this
run are kept.
"""
from __future__ import annotations

import argparse
import datetime
import os
import re
import sys
import tempfile
import time

HERE = os.path.dirname(os.path.abspath(__file__))

CAND = re.compile(r"^mi_hgemm_tune (\d+) (\d+) (\d+) (\S+) g(\d+) x(\d) s(\d+) ([\d.]+) us$")
FINAL = re.compile(r"^mi_hgemm_tune final (\d+) (\d+) (\d+) (\S+) g(\d+) x(\d) s(\d+) median ([\d.]+) us "
                   r"min ([\d.]+) max ([\d.]+) over (\d+) replays$")


GRID = tuple(1 << e for e in range(6, 14))


def grid_shapes():
    """The binary16 power-of-two grid, less the named shapes."""
    named = set(default_shapes(False))
    return [(m, n, k) for m in GRID for n in GRID for k in GRID if (m, n, k) not in named]


def default_shapes(int8=False):
    from . import inputs
    seen, out = set(), []
    for p in (inputs.i8_llm() + [inputs.i8_square()] if int8 else inputs.all_named()):
        key = (p.M, p.N, p.K)
        if key not in seen:
            seen.add(key)
            out.append(key)
    return out


def tune_logged(h, M, N, K, flags):
    """h.tune with the tuner's log (MI_HGEMM_TUNE_LOG) captured from fd 2."""
    import torch
    os.environ["MI_HGEMM_TUNE_LOG"] = "1"
    with tempfile.TemporaryFile(mode="w+b") as tf:
        sys.stderr.flush()
        saved = os.dup(2)
        os.dup2(tf.fileno(), 2)
        try:
            h.tune(M, N, K, flags)
            torch.cuda.synchronize()
        finally:
            os.dup2(saved, 2)
            os.close(saved)
        tf.seek(0)
        return tf.read().decode(errors="replace")


def evidence_of(log: str):
    cands, finals = [], []
    for line in log.splitlines():
        m = FINAL.match(line.strip())
        if m:
            finals.append(m.groups())
            continue
        m = CAND.match(line.strip())
        if m:
            cands.append(m.groups())
    return cands, finals


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--out", default=os.path.join(HERE, "tables", "gfx950.tsv"))
    ap.add_argument("--evidence", default=None,
                    help="where to write the evidence of each choice (default: beside --out)")
    ap.add_argument("--fresh", action="store_true",
                    help="start from an empty table instead of the shipped one")
    ap.add_argument("--heuristic", action="store_true", help="pruned candidate list")
    ap.add_argument("--shapes", nargs="*", default=None, metavar="M_N_K")
    ap.add_argument("--int8", action="store_true", help="tune the int8 variant")
    ap.add_argument("--all", action="store_true", help="tune the fp16 and the int8 default shapes")
    ap.add_argument("--grid", action="store_true",
                    help="tune the power-of-two grid (64..8192 each) less the named shapes, "
                         "over the pruned candidate list")
    ap.add_argument("--part", default=None, metavar="I/N",
                    help="with --grid: tune only every N-th grid shape from the I-th (1-based)")
    ap.add_argument("--log", default=None, metavar="PATH",
                    help="also write the tuner's log (every timed candidate) to PATH")
    args = ap.parse_args(argv)

    import torch
    from . import Hgemm, MI_HGEMM_TUNE_EXHAUSTIVE, MI_HGEMM_TUNE_HEURISTIC, MI_HGEMM_TUNE_INT8
    from .provenance import library_version, source_digest

    if not torch.cuda.is_available():
        raise SystemExit("make_table needs a GPU")
    torch.cuda.set_device(0)
    base = MI_HGEMM_TUNE_HEURISTIC if args.heuristic else MI_HGEMM_TUNE_EXHAUSTIVE
    if args.shapes:
        jobs = [(tuple(int(x) for x in s.split("_")), args.int8, base) for s in args.shapes]
    elif args.all:
        jobs = ([(s, False, base) for s in default_shapes(False)] +
                [(s, True, base) for s in default_shapes(True)])
    elif args.grid:
        jobs = []
    else:
        jobs = [(s, args.int8, base) for s in default_shapes(args.int8)]
    if args.grid:
        grid = grid_shapes()
        if args.part:
            i, n = (int(v) for v in args.part.split("/"))
            if not 1 <= i <= n:
                raise SystemExit("--part I/N needs 1 <= I <= N")
            grid = grid[i - 1::n]
        jobs += [(s, False, MI_HGEMM_TUNE_HEURISTIC) for s in grid]
    table = os.devnull + ".absent" if args.fresh else None
    h = Hgemm(table_path=table)
    out = os.path.abspath(args.out)
    ev = args.evidence or os.path.splitext(out)[0] + "_evidence.md"
    # without --fresh the table grows from the one loaded: keep its provenance
    # lines and the evidence of the shapes not tuned again
    # (the loaded table: MI_HGEMM_TABLE when set, else the one beside the library)
    src = None if args.fresh else (os.environ.get("MI_HGEMM_TABLE") or
                                   os.path.join(HERE, "tables", "gfx950.tsv"))
    kept_head = []
    if src and os.path.exists(src):
        with open(src, encoding="utf-8") as f:
            kept_head = [ln for ln in f if ln.startswith("# written") or ln.startswith("#   then")]
    evidence = []
    logf = open(args.log, "w", encoding="utf-8") if args.log else None
    try:
        for (M, N, K), int8, mode in jobs:
            t0 = time.perf_counter()
            flags = mode | (MI_HGEMM_TUNE_INT8 if int8 else 0)
            log = tune_logged(h, M, N, K, flags)
            if logf:
                logf.write(log)
                logf.flush()
            dev = torch.device("cuda", 0)
            et = torch.int8 if int8 else torch.float16
            a = torch.empty((M, K), dtype=et, device=dev)
            b = torch.empty((N, K), dtype=et, device=dev)
            name, g, x, s = h.plan(a, b)
            secs = time.perf_counter() - t0
            print(f"tuned {'int8 ' if int8 else ''}{M}x{N}x{K}: {name} group_m {g} xcd {x} "
                  f"split {s} ({secs:.1f} s)", flush=True)
            cands, finals = evidence_of(log)
            evidence.append(((M, N, K), int8, (name, g, x, s), cands, finals, secs,
                             mode == MI_HGEMM_TUNE_HEURISTIC))
            del a, b
        os.makedirs(os.path.dirname(out), exist_ok=True)
        h.save_table(out)
        gpu = torch.cuda.get_device_properties(0)
        cmd = (f"{datetime.date.today().isoformat()} by python -m dense_fp16_gemm_hgemm_amd.make_table "
               f"{' '.join(argv if argv is not None else sys.argv[1:])}")
        written = "".join(kept_head) + (f"#   then {cmd}\n" if kept_head else f"# written {cmd}\n")
        head = (f"# Shape -> config table for {getattr(gpu, 'gcnArchName', 'gfx950')} ({gpu.name}), "
                f"libmi_hgemm {library_version()}, device-source digest {source_digest()},\n"
                + written +
                "# Each entry: the fastest correct candidate of a timed search (every compiled "
                "instance x raster x K split, or the pruned list\n# for the grid shapes), bit-exact "
                "against the element-wise instance on integer operands, timed as graph replays\n# on "
                "random operands over copies that overflow the MALL; its three fastest re-timed in "
                "interleaved rounds;\n# evidence in the companion *_evidence.md.\n")
        with open(out, encoding="utf-8") as f:
            body = f.read()
        with open(out, "w", encoding="utf-8") as f:
            f.write(head + body)
        print(f"wrote {h.table_size()} entries to {out}", flush=True)
        write_evidence(ev, evidence, gpu.name,
                       keep_from=os.path.splitext(src)[0] + "_evidence.md" if src else None)
        print(f"wrote the evidence to {ev}", flush=True)
    finally:
        h.close()
        if logf:
            logf.close()


def read_sections(path):
    """The '## shape' sections of an evidence file, in order: [(title, text)]."""
    if not os.path.exists(path):
        return []
    out, title, buf = [], None, []
    with open(path, encoding="utf-8") as f:
        for line in f.read().splitlines():
            if line.startswith("## "):
                if title is not None:
                    out.append((title, "\n".join(buf).rstrip("\n")))
                title, buf = line, [line]
            elif title is not None:
                buf.append(line)
    if title is not None:
        out.append((title, "\n".join(buf).rstrip("\n")))
    return out


def write_evidence(path, evidence, gpu_name, keep_from=None):
    from .provenance import library_version, source_digest
    lines = [f"# Evidence of the tuned table ({gpu_name}, libmi_hgemm {library_version()}, "
             f"device-source digest {source_digest()})", "",
             "Per shape: the candidates timed (instance x raster x K split, each a median of 5 graph "
             "replays on cold operands; the full list, or the pruned one where marked), the three "
             "finalists re-timed in three interleaved rounds (median, min and max over their 15 "
             "replays, in µs per call), and the winner.", ""]
    new = {}
    for (M, N, K), int8, (name, g, x, s), cands, finals, secs, pruned in evidence:
        sec = []
        sec.append(f"## {'int8 ' if int8 else ''}{M}x{N}x{K}")
        sec.append("")
        sec.append(f"Winner: `{name}` group_m {g} xcd_remap {x} split {s}; {len(cands)} candidates "
                   f"timed in {secs:.1f} s{' (pruned list)' if pruned else ''}.")
        if finals:
            sec.append("")
            sec.append("| finalist | raster | split | median µs | min µs | max µs | replays |")
            sec.append("|---|---|---|---|---|---|---|")
            for (_, _, _, kern, gg, xx, ss, med, mn, mx, n) in finals:
                sec.append(f"| `{kern}` | g{gg} x{xx} | {ss} | {med} | {mn} | {mx} | {n} |")
            meds = sorted(float(f[7]) for f in finals)
            if len(meds) > 1:
                sec.append("")
                sec.append(f"Runner-up gap: {100 * (meds[1] / meds[0] - 1):.2f}%.")
        new[sec[0]] = "\n".join(sec)
    sections = read_sections(keep_from) if keep_from else []
    seen = set()
    for title, text in sections:
        lines.append(new.get(title, text))
        lines.append("")
        seen.add(title)
    for title, text in new.items():
        if title not in seen:
            lines.append(text)
            lines.append("")
    with open(path, "w", encoding="utf-8") as f:
        f.write("\n".join(lines))


if __name__ == "__main__":
    sys.exit(main())
