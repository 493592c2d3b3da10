"""Tune the shape -> config table that ships beside the library.

    python -m dense_fp16_gemm_hgemm_amd.make_table [--out PATH] [--fresh] [--all]
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

writes the shipped table from nothing.  The evidence of each choice (the
finalists' medians and spreads, how many candidates were timed, the runner-up)
goes to ``tables/gfx950_evidence.md`` (or ``--evidence``).
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
    ap.add_argument("--log", default=None, metavar="PATH",
                    help="also write the tuner's log (every timed candidate) to PATH")
    args = ap.parse_args(argv)

    import torch
    from . import Hgemm, MI_HGEMM_TUNE_EXHAUSTIVE, MI_HGEMM_TUNE_HEURISTIC, MI_HGEMM_TUNE_INT8
    from .provenance import library_version, source_digest

    if not torch.cuda.is_available():
        raise SystemExit("make_table needs a GPU")
    torch.cuda.set_device(0)
    if args.shapes:
        jobs = [(tuple(int(x) for x in s.split("_")), args.int8) for s in args.shapes]
    elif args.all:
        jobs = [(s, False) for s in default_shapes(False)] + [(s, True) for s in default_shapes(True)]
    else:
        jobs = [(s, args.int8) for s in default_shapes(args.int8)]
    table = os.devnull + ".absent" if args.fresh else None
    h = Hgemm(table_path=table)
    base = MI_HGEMM_TUNE_HEURISTIC if args.heuristic else MI_HGEMM_TUNE_EXHAUSTIVE
    evidence = []
    logf = open(args.log, "w", encoding="utf-8") if args.log else None
    try:
        for (M, N, K), int8 in jobs:
            t0 = time.perf_counter()
            flags = base | (MI_HGEMM_TUNE_INT8 if int8 else 0)
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
            evidence.append(((M, N, K), int8, (name, g, x, s), cands, finals, secs))
            del a, b
        out = os.path.abspath(args.out)
        os.makedirs(os.path.dirname(out), exist_ok=True)
        h.save_table(out)
        gpu = torch.cuda.get_device_properties(0)
        head = (f"# Shape -> config table for {getattr(gpu, 'gcnArchName', 'gfx950')} ({gpu.name}), "
                f"libmi_hgemm {library_version()}, device-source digest {source_digest()},\n"
                f"# written {datetime.date.today().isoformat()} by python -m "
                f"dense_fp16_gemm_hgemm_amd.make_table {' '.join(argv if argv is not None else sys.argv[1:])}\n"
                "# Each entry: the fastest correct candidate of an exhaustive timed search (every "
                "compiled instance x raster x K split,\n# bit-exact against the element-wise "
                "instance on integer operands, timed as graph replays on random operands over "
                "copies\n# that overflow the MALL), its three fastest re-timed in interleaved "
                "rounds; evidence in the companion *_evidence.md.\n")
        with open(out, encoding="utf-8") as f:
            body = f.read()
        with open(out, "w", encoding="utf-8") as f:
            f.write(head + body)
        print(f"wrote {h.table_size()} entries to {out}", flush=True)
        ev = args.evidence or os.path.splitext(out)[0] + "_evidence.md"
        write_evidence(ev, evidence, gpu.name)
        print(f"wrote the evidence to {ev}", flush=True)
    finally:
        h.close()
        if logf:
            logf.close()


def write_evidence(path, evidence, gpu_name):
    from .provenance import library_version, source_digest
    lines = [f"# Evidence of the tuned table ({gpu_name}, libmi_hgemm {library_version()}, "
             f"device-source digest {source_digest()})", "",
             "Per shape: the candidates timed (instance x raster x K split, each a median of 5 graph "
             "replays on cold operands), the three finalists re-timed in three interleaved rounds "
             "(median, min and max over their 15 replays, in µs per call), and the winner.", ""]
    for (M, N, K), int8, (name, g, x, s), cands, finals, secs in evidence:
        lines.append(f"## {'int8 ' if int8 else ''}{M}x{N}x{K}")
        lines.append("")
        lines.append(f"Winner: `{name}` group_m {g} xcd_remap {x} split {s}; {len(cands)} candidates "
                     f"timed in {secs:.1f} s.")
        if finals:
            lines.append("")
            lines.append("| finalist | raster | split | median µs | min µs | max µs | replays |")
            lines.append("|---|---|---|---|---|---|---|")
            for (_, _, _, kern, gg, xx, ss, med, mn, mx, n) in finals:
                lines.append(f"| `{kern}` | g{gg} x{xx} | {ss} | {med} | {mn} | {mx} | {n} |")
            meds = sorted(float(f[7]) for f in finals)
            if len(meds) > 1:
                lines.append("")
                lines.append(f"Runner-up gap: {100 * (meds[1] / meds[0] - 1):.2f}%.")
        lines.append("")
    with open(path, "w", encoding="utf-8") as f:
        f.write("\n".join(lines))


if __name__ == "__main__":
    sys.exit(main())
