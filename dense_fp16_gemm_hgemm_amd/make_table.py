"""Tune the shape -> config table that ships beside the library.

    python -m dense_fp16_gemm_hgemm_amd.make_table [--out PATH] [--fresh]
                                                   [--heuristic] [--shapes M_N_K ...]
                                                   [--int8]

For every shape, ``mi_hgemm_tune`` times each compiled instance, raster setting
and K split on the current GPU (exhaustive unless ``--heuristic``), keeps the
fastest one whose result is bit-identical to the element-wise instance, and
stores it in the handle; the handle's table is then written to PATH (default:
``tables/gfx950.tsv`` beside the library, which new handles load).  Without
``--shapes`` the shapes are the named benchmark problems: the LLM projection
shapes, the two small cases and the large square.  ``--int8`` tunes the int8
variant instead (entries of class i8a16; default shapes: the LLM projection
shapes and the large square).
"""
from __future__ import annotations

import argparse
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))


def default_shapes(int8=False):
    from . import inputs
    seen, out = set(), []
    for p in (inputs.i8_llm() + [inputs.i8_square()] if int8 else inputs.all_named()):
        key = (p.M, p.N, p.K)
        if key not in seen:
            seen.add(key)
            out.append(key)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--out", default=os.path.join(HERE, "tables", "gfx950.tsv"))
    ap.add_argument("--fresh", action="store_true",
                    help="start from an empty table instead of the shipped one")
    ap.add_argument("--heuristic", action="store_true", help="pruned candidate list")
    ap.add_argument("--shapes", nargs="*", default=None, metavar="M_N_K")
    ap.add_argument("--int8", action="store_true", help="tune the int8 variant")
    args = ap.parse_args(argv)

    import torch
    from . import Hgemm, MI_HGEMM_TUNE_EXHAUSTIVE, MI_HGEMM_TUNE_HEURISTIC, MI_HGEMM_TUNE_INT8

    if not torch.cuda.is_available():
        raise SystemExit("make_table needs a GPU")
    torch.cuda.set_device(0)
    shapes = ([tuple(int(x) for x in s.split("_")) for s in args.shapes]
              if args.shapes else default_shapes(args.int8))
    table = os.devnull + ".absent" if args.fresh else None
    h = Hgemm(table_path=table)
    flags = MI_HGEMM_TUNE_HEURISTIC if args.heuristic else MI_HGEMM_TUNE_EXHAUSTIVE
    if args.int8:
        flags |= MI_HGEMM_TUNE_INT8
    try:
        for M, N, K in shapes:
            t0 = time.perf_counter()
            h.tune(M, N, K, flags)
            torch.cuda.synchronize()
            dev = torch.device("cuda", 0)
            et = torch.int8 if args.int8 else torch.float16
            a = torch.empty((M, K), dtype=et, device=dev)
            b = torch.empty((N, K), dtype=et, device=dev)
            name, g, x, s = h.plan(a, b)
            print(f"tuned {M}x{N}x{K}: {name} group_m {g} xcd {x} split {s} "
                  f"({time.perf_counter() - t0:.1f} s)", flush=True)
            del a, b
        os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
        h.save_table(args.out)
        print(f"wrote {h.table_size()} entries to {args.out}", flush=True)
    finally:
        h.close()


if __name__ == "__main__":
    sys.exit(main())
