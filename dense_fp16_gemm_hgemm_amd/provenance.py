"""Provenance of measurements and tuned tables: the library version and a
digest of the device code.

``source_digest()`` hashes the code of the device sources (kernels, instance
list, shared declarations, LDS ring arithmetic) with comments and blank lines
removed, so a comment edit does not invalidate a profile or a table while any
change to what the kernels compute or how they are scheduled does.
"""
from __future__ import annotations

import hashlib
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
DEVICE_SOURCES = ("kernels.hpp", "instances.hip", "internal.h", "ring_schedule.h")


def _code_only(text: str) -> str:
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def source_digest() -> str:
    h = hashlib.sha256()
    for name in DEVICE_SOURCES:
        with open(os.path.join(PKG, "csrc", name), encoding="utf-8") as fh:
            h.update(name.encode())
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def library_version() -> str:
    text = open(os.path.join(ROOT, "include", "mi_hgemm.h"), encoding="utf-8").read()
    major = re.search(r"MI_HGEMM_VERSION_MAJOR (\d+)", text).group(1)
    minor = re.search(r"MI_HGEMM_VERSION_MINOR (\d+)", text).group(1)
    return f"{major}.{minor}"
