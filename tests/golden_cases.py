"""Loader for the hand-derived cases under ``tests/golden/``.

Each file states one row of x, its cos/sin tables over the slice, the slice,
mode and direction, and the expected row; the derivation and the passage it
follows are in the file's comment lines. Every value is a short dyadic
fraction, exact in the case's storage type.
"""
from __future__ import annotations

import glob
import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(path: str) -> dict:
    case = {"name": os.path.basename(path)}
    with open(path, encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            vals = rest.split()
            if key in ("dtype", "table_dtype", "mode", "direction"):
                case[key] = vals[0]
            elif key == "slice":
                case[key] = (int(vals[0]), int(vals[1]))
            else:
                case[key] = np.array([float(v) for v in vals], np.float64)
    case.setdefault("table_dtype", case.get("dtype"))
    return case


def all_cases() -> list[dict]:
    return [load(p) for p in sorted(glob.glob(os.path.join(GOLDEN_DIR, "*.txt")))]
