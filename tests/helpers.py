"""Shared test helpers: golden-file reader and the parity criteria."""
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    """Parse a tests/golden fixture into a dict with A, B, C as Fraction lists."""
    path = os.path.join(GOLDEN, name)
    meta, blocks, cur = {}, {"A": [], "B": [], "C": []}, None
    with open(path) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            if line in blocks:
                cur = line
                continue
            if cur is None and ":" in line:
                k, v = line.split(":", 1)
                meta[k.strip()] = v.strip()
                continue
            blocks[cur].append([Fraction(t) for t in line.split()])
    meta["M"], meta["N"], meta["K"] = int(meta["M"]), int(meta["N"]), int(meta["K"])
    meta["transB"] = int(meta["transB"])
    meta.update(blocks)
    return meta


def tolerance(ref, K):
    """Per-element bound for random inputs: 2^-9 |ref| + 1e-3 sqrt(K)."""
    return np.abs(ref) * 2.0 ** -9 + 1e-3 * math.sqrt(max(K, 0))


def fp32_sum_bound(absum, ref, K, out_unit_roundoff):
    """Forward error bound of a binary32 sum of K exact products, plus output rounding.

    |gpu - ref| <= K * 2^-24 * S + u_out * |ref| + 2^-24, S = sum_k |a b|.
    """
    return K * 2.0 ** -24 * absum + out_unit_roundoff * np.abs(ref) + 2.0 ** -24
