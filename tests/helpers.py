"""Shared test helpers: golden-file reader and the parity criteria."""
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    """Parse a tests/golden fixture into a dict with A, B, C as Fraction lists."""
    path = os.path.join(GOLDEN, name)
    meta, blocks, cur = {}, {"A": [], "B": [], "C": [], "AS": [], "E": []}, None
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


# Comparison configurations: compiled only into a library built with
# GEMM_RELU_COMPARISON_CONFIGS=1 (never chosen by plan selection).
COMPARISON_CONFIGS = ("d256x256x64_s2", "d256x256x32_s4", "d256x256x32_s5", "d256x256x64_s2_16",
                      "d256x256x32_s4_ip", "d256x256x32_s4_isk", "d256x256x32_s4_w8i",
                      "d256x256x32_s5_w8i", "d256x256x64_s2_w8", "d256x128x64_s2",
                      "d256x256x32_s4_i16p", "d64x256x64_s3_splitk", "d64x128x128_s3_splitk",
                      "d64x128x64_s3_splitk", "sp256x256x64_s3", "d128x384x32_s4_i16w8",
                      "d256x256x32_s4_i16w8+d128x384x32_s4_i16w8", "d256x256x32_s4_i16w8sk")


def built_configs(names):
    """The configurations of `names` that the library in the tree holds: every
    plan-selection configuration, and the comparison ones only in a build made
    with them (asked of the library; none if it cannot be loaded)."""
    try:
        import dense_tiled_gemm_relu_amd as gr
        have = set(gr.gemm_relu_configs())
    except Exception:
        have = set()
    return [n for n in names if n not in COMPARISON_CONFIGS or n in have]


# ------------------------------------------------------------------ GPU side
def to_device(bits, dtype_code, shape):
    """Storage patterns (uint16 for fp16/bf16, uint8 for the 8-bit formats) ->
    contiguous CUDA tensor of the input type."""
    import torch
    bits = np.ascontiguousarray(bits).reshape(shape)
    if dtype_code in (3, 4):
        t = torch.from_numpy(bits.view(np.uint8)).cuda()
        return t.view(torch.float8_e4m3fn if dtype_code == 3 else torch.float8_e5m2)
    t = torch.from_numpy(bits.view(np.int16)).cuda()
    return t.view(torch.float16 if dtype_code == 0 else torch.bfloat16)


def out_tensor(M, N, out_code, fill=float("nan")):
    import torch
    dt = {0: torch.float16, 1: torch.bfloat16, 2: torch.float32}[out_code]
    return torch.full((M, N), fill, dtype=dt, device="cuda")


def from_device(C):
    """CUDA tensor (fp16 / bf16 / fp32) -> exact binary64 numpy values."""
    import torch
    if C.dtype == torch.float32:
        return C.cpu().numpy().astype(np.float64)
    bits = C.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    if C.dtype == torch.float16:
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def unit_roundoff(out_code):
    return {0: 2.0 ** -11, 1: 2.0 ** -8, 2: 2.0 ** -24}[out_code]


def rel_tolerance(out_code):
    """Relative term of the random-input bound: 2^-9 for fp16/fp32 outputs; a
    bf16 output rounds with unit roundoff 2^-8, so its bound uses 2^-8."""
    return 2.0 ** -8 if out_code == 1 else 2.0 ** -9


def check_close(gpu, ref, K, out_code):
    bound = np.abs(ref) * rel_tolerance(out_code) + 1e-3 * math.sqrt(max(K, 0))
    err = np.abs(gpu - ref)
    bad = ~(err <= bound)
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%d elements out of tolerance, first %s: gpu %s ref %s"
                             % (bad.sum(), idx.tolist(), gpu[bad][:5], ref[bad][:5]))
    return float(err.max()) if err.size else 0.0
