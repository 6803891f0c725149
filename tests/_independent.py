"""Independent decoders used to pin the oracle (tests only).

Nothing here calls the oracle.  E2M1 values come from the table printed on the
pages (tests/golden/e2m1_values.txt); E4M3 values come from PyTorch's
float8_e4m3fn conversion (a library routine); products and sums come from
numpy float64 (exact for the sizes used: see each test); rounding to fp16 comes
from numpy's float64 -> float16 conversion (round-to-nearest-even).
"""
from __future__ import annotations

import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def e2m1_table() -> np.ndarray:
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    assert sorted(vals) == list(range(16))
    return np.array([vals[c] for c in range(16)], dtype=np.float64)


def e4m3_table() -> np.ndarray:
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def unpack_fp4(packed: np.ndarray, rows: int, K: int) -> np.ndarray:
    """Codes (rows x K): element 2j is the low nibble of byte j, element 2j+1
    the high nibble (page kernelbot-nvfp4-group-gemm-505431, dequantize_fp4)."""
    p = np.asarray(packed, dtype=np.uint8).reshape(rows, K // 2)
    out = np.empty((rows, K), dtype=np.uint8)
    out[:, 0::2] = p & 0x0F
    out[:, 1::2] = p >> 4
    return out


def decode(packed, scales, rows, K) -> np.ndarray:
    """Decoded real values: table value times the row's scale for k // 16."""
    codes = unpack_fp4(packed, rows, K)
    vals = e2m1_table()[codes]
    sc = e4m3_table()[np.asarray(scales, dtype=np.uint8).reshape(rows, K // 16)]
    return vals * np.repeat(sc, 16, axis=1)


def brute_group(A, B, SFA, SFB, M, N, K):
    """fp16 result of one group by float64 matmul + numpy rounding."""
    a = decode(A, SFA, M, K)
    b = decode(B, SFB, N, K)
    exact = a @ b.T
    return exact.astype(np.float16), exact


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def decode_mx(packed, scales, rows, K) -> np.ndarray:
    """MXFP4 values: table value times 2^(code - 127) of the row's scale for
    k // 32 (the power of two from Python's float exponentiation)."""
    codes = unpack_fp4(packed, rows, K)
    vals = e2m1_table()[codes]
    sc = np.array([2.0 ** (int(c) - 127) for c in range(255)] + [np.nan])[
        np.asarray(scales, dtype=np.uint8).reshape(rows, K // 32)]
    return vals * np.repeat(sc, 32, axis=1)


def brute_mx_group(A, B, SFA, SFB, M, N, K):
    """fp16 result of one MXFP4 group by float64 matmul + numpy rounding
    (exact while the scale exponents of a dot product stay within a few
    dozen binades, as in the shapes the pins use)."""
    exact = decode_mx(A, SFA, M, K) @ decode_mx(B, SFB, N, K).T
    return exact.astype(np.float16), exact


def exact_mx_element(a_codes, a_scales, b_codes, b_scales):
    """One MXFP4 dot product as an exact Python fraction (codes per K, E8M0
    scale codes per 32 K), for exponent spreads float64 cannot hold."""
    from fractions import Fraction
    t = e2m1_table()
    s = Fraction(0)
    for k in range(len(a_codes)):
        ea = int(a_scales[k // 32]) - 127
        eb = int(b_scales[k // 32]) - 127
        s += Fraction(t[a_codes[k]]) * Fraction(t[b_codes[k]]) * Fraction(2) ** (ea + eb)
    return s
