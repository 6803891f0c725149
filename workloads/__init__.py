"""Seeded synthetic inputs for the NVFP4 grouped GEMM (shared by tests and bench).

This module holds no arithmetic of the method: it only draws random bytes and
packs randomly chosen code fields into bytes.  Both the oracle and the HIP path
receive the same arrays from here.

Random numbers come from SplitMix64 used as a counter-based generator
(Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
OOPSLA 2014; finaliser constants as in Vigna's public-domain splitmix64.c):
draw i of stream ``key`` is ``mix(key + (i + 1) * 0x9E3779B97F4A7C15)``.

Input recipe (the workloads the pages benchmark, with the value distributions
stated for them):
  * A, B: every byte uniform over 0..255, i.e. two independent uniform E2M1
    codes per byte (all 16 codes, including -0).
  * SFA, SFB ("pos" distribution): sign 0, unbiased exponent uniform over
    {-3..3} (exponent field 4..10), mantissa field uniform over 0..7, so every
    scale is a positive normal E4M3 value in [0.125, 15].
  * Other scale distributions for edge tests: "unit" (every scale 1.0, code
    0x38), "finite" (any non-NaN E4M3 code, signs and subnormals included).
  * MXFP4 form: the same A, B bytes; E8M0 scales (one per 32 K) with the
    exponent uniform over {-3..3} (codes 124..130), the range of the NVFP4
    scales' exponents; "unit" (code 127) and "wide" (codes 107..147, a
    product spread up to 2^80) for edge tests.
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def stream_key(*parts: int) -> np.uint64:
    """Derive a stream key from integers (seed, group, tensor id, ...)."""
    k = np.zeros(1, dtype=np.uint64)
    for p in parts:
        k = _mix(k ^ np.uint64(p & 0xFFFFFFFFFFFFFFFF)) + GOLDEN
    return np.uint64(k[0])


def draws(key: np.uint64, n: int, start: int = 0) -> np.ndarray:
    """n 64-bit draws (counters start+1 .. start+n) of stream ``key``."""
    with np.errstate(over="ignore"):
        ctr = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        return _mix(np.uint64(key) + ctr * GOLDEN)


def random_bytes(key: np.uint64, nbytes: int) -> np.ndarray:
    """nbytes uniform bytes (8 per draw, little-endian)."""
    d = draws(key, (nbytes + 7) // 8)
    return d.view(np.uint8)[:nbytes].copy()


def scale_codes(key: np.uint64, count: int, dist: str = "pos") -> np.ndarray:
    """E4M3 scale codes drawn from one of the distributions in the module doc."""
    d = draws(key, count)
    if dist == "pos":
        e_field = ((d >> np.uint64(32)) % np.uint64(7)) + np.uint64(4)
        f_field = d & np.uint64(7)
        return ((e_field << np.uint64(3)) | f_field).astype(np.uint8)
    if dist == "unit":
        return np.full(count, 0x38, dtype=np.uint8)
    if dist == "finite":
        c = (d & np.uint64(0xFF)).astype(np.uint8)
        nan = (c & 0x7F) == 0x7F
        c[nan] = c[nan] & 0xF8          # replace a NaN code by a finite one
        return c
    raise ValueError("unknown scale distribution %r" % dist)


# The five workloads: one small case, then the four shapes the pages time
# (page kernelbot-nvfp4-group-gemm-495528, the timing docstring at the top).
CONFIGS = [
    dict(name="g2_k512_n256", g=2, M=[64, 96], N=[256, 256], K=[512, 512], seed=0),
    dict(name="g2_k1536_n4096", g=2, M=[128, 384], N=[4096] * 2, K=[1536] * 2, seed=1111),
    dict(name="g2_k4096_n3072", g=2, M=[192, 320], N=[3072] * 2, K=[4096] * 2, seed=1111),
    dict(name="g8_k2048_n7168", g=8, M=[40, 76, 168, 72, 164, 148, 196, 160],
         N=[7168] * 8, K=[2048] * 8, seed=1111),
    dict(name="g8_k7168_n4096", g=8, M=[80, 176, 128, 72, 64, 248, 96, 160],
         N=[4096] * 8, K=[7168] * 8, seed=1111),
]


def config(name: str) -> dict:
    """The workload called ``name`` (one of CONFIGS' names)."""
    for cfg in CONFIGS:
        if cfg["name"] == name:
            return cfg
    raise KeyError("unknown workload %r" % name)


SMALL = config("g2_k512_n256")
HEADLINE = config("g8_k7168_n4096")

_T_A, _T_B, _T_SFA, _T_SFB = 1, 2, 3, 4


def make_group(seed: int, gi: int, M: int, N: int, K: int, *,
               dist: str = "pos", variant: int = 0):
    """Packed inputs of one group as uint8 arrays:
    A (M, K/2), B (N, K/2), SFA (M, K/16), SFB (N, K/16)."""
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    kA = stream_key(seed, variant, gi, _T_A)
    kB = stream_key(seed, variant, gi, _T_B)
    kSA = stream_key(seed, variant, gi, _T_SFA)
    kSB = stream_key(seed, variant, gi, _T_SFB)
    A = random_bytes(kA, M * K // 2).reshape(M, K // 2)
    B = random_bytes(kB, N * K // 2).reshape(N, K // 2)
    SFA = scale_codes(kSA, M * K // 16, dist).reshape(M, K // 16)
    SFB = scale_codes(kSB, N * K // 16, dist).reshape(N, K // 16)
    return A, B, SFA, SFB


def make_inputs(M, N, K, seed: int, *, dist: str = "pos", variant: int = 0):
    """Lists (A, B, SFA, SFB) over the groups of one problem."""
    A, B, SA, SB = [], [], [], []
    for gi, (m, n, k) in enumerate(zip(M, N, K)):
        a, b, sa, sb = make_group(seed, gi, m, n, k, dist=dist, variant=variant)
        A.append(a)
        B.append(b)
        SA.append(sa)
        SB.append(sb)
    return A, B, SA, SB


def config_inputs(cfg: dict, variant: int = 0):
    return make_inputs(cfg["M"], cfg["N"], cfg["K"], cfg["seed"], variant=variant)


def mx_scale_codes(key: np.uint64, count: int, dist: str = "pos") -> np.ndarray:
    """E8M0 scale codes: "pos" 124..130, "unit" 127, "wide" 107..147."""
    d = draws(key, count)
    if dist == "pos":
        return ((d >> np.uint64(32)) % np.uint64(7) + np.uint64(124)).astype(np.uint8)
    if dist == "unit":
        return np.full(count, 127, dtype=np.uint8)
    if dist == "wide":
        return ((d >> np.uint64(32)) % np.uint64(41) + np.uint64(107)).astype(np.uint8)
    raise ValueError("unknown E8M0 scale distribution %r" % dist)


_T_MXSFA, _T_MXSFB = 5, 6


def make_mx_inputs(M, N, K, seed: int, *, dist: str = "pos", variant: int = 0):
    """MXFP4 inputs: the A, B bytes of make_inputs and E8M0 scales,
    SFA (M, K/32), SFB (N, K/32)."""
    A, B, SA, SB = [], [], [], []
    for gi, (m, n, k) in enumerate(zip(M, N, K)):
        if k % 32:
            raise ValueError("K must be a multiple of 32")
        a, b, _, _ = make_group(seed, gi, m, n, k, variant=variant)
        A.append(a)
        B.append(b)
        SA.append(mx_scale_codes(stream_key(seed, variant, gi, _T_MXSFA), m * k // 32, dist).reshape(m, k // 32))
        SB.append(mx_scale_codes(stream_key(seed, variant, gi, _T_MXSFB), n * k // 32, dist).reshape(n, k // 32))
    return A, B, SA, SB


def algorithmic_bytes(M, N, K, scale_block: int = 16) -> int:
    """Bytes each input is read once plus C written once (fp16); one scale
    byte per scale_block K of a row (16 for NVFP4, 32 for MXFP4)."""
    tot = 0
    for m, n, k in zip(M, N, K):
        tot += m * k // 2 + n * k // 2 + m * k // scale_block + n * k // scale_block + 2 * m * n
    return tot


def algorithmic_flops(M, N, K) -> int:
    return sum(2 * m * n * k for m, n, k in zip(M, N, K))
