"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Every test here runs on the CPU.  None of them derives its expected value from
the oracle's own code: see tests/_independent.py for the sources used.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest

import workloads
from tests import _independent as ind


# ---------------------------------------------------------------- decoding

def test_e2m1_matches_printed_table(oracle_lib):
    table = ind.e2m1_table()
    for code in range(16):
        got = oracle_lib.e2m1(code)
        assert got == table[code], code
        assert math.copysign(1.0, got) == math.copysign(1.0, table[code]), code


def test_e4m3_closed_form_points(oracle_lib):
    # OCP OFP8 E4M3: bias 7, subnormal step 2^-9, max finite 448, S.1111.111 NaN.
    assert oracle_lib.e4m3(0x00) == 0.0
    assert oracle_lib.e4m3(0x01) == 2.0 ** -9
    assert oracle_lib.e4m3(0x07) == 7 * 2.0 ** -9
    assert oracle_lib.e4m3(0x08) == 2.0 ** -6
    assert oracle_lib.e4m3(0x38) == 1.0
    assert oracle_lib.e4m3(0x3C) == 1.5
    assert oracle_lib.e4m3(0x7E) == 448.0
    assert math.isnan(oracle_lib.e4m3(0x7F))
    assert math.isnan(oracle_lib.e4m3(0xFF))


def test_e4m3_sign_symmetry_and_order(oracle_lib):
    pos = [oracle_lib.e4m3(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(pos, pos[1:]))
    for c in range(0x7F):
        assert oracle_lib.e4m3(c | 0x80) == -pos[c]


def test_e4m3_matches_library_on_all_codes(oracle_lib):
    lib = ind.e4m3_table()
    for c in range(256):
        got = oracle_lib.e4m3(c)
        if math.isnan(lib[c]):
            assert math.isnan(got), c
        else:
            assert got == lib[c], c


# ---------------------------------------------------------------- rounding

def _np_f16_bits(x: float) -> int:
    return int(np.array([x], dtype=np.float64).astype(np.float16).view(np.uint16)[0])


def test_round_f16_all_values_midpoints_and_neighbours(oracle_lib):
    """Every positive finite fp16 value h, the midpoint to the next value and
    one 2^-20 unit either side of it, where those are multiples of 2^-20,
    rounded by the oracle and by numpy's float64 -> float16 conversion."""
    hs = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt = np.append(hs[1:], 65536.0)          # 65536 = first value past max
    checked = 0
    for h, n in zip(hs, nxt):
        for x in (h, (h + n) / 2):
            X = x * 2.0 ** 20
            if X != math.floor(X):
                continue
            for d in (-1, 0, 1):
                Xi = int(X) + d
                v = Xi * 2.0 ** -20
                for s in ((1, -1) if Xi else (1,)):   # exact zero rounds to +0
                    assert oracle_lib.round_f16_fixed20(s * Xi) == _np_f16_bits(s * v), (s * Xi)
                checked += 1
    assert checked > 60000


def test_round_f16_overflow_boundary(oracle_lib):
    u = 2 ** 20
    assert oracle_lib.round_f16_fixed20(65504 * u) == 0x7BFF
    assert oracle_lib.round_f16_fixed20(65520 * u - 1) == 0x7BFF
    assert oracle_lib.round_f16_fixed20(65520 * u) == 0x7C00        # tie -> even -> inf
    assert oracle_lib.round_f16_fixed20(-65520 * u) == 0xFC00
    assert oracle_lib.round_f16_fixed20(2 ** 62) == 0x7C00
    assert oracle_lib.round_f16_fixed20(0) == 0x0000
    assert oracle_lib.round_f16_fixed20(1) == 0x0010               # 2^-20 = 16 * 2^-24


def test_round_f16_random_vs_numpy(oracle_lib):
    rng = np.random.default_rng(7)
    for mag in (2 ** 10, 2 ** 24, 2 ** 34, 2 ** 40):
        for X in rng.integers(-mag, mag, size=3000):
            X = int(X)
            assert oracle_lib.round_f16_fixed20(X) == _np_f16_bits(X * 2.0 ** -20), X


# ------------------------------------------------------- structure and values

def _onehot_case(M, N, K, m, n, k, ca, cb, sa_code, sb_code):
    A = np.zeros((M, K), np.uint8)
    B = np.zeros((N, K), np.uint8)
    A[m, k] = ca
    B[n, k] = cb
    # distinct scales on every block, the chosen one on block k // 16
    SFA = np.full((M, K // 16), 0x30, np.uint8)
    SFB = np.full((N, K // 16), 0x40, np.uint8)
    SFA[:, :] = (0x30 + np.arange(K // 16)) % 0x70 + 1
    SFB[:, :] = (0x48 + 3 * np.arange(K // 16)) % 0x70 + 1
    SFA[m, k // 16] = sa_code
    SFB[n, k // 16] = sb_code
    return ind.pack_fp4(A), ind.pack_fp4(B), SFA, SFB


@pytest.mark.parametrize("k", [0, 1, 14, 15, 16, 17, 30, 31, 63])
def test_onehot_nibble_order_and_scale_index(oracle_lib, k):
    M, N, K = 3, 5, 64
    m, n = 2, 3
    t = ind.e2m1_table()
    s = ind.e4m3_table()
    ca, cb, sa, sb = 7, 13, 0x3D, 0x2A     # 6.0, -3.0, 1.625, 0.3125
    A, B, SFA, SFB = _onehot_case(M, N, K, m, n, k, ca, cb, sa, sb)
    C, X = oracle_lib.group_gemm([M], [N], [K], [A], [B], [SFA], [SFB], exact=True)
    want = t[ca] * s[sa] * t[cb] * s[sb]
    expect = np.zeros((M, N))
    expect[m, n] = want
    np.testing.assert_array_equal(X[0], expect)
    assert C[0].view(np.uint16)[m, n] == _np_f16_bits(want)
    assert np.count_nonzero(C[0].astype(np.float64)) == 1


@pytest.mark.parametrize("shape", [(1, 1, 16), (3, 5, 32), (8, 7, 64), (4, 8, 48)])
def test_bruteforce_unit_scales(oracle_lib, shape):
    M, N, K = shape
    key = workloads.stream_key(99, M, N, K)
    A = workloads.random_bytes(key, M * K // 2).reshape(M, K // 2)
    B = workloads.random_bytes(key + np.uint64(1), N * K // 2).reshape(N, K // 2)
    SFA = np.full((M, K // 16), 0x38, np.uint8)
    SFB = np.full((N, K // 16), 0x38, np.uint8)
    want16, want = ind.brute_group(A, B, SFA, SFB, M, N, K)
    C, X = oracle_lib.group_gemm([M], [N], [K], [A], [B], [SFA], [SFB], exact=True)
    np.testing.assert_array_equal(X[0], want)
    np.testing.assert_array_equal(C[0].view(np.uint16), want16.view(np.uint16))


@pytest.mark.parametrize("dist", ["pos", "finite"])
@pytest.mark.parametrize("shape", [(5, 6, 64), (8, 8, 64), (2, 9, 16)])
def test_bruteforce_random_scales(oracle_lib, dist, shape):
    """Float64 sums are exact here: every product is a multiple of 2^-20 below
    2^23 and K <= 64, so partial sums stay below 2^29 (49 bits)."""
    M, N, K = shape
    A, B, SFA, SFB = workloads.make_group(5, 0, M, N, K, dist=dist)
    want16, want = ind.brute_group(A, B, SFA, SFB, M, N, K)
    C, X = oracle_lib.group_gemm([M], [N], [K], [A], [B], [SFA], [SFB], exact=True)
    np.testing.assert_array_equal(X[0], want)
    got = C[0].view(np.uint16)
    w = want16.view(np.uint16)
    zero = want == 0                       # the sign of an exact zero is not pinned
    np.testing.assert_array_equal(got[~zero], w[~zero])
    assert np.all(C[0][zero] == 0)


def test_int64_and_f64_paths_agree_on_config_inputs(oracle_lib):
    cfg = workloads.SMALL
    A, B, SA, SB = workloads.config_inputs(cfg)
    C1, X1 = oracle_lib.group_gemm(cfg["M"], cfg["N"], cfg["K"], A, B, SA, SB, exact=True)
    C2, X2 = oracle_lib.group_gemm(cfg["M"], cfg["N"], cfg["K"], A, B, SA, SB,
                                   exact=True, use_f64=True)
    for i in range(cfg["g"]):
        np.testing.assert_array_equal(X1[i], X2[i])
        np.testing.assert_array_equal(C1[i].view(np.uint16), C2[i].view(np.uint16))


def test_config1_matches_bruteforce(oracle_lib):
    """The whole small workload against float64 matmul: products are multiples
    of 2^-14 below 2^13, K = 512, so sums stay below 2^22 / 2^-14 = 2^36."""
    cfg = workloads.SMALL
    A, B, SA, SB = workloads.config_inputs(cfg)
    C = oracle_lib.group_gemm(cfg["M"], cfg["N"], cfg["K"], A, B, SA, SB)
    for i in range(cfg["g"]):
        w16, _ = ind.brute_group(A[i], B[i], SA[i], SB[i], cfg["M"][i], cfg["N"][i], cfg["K"][i])
        np.testing.assert_array_equal(C[i].view(np.uint16), w16.view(np.uint16))


def test_group_independence(oracle_lib):
    M, N, K = [16, 8, 24], [32, 16, 8], [64, 128, 32]
    A, B, SA, SB = workloads.make_inputs(M, N, K, 3)
    C = oracle_lib.group_gemm(M, N, K, A, B, SA, SB)
    A2 = list(A)
    A2[1] = A[1] ^ np.uint8(0x5A)
    C2 = oracle_lib.group_gemm(M, N, K, A2, B, SA, SB)
    for i in (0, 2):
        np.testing.assert_array_equal(C[i].view(np.uint16), C2[i].view(np.uint16))
    assert not np.array_equal(C[1].view(np.uint16), C2[1].view(np.uint16))
    for i in range(3):
        Ci = oracle_lib.group_gemm([M[i]], [N[i]], [K[i]], [A[i]], [B[i]], [SA[i]], [SB[i]])
        np.testing.assert_array_equal(Ci[0].view(np.uint16), C[i].view(np.uint16))


def test_transpose_symmetry(oracle_lib):
    M, N, K = 12, 20, 96
    A, B, SA, SB = workloads.make_group(8, 0, M, N, K, dist="finite")
    C = oracle_lib.group_gemm([M], [N], [K], [A], [B], [SA], [SB])[0]
    Ct = oracle_lib.group_gemm([N], [M], [K], [B], [A], [SB], [SA])[0]
    np.testing.assert_array_equal(C.view(np.uint16), Ct.T.view(np.uint16))


def test_element_matches_full(oracle_lib):
    M, N, K = 7, 9, 160
    A, B, SA, SB = workloads.make_group(4, 1, M, N, K)
    C, X = oracle_lib.group_gemm([M], [N], [K], [A], [B], [SA], [SB], exact=True)
    for m in range(M):
        for n in range(N):
            c16, ex = oracle_lib.gemm_element(M, N, K, A, B, SA, SB, m, n)
            assert c16 == int(C[0].view(np.uint16)[m, n])
            assert ex == X[0][m, n]


def test_dequant_matches_independent_decode(oracle_lib):
    rows, K = 256, 32
    X = ind.pack_fp4(np.tile(np.arange(16, dtype=np.uint8), (rows, K // 16)))
    SF = np.repeat(np.arange(256, dtype=np.uint8)[:, None], K // 16, axis=1)
    got = oracle_lib.dequant(X, SF, rows, K)
    want = ind.decode(X, SF, rows, K)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])


def test_nan_scale_gives_nan(oracle_lib):
    """Reading taken where the pages are silent: a NaN scale code used by an
    output makes that output NaN (IEEE: NaN times anything is NaN)."""
    M, N, K = 2, 3, 32
    A, B, SA, SB = workloads.make_group(1, 0, M, N, K)
    SA = SA.copy()
    SA[1, 1] = 0x7F
    C = oracle_lib.group_gemm([M], [N], [K], [A], [B], [SA], [SB])[0]
    assert not np.isnan(C[0].astype(np.float32)).any()
    assert np.isnan(C[1].astype(np.float32)).all()


def test_degenerate_sizes(oracle_lib):
    C = oracle_lib.group_gemm([0, 3], [4, 0], [32, 32],
                              [np.zeros(0, np.uint8), np.zeros(48, np.uint8)],
                              [np.zeros(64, np.uint8), np.zeros(0, np.uint8)],
                              [np.zeros(0, np.uint8), np.zeros(6, np.uint8)],
                              [np.zeros(8, np.uint8), np.zeros(0, np.uint8)])
    assert C[0].shape == (0, 4) and C[1].shape == (3, 0)
    # K = 0: empty sums are exactly zero
    C = oracle_lib.group_gemm([2], [2], [0], [np.zeros(0, np.uint8)], [np.zeros(0, np.uint8)],
                              [np.zeros(0, np.uint8)], [np.zeros(0, np.uint8)])
    assert np.all(C[0].view(np.uint16) == 0)


# ------------------------------------------- sensitivity of the pins above

def test_pins_detect_plausible_mistakes(oracle_lib):
    """The brute-force pin would catch an oracle that swapped the nibble order,
    transposed B, or indexed scales per 32 instead of 16: each such change
    alters the expected values on these inputs."""
    M, N, K = 4, 4, 64
    A, B, SA, SB = workloads.make_group(11, 0, M, N, K)
    base16, base = ind.brute_group(A, B, SA, SB, M, N, K)
    swapped = ((A >> 4) | (A << 4)).astype(np.uint8)
    assert not np.array_equal(ind.brute_group(swapped, B, SA, SB, M, N, K)[1], base)
    assert not np.array_equal(ind.brute_group(A, B.reshape(N, K // 2)[::-1].copy(), SA, SB, M, N, K)[1], base)
    SA32 = np.repeat(SA[:, ::2], 2, axis=1)
    assert not np.array_equal(ind.brute_group(A, B, SA32, SB, M, N, K)[1], base)
    C = oracle_lib.group_gemm([M], [N], [K], [A], [B], [SA], [SB])[0]
    np.testing.assert_array_equal(C.view(np.uint16), base16.view(np.uint16))


# ------------------------------------------------------ blocked scale layout

def _cute_atom_offsets(rows, cols):
    """Byte offset of every (row, scale column) of a rows x cols scale matrix,
    evaluated from the layout algebra printed with page 482006's CuTe kernel:
    the atom has shape ((32, 4), (16, 4)) and strides ((16, 4), (0, 1)) over
    (row, K), so a row r = r0 + 32 r1 contributes 16 r0 + 4 r1 and a K index
    k = k0 + 16 k1 (k0 < 16 shares one scale) contributes k1; atoms are tiled
    over (M, K) with the K tiles first (tile order (2, 1, 3)), 512 bytes each.
    Independent of the oracle's row-band/run formulation."""
    ktiles = -(-cols // 4)
    r = np.arange(rows)[:, None]
    s = np.arange(cols)[None, :]
    k = 16 * s                                    # first K index of scale column s
    r0, r1, tm = r % 32, (r // 32) % 4, r // 128
    k1, tk = (k // 16) % 4, k // 64
    return 16 * r0 + 4 * r1 + 0 * (k % 16) + k1 + 512 * (tk + ktiles * tm)


@pytest.mark.parametrize("rows,cols", [(1, 4), (128, 4), (130, 8), (300, 12), (64, 448)])
def test_blocked_layout_matches_cute_atom(oracle_lib, rows, cols):
    rng = np.random.default_rng(rows * 1000 + cols)
    plain = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
    blocked = oracle_lib.block_scales(plain, rows, cols, pad_value=0)
    assert blocked.size == (-(-rows // 128) * 128) * (-(-cols // 4) * 4)
    off = _cute_atom_offsets(rows, cols)
    np.testing.assert_array_equal(blocked[off], plain)
    # the layout is a bijection: every byte of the padded matrix has its own place
    assert len(np.unique(off)) == rows * cols
    np.testing.assert_array_equal(oracle_lib.unblock_scales(blocked, rows, cols), plain)


def test_blocked_layout_golden(oracle_lib):
    """Hand-placed positions (tests/golden/blocked_scales_130x8.txt) of a
    130 x 8 scale matrix whose byte at (r, c) is a distinct tag."""
    rows, cols = 130, 8
    plain = ((np.arange(rows)[:, None] * 7 + np.arange(cols)[None, :] * 3) % 251).astype(np.uint8)
    blocked = oracle_lib.block_scales(plain, rows, cols, pad_value=255)
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "blocked_scales_130x8.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        r, c, pos = (int(v) for v in line.split())
        assert blocked[pos] == plain[r, c], (r, c, pos)
    # rows 130..255 of the second band are padding
    assert np.count_nonzero(blocked == 255) >= (256 - 130) * cols


def test_blocked_pins_detect_plausible_mistakes(oracle_lib):
    """A layout with the 32-row groups and the runs swapped, or with the atoms
    of a band laid out row-first, fails the CuTe-atom pin."""
    rows, cols = 256, 8
    off = _cute_atom_offsets(rows, cols)
    r = np.arange(rows)[:, None]
    s = np.arange(cols)[None, :]
    swapped = 512 * ((r // 128) * 2 + s // 4) + 4 * (r % 32) + 16 * ((r // 32) % 4) + s % 4
    row_first = 512 * ((s // 4) * 2 + r // 128) + 16 * (r % 32) + 4 * ((r // 32) % 4) + s % 4
    assert not np.array_equal(swapped, off)
    assert not np.array_equal(row_first, off)


# ------------------------------------------------------------------- MXFP4

def test_e8m0_closed_form(oracle_lib):
    assert oracle_lib.e8m0(127) == 1.0
    assert oracle_lib.e8m0(128) == 2.0
    assert oracle_lib.e8m0(126) == 0.5
    assert oracle_lib.e8m0(0) == 2.0 ** -127
    assert oracle_lib.e8m0(254) == 2.0 ** 127
    assert math.isnan(oracle_lib.e8m0(255))
    for c in range(254):
        assert oracle_lib.e8m0(c + 1) == 2.0 * oracle_lib.e8m0(c)


@pytest.mark.parametrize("dist", ["pos", "unit"])
@pytest.mark.parametrize("shape", [(1, 1, 32), (3, 5, 64), (8, 8, 128), (7, 4, 96)])
def test_mx_bruteforce(oracle_lib, dist, shape):
    """float64 matmul is exact here: products of two E2M1 values scaled by at
    most 2^+-6, summed over at most 128 terms."""
    M, N, K = shape
    A, B, SA, SB = workloads.make_mx_inputs([M], [N], [K], 9, dist=dist)
    want16, want = ind.brute_mx_group(A[0], B[0], SA[0], SB[0], M, N, K)
    C, X = oracle_lib.mx_group_gemm([M], [N], [K], A, B, SA, SB, exact=True)
    np.testing.assert_array_equal(X[0], want)
    np.testing.assert_array_equal(C[0].view(np.uint16), want16.view(np.uint16))


@pytest.mark.parametrize("shape", [(3, 5, 64), (4, 3, 128)])
def test_mx_wide_scales_exact(oracle_lib, shape):
    """Scales 2^-20 .. 2^20 (term exponents spread over 80 binades, beyond
    float64): every output against the exact rational sum, rounded to the
    nearest fp16 (ties to even) by exact comparison with the fp16 values
    around it."""
    from fractions import Fraction
    M, N, K = shape
    A, B, SA, SB = workloads.make_mx_inputs([M], [N], [K], 10, dist="wide")
    a = ind.unpack_fp4(A[0], M, K)
    b = ind.unpack_fp4(B[0], N, K)
    C = oracle_lib.mx_group_gemm([M], [N], [K], A, B, SA, SB)[0]
    for m in range(M):
        for n in range(N):
            x = ind.exact_mx_element(a[m], SA[0][m], b[n], SB[0][n])
            got = float(C[m, n])
            cand = np.float16(float(x))
            near = sorted({float(v) for v in (cand, np.nextafter(cand, np.float16(-np.inf)),
                                              np.nextafter(cand, np.float16(np.inf))) if np.isfinite(v)},
                          key=lambda v: abs(Fraction(v) - x))
            best = near[0]
            if len(near) > 1 and abs(Fraction(near[1]) - x) == abs(Fraction(near[0]) - x):
                best = [v for v in near[:2] if (int(np.float16(v).view(np.uint16)) & 1) == 0][0]
            if x == 0:
                assert got == 0.0
            elif abs(x) >= 65520:
                assert np.isinf(got) and (got > 0) == (x > 0)
            else:
                assert got == best, (m, n, float(x), got, best)


def test_mx_onehot_block_index(oracle_lib):
    """A single non-zero code at K index k in A and in B, with a distinct
    scale per 32-K block: the one output is e2m1 * e2m1 * 2^(ea + eb - 254)
    with the scales of block k // 32 (block edges 31, 32, 63, 64)."""
    M, N, K = 2, 3, 128
    table = ind.e2m1_table()
    sa = np.array([[120, 125, 130, 135]] * M, dtype=np.uint8)
    sb = np.array([[131, 126, 121, 129]] * N, dtype=np.uint8)
    for k in (0, 1, 31, 32, 63, 64, 127):
        a = np.zeros((M, K), np.uint8)
        b = np.zeros((N, K), np.uint8)
        a[1, k] = 3      # 1.5
        b[2, k] = 13     # -3
        C, X = oracle_lib.mx_group_gemm([M], [N], [K], [ind.pack_fp4(a)], [ind.pack_fp4(b)], [sa], [sb], exact=True)
        want = table[3] * table[13] * 2.0 ** (int(sa[1, k // 32]) + int(sb[2, k // 32]) - 254)
        assert X[0][1, 2] == want, k
        assert np.count_nonzero(X[0]) == 1


def test_mx_unit_scales_equal_nvfp4_unit_scales(oracle_lib):
    """With every scale 1.0 the two formats compute the same sum of E2M1
    products: the MX oracle equals the (separately pinned) NVFP4 oracle."""
    M, N, K = [5, 9], [7, 3], [256, 96]
    A, B, _, _ = workloads.make_mx_inputs(M, N, K, 4)
    nsa = [np.full((m, k // 16), 0x38, np.uint8) for m, k in zip(M, K)]
    nsb = [np.full((n, k // 16), 0x38, np.uint8) for n, k in zip(N, K)]
    msa = [np.full((m, k // 32), 127, np.uint8) for m, k in zip(M, K)]
    msb = [np.full((n, k // 32), 127, np.uint8) for n, k in zip(N, K)]
    Cn = oracle_lib.group_gemm(M, N, K, A, B, nsa, nsb)
    Cm = oracle_lib.mx_group_gemm(M, N, K, A, B, msa, msb)
    for a, b in zip(Cn, Cm):
        np.testing.assert_array_equal(a.view(np.uint16), b.view(np.uint16))


def test_mx_exponent_spread_limit(oracle_lib):
    """Scales 2^-67 and 2^+23 in one dot product (a 90-binade spread): the
    oracle's integer sum matches an exact rational computation; a spread
    beyond 96 binades is reported, not approximated."""
    K = 64
    rng = np.random.default_rng(3)
    a = rng.integers(0, 16, size=(1, K), dtype=np.uint8)
    b = rng.integers(0, 16, size=(1, K), dtype=np.uint8)
    sb = np.array([[127, 127]], np.uint8)
    sa = np.array([[60, 150]], np.uint8)
    c16, x = oracle_lib.mx_gemm_element(1, 1, K, ind.pack_fp4(a), ind.pack_fp4(b), sa, sb, 0, 0)
    want = ind.exact_mx_element(a[0], sa[0], b[0], sb[0])
    assert x == float(want)
    assert c16 == int(np.float16(float(want)).view(np.uint16))
    with pytest.raises(ValueError):
        oracle_lib.mx_gemm_element(1, 1, K, ind.pack_fp4(a), ind.pack_fp4(b), np.array([[20, 150]], np.uint8),
                                   sb, 0, 0)


def test_mx_pins_detect_plausible_mistakes(oracle_lib):
    """A scale per 16 K instead of 32, or a missing -127 bias, changes the
    brute-force values the MX pins compare against."""
    M, N, K = 4, 4, 128
    A, B, SA, SB = workloads.make_mx_inputs([M], [N], [K], 12)
    _, base = ind.brute_mx_group(A[0], B[0], SA[0], SB[0], M, N, K)
    sa16 = np.repeat(SA[0], 2, axis=1)[:, : K // 32]       # block k//16 read as k//32
    assert not np.array_equal(ind.brute_mx_group(A[0], B[0], sa16, SB[0], M, N, K)[1], base)
    C = oracle_lib.mx_group_gemm([M], [N], [K], A, B, SA, SB, exact=True)[1][0]
    assert not np.array_equal(C * 2.0, base)
    np.testing.assert_array_equal(C, base)


# ------------------------------------------------------------------ batched

def test_batched_is_independent_slices(oracle_lib):
    """(M, N, K, L) problems: slice l of every operand is its l-th consecutive
    block, and each output slice is the single product of those slices
    (checked against separate single-problem calls); changing one slice of
    A changes that output slice only."""
    M, N, K, L = [5, 9], [7, 3], [128, 256], [3, 2]
    A, B, SA, SB = [], [], [], []
    for i in range(2):
        parts = [workloads.make_group(40 + l, i, M[i], N[i], K[i]) for l in range(L[i])]
        A.append(np.concatenate([p[0].reshape(-1) for p in parts]))
        B.append(np.concatenate([p[1].reshape(-1) for p in parts]))
        SA.append(np.concatenate([p[2].reshape(-1) for p in parts]))
        SB.append(np.concatenate([p[3].reshape(-1) for p in parts]))
    C = oracle_lib.group_gemm_batched(M, N, K, L, A, B, SA, SB)
    for i in range(2):
        for l in range(L[i]):
            p = workloads.make_group(40 + l, i, M[i], N[i], K[i])
            want = oracle_lib.group_gemm([M[i]], [N[i]], [K[i]], [p[0]], [p[1]], [p[2]], [p[3]])[0]
            np.testing.assert_array_equal(C[i][l].view(np.uint16), want.view(np.uint16))
    A2 = [a.copy() for a in A]
    A2[0][M[0] * K[0] // 2: 2 * M[0] * K[0] // 2] ^= 0x11          # slice 1 of group 0
    C2 = oracle_lib.group_gemm_batched(M, N, K, L, A2, B, SA, SB)
    assert not np.array_equal(C2[0][1].view(np.uint16), C[0][1].view(np.uint16))
    for i, l in [(0, 0), (0, 2), (1, 0), (1, 1)]:
        np.testing.assert_array_equal(C2[i][l].view(np.uint16), C[i][l].view(np.uint16))
