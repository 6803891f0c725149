"""Parity of mxfp4_group_gemm (E8M0 scale per 32 K, native block-scaled FP4
MFMA) with the MXFP4 oracle, on the GPU through the C ABI.

Small and ragged problems element by element (the larger workloads at full
size, element by element, are in test_gpu_full.py).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import workloads
from tests import _compare

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SENTINEL = 0x7E00


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_block_scaled_grouped_amd as nv
    nv.load()
    return nv


def _dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _run(nv, M, N, K, A, B, SA, SB):
    dC = [torch.full((m, n), 0, dtype=torch.int16, device="cuda").fill_(SENTINEL).view(torch.float16)
          for m, n in zip(M, N)]
    nv.group_gemm([_dev(a) for a in A], [_dev(b) for b in B], [_dev(s) for s in SA], [_dev(s) for s in SB],
                  dC, M=M, N=N, K=K, fmt="mxfp4")
    torch.cuda.synchronize()
    return [c.cpu().numpy() for c in dC]


@pytest.mark.parametrize("M,N,K,dist", [
    ([1], [256], [128], "pos"),
    ([16], [16], [128], "unit"),
    ([17, 130], [100, 300], [512, 1280], "pos"),
    ([385, 129, 192], [520, 260, 33], [384, 640, 128], "pos"),
    ([200], [300], [1792], "pos"),
    ([64, 96], [256, 256], [512, 512], "wide"),
])
def test_mx_parity(nv, oracle_lib, M, N, K, dist):
    """For the "wide" scales (2^-20 .. 2^20) single terms reach 4e13 and
    cancel, and no fp32 accumulation meets 2e-3 relative accuracy on the
    remainder; there the tolerance adds the standard bound of a sum
    accumulated in fp32 in chunks, (K/32) 2^-24 sum|terms| (the same rule as
    the NVFP4 "finite" scale test)."""
    _say("mx case M=%s N=%s K=%s dist=%s" % (M, N, K, dist))
    A, B, SA, SB = workloads.make_mx_inputs(M, N, K, 61, dist=dist)
    C_ref, X = oracle_lib.mx_group_gemm(M, N, K, A, B, SA, SB, exact=True)
    C = _run(nv, M, N, K, A, B, SA, SB)
    extra = None
    if dist == "wide":
        ab = lambda xs: [x & np.uint8(0x77) for x in xs]
        S = oracle_lib.mx_group_gemm(M, N, K, ab(A), ab(B), SA, SB, exact=True)[1]
        extra = [S[i] * (K[i] / 32) * 2.0 ** -24 for i in range(len(M))]
    for i in range(len(M)):
        _compare.assert_close(C[i], C_ref[i], X[i], "group %d" % i,
                              extra_tol=None if extra is None else extra[i])


def test_mx_many_groups(nv, oracle_lib):
    g = 37
    M = [1 + (7 * i) % 50 for i in range(g)]
    N = [16 + (13 * i) % 90 for i in range(g)]
    K = [128 * (1 + i % 3) for i in range(g)]
    A, B, SA, SB = workloads.make_mx_inputs(M, N, K, 62)
    C_ref, X = oracle_lib.mx_group_gemm(M, N, K, A, B, SA, SB, exact=True)
    C = _run(nv, M, N, K, A, B, SA, SB)
    for i in range(g):
        _compare.assert_close(C[i], C_ref[i], X[i], "group %d" % i)


def test_mx_long_segments_run_as_several_chains(nv, oracle_lib):
    """K = 17408 (136 stages of 128) over 128 column blocks, as the NVFP4
    chain test: a workgroup's segment runs as several chains, each restarting
    the scale blocks at its first stage.  Checked on sampled elements
    (corners, centre and random points) against the oracle's one-element
    form."""
    M, N, K = [96], [32768], [17408]
    _say("mx long segments M=%s N=%s K=%s" % (M, N, K))
    A, B, SA, SB = workloads.make_mx_inputs(M, N, K, 63)
    C = _run(nv, M, N, K, A, B, SA, SB)[0]
    assert not np.isnan(C.astype(np.float32)).any()
    rng = np.random.default_rng(8)
    pts = {(m, n) for m in (0, M[0] // 2, M[0] - 1) for n in (0, N[0] // 2, N[0] - 1)}
    pts |= {(int(m), int(n)) for m, n in zip(rng.integers(0, M[0], 300), rng.integers(0, N[0], 300))}
    y, r, x = [], [], []
    for m, n in sorted(pts):
        c16, ex = oracle_lib.mx_gemm_element(M[0], N[0], K[0], A[0], B[0], SA[0], SB[0], m, n)
        y.append(C[m, n])
        r.append(np.uint16(c16).view(np.float16))
        x.append(ex)
    _compare.assert_close(np.array(y), np.array(r), np.array(x), "mx long segments")
