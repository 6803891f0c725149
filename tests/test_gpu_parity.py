"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Small and medium problems are compared element by element with the full
oracle output (the larger workloads at full size are in test_gpu_full.py);
one problem too large for the whole oracle output, whose segments run as
several chains, is checked on sampled elements the oracle computes one by
one.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import workloads
from tests import _compare

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SENTINEL = 0x7E00   # fp16 NaN: any output the kernel fails to write shows up


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


def _run_gpu(nv, M, N, K, A, B, SA, SB, stream=None):
    dA = [_dev(a) for a in A]
    dB = [_dev(b) for b in B]
    dSA = [_dev(s) for s in SA]
    dSB = [_dev(s) for s in SB]
    dC = [torch.full((m, n), 0, dtype=torch.int16, device="cuda").fill_(SENTINEL).view(torch.float16)
          for m, n in zip(M, N)]
    nv.group_gemm(dA, dB, dSA, dSB, dC, M=M, N=N, K=K, stream=stream)
    torch.cuda.synchronize()
    return [c.cpu().numpy() for c in dC]


def _abs_sums(oracle_lib, M, N, K, A, B, SA, SB):
    """sum_k |a_k b_k| per output, from the oracle run on sign-cleared codes
    and scales (clearing bit 3 of every nibble and bit 7 of every scale)."""
    ab = lambda xs: [x & np.uint8(0x77) for x in xs]
    sc = lambda xs: [x & np.uint8(0x7F) for x in xs]
    return oracle_lib.group_gemm(M, N, K, ab(A), ab(B), sc(SA), sc(SB), exact=True)[1]


def _full_parity(nv, oracle_lib, M, N, K, seed, dist="pos"):
    """Element-wise parity.  For the workload distribution ("pos": scales in
    [1/8, 15]) the stated tolerance applies as is.  For "finite" (scales up to
    448, so single terms reach 1e7 and cancel) no fp32 accumulation can reach
    1e-2 absolute accuracy near zero; there the tolerance adds the standard
    bound for a sum accumulated in fp32 in chunks, (K/16) * 2^-24 * sum|terms|."""
    _say("case M=%s N=%s K=%s seed=%d dist=%s" % (M, N, K, seed, dist))
    A, B, SA, SB = workloads.make_inputs(M, N, K, seed, dist=dist)
    C_ref, X = oracle_lib.group_gemm(M, N, K, A, B, SA, SB, exact=True)
    C_gpu = _run_gpu(nv, M, N, K, A, B, SA, SB)
    extra = None
    if dist == "finite":
        S = _abs_sums(oracle_lib, M, N, K, A, B, SA, SB)
        extra = [S[i] * (K[i] / 16) * 2.0 ** -24 for i in range(len(M))]
    worst = 0.0
    for i in range(len(M)):
        worst = max(worst, _compare.assert_close(C_gpu[i], C_ref[i], X[i], "group %d" % i,
                                                 extra_tol=None if extra is None else extra[i]))
    return worst


# ------------------------------------------------------------------ dequant

@pytest.mark.parametrize("K", [64, 48, 16, 1024])
def test_dequant_exhaustive(nv, oracle_lib, K):
    """Every (E2M1 code, E4M3 scale code) pair: one row per scale code, each
    row cycling through the 16 codes.  fp16 holds every product exactly, so
    the result must equal the oracle's decoded value bit for bit."""
    rows = 256
    codes = np.tile(np.arange(16, dtype=np.uint8), (rows, K // 16))
    codes = (codes + np.arange(rows, dtype=np.uint8)[:, None]) % 16
    X = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    SF = np.repeat(np.arange(256, dtype=np.uint8)[:, None], K // 16, axis=1).copy()
    SF[:, 1::2] = SF[:, 1::2] ^ 0x80          # odd blocks: the negated scale
    want = oracle_lib.dequant(X, SF, rows, K)
    out = torch.zeros(rows * K, dtype=torch.float16, device="cuda")
    nv.dequant_f16(_dev(X), _dev(SF), out, rows, K)
    got = out.cpu().numpy().reshape(rows, K).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])


# ------------------------------------------------------------ small / medium

def test_config1_full(nv, oracle_lib):
    cfg = workloads.SMALL
    _full_parity(nv, oracle_lib, cfg["M"], cfg["N"], cfg["K"], cfg["seed"])


@pytest.mark.parametrize("M,N,K", [
    ([1], [256], [256]),
    ([17], [100], [512]),
    ([40, 76], [520, 130], [768, 256]),
    ([64, 65, 130], [256, 257, 259], [256, 512, 256]),
    ([200], [300], [1792]),
    ([5, 0, 7], [9, 11, 0], [256, 256, 256]),
    ([385, 129, 192], [520, 260, 33], [384, 640, 128]),
])
def test_ragged_shapes(nv, oracle_lib, M, N, K):
    _full_parity(nv, oracle_lib, M, N, K, seed=21)


def test_many_groups_span_launch_batches(nv, oracle_lib):
    g = 37
    M = [1 + (7 * i) % 50 for i in range(g)]
    N = [16 + (13 * i) % 90 for i in range(g)]
    K = [256 * (1 + i % 3) for i in range(g)]
    _full_parity(nv, oracle_lib, M, N, K, seed=5)


@pytest.mark.parametrize("dist", ["finite", "unit"])
def test_other_scale_distributions(nv, oracle_lib, dist):
    _full_parity(nv, oracle_lib, [48, 96], [512, 256], [512, 1024], seed=8, dist=dist)


def test_zero_k_writes_zeros(nv):
    M, N = [4, 3], [8, 5]
    e = torch.zeros(4096, dtype=torch.uint8, device="cuda")   # valid, never read
    C = [torch.full((m, n), 1.0, dtype=torch.float16, device="cuda") for m, n in zip(M, N)]
    pa = [e.data_ptr()] * 2
    rc = nv.group_gemm_ptrs(M, N, [0, 0], pa, pa, pa, pa, [c.data_ptr() for c in C],
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == nv.OK
    for c in C:
        assert torch.all(c == 0)
    del e


def test_non_default_stream_and_determinism(nv, oracle_lib):
    M, N, K = [33, 70], [384, 200], [512, 768]
    A, B, SA, SB = workloads.make_inputs(M, N, K, 17)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        C1 = _run_gpu(nv, M, N, K, A, B, SA, SB, stream=s)
    C2 = _run_gpu(nv, M, N, K, A, B, SA, SB)
    for a, b in zip(C1, C2):
        np.testing.assert_array_equal(a.view(np.uint16), b.view(np.uint16))
    C_ref, X = oracle_lib.group_gemm(M, N, K, A, B, SA, SB, exact=True)
    for i in range(2):
        _compare.assert_close(C1[i], C_ref[i], X[i])


# ------------------------------------------------------------- long segments

def _sample_points(M, N, rng, n_rand):
    pts = set()
    for m in {0, M - 1, M // 2}:
        for n in {0, N - 1, N // 2}:
            pts.add((m, n))
    for m, n in zip(rng.integers(0, M, n_rand), rng.integers(0, N, n_rand)):
        pts.add((int(m), int(n)))
    return sorted(pts)


def test_long_segments_run_as_several_chains(nv, oracle_lib):
    """K = 17408 (136 stages of 128) over 128 column blocks: a workgroup's
    range covers more than 64 stages of a tile, so its segment runs as two
    chains that meet in the scratch slot.  Checked on sampled elements."""
    M, N, K = [96], [32768], [17408]
    _say("long segments M=%s N=%s K=%s" % (M, N, K))
    A, B, SA, SB = workloads.make_inputs(M, N, K, 31)
    C = _run_gpu(nv, M, N, K, A, B, SA, SB)[0]
    assert not np.isnan(C.astype(np.float32)).any()
    rng = np.random.default_rng(7)
    y, r, x = [], [], []
    for m, n in _sample_points(M[0], N[0], rng, 300):
        c16, ex = oracle_lib.gemm_element(M[0], N[0], K[0], A[0], B[0], SA[0], SB[0], m, n)
        y.append(C[m, n])
        r.append(np.uint16(c16).view(np.float16))
        x.append(ex)
    _compare.assert_close(np.array(y), np.array(r), np.array(x), "long segments")


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_fixup_hand_over_path(nv, oracle_lib, fmt):
    """With a wait limit of 0, the first contributor of every split tile
    hands the fix-up over to the last of the others (the path taken when a
    wait runs out).  Shapes whose tiles are split over 2 to 7 workgroups."""
    M, N, K = [192, 320], [3072, 1024], [4096, 2048]
    _say("hand-over fix-up %s M=%s N=%s K=%s" % (fmt, M, N, K))
    if fmt == "mxfp4":
        A, B, SA, SB = workloads.make_mx_inputs(M, N, K, 71)
        C_ref, X = oracle_lib.mx_group_gemm(M, N, K, A, B, SA, SB, exact=True)
    else:
        A, B, SA, SB = workloads.make_inputs(M, N, K, 71)
        C_ref, X = oracle_lib.group_gemm(M, N, K, A, B, SA, SB, exact=True)
    dC = [torch.full((m, n), 0, dtype=torch.int16, device="cuda").fill_(SENTINEL).view(torch.float16)
          for m, n in zip(M, N)]
    nv.set_wait_limit(0)
    try:
        nv.group_gemm([_dev(a) for a in A], [_dev(b) for b in B], [_dev(s) for s in SA], [_dev(s) for s in SB],
                      dC, M=M, N=N, K=K, fmt=fmt)
        torch.cuda.synchronize()
    finally:
        nv.set_wait_limit(1 << 20)
    for i in range(len(M)):
        _compare.assert_close(dC[i].cpu().numpy(), C_ref[i], X[i], "group %d" % i)
