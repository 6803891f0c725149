"""Parity of nvfp4_group_gemm_blocked (scales in the blocked 128 x 4 atom
layout) on the GPU, through the C ABI.

The blocked scale arrays are made from the row-major ones by the oracle's
layout function (pad bytes 0x7F, an E4M3 NaN, so a kernel that read a pad
byte into a result would produce NaN there).  Problems are compared
element by element with the oracle (the larger workloads at full size are in
test_gpu_full.py).
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
NAN_SCALE = 0x7F


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


def _run(nv, M, N, K, A, B, SA, SB, blocked):
    dC = [torch.full((m, n), 0, dtype=torch.int16, device="cuda").fill_(SENTINEL).view(torch.float16)
          for m, n in zip(M, N)]
    nv.group_gemm([_dev(a) for a in A], [_dev(b) for b in B], [_dev(s) for s in SA], [_dev(s) for s in SB],
                  dC, M=M, N=N, K=K, blocked=blocked)
    torch.cuda.synchronize()
    return [c.cpu().numpy() for c in dC]


def _blocked(oracle_lib, S, rows, K):
    return [oracle_lib.block_scales(s, r, k // 16, pad_value=NAN_SCALE) for s, r, k in zip(S, rows, K)]


@pytest.mark.parametrize("M,N,K", [
    ([1], [256], [256]),
    ([17, 130], [100, 300], [512, 1280]),
    ([385, 129, 192], [520, 260, 33], [384, 640, 128]),
    ([248, 64], [512, 1024], [7168, 1024]),
])
def test_blocked_parity(nv, oracle_lib, M, N, K):
    _say("blocked case M=%s N=%s K=%s" % (M, N, K))
    A, B, SA, SB = workloads.make_inputs(M, N, K, 44)
    C_ref, X = oracle_lib.group_gemm(M, N, K, A, B, SA, SB, exact=True)
    C = _run(nv, M, N, K, A, B, _blocked(oracle_lib, SA, M, K), _blocked(oracle_lib, SB, N, K), True)
    for i in range(len(M)):
        _compare.assert_close(C[i], C_ref[i], X[i], "group %d" % i)
