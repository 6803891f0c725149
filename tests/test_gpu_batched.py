"""Parity of nvfp4_group_gemm_batched ((M, N, K, L) per group, slices
consecutive in every operand) with the oracle, on the GPU through the C ABI."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import workloads
from tests import _compare

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SENTINEL = 0x7E00


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_block_scaled_grouped_amd as nv
    nv.load()
    return nv


def _inputs(M, N, K, L, seed):
    A, B, SA, SB = [], [], [], []
    for i in range(len(M)):
        parts = [workloads.make_group(seed + l, i, M[i], N[i], K[i]) for l in range(L[i])]
        cat = lambda j: (np.concatenate([p[j].reshape(-1) for p in parts]) if parts
                         else np.zeros(0, np.uint8))
        A.append(cat(0))
        B.append(cat(1))
        SA.append(cat(2))
        SB.append(cat(3))
    return A, B, SA, SB


@pytest.mark.parametrize("M,N,K,L", [
    ([16, 40], [64, 96], [256, 512], [3, 2]),
    ([64, 8, 200], [256, 128, 320], [1024, 128, 768], [1, 0, 4]),
    ([17], [100], [512], [1]),
])
def test_batched_parity(nv, oracle_lib, M, N, K, L):
    print("batched M=%s N=%s K=%s L=%s" % (M, N, K, L), flush=True)
    A, B, SA, SB = _inputs(M, N, K, L, 81)
    C_ref, X = oracle_lib.group_gemm_batched(M, N, K, L, A, B, SA, SB, exact=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    dC = [torch.full((max(l * m * n, 1),), 0, dtype=torch.int16, device="cuda").fill_(SENTINEL)
          .view(torch.float16)[:l * m * n] for m, n, l in zip(M, N, L)]
    nv.group_gemm_batched([dev(a) for a in A], [dev(b) for b in B], [dev(s) for s in SA], [dev(s) for s in SB],
                          dC, M, N, K, L)
    torch.cuda.synchronize()
    for i in range(len(M)):
        got = dC[i].cpu().numpy().reshape(L[i], M[i], N[i]) if L[i] else None
        for l in range(L[i]):
            _compare.assert_close(got[l], C_ref[i][l], X[i][l], "group %d slice %d" % (i, l))
