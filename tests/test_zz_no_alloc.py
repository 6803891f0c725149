"""nvfp4_group_gemm_noalloc (split-tile workspace in the library's static
device scratch, no allocation) against nvfp4_group_gemm and the oracle, on
the GPU through the C ABI: two calls in a row, the second with a smaller
problem, each compared bit for bit with the allocating entry point's output
on the same inputs (the same kernels and schedule run, so the results are
identical) and element by element with the oracle under the stated
tolerance."""
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


def _run(nv, M, N, K, dev, noalloc):
    dC = [torch.full((m, n), 0, dtype=torch.int16, device="cuda").fill_(SENTINEL).view(torch.float16)
          for m, n in zip(M, N)]
    nv.group_gemm(*dev, dC, M=M, N=N, K=K, noalloc=noalloc)
    torch.cuda.synchronize()
    return [c.cpu().numpy() for c in dC]


def test_noalloc_matches_allocating_entry_point(nv, oracle_lib):
    # The larger problem splits most tiles over several workgroups (so the
    # partial slots and counters are used), the smaller one reuses what the
    # larger one left in the scratch.
    cases = [([80, 176, 128, 248], [4096] * 4, [2048] * 4, 91), ([64, 96], [256, 256], [512, 512], 92)]
    inputs, outs = [], []
    for M, N, K, seed in cases:          # the two no-alloc calls, in a row
        _say("no-alloc M=%s N=%s K=%s seed=%d" % (M, N, K, seed))
        A, B, SA, SB = workloads.make_inputs(M, N, K, seed)
        dev = ([_dev(a) for a in A], [_dev(b) for b in B], [_dev(s) for s in SA], [_dev(s) for s in SB])
        inputs.append((A, B, SA, SB, dev))
        outs.append(_run(nv, M, N, K, dev, noalloc=True))
    for (M, N, K, seed), (A, B, SA, SB, dev), C_na in zip(cases, inputs, outs):
        _say("allocating entry point and oracle M=%s" % (M,))
        C_al = _run(nv, M, N, K, dev, noalloc=False)
        C_ref, X = oracle_lib.group_gemm(M, N, K, A, B, SA, SB, exact=True)
        for i in range(len(M)):
            np.testing.assert_array_equal(C_na[i].view(np.uint16), C_al[i].view(np.uint16))
            _compare.assert_close(C_na[i], C_ref[i], X[i], "no-alloc group %d" % i)


def test_noalloc_rejects_bad_arguments_before_any_hip_call(nv):
    assert nv.group_gemm_ptrs([4], [8], [24], [0x10000], [0x10000], [0x10000], [0x10000], [0x10000],
                              0, noalloc=True) == nv.INVALID_ARG
    assert "multiple of 16" in nv.last_error()
