"""Full-output parity of the three grouped-GEMM kernels with the oracle, on the
GPU through the C ABI, at the workloads' full sizes and on every m-block size.

Every output element of the HIP path is compared with the oracle's (exact sum
rounded once to fp16) under the stated tolerance, and the worst |err| / tol
is printed per case.  The oracle runs once per (format, problem) and its result
is shared by the cases that use it: the blocked-scale kernel computes the same
values as the row-major one from the same scales, so both are compared with
the one NVFP4 oracle result.

Shapes:
  * the four larger workloads (the timing shapes of page
    kernelbot-nvfp4-group-gemm-495528, whose per-element definition is
    custom_kernel_fallback on page kernelbot-nvfp4-group-gemm-505431), run
    twice for bitwise determinism;
  * M = [176, 128, 248, 160], N = 8192, K = 1024 with the m-block size forced
    to each of 1..12 fragments of 16 rows (so every instantiation of every
    kernel runs its steady-state loop and its split-tile fix-up), and with
    the wait limit 0 at 8, 11 and 12 fragments (the fix-up handed over to the
    last contributor, in its one-contributor-at-a-time and half-tile forms);
  * a larger problem after a smaller one on one stream (the workspace is
    sized once per stream and reused).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import workloads
from tests import _compare

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SENTINEL = 0x7E00    # fp16 NaN: an output the kernel fails to write shows up
NAN_SCALE = 0x7F     # E4M3 NaN in the blocked layout's pad bytes
FMTS = ["nvfp4", "blocked", "mxfp4"]
LARGE = [workloads.config(n) for n in ("g2_k1536_n4096", "g2_k4096_n3072", "g8_k2048_n7168", "g8_k7168_n4096")]
SWEEP = dict(name="sweep", M=[176, 128, 248, 160], N=[8192] * 4, K=[1024] * 4, seed=404)

_inputs = {}
_refs = {}


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


def _problem(cfg, fmt, oracle_lib):
    """Device operands of (cfg, fmt) and the oracle's (C, X) for them."""
    okey = "mxfp4" if fmt == "mxfp4" else "nvfp4"
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    if (cfg["name"], okey) not in _inputs:
        make = workloads.make_mx_inputs if okey == "mxfp4" else workloads.make_inputs
        _inputs[(cfg["name"], okey)] = make(M, N, K, cfg["seed"])
    A, B, SA, SB = _inputs[(cfg["name"], okey)]
    if (cfg["name"], okey) not in _refs:
        _say("oracle %s %s" % (okey, cfg["name"]))
        run = oracle_lib.mx_group_gemm if okey == "mxfp4" else oracle_lib.group_gemm
        _refs[(cfg["name"], okey)] = run(M, N, K, A, B, SA, SB, exact=True)
    if fmt == "blocked":
        SA = [oracle_lib.block_scales(s, r, k // 16, pad_value=NAN_SCALE) for s, r, k in zip(SA, M, K)]
        SB = [oracle_lib.block_scales(s, r, k // 16, pad_value=NAN_SCALE) for s, r, k in zip(SB, N, K)]
    dev = ([_dev(a) for a in A], [_dev(b) for b in B], [_dev(s) for s in SA], [_dev(s) for s in SB])
    return dev, _refs[(cfg["name"], okey)]


def _run(nv, cfg, fmt, dev, stream=None):
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    dC = [torch.full((m, n), 0, dtype=torch.int16, device="cuda").fill_(SENTINEL).view(torch.float16)
          for m, n in zip(M, N)]
    nv.group_gemm(*dev, dC, M=M, N=N, K=K, stream=stream, blocked=(fmt == "blocked"),
                  fmt="mxfp4" if fmt == "mxfp4" else "nvfp4")
    torch.cuda.synchronize()
    return [c.cpu().numpy() for c in dC]


def _compare_all(C, ref, what):
    C_ref, X = ref
    worst = 0.0
    for i in range(len(C)):
        worst = max(worst, _compare.assert_close(C[i], C_ref[i], X[i], "%s group %d" % (what, i)))
    _say("  %s: worst |err|/tol %.4f" % (what, worst))
    return worst


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("cfg", LARGE, ids=[c["name"] for c in LARGE])
def test_workload_full(nv, oracle_lib, cfg, fmt):
    _say("full workload %s %s" % (fmt, cfg["name"]))
    dev, ref = _problem(cfg, fmt, oracle_lib)
    C1 = _run(nv, cfg, fmt, dev)
    C2 = _run(nv, cfg, fmt, dev)
    for a, b in zip(C1, C2):
        np.testing.assert_array_equal(a.view(np.uint16), b.view(np.uint16))
    _compare_all(C1, ref, "%s %s" % (fmt, cfg["name"]))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("maxf", list(range(1, 13)))
def test_every_mblock_size(nv, oracle_lib, maxf, fmt):
    _say("m-block size %d, %s, M=%s N=%s K=%s" % (maxf, fmt, SWEEP["M"], SWEEP["N"][0], SWEEP["K"][0]))
    dev, ref = _problem(SWEEP, fmt, oracle_lib)
    nv.set_max_frags(maxf)
    try:
        C = _run(nv, SWEEP, fmt, dev)
    finally:
        nv.set_max_frags(0)
    _compare_all(C, ref, "%s m-block %d" % (fmt, maxf))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("maxf", [8, 11, 12])
def test_hand_over_every_large_mblock(nv, oracle_lib, maxf, fmt):
    """Wait limit 0: the first contributor of every split tile stores its
    partial and hands the fix-up over; the last to arrive sums them all."""
    _say("hand-over, m-block size %d, %s" % (maxf, fmt))
    dev, ref = _problem(SWEEP, fmt, oracle_lib)
    nv.set_max_frags(maxf)
    nv.set_wait_limit(0)
    try:
        C = _run(nv, SWEEP, fmt, dev)
    finally:
        nv.set_wait_limit(1 << 20)
        nv.set_max_frags(0)
    _compare_all(C, ref, "%s hand-over m-block %d" % (fmt, maxf))


def test_larger_after_smaller_on_one_stream(nv, oracle_lib):
    """The first call on a new stream sizes its workspace; a larger problem
    after a smaller one reuses it, with no reallocation."""
    s = torch.cuda.Stream()
    small = workloads.SMALL
    for cfg in (small, SWEEP, small):
        _say("stream reuse %s" % cfg["name"])
        dev, ref = _problem(cfg, "nvfp4", oracle_lib)
        with torch.cuda.stream(s):
            C = _run(nv, cfg, "nvfp4", dev, stream=s)
        _compare_all(C, ref, "stream reuse %s" % cfg["name"])


LOW_M = dict(name="low_m", M=[40, 72, 164, 148, 8, 24], N=[520, 260, 1024, 300, 64, 33],
             K=[512, 1024, 384, 768, 256, 128], seed=405)


@pytest.mark.parametrize("fmt", FMTS)
def test_low_m_groups(nv, oracle_lib, fmt):
    """Groups whose row count ends in a half-used 16-row fragment (M = 40,
    72, 164, 148: 8, 8, 4 and 4 rows past a multiple of 32), and tiny M:
    the last fragment's padding rows are computed from zeros and never
    stored."""
    _say("low M %s M=%s" % (fmt, LOW_M["M"]))
    dev, ref = _problem(LOW_M, fmt, oracle_lib)
    _compare_all(_run(nv, LOW_M, fmt, dev), ref, "%s low M" % fmt)
