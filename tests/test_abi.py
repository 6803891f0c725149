"""CPU tests of the C ABI: the library loads, exports what the header declares,
and rejects bad arguments before any HIP call (no GPU needed)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import nvfp4_block_scaled_grouped_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(nv._lib.LIB_PATH):
        from nvfp4_block_scaled_grouped_amd import build
        build.build()
    return nv.load()


def _declared_functions():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", txt, flags=re.M)
    return names


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert "nvfp4_group_gemm" in names and "nvfp4_dequant_f16" in names
    for n in names:
        assert hasattr(lib, n), n


def test_version(lib):
    assert nv.version() == 7


A16 = 0x10000          # fake, aligned addresses: never dereferenced, every case
MIS = 0x10008          # below is rejected before a kernel could be launched


def _call(M, N, K, A=None, C=None, g=None):
    g = len(M) if g is None else g
    A = A or [A16] * len(M)
    C = C or [A16] * len(M)
    return nv.group_gemm_ptrs(M, N, K, A, [A16] * len(M), [A16] * len(M), [A16] * len(M), C, 0)


def test_rejects_bad_group_count(lib):
    assert lib.nvfp4_group_gemm(0, None, None, None, None, None, None, None, None, None) == nv.INVALID_ARG
    assert "g must be" in nv.last_error()


def test_rejects_null_arrays(lib):
    one = (ctypes.c_int * 1)(16)
    assert lib.nvfp4_group_gemm(1, one, one, None, None, None, None, None, None, None) == nv.INVALID_ARG


@pytest.mark.parametrize("M,N,K", [([-1], [8], [32]), ([8], [-2], [32]), ([8], [8], [-16])])
def test_rejects_negative_sizes(lib, M, N, K):
    assert _call(M, N, K) == nv.INVALID_ARG
    assert "negative" in nv.last_error()


def test_rejects_k_not_multiple_of_16(lib):
    assert _call([8], [8], [24]) == nv.INVALID_ARG
    assert "multiple of 16" in nv.last_error()


def test_rejects_null_and_misaligned_pointers(lib):
    assert _call([8], [8], [256], A=[0]) == nv.INVALID_ARG
    assert _call([8], [8], [256], A=[MIS]) == nv.INVALID_ARG
    assert _call([8], [8], [256], C=[MIS]) == nv.INVALID_ARG
    assert "aligned" in nv.last_error()


def test_second_group_is_validated(lib):
    assert _call([8, 8], [8, 8], [256, 40]) == nv.INVALID_ARG
    assert "group 1" in nv.last_error()


def test_unsupported_k(lib):
    assert _call([8], [8], [144]) == nv.UNSUPPORTED
    assert "K % 128" in nv.last_error()


def test_unsupported_huge_operand(lib):
    assert _call([8], [1 << 20], [8192]) == nv.UNSUPPORTED


def test_empty_groups_are_ok_without_launch(lib):
    assert _call([0, 5], [7, 0], [256, 256]) == nv.OK
    assert nv.last_error() == ""


def test_dequant_validation(lib):
    assert lib.nvfp4_dequant_f16(-1, 16, A16, A16, A16, None) == nv.INVALID_ARG
    assert lib.nvfp4_dequant_f16(4, 24, A16, A16, A16, None) == nv.INVALID_ARG
    assert lib.nvfp4_dequant_f16(4, 32, MIS, A16, A16, None) == nv.INVALID_ARG
    assert lib.nvfp4_dequant_f16(0, 32, A16, A16, A16, None) == nv.OK


def test_binding_rejects_host_tensors(lib):
    import torch
    t = torch.zeros(128, dtype=torch.uint8)
    c = torch.zeros(16, dtype=torch.float16)
    with pytest.raises(ValueError):
        nv.group_gemm([t], [t], [t[:16]], [t[:16]], [c.view(4, 4)], M=[4], N=[4], K=[64])


def test_blocked_entry_validates_like_the_plain_one(lib):
    assert lib.nvfp4_group_gemm_blocked(0, None, None, None, None, None, None, None, None, None) == nv.INVALID_ARG
    rc = nv.group_gemm_ptrs([8], [8], [144], [A16], [A16], [A16], [A16], [A16], 0, blocked=True)
    assert rc == nv.UNSUPPORTED and "K % 128" in nv.last_error()
    rc = nv.group_gemm_ptrs([8], [8], [256], [MIS], [A16], [A16], [A16], [A16], 0, blocked=True)
    assert rc == nv.INVALID_ARG


def test_blocked_scale_bytes():
    assert nv.blocked_scale_bytes(1, 128) == 128 * 8
    assert nv.blocked_scale_bytes(128, 7168) == 128 * 448
    assert nv.blocked_scale_bytes(129, 256) == 256 * 16


def test_mxfp4_entry_validates(lib):
    assert lib.mxfp4_group_gemm(0, None, None, None, None, None, None, None, None, None) == nv.INVALID_ARG
    rc = nv.group_gemm_ptrs([8], [8], [144], [A16], [A16], [A16], [A16], [A16], 0, fmt="mxfp4")
    assert rc == nv.UNSUPPORTED and "K % 128" in nv.last_error()
    rc = nv.group_gemm_ptrs([8], [8], [256], [MIS], [A16], [A16], [A16], [A16], 0, fmt="mxfp4")
    assert rc == nv.INVALID_ARG


def test_wait_limit_validation(lib):
    assert lib.nvfp4_group_gemm_set_wait_limit(-1) == nv.INVALID_ARG
    assert lib.nvfp4_group_gemm_set_wait_limit(1 << 20) == nv.OK


def test_batched_entry_validates(lib):
    ip = lambda v: (ctypes.c_int * len(v))(*v)
    pp = lambda v: (ctypes.c_void_p * len(v))(*v)
    f = lib.nvfp4_group_gemm_batched
    assert f(0, None, None, None, None, None, None, None, None, None, None) == nv.INVALID_ARG
    args = lambda M, N, K, L: (1, ip([M]), ip([N]), ip([K]), ip([L]), pp([A16]), pp([A16]), pp([A16]), pp([A16]),
                               pp([A16]), None)
    assert f(*args(8, 8, 256, -1)) == nv.INVALID_ARG
    assert f(*args(3, 8, 128, 2)) == nv.UNSUPPORTED and "16 bytes" in nv.last_error()   # SFA slice of 24 bytes
    assert f(*args(8, 8, 256, 0)) == nv.OK                                                # no slices: nothing to do
