"""ctypes binding of libnvfp4gg.so (argument marshalling only).

Every step of the computation runs in the HIP kernels of csrc/nvfp4gg.hip; this
module only turns torch tensors into device pointers and a HIP stream.  It
fails loudly when the library has not been built: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libnvfp4gg.so")

OK, INVALID_ARG, UNSUPPORTED, HIP_ERROR = 0, -1, -2, -3
_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("nvfp4gg error %d: %s" % (code, msg))
        self.code = code


def load():
    """Load the built library (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libnvfp4gg.so is not built; run __graft_entry__.build() "
                           "or python nvfp4_block_scaled_grouped_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    ip = ctypes.POINTER(ctypes.c_int)
    pp = ctypes.POINTER(ctypes.c_void_p)
    for fn in (lib.nvfp4_group_gemm, lib.nvfp4_group_gemm_blocked, lib.mxfp4_group_gemm,
               lib.nvfp4_group_gemm_noalloc):
        fn.argtypes = [ctypes.c_int, ip, ip, ip, pp, pp, pp, pp, pp, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    lib.nvfp4_dequant_f16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p]
    lib.nvfp4_dequant_f16.restype = ctypes.c_int
    lib.nvfp4_group_gemm_batched.argtypes = [ctypes.c_int, ip, ip, ip, ip, pp, pp, pp, pp, pp, ctypes.c_void_p]
    lib.nvfp4_group_gemm_batched.restype = ctypes.c_int
    lib.nvfp4_group_gemm_set_wait_limit.argtypes = [ctypes.c_int]
    lib.nvfp4_group_gemm_set_wait_limit.restype = ctypes.c_int
    lib.nvfp4_group_gemm_set_max_frags.argtypes = [ctypes.c_int]
    lib.nvfp4_group_gemm_set_max_frags.restype = ctypes.c_int
    lib.nvfp4_group_gemm_last_error.argtypes = []
    lib.nvfp4_group_gemm_last_error.restype = ctypes.c_char_p
    lib.nvfp4_group_gemm_version.argtypes = []
    lib.nvfp4_group_gemm_version.restype = ctypes.c_int
    _lib = lib
    return lib


def last_error() -> str:
    return load().nvfp4_group_gemm_last_error().decode()


def _check(rc: int):
    if rc != OK:
        raise Nvfp4Error(rc, last_error())


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t, name, dtype_names):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if str(t.dtype).replace("torch.", "") not in dtype_names:
        raise ValueError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtype_names))
    return t.data_ptr()


_BYTES = ("uint8", "int8", "float4_e2m1fn_x2", "float8_e4m3fn")


def _entry(lib, blocked, fmt, noalloc=False):
    if noalloc:
        if blocked or fmt != "nvfp4":
            raise ValueError("the no-allocation entry point takes NVFP4 row-major scales only")
        return lib.nvfp4_group_gemm_noalloc
    if fmt == "mxfp4":
        if blocked:
            raise ValueError("the MXFP4 entry point takes row-major scales only")
        return lib.mxfp4_group_gemm
    if fmt != "nvfp4":
        raise ValueError("fmt must be 'nvfp4' or 'mxfp4'")
    return lib.nvfp4_group_gemm_blocked if blocked else lib.nvfp4_group_gemm


def group_gemm_ptrs(M, N, K, A, B, SFA, SFB, C, stream=0, blocked=False, fmt="nvfp4", noalloc=False) -> int:
    """Raw call: sizes are Python ints, operands are integer device addresses.
    blocked selects nvfp4_group_gemm_blocked (scales in the blocked layout),
    fmt="mxfp4" mxfp4_group_gemm, noalloc nvfp4_group_gemm_noalloc.  Returns
    the library's status code without raising."""
    g = len(M)
    lib = load()
    arr = lambda vals, ct: (ct * g)(*vals)
    fn = _entry(lib, blocked, fmt, noalloc)
    return fn(
        g, arr([int(v) for v in M], ctypes.c_int), arr([int(v) for v in N], ctypes.c_int),
        arr([int(v) for v in K], ctypes.c_int),
        arr(A, ctypes.c_void_p), arr(B, ctypes.c_void_p), arr(SFA, ctypes.c_void_p),
        arr(SFB, ctypes.c_void_p), arr(C, ctypes.c_void_p), ctypes.c_void_p(stream))


def group_gemm_batched_ptrs(M, N, K, L, A, B, SFA, SFB, C, stream=0) -> int:
    """Raw nvfp4_group_gemm_batched call (L_i slices per group, each operand
    holding its slices consecutively).  Returns the status code."""
    g = len(M)
    lib = load()
    arr = lambda vals, ct: (ct * g)(*vals)
    return lib.nvfp4_group_gemm_batched(
        g, arr([int(v) for v in M], ctypes.c_int), arr([int(v) for v in N], ctypes.c_int),
        arr([int(v) for v in K], ctypes.c_int), arr([int(v) for v in L], ctypes.c_int),
        arr(A, ctypes.c_void_p), arr(B, ctypes.c_void_p), arr(SFA, ctypes.c_void_p),
        arr(SFB, ctypes.c_void_p), arr(C, ctypes.c_void_p), ctypes.c_void_p(stream))


class GroupGemmCall:
    """A grouped GEMM call whose argument arrays are marshalled once.

    Holds the ctypes copies of the sizes, the device addresses and the stream
    handle, so that calling it repeats the same nvfp4_group_gemm call with no
    per-call Python list work.  The addresses must stay valid while it is used.
    """

    def __init__(self, M, N, K, A, B, SFA, SFB, C, stream=0, blocked=False, fmt="nvfp4"):
        g = len(M)
        lib = load()
        arr = lambda vals, ct: (ct * g)(*vals)
        self._fn = _entry(lib, blocked, fmt)
        self._args = (g, arr([int(v) for v in M], ctypes.c_int), arr([int(v) for v in N], ctypes.c_int),
                      arr([int(v) for v in K], ctypes.c_int), arr(A, ctypes.c_void_p),
                      arr(B, ctypes.c_void_p), arr(SFA, ctypes.c_void_p), arr(SFB, ctypes.c_void_p),
                      arr(C, ctypes.c_void_p), ctypes.c_void_p(stream))

    def __call__(self) -> int:
        return self._fn(*self._args)


def blocked_scale_bytes(rows: int, K: int) -> int:
    """Bytes of a blocked-layout scale array of `rows` rows and K/16 scale
    columns: rows padded to a multiple of 128, columns to a multiple of 4."""
    return -(-rows // 128) * 128 * (-(-(K // 16) // 4) * 4)


def group_gemm_batched(A, B, SFA, SFB, C, M, N, K, L, stream=None):
    """C_i[l] = A_i[l] . B_i[l]^T for l < L_i (nvfp4_group_gemm_batched): each
    operand a contiguous device tensor of L_i slices (A_i: L_i*M_i*K_i/2 bytes,
    SFA_i: L_i*M_i*K_i/16, ..., C_i: L_i*M_i*N_i fp16)."""
    g = len(A)
    if not (len(B) == len(SFA) == len(SFB) == len(C) == len(M) == len(N) == len(K) == len(L) == g):
        raise ValueError("operand and size lists differ in length")
    for i in range(g):
        need = {"A": (A[i], L[i] * M[i] * K[i] // 2), "B": (B[i], L[i] * N[i] * K[i] // 2),
                "SFA": (SFA[i], L[i] * M[i] * K[i] // 16), "SFB": (SFB[i], L[i] * N[i] * K[i] // 16),
                "C": (C[i], L[i] * M[i] * N[i])}
        for name, (t, n) in need.items():
            if t.numel() != n:
                raise ValueError("group %d: %s has %d elements, expected %d" % (i, name, t.numel(), n))
    _check(group_gemm_batched_ptrs(M, N, K, L, [_ptr(t, "A", _BYTES) for t in A], [_ptr(t, "B", _BYTES) for t in B],
                                   [_ptr(t, "SFA", _BYTES) for t in SFA], [_ptr(t, "SFB", _BYTES) for t in SFB],
                                   [_ptr(t, "C", ("float16",)) for t in C], _stream_handle(stream)))
    return C


def group_gemm(A, B, SFA, SFB, C, M=None, N=None, K=None, stream=None, blocked=False, fmt="nvfp4",
               noalloc=False):
    """C_i = A_i . B_i^T for every group (see include/nvfp4gg.h).

    A, B, SFA, SFB: lists of contiguous uint8 device tensors holding the packed
    codes (A_i: M_i*K_i/2 bytes, SFA_i: M_i*K_i/16 bytes, ...; with
    blocked=True the scales are in the blocked layout, blocked_scale_bytes
    each; with fmt="mxfp4" they are E8M0, M_i*K_i/32 and N_i*K_i/32 bytes).
    C: list of contiguous float16 device tensors (M_i*N_i elements), written.
    M, N, K: sizes; taken from C's and A's shapes when omitted
    (C_i as (M_i, N_i), A_i as (M_i, K_i/2)).
    noalloc: call nvfp4_group_gemm_noalloc (static workspace, NVFP4 only).
    """
    g = len(A)
    if not (len(B) == len(SFA) == len(SFB) == len(C) == g):
        raise ValueError("operand lists differ in length")
    if M is None:
        M = [int(c.shape[0]) for c in C]
    if N is None:
        N = [int(c.shape[1]) for c in C]
    if K is None:
        K = [int(a.shape[-1]) * 2 for a in A]
    for i in range(g):
        per = 32 if fmt == "mxfp4" else 16
        sfa_n = blocked_scale_bytes(M[i], K[i]) if blocked else M[i] * K[i] // per
        sfb_n = blocked_scale_bytes(N[i], K[i]) if blocked else N[i] * K[i] // per
        need = {"A": (A[i], M[i] * K[i] // 2), "B": (B[i], N[i] * K[i] // 2),
                "SFA": (SFA[i], sfa_n), "SFB": (SFB[i], sfb_n), "C": (C[i], M[i] * N[i])}
        for name, (t, n) in need.items():
            if t.numel() != n:
                raise ValueError("group %d: %s has %d elements, expected %d" % (i, name, t.numel(), n))
    pa = [_ptr(t, "A", _BYTES) for t in A]
    pb = [_ptr(t, "B", _BYTES) for t in B]
    psa = [_ptr(t, "SFA", _BYTES) for t in SFA]
    psb = [_ptr(t, "SFB", _BYTES) for t in SFB]
    pc = [_ptr(t, "C", ("float16",)) for t in C]
    _check(group_gemm_ptrs(M, N, K, pa, pb, psa, psb, pc, _stream_handle(stream), blocked=blocked, fmt=fmt,
                           noalloc=noalloc))
    return C


def dequant_f16(X, SFX, out, rows: int, K: int, stream=None):
    """out = fp16 dequantisation of packed FP4 X (rows x K) with scales SFX."""
    if X.numel() != rows * K // 2 or SFX.numel() != rows * K // 16 or out.numel() != rows * K:
        raise ValueError("dequant_f16: wrong tensor sizes")
    lib = load()
    _check(lib.nvfp4_dequant_f16(int(rows), int(K), _ptr(X, "X", _BYTES), _ptr(SFX, "SFX", _BYTES),
                                 _ptr(out, "out", ("float16",)), ctypes.c_void_p(_stream_handle(stream))))
    return out


def set_wait_limit(polls: int):
    """Bound on a split tile's finisher waiting for the other contributors
    (see include/nvfp4gg.h); 0 hands every fix-up to the last arriver."""
    _check(load().nvfp4_group_gemm_set_wait_limit(int(polls)))


def set_max_frags(frags: int):
    """m-block size (fragments of 16 rows, 1..12) forced for every launch;
    0 chooses it per launch (see include/nvfp4gg.h)."""
    _check(load().nvfp4_group_gemm_set_max_frags(int(frags)))


def version() -> int:
    return int(load().nvfp4_group_gemm_version())
