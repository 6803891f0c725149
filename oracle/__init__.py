"""CPU oracle for the NVFP4 block-scaled grouped GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports it and shares no code with it.

The arithmetic lives in ``nvfp4_oracle.c`` (plain C, exact int64 accumulation,
one round-to-nearest-even to fp16); this module only builds that file with gcc
and marshals numpy arrays into it.  See the C file's header for the definition
and the passages of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O3, OpenMP).  Returns the library path."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    lib.oracle_e2m1_x2.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1_x2.restype = ctypes.c_int
    lib.oracle_e2m1.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1.restype = ctypes.c_double
    lib.oracle_e4m3.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3.restype = ctypes.c_double
    lib.oracle_round_f16_fixed20.argtypes = [ctypes.c_int64]
    lib.oracle_round_f16_fixed20.restype = ctypes.c_uint16
    lib.oracle_round_f16_double.argtypes = [ctypes.c_double]
    lib.oracle_round_f16_double.restype = ctypes.c_uint16
    lib.oracle_gemm_element.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, u8p, u8p, u8p, u8p,
        ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_uint16),
        ctypes.POINTER(ctypes.c_double)]
    lib.oracle_gemm_element.restype = ctypes.c_int
    pp = ctypes.POINTER(ctypes.c_void_p)
    ip = ctypes.POINTER(ctypes.c_int)
    lib.oracle_group_gemm.argtypes = [ctypes.c_int, ip, ip, ip, pp, pp, pp, pp,
                                      pp, pp, ctypes.c_int, ctypes.c_int]
    lib.oracle_group_gemm.restype = ctypes.c_int
    lib.oracle_dequant.argtypes = [ctypes.c_int, ctypes.c_int, u8p, u8p,
                                   ctypes.POINTER(ctypes.c_double)]
    lib.oracle_dequant.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _u8ptr(a: np.ndarray):
    assert a.dtype == np.uint8 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def e2m1(code: int) -> float:
    return _load().oracle_e2m1(code)


def e4m3(code: int) -> float:
    return _load().oracle_e4m3(code)


def round_f16_fixed20(x: int) -> int:
    """fp16 bits of the exact value x * 2**-20 (RNE, overflow to inf)."""
    return int(_load().oracle_round_f16_fixed20(int(x)))


def round_f16_double(x: float) -> int:
    return int(_load().oracle_round_f16_double(float(x)))


def e8m0(code: int) -> float:
    lib = _load()
    lib.oracle_e8m0.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0.restype = ctypes.c_double
    return float(lib.oracle_e8m0(int(code)))


def mx_group_gemm(M, N, K, A, B, SFA, SFB, *, exact: bool = False, nthreads: int = 0):
    """The MXFP4 oracle (E8M0 scales, M_i x K_i/32 and N_i x K_i/32 bytes).
    Returns the fp16 outputs, plus the exact sums when ``exact`` is set."""
    g = len(M)
    lib = _load()
    pp = ctypes.POINTER(ctypes.c_void_p)
    ip = ctypes.POINTER(ctypes.c_int)
    lib.oracle_mx_group_gemm.argtypes = [ctypes.c_int, ip, ip, ip, pp, pp, pp, pp, pp, pp, ctypes.c_int]
    lib.oracle_mx_group_gemm.restype = ctypes.c_int
    keep = []

    def ptrs(arrs):
        out = (ctypes.c_void_p * g)()
        for i, a in enumerate(arrs):
            keep.append(a)
            out[i] = a.ctypes.data
        return out

    A = [np.ascontiguousarray(a, dtype=np.uint8) for a in A]
    B = [np.ascontiguousarray(a, dtype=np.uint8) for a in B]
    SFA = [np.ascontiguousarray(a, dtype=np.uint8) for a in SFA]
    SFB = [np.ascontiguousarray(a, dtype=np.uint8) for a in SFB]
    for i in range(g):
        if (A[i].size != M[i] * K[i] // 2 or B[i].size != N[i] * K[i] // 2
                or SFA[i].size != M[i] * K[i] // 32 or SFB[i].size != N[i] * K[i] // 32):
            raise ValueError("oracle.mx_group_gemm: group %d has wrong byte counts" % i)
    C = [np.empty((M[i], N[i]), dtype=np.uint16) for i in range(g)]
    X = [np.empty((M[i], N[i]), dtype=np.float64) for i in range(g)] if exact else None
    rc = lib.oracle_mx_group_gemm(g, (ctypes.c_int * g)(*M), (ctypes.c_int * g)(*N), (ctypes.c_int * g)(*K),
                                  ptrs(A), ptrs(B), ptrs(SFA), ptrs(SFB), ptrs(C),
                                  ptrs(X) if exact else None, int(nthreads))
    if rc == -2:
        raise ValueError("oracle_mx_group_gemm: scale exponents spread too wide for the exact sum")
    if rc != 0:
        raise ValueError("oracle_mx_group_gemm: bad sizes")
    C = [c.view(np.float16) for c in C]
    return (C, X) if exact else C


def mx_gemm_element(M, N, K, A, B, SFA, SFB, m, n):
    """One MXFP4 output element of a single group: (fp16 bits, exact value)."""
    lib = _load()
    u8p = ctypes.POINTER(ctypes.c_uint8)
    lib.oracle_mx_gemm_element.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, u8p, u8p, u8p, u8p,
                                           ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_uint16),
                                           ctypes.POINTER(ctypes.c_double)]
    lib.oracle_mx_gemm_element.restype = ctypes.c_int
    c16 = ctypes.c_uint16()
    ex = ctypes.c_double()
    rc = lib.oracle_mx_gemm_element(int(M), int(N), int(K), _u8ptr(A), _u8ptr(B), _u8ptr(SFA), _u8ptr(SFB),
                                    int(m), int(n), ctypes.byref(c16), ctypes.byref(ex))
    if rc != 0:
        raise ValueError("oracle_mx_gemm_element: bad index or exponent spread")
    return int(c16.value), float(ex.value)


def blocked_scale_bytes(rows: int, cols: int) -> int:
    """Size of the blocked layout of a rows x cols scale matrix."""
    lib = _load()
    lib.oracle_blocked_scale_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.oracle_blocked_scale_bytes.restype = ctypes.c_int64
    return int(lib.oracle_blocked_scale_bytes(int(rows), int(cols)))


def block_scales(plain: np.ndarray, rows: int, cols: int, pad_value: int = 0) -> np.ndarray:
    """The blocked layout (flat uint8) of a row-major rows x cols scale matrix;
    pad bytes are pad_value."""
    plain = np.ascontiguousarray(plain, dtype=np.uint8)
    assert plain.size == rows * cols
    out = np.empty(blocked_scale_bytes(rows, cols), dtype=np.uint8)
    lib = _load()
    lib.oracle_block_scales.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_uint8),
                                        ctypes.POINTER(ctypes.c_uint8), ctypes.c_uint8]
    if lib.oracle_block_scales(int(rows), int(cols), _u8ptr(plain), _u8ptr(out), int(pad_value)) != 0:
        raise ValueError("oracle_block_scales: bad sizes")
    return out


def unblock_scales(blocked: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """The row-major rows x cols scale matrix held in a blocked array."""
    blocked = np.ascontiguousarray(blocked, dtype=np.uint8)
    assert blocked.size >= blocked_scale_bytes(rows, cols)
    out = np.empty((rows, cols), dtype=np.uint8)
    lib = _load()
    lib.oracle_unblock_scales.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_uint8),
                                          ctypes.POINTER(ctypes.c_uint8)]
    if lib.oracle_unblock_scales(int(rows), int(cols), _u8ptr(blocked), _u8ptr(out)) != 0:
        raise ValueError("oracle_unblock_scales: bad sizes")
    return out


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def dequant(x: np.ndarray, sfx: np.ndarray, rows: int, K: int) -> np.ndarray:
    """Decoded values (float64, rows x K) of a packed FP4 matrix and its scales."""
    x = np.ascontiguousarray(x, dtype=np.uint8)
    sfx = np.ascontiguousarray(sfx, dtype=np.uint8)
    assert x.size == rows * K // 2 and sfx.size == rows * K // 16
    out = np.empty((rows, K), dtype=np.float64)
    rc = _load().oracle_dequant(rows, K, _u8ptr(x), _u8ptr(sfx),
                                out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc != 0:
        raise ValueError("oracle_dequant: bad sizes")
    return out


def group_gemm(M, N, K, A, B, SFA, SFB, *, exact: bool = False,
               use_f64: bool = False, nthreads: int = 0):
    """Run the oracle.  A/B/SFA/SFB are lists of uint8 numpy arrays holding the
    packed codes (row-major, any shape with the right byte count).  Returns the
    list of fp16 outputs (np.float16, M_i x N_i), plus the list of exact sums
    (float64) when ``exact`` is set."""
    g = len(M)
    lib = _load()
    Ms = (ctypes.c_int * g)(*[int(v) for v in M])
    Ns = (ctypes.c_int * g)(*[int(v) for v in N])
    Ks = (ctypes.c_int * g)(*[int(v) for v in K])
    keep = []

    def ptrs(arrs):
        out = (ctypes.c_void_p * g)()
        for i, a in enumerate(arrs):
            keep.append(a)
            out[i] = a.ctypes.data
        return out

    A = [np.ascontiguousarray(a, dtype=np.uint8) for a in A]
    B = [np.ascontiguousarray(a, dtype=np.uint8) for a in B]
    SFA = [np.ascontiguousarray(a, dtype=np.uint8) for a in SFA]
    SFB = [np.ascontiguousarray(a, dtype=np.uint8) for a in SFB]
    for i in range(g):
        if (A[i].size != M[i] * K[i] // 2 or B[i].size != N[i] * K[i] // 2
                or SFA[i].size != M[i] * K[i] // 16 or SFB[i].size != N[i] * K[i] // 16):
            raise ValueError("oracle.group_gemm: group %d has wrong byte counts" % i)
    C = [np.empty((M[i], N[i]), dtype=np.uint16) for i in range(g)]
    X = [np.empty((M[i], N[i]), dtype=np.float64) for i in range(g)] if exact else None
    rc = lib.oracle_group_gemm(g, Ms, Ns, Ks, ptrs(A), ptrs(B), ptrs(SFA), ptrs(SFB),
                               ptrs(C), ptrs(X) if exact else None,
                               1 if use_f64 else 0, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_group_gemm: bad sizes")
    C = [c.view(np.float16) for c in C]
    return (C, X) if exact else C


def group_gemm_batched(M, N, K, L, A, B, SFA, SFB, *, exact: bool = False, nthreads: int = 0):
    """The batched form, (M, N, K, L) per group (page 505431,
    custom_kernel_fallback: C[m,n,l] = sum_k A[m,k,l] B[n,k,l]; page 482006:
    the batch stride is a whole slice): slice l of every operand is the l-th
    consecutive block of its array, and each slice is the ordinary product.
    Returns per group the list of L_i fp16 outputs (and exact sums)."""
    C, X = [], []
    for i in range(len(M)):
        m, n, k, l_count = M[i], N[i], K[i], L[i]
        a = np.ascontiguousarray(A[i], dtype=np.uint8).reshape(-1)
        b = np.ascontiguousarray(B[i], dtype=np.uint8).reshape(-1)
        sa = np.ascontiguousarray(SFA[i], dtype=np.uint8).reshape(-1)
        sb = np.ascontiguousarray(SFB[i], dtype=np.uint8).reshape(-1)
        sl = lambda arr, size, j: arr[j * size:(j + 1) * size]
        Ms, Ns, Ks = [m] * l_count, [n] * l_count, [k] * l_count
        out = group_gemm(Ms, Ns, Ks, [sl(a, m * k // 2, j) for j in range(l_count)],
                         [sl(b, n * k // 2, j) for j in range(l_count)],
                         [sl(sa, m * k // 16, j) for j in range(l_count)],
                         [sl(sb, n * k // 16, j) for j in range(l_count)], exact=True, nthreads=nthreads) \
            if l_count else ([], [])
        C.append(out[0])
        X.append(out[1])
    return (C, X) if exact else C


def gemm_element(M, N, K, A, B, SFA, SFB, m, n):
    """One output element of a single group: (fp16 bits, exact value)."""
    c16 = ctypes.c_uint16()
    ex = ctypes.c_double()
    rc = _load().oracle_gemm_element(int(M), int(N), int(K), _u8ptr(A), _u8ptr(B),
                                     _u8ptr(SFA), _u8ptr(SFB), int(m), int(n),
                                     ctypes.byref(c16), ctypes.byref(ex))
    if rc != 0:
        raise ValueError("oracle_gemm_element: bad index")
    return int(c16.value), float(ex.value)
