"""Plain CPU oracle for ternary-weight GEMV/GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does; the
two share no code.  The arithmetic lives in ``tq_oracle.c`` (plain C, fp64
accumulation); this module only compiles it and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GROUP = 128
FMT_B3 = 0
FMT_2B = 1
FMT_BP = 2


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: no FMA contraction, OpenMP row loops."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", _LIB, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        # A mutated copy of the oracle may be substituted by the pin-sensitivity
        # test (tests/test_oracle_mutations.py); nothing else sets this.
        path = os.environ.get("TQ_ORACLE_LIB_OVERRIDE") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.orc_half_to_float.argtypes = [ctypes.c_uint16]
        L.orc_half_to_float.restype = ctypes.c_float
        for name in ("orc_b3_bytes", "orc_2b_bytes"):
            getattr(L, name).argtypes = [I64, I64]
            getattr(L, name).restype = ctypes.c_size_t
        for name in ("orc_pack_b3", "orc_unpack_b3", "orc_pack_2b", "orc_unpack_2b", "orc_pack_bp",
                     "orc_unpack_bp"):
            getattr(L, name).argtypes = [I64, I64, P, P, P]
            getattr(L, name).restype = ctypes.c_int
        for name in ("orc_quant_f16", "orc_quant_f32"):
            getattr(L, name).argtypes = [I64, I64, P, P, P]
            getattr(L, name).restype = ctypes.c_int
        L.orc_group_sums.argtypes = [I64, I64, I64, P, P, P]
        L.orc_group_sums.restype = ctypes.c_int
        L.orc_gemv.argtypes = [I64, I64, I64, P, P, P, P, P]
        L.orc_gemv.restype = ctypes.c_int
        L.orc_gemv_rows.argtypes = [I64, I64, I64, P, P, P, P, I64, P, P]
        L.orc_gemv_rows.restype = ctypes.c_int
        L.orc_swiglu.argtypes = [I64, P, P, P]
        L.orc_swiglu.restype = ctypes.c_int
        L.orc_project_packed.argtypes = [ctypes.c_int, I64, I64, I64, P, P, P, P]
        L.orc_project_packed.restype = ctypes.c_int
        L.orc_ternarize.argtypes = [I64, I64, P, P, P]
        L.orc_ternarize.restype = ctypes.c_int
        L.orc_hadamard_f32.argtypes = [I64, I64, P, P, P]
        L.orc_hadamard_f32.restype = ctypes.c_int
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_get_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what} failed with status {rc}")


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def half_to_float(h: int) -> float:
    return float(lib().orc_half_to_float(int(h)))


def packed_bytes(fmt: int, N: int, K: int) -> int:
    return int((lib().orc_b3_bytes if fmt == FMT_B3 else lib().orc_2b_bytes)(N, K))  # BP: as 2B


def pack(fmt: int, trits: np.ndarray, scales: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(trits, dtype=np.int8)
    s = np.ascontiguousarray(scales, dtype=np.uint16)
    N, K = t.shape
    nbytes = packed_bytes(fmt, N, K)
    if nbytes == 0:
        raise OracleError("bad shape")
    out = np.empty(nbytes, dtype=np.uint8)
    fn = {FMT_B3: lib().orc_pack_b3, FMT_2B: lib().orc_pack_2b, FMT_BP: lib().orc_pack_bp}[fmt]
    _check(fn(N, K, _p(t), _p(s), _p(out)), "pack")
    return out


def unpack(fmt: int, blob: np.ndarray, N: int, K: int):
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    t = np.empty((N, K), dtype=np.int8)
    s = np.empty((N, K // GROUP), dtype=np.uint16)
    fn = {FMT_B3: lib().orc_unpack_b3, FMT_2B: lib().orc_unpack_2b, FMT_BP: lib().orc_unpack_bp}[fmt]
    rc = fn(N, K, _p(b), _p(t), _p(s))
    return rc, t, s


def quant(x: np.ndarray):
    """x: [M][K] float16 or float32 -> (q int8 [M][K], scale fp32 [M])."""
    x = np.ascontiguousarray(x)
    if x.ndim == 1:
        x = x[None, :]
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int8)
    sc = np.empty(M, dtype=np.float32)
    if x.dtype == np.float16:
        rc = lib().orc_quant_f16(M, K, _p(x.view(np.uint16)), _p(q), _p(sc))
    elif x.dtype == np.float32:
        rc = lib().orc_quant_f32(M, K, _p(x), _p(q), _p(sc))
    else:
        raise TypeError(x.dtype)
    _check(rc, "quant")
    return q, sc


def group_sums(trits: np.ndarray, q: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(trits, dtype=np.int8)
    q = np.ascontiguousarray(q, dtype=np.int8)
    if q.ndim == 1:
        q = q[None, :]
    N, K = t.shape
    M = q.shape[0]
    S = np.empty((M, N, K // GROUP), dtype=np.int32)
    _check(lib().orc_group_sums(M, N, K, _p(t), _p(q), _p(S)), "group_sums")
    return S


def gemv(trits, scales, q, a) -> np.ndarray:
    t = np.ascontiguousarray(trits, dtype=np.int8)
    s = np.ascontiguousarray(scales, dtype=np.uint16)
    q = np.ascontiguousarray(q, dtype=np.int8)
    if q.ndim == 1:
        q = q[None, :]
    a = np.ascontiguousarray(np.atleast_1d(a), dtype=np.float32)
    N, K = t.shape
    M = q.shape[0]
    y = np.empty((M, N), dtype=np.float32)
    _check(lib().orc_gemv(M, N, K, _p(t), _p(s), _p(q), _p(a), _p(y)), "gemv")
    return y


def gemv_rows(trits, scales, q, a, rows) -> np.ndarray:
    t = np.ascontiguousarray(trits, dtype=np.int8)
    s = np.ascontiguousarray(scales, dtype=np.uint16)
    q = np.ascontiguousarray(q, dtype=np.int8)
    if q.ndim == 1:
        q = q[None, :]
    a = np.ascontiguousarray(np.atleast_1d(a), dtype=np.float32)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    N, K = t.shape
    M = q.shape[0]
    y = np.empty((M, r.size), dtype=np.float32)
    _check(lib().orc_gemv_rows(M, N, K, _p(t), _p(s), _p(q), _p(a), r.size, _p(r), _p(y)),
           "gemv_rows")
    return y


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    h = np.empty_like(g)
    _check(lib().orc_swiglu(g.size, _p(g), _p(u), _p(h)), "swiglu")
    return h


def project_packed(fmt: int, blob: np.ndarray, N: int, K: int, q, a) -> np.ndarray:
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.int8)
    if q.ndim == 1:
        q = q[None, :]
    a = np.ascontiguousarray(np.atleast_1d(a), dtype=np.float32)
    M = q.shape[0]
    y = np.empty((M, N), dtype=np.float32)
    _check(lib().orc_project_packed(fmt, M, N, K, _p(b), _p(q), _p(a), _p(y)), "project")
    return y


HBLOCK = 64


def hadamard(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Rotate each row of x ([M][K] or [K], fp16 widened exactly, or fp32) by
    the block Hadamard transform and the sign vector signs [K] (+-1)."""
    x = np.ascontiguousarray(x)
    squeeze = x.ndim == 1
    if squeeze:
        x = x[None, :]
    x = np.ascontiguousarray(x.astype(np.float32))
    s = np.ascontiguousarray(signs, dtype=np.int8)
    M, K = x.shape
    y = np.empty((M, K), dtype=np.float32)
    _check(lib().orc_hadamard_f32(M, K, _p(x), _p(s), _p(y)), "hadamard")
    return y[0] if squeeze else y


def ternarize(w: np.ndarray):
    """fp32 weights [N][K] -> (trits int8 [N][K], fp16 scales as uint16 [N][K/128])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    t = np.empty((N, K), dtype=np.int8)
    s = np.empty((N, K // GROUP), dtype=np.uint16)
    _check(lib().orc_ternarize(N, K, _p(w), _p(t), _p(s)), "ternarize")
    return t, s
