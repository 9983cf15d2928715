"""Seeded synthetic inputs (trits, fp16 group scales, activations).

A module of its own: it holds none of the ternary method's arithmetic and is
used by the oracle tests, the GPU parity tests and the benchmark alike.  The
draws are counter-based SplitMix64 (see ``synth.c``), so the same seed gives
the same tensor on any machine and any slice can be drawn on its own.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
GROUP = 128


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall",
                        "-o", _LIB, _SRC, "-lm"], check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        U64, I64, P = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        L.synth_word.argtypes = [U64, U64]
        L.synth_word.restype = U64
        L.synth_seed.argtypes = [U64, U64, U64, U64]
        L.synth_seed.restype = U64
        L.synth_f16_from_double.argtypes = [ctypes.c_double]
        L.synth_f16_from_double.restype = ctypes.c_uint16
        L.synth_trits.argtypes = [U64, U64, I64, P]
        L.synth_scales.argtypes = [U64, I64, P]
        L.synth_normal_f16.argtypes = [U64, I64, P]
        L.synth_normal_f32.argtypes = [U64, I64, P]
        L.synth_signs.argtypes = [U64, I64, P]
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def seed(*parts: int) -> int:
    p = list(parts) + [0] * (4 - len(parts))
    return int(lib().synth_seed(*[int(v) & (2**64 - 1) for v in p[:4]]))


def trits(seed_: int, N: int, K: int, start: int = 0) -> np.ndarray:
    """[N][K] int8 trits, P(0)=1/2, P(+1)=P(-1)=1/4."""
    out = np.empty((N, K), dtype=np.int8)
    lib().synth_trits(seed_, start, N * K, _p(out))
    return out


def scales(seed_: int, N: int, K: int) -> np.ndarray:
    """[N][K/128] fp16 scales (as uint16 bit patterns), uniform in [0.005, 0.05]."""
    out = np.empty((N, K // GROUP), dtype=np.uint16)
    lib().synth_scales(seed_, out.size, _p(out))
    return out


def normal_f16(seed_: int, *shape: int) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)
    lib().synth_normal_f16(seed_, out.size, _p(out))
    return out.view(np.float16)


def normal_f32(seed_: int, *shape: int) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    lib().synth_normal_f32(seed_, out.size, _p(out))
    return out


def signs(seed_: int, n: int) -> np.ndarray:
    """[n] int8 random signs, +1 or -1 with probability 1/2 each."""
    out = np.empty(n, dtype=np.int8)
    lib().synth_signs(seed_, n, _p(out))
    return out


def f16_bits(x: float) -> int:
    return int(lib().synth_f16_from_double(float(x)))
