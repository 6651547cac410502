"""Seeded synthetic inputs shared by the oracle and the GPU library.

The generator lives in ``gen.c`` (SplitMix64 + Box-Muller, stateless, so the
bytes do not depend on the thread count).  This module only compiles it, calls
it through ctypes and names the workloads.  It holds none of the decoder
block's arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .configs import CONFIGS, Config, TENSOR_IDS, tensor_id  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None


def build() -> str:
    """Compile gen.c into libsynth.so (always recompiles)."""
    tmp = _SO + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           os.path.join(_HERE, "gen.c"), "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        lib.synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_double,
                                     ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_normal.restype = None
        lib.synth_int.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_int64, ctypes.c_void_p]
        lib.synth_int.restype = None
        lib.synth_round_bf16.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_round_bf16.restype = None
        lib.synth_mix.argtypes = [ctypes.c_uint64]
        lib.synth_mix.restype = ctypes.c_uint64
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def normal(seed: int, tid: int, shape, sigma: float, bf16: bool):
    """Draw N(0, sigma) values.

    Returns ``(f32, bits)``: ``f32`` is the stored value as float32 (exactly the
    bf16 value widened when ``bf16``); ``bits`` is the uint16 bf16 array or None.
    """
    lib = _load()
    n = int(np.prod(shape)) if len(shape) else 1
    f = np.empty(shape, dtype=np.float32)
    bits = np.empty(shape, dtype=np.uint16) if bf16 else None
    lib.synth_normal(seed, tid, n, float(sigma), 1 if bf16 else 0, _ptr(f),
                     _ptr(bits) if bits is not None else None)
    return f, bits


def integers(seed: int, tid: int, shape, lo: int, hi: int) -> np.ndarray:
    """Integers uniform in [lo, hi] (inclusive)."""
    lib = _load()
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(shape, dtype=np.int32)
    lib.synth_int(seed, tid, n, int(lo), int(hi), _ptr(out))
    return out


def to_bf16(f32: np.ndarray):
    """Round float32 values to bf16 (RNE); returns (bits, widened float32)."""
    lib = _load()
    f32 = np.ascontiguousarray(f32, dtype=np.float32)
    bits = np.empty(f32.shape, dtype=np.uint16)
    wide = np.empty(f32.shape, dtype=np.float32)
    lib.synth_round_bf16(f32.size, _ptr(f32), _ptr(bits), _ptr(wide))
    return bits, wide


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def mix(z: int) -> int:
    return int(_load().synth_mix(z))
