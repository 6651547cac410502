"""Seeded inputs for tests, drawn with ``synth`` (no block arithmetic here)."""
from __future__ import annotations

import numpy as np

from synth.configs import Config
from synth.inputs import activations, block_weights  # noqa: F401  (seeded inputs live with the generator)


def small_cfg(d=64, H=4, Hkv=2, f=192, dtype="f32", base=10000.0, number=1, eps=1e-6, window=0):
    return Config("test", number, d=d, n_heads=H, n_kv_heads=Hkv, d_ff=f, rope_base=base, dtype=dtype,
                  B=1, T=16, rms_eps=eps, window=window)


def rms(a) -> float:
    a = np.asarray(a, np.float64)
    return float(np.sqrt(np.mean(a * a)))


def rel_err(got, ref) -> float:
    """max |got - ref| / rms(ref)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    r = rms(ref)
    return float(np.max(np.abs(got - ref)) / (r if r > 0 else 1.0))
