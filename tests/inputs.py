"""Seeded inputs for tests, drawn with ``synth`` (no block arithmetic here)."""
from __future__ import annotations

import numpy as np

import synth
from synth.configs import Config, tensor_id
from oracle.formulas import block_weight_shapes


def block_weights(cfg: Config, layer: int | None = None, gains: str = "ones"):
    """Returns (f32 dict, bits dict or None).  Gains are 1 unless gains='random'
    (1 + N(0, 0.1)), used by one extra parity case."""
    bf = cfg.dtype == "bf16"
    shapes = block_weight_shapes(cfg.d, cfg.n_heads, cfg.n_kv_heads, cfg.d_ff)
    f32, bits = {}, {}
    for name, shp in shapes.items():
        if name.startswith("g_"):
            if gains == "random":
                n, _ = synth.normal(cfg.seed, tensor_id(name, layer), shp, 0.1, False)
                v = 1.0 + n
            else:
                v = np.ones(shp, np.float32)
            if bf:
                b, v = synth.to_bf16(v)
                bits[name] = b
            f32[name] = v.astype(np.float32)
        else:
            v, b = synth.normal(cfg.seed, tensor_id(name, layer), shp, cfg.w_sigma, bf)
            f32[name] = v
            if bf:
                bits[name] = b
    return f32, (bits if bf else None)


def activations(cfg: Config, B: int, T: int, name: str = "x", sigma: float | None = None):
    shp = (B, T, cfg.d)
    return synth.normal(cfg.seed, tensor_id(name), shp, cfg.x_sigma if sigma is None else sigma,
                        cfg.dtype == "bf16")


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
