"""Seeded block inputs: weights, gains and activations of the workloads, drawn
with the generator in this package.  Shapes only, no block arithmetic.

Weights are stored [in, out] (tirogla "Transformer block", Code: y = x W):
Wq [d, H dh], Wk and Wv [d, Hkv dh], Wo [H dh, d], W1 and W3 [d, f],
W2 [f, d]; the RMSNorm gains are [d].
"""
from __future__ import annotations

import numpy as np

from . import normal, to_bf16
from .configs import Config, tensor_id


def weight_shapes(d: int, H: int, Hkv: int, f: int) -> dict:
    dh = d // H
    return {"g_attn": (d,), "g_mlp": (d,), "wq": (d, H * dh), "wk": (d, Hkv * dh), "wv": (d, Hkv * dh),
            "wo": (H * dh, d), "w1": (d, f), "w3": (d, f), "w2": (f, d)}


def block_weights(cfg: Config, layer: int | None = None, gains: str = "ones"):
    """Returns (f32 dict, bits dict or None).  Gains are 1 unless gains='random'
    (1 + N(0, 0.1)), used by one extra parity case."""
    bf = cfg.dtype == "bf16"
    shapes = weight_shapes(cfg.d, cfg.n_heads, cfg.n_kv_heads, cfg.d_ff)
    f32, bits = {}, {}
    for name, shp in shapes.items():
        if name.startswith("g_"):
            if gains == "random":
                n, _ = normal(cfg.seed, tensor_id(name, layer), shp, 0.1, False)
                v = 1.0 + n
            else:
                v = np.ones(shp, np.float32)
            if bf:
                b, v = to_bf16(v)
                bits[name] = b
            f32[name] = v.astype(np.float32)
        else:
            v, b = normal(cfg.seed, tensor_id(name, layer), shp, cfg.w_sigma, bf)
            f32[name] = v
            if bf:
                bits[name] = b
    return f32, (bits if bf else None)


def activations(cfg: Config, B: int, T: int, name: str = "x", sigma: float | None = None):
    shp = (B, T, cfg.d)
    return normal(cfg.seed, tensor_id(name), shp, cfg.x_sigma if sigma is None else sigma, cfg.dtype == "bf16")
