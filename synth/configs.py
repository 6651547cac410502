"""The five workloads of the decoder-block path and how their inputs are drawn.

Shapes follow the pages' notation (tirogla "Transformer block", How it works):
B batch, T sequence, d width, H query heads, Hkv KV heads, dh = d/H, f MLP
width, L layers, V vocabulary.  Every tensor is drawn by ``synth.normal`` or
``synth.integers`` with seed ``1000 + config number`` and the tensor ids below
(per layer l the id is offset by ``100 * (l + 1)``).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

TENSOR_IDS = {
    "x": 1, "g_attn": 2, "g_mlp": 3, "wq": 4, "wk": 5, "wv": 6, "wo": 7, "w1": 8, "w3": 9, "w2": 10,
    "kc": 11, "vc": 12, "lens": 13, "ids": 14, "embed": 15, "g_final": 16, "w_unembed": 17,
}


def tensor_id(name: str, layer: int | None = None) -> int:
    base = TENSOR_IDS[name]
    return base if layer is None else base + 100 * (layer + 1)


@dataclass(frozen=True)
class Config:
    name: str
    number: int
    d: int
    n_heads: int
    n_kv_heads: int
    d_ff: int
    rope_base: float
    dtype: str            # "f32" or "bf16" (storage; accumulation is fp32)
    B: int
    T: int                # prefill length (decode: 1 new token per sequence)
    rms_eps: float = 1e-6
    n_layers: int = 1
    vocab: int = 0
    mode: str = "prefill"  # "prefill", "decode" or "model"
    t_max: int = 0         # KV cache rows per sequence
    lens_lo: int = 0       # decode: cache length range (inclusive)
    lens_hi: int = 0
    decode_steps: int = 0
    w_sigma: float = 0.02
    x_sigma: float = 1.0
    window: int = 0        # sliding-window attention: keys per query (0 = full causal)
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def head_dim(self) -> int:
        return self.d // self.n_heads

    @property
    def seed(self) -> int:
        return 1000 + self.number

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


C1 = Config("C1 tiny fp32 block", 1, d=64, n_heads=4, n_kv_heads=2, d_ff=192, rope_base=10000.0,
            dtype="f32", B=1, T=16, mode="prefill", t_max=32, decode_steps=4)
C2 = Config("C2 Llama-2-7B block prefill", 2, d=4096, n_heads=32, n_kv_heads=32, d_ff=11008,
            rope_base=10000.0, dtype="bf16", B=1, T=2048, mode="prefill", t_max=2048)
C3 = Config("C3 GQA long-context block prefill", 3, d=4096, n_heads=32, n_kv_heads=8, d_ff=14336,
            rope_base=500000.0, dtype="bf16", B=2, T=8192, mode="prefill", t_max=8192)
C4 = Config("C4 GQA decode step", 4, d=4096, n_heads=32, n_kv_heads=8, d_ff=14336, rope_base=500000.0,
            dtype="bf16", B=64, T=1, mode="decode", t_max=4224, lens_lo=1024, lens_hi=4096)
C5 = Config("C5 32-layer model", 5, d=4096, n_heads=32, n_kv_heads=8, d_ff=14336, rope_base=500000.0,
            dtype="bf16", B=4, T=1024, n_layers=32, vocab=32000, mode="model", t_max=1152,
            decode_steps=128)

CONFIGS = {1: C1, 2: C2, 3: C3, 4: C4, 5: C5}
