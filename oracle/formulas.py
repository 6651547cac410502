"""ORACLE — test infrastructure: the pages' closed-form counting formulas.

Page short names as in oracle.c: [TIR] tirogla "Transformer block",
[KIR] kirito-excalibur "The Transformer", [PID] pidoku "The Transformer",
[GEN] thegeniusblogs "The Transformer Architecture".
FLOPs count one multiply-add as 2 FLOPs ([TIR] How it works, FLOPs per token;
[KIR] 4. FLOP counting).
"""
from __future__ import annotations

import math


def block_weight_shapes(d: int, H: int, Hkv: int, f: int) -> dict:
    """Weight shapes of one block ([TIR] Code, struct Block; [TIR] How it works)."""
    dh = d // H
    return {"g_attn": (d,), "g_mlp": (d,), "wq": (d, H * dh), "wk": (d, Hkv * dh), "wv": (d, Hkv * dh),
            "wo": (H * dh, d), "w1": (d, f), "w3": (d, f), "w2": (f, d)}


def block_matrix_params(d: int, H: int, Hkv: int, f: int) -> int:
    """Weight-matrix parameters of one block, gains excluded ([KIR] 3. Parameter counting,
    exactly: Q, K, V, O plus three SwiGLU matrices; [PID] Counting everything, GQA-adjusted)."""
    dh = d // H
    return d * H * dh + 2 * d * Hkv * dh + H * dh * d + 3 * d * f


def model_params(L: int, d: int, H: int, Hkv: int, f: int, V: int, untied: bool = True,
                 norms: bool = False) -> int:
    """L blocks plus embedding (and an untied head) ([KIR] 3: N ~ 12 L d^2 + V d, x2 untied;
    [PID] Counting everything: L (4d^2 adj. for GQA + 3 d d_ff) + 2 V d)."""
    n = L * block_matrix_params(d, H, Hkv, f) + V * d * (2 if untied else 1)
    if norms:
        n += L * 2 * d + d
    return n


def gpt2_params(L: int = 12, d: int = 768, V: int = 50257, n_ctx: int = 1024) -> int:
    """GPT-2 style count with a 4d GELU MLP, tied embedding and learned positions:
    12 L d^2 + V d + n_ctx d ([TIR] How it works, Parameter count)."""
    return 12 * L * d * d + V * d + n_ctx * d


def d_ff_swiglu(d: int) -> int:
    """f = 8d/3 rounded up to a multiple of 256 ([KIR] 7. The full modern block)."""
    f = int(2 * (4 * d) / 3)
    return 256 * ((f + 255) // 256)


def forward_flops_per_token(N: int, L: int, T: int, d: int) -> int:
    """2N + 4 L T d, counting the full T x T score matrix ([TIR] How it works, Cost)."""
    return 2 * N + 4 * L * T * d


def block_prefill_flops_causal(B: int, T: int, d: int, H: int, Hkv: int, f: int) -> int:
    """Algorithmic prefill FLOPs of one block when only keys j <= i are visited:
    2 N_blk per token for the weight matmuls, plus q.k and p.v over T(T+1)/2 pairs
    per head ([TIR] How it works: causal kernels do about half of 4 T d)."""
    dh = d // H
    return 2 * B * T * block_matrix_params(d, H, Hkv, f) + 4 * dh * H * B * T * (T + 1) // 2


def block_prefill_flops_full(B: int, T: int, d: int, H: int, Hkv: int, f: int) -> int:
    """The page formula per token summed over B T tokens (full T x T)."""
    dh = d // H
    return 2 * B * T * block_matrix_params(d, H, Hkv, f) + 4 * dh * H * B * T * T


def attention_share(d: int, T: int) -> float:
    """4Td / (24 d^2 + 4 T d) ([KIR] 4. FLOP counting, When does attention start to matter)."""
    return 4 * T * d / (24 * d * d + 4 * T * d)


def kv_bytes_per_token(L: int, Hkv: int, dh: int, bytes_per_value: int) -> int:
    """2 L Hkv dh bytes ([TIR] How it works, KV cache; [PID] Counting everything)."""
    return 2 * L * Hkv * dh * bytes_per_value


def kv_cache_bytes(L: int, Hkv: int, dh: int, n: int, bytes_per_value: int) -> int:
    """Whole cache for n tokens ([GEN] KV cache size, 2 L d n bytes for MHA)."""
    return kv_bytes_per_token(L, Hkv, dh, bytes_per_value) * n


def decode_attention_bytes(lens, Hkv: int, dh: int, bytes_per_value: int = 2) -> int:
    """K and V bytes one decode step must read: rows 0..len_b (the new row included)."""
    return sum((int(n) + 1) * Hkv * dh * 2 * bytes_per_value for n in lens)


def isclose_rel(a: float, b: float, rel: float) -> bool:
    return math.isclose(a, b, rel_tol=rel)
