"""Pins for the CPU oracle: each test ties it to something other than itself.

Page short names: [TIR] tirogla "Transformer block", [KIR] kirito-excalibur
"The Transformer", [PID] pidoku "The Transformer", [GEN] thegeniusblogs
"The Transformer Architecture", [MSA] msaqlain "AI engineering: transformers".
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from oracle import formulas as FM
from tests.inputs import activations, block_weights, rel_err, small_cfg

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")


from tests.exact import _bf16, torch_block_f64  # noqa: E402  (the fp64 library composition)


TINY_SHAPES = [
    dict(d=64, H=4, Hkv=2, f=192, T=16),    # the tiny fp32 workload's shape
    dict(d=16, H=4, Hkv=2, f=48, T=5),      # the shape of [TIR] Code's test
    dict(d=32, H=4, Hkv=1, f=96, T=33),     # MQA
    dict(d=32, H=2, Hkv=2, f=64, T=9),      # MHA
    dict(d=64, H=2, Hkv=1, f=128, T=20),    # dh = 32
]


def _run_pins_vs_torch(orc, shapes=TINY_SHAPES, gains="random", dtype="f32"):
    worst = 0.0
    for i, s in enumerate(shapes):
        cfg = small_cfg(d=s["d"], H=s["H"], Hkv=s["Hkv"], f=s["f"], number=40 + i, dtype=dtype)
        w, _ = block_weights(cfg, gains=gains)
        x, _ = activations(cfg, 2, s["T"])
        got, inter = orc.block_forward(cfg, w, x, intermediates=True)
        ref, rint = torch_block_f64(cfg, w, x, bf16=dtype == "bf16")
        worst = max(worst, rel_err(got, ref))
        for key in ("q", "att", "r", "act"):
            worst = max(worst, rel_err(inter[key], rint[key]))
    return worst


def test_block_matches_fp64_library_composition(oracle):
    """Every step at once, against library routines in fp64 ([TIR] How it works)."""
    assert _run_pins_vs_torch(oracle) <= 1e-5
    assert _run_pins_vs_torch(oracle, gains="ones") <= 1e-5


def _bf16_gap(got, ref):
    """(largest gap, number of values) between two arrays of bf16 values that
    are not bitwise equal: 1 means neighbouring bf16 values, more is a real
    difference."""
    a = np.asarray(got, np.float32).view(np.uint32).astype(np.int64)
    b = np.asarray(ref, np.float64).astype(np.float32).view(np.uint32).astype(np.int64)
    assert not np.any((a | b) & 0xFFFF), "operands must be bf16 values"
    diff = np.abs((a >> 16) - (b >> 16))
    diff[(a >> 31) != (b >> 31)] = 1 << 16  # sign differs
    return int(diff.max(initial=0)), int(np.count_nonzero(diff))


def test_bf16_operands_match_fp64_composition(oracle):
    """bf16 storage: the oracle rounds each GEMM operand to bf16 and nothing
    else ([TIR] Implementation notes).  Against the fp64 composition that rounds
    at the same places with torch's conversion, the only gap is fp32 vs fp64
    arithmetic: the output agrees to 1e-5 rms, and each rounded operand (q, att,
    act) is bitwise equal except where a value fell so close to a rounding
    boundary that the two sides picked neighbouring bf16 values (rare).  A
    dropped or misplaced rounding leaves non-bf16 values or moves many values."""
    for gains in ("random", "ones"):
        for i, s in enumerate(TINY_SHAPES):
            cfg = small_cfg(d=s["d"], H=s["H"], Hkv=s["Hkv"], f=s["f"], number=40 + i, dtype="bf16")
            w, _ = block_weights(cfg, gains=gains)
            x, _ = activations(cfg, 2, s["T"])
            got, inter = oracle.block_forward(cfg, w, x, intermediates=True)
            ref, rint = torch_block_f64(cfg, w, x, bf16=True)
            assert rel_err(got, ref) <= 1e-5
            assert rel_err(inter["r"], rint["r"]) <= 1e-5
            for key in ("q", "att", "act"):
                gap, n = _bf16_gap(inter[key], rint[key])
                assert gap <= 1 and n <= max(2, inter[key].size // 500), (key, gap, n)


def test_values_before_rounding(oracle):
    """The oracle's *_pre intermediates are the operands before their bf16
    rounding: torch's own fp32 -> bf16 conversion of each gives the operand the
    oracle handed on bit for bit, with fp32 storage they are the operands, and
    they follow the fp64 composition's unrounded values (q and k after RoPE,
    v, the attention output, the SwiGLU product)."""
    for i, s in enumerate(TINY_SHAPES[:3]):
        for dtype in ("f32", "bf16"):
            cfg = small_cfg(d=s["d"], H=s["H"], Hkv=s["Hkv"], f=s["f"], number=60 + i, dtype=dtype)
            w, _ = block_weights(cfg, gains="random")
            x, _ = activations(cfg, 2, s["T"])
            _, inter = oracle.block_forward(cfg, w, x, intermediates=True)
            _, rint = torch_block_f64(cfg, w, x, bf16=dtype == "bf16")
            for key in ("q", "att", "act"):
                pre = inter[key + "_pre"]
                if dtype == "f32":
                    assert np.array_equal(pre, inter[key]), key
                else:
                    rounded = torch.from_numpy(pre).to(torch.bfloat16).to(torch.float32).numpy()
                    assert np.array_equal(rounded, inter[key]), key
                    assert np.any(pre.view(np.uint32) & 0xFFFF), key
            for key in ("q_pre", "k_pre", "v_pre", "att_pre", "act_pre"):
                assert rel_err(inter[key], rint[key]) <= 1e-5, (dtype, key, rel_err(inter[key], rint[key]))


def test_kv_append_places_every_value(oracle):
    """[TIR] How it works, KV cache paragraph: the keys and values of new
    tokens go to rows start[b] + t of their sequence and KV head.  Each value
    encodes its own (b, t, g, e), so the cache shows where every value landed;
    every other row keeps its sentinel."""
    B, Hkv, dh, t_max, n = 3, 2, 6, 11, 4
    start = np.array([0, 5, 7], np.int32)
    b, t, g, e = np.meshgrid(np.arange(B), np.arange(n), np.arange(Hkv), np.arange(dh), indexing="ij")
    code = (1000 * b + 100 * t + 10 * g + e).astype(np.float32) + 1.0
    kc = np.full((B, Hkv, t_max, dh), -7.0, np.float32)
    vc = np.full_like(kc, -9.0)
    oracle.kv_append(kc, vc, code, -code, start)
    for bb in range(B):
        for gg in range(Hkv):
            for row in range(t_max):
                tt = row - start[bb]
                if 0 <= tt < n:
                    want = 1.0 + 1000 * bb + 100 * tt + 10 * gg + np.arange(dh)
                    assert np.array_equal(kc[bb, gg, row], want) and np.array_equal(vc[bb, gg, row], -want)
                else:
                    assert np.all(kc[bb, gg, row] == -7.0) and np.all(vc[bb, gg, row] == -9.0)
    # a start that would run past t_max is refused and writes nothing
    before = kc.copy()
    with pytest.raises(ValueError):
        oracle.kv_append(kc, vc, code, -code, np.array([0, 5, 8], np.int32))
    assert np.array_equal(kc, before)


def test_kv_append_equals_the_block_cache_write(oracle):
    """Appending a block's own post-RoPE k and v (bf16 operands, as stored)
    gives bit for bit the cache rows the block itself writes, at a nonzero start."""
    cfg = small_cfg(d=64, H=4, Hkv=2, f=192, number=48, dtype="bf16")
    w, _ = block_weights(cfg, gains="random")
    x, _ = activations(cfg, 2, 9)
    start = np.array([3, 6], np.int32)
    B, T, dh, t_max = 2, 9, 16, 20
    kc = np.zeros((B, 2, t_max, dh), np.float32)
    vc = np.zeros_like(kc)
    # earlier rows the block reads, and rows after the write, hold sentinels
    kc[:], vc[:] = 0.25, -0.25
    _, inter = oracle.block_forward(cfg, w, x, start=start, kc=kc, vc=vc, intermediates=True)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()  # noqa: E731
    k_new = bf(inter["k_pre"]).reshape(B, T, 2, dh)
    v_new = bf(inter["v_pre"]).reshape(B, T, 2, dh)
    kc2 = np.full_like(kc, 0.25)
    vc2 = np.full_like(vc, -0.25)
    oracle.kv_append(kc2, vc2, k_new, v_new, start)
    assert np.array_equal(kc2, kc) and np.array_equal(vc2, vc)


def test_bf16_operands_are_bf16_values(oracle):
    """The GEMM operands the oracle hands on are bf16 values (the low 16 bits of
    their fp32 patterns are zero); the residual inside the block is not rounded."""
    cfg = small_cfg(d=64, H=4, Hkv=2, f=192, number=47, dtype="bf16")
    w, _ = block_weights(cfg, gains="random")
    x, _ = activations(cfg, 2, 16)
    _, inter = oracle.block_forward(cfg, w, x, intermediates=True)
    for key in ("q", "att", "act"):
        assert not np.any(inter[key].view(np.uint32) & 0xFFFF), key
    assert np.any(inter["r"].view(np.uint32) & 0xFFFF)
    # the fp32 storage configuration rounds nothing
    _, i32 = oracle.block_forward(cfg.with_(dtype="f32"), w, x, intermediates=True)
    assert np.any(i32["act"].view(np.uint32) & 0xFFFF)


def test_sliding_window_first_key_matches_page_example(oracle):
    """[PID] Sliding-window attention: with W = 4096 the query at position
    10000 attends to tokens 5905..10000; W = 0 is full causal attention."""
    g = json.load(open(GOLDEN))["sliding_window_example"]
    assert oracle.window_first_key(g["query"], g["window"]) == g["first_key"]
    assert oracle.window_first_key(g["query"], 0) == 0
    assert oracle.window_first_key(3, 10) == 0 and oracle.window_first_key(9, 1) == 9


def test_sliding_window_attention_reads_exactly_the_window(oracle):
    """q = 0 gives equal weights, so with v_j = (j, j^2, 1) the output is the
    mean of j and of j^2 over the keys read: that fixes the key range."""
    n, W = 40, 7
    kc = np.random.default_rng(9).normal(size=(n, 16)).astype(np.float32)
    j = np.arange(n, dtype=np.float64)
    vc = np.zeros((n, 16), np.float32)
    vc[:, 0], vc[:, 1], vc[:, 2] = j, j * j, 1.0
    for p in (0, 3, 6, 7, 20, 39):
        j0 = oracle.window_first_key(p, W)
        o = oracle.attend_row(np.zeros(16, np.float32), kc, vc, p + 1, first_key=j0)
        sel = j[j0:p + 1]
        assert len(sel) == min(W, p + 1)
        assert abs(o[0] - sel.mean()) <= 1e-5 * max(1.0, sel.mean())
        assert abs(o[1] - (sel * sel).mean()) <= 1e-5 * max(1.0, (sel * sel).mean())
        assert abs(o[2] - 1.0) <= 1e-6


def test_sliding_window_block_matches_fp64_band_mask(oracle):
    """The block with a window against SDPA with an explicit band mask; a
    window at least T long is full causal attention, bitwise."""
    for W in (1, 3, 8):
        cfg = small_cfg(number=74, window=W)
        w, _ = block_weights(cfg, gains="random")
        x, _ = activations(cfg, 2, 13)
        got, inter = oracle.block_forward(cfg, w, x, intermediates=True)
        ref, rint = torch_block_f64(cfg, w, x, window=W)
        assert rel_err(got, ref) <= 1e-5 and rel_err(inter["att"], rint["att"]) <= 1e-5
        if W == 1:  # each query sees only itself: the attention output is its own v
            v = np.stack([oracle.matmul(oracle.rms_norm(x[b], w["g_attn"], cfg.rms_eps), w["wv"]) for b in range(2)])
            g = cfg.n_heads // cfg.n_kv_heads
            v = v.reshape(2, 13, cfg.n_kv_heads, 1, cfg.head_dim).repeat(g, axis=3).reshape(2, 13, -1)
            assert np.array_equal(inter["att"], v)
    cfg = small_cfg(number=75)
    w, _ = block_weights(cfg)
    x, _ = activations(cfg, 1, 10)
    assert np.array_equal(oracle.block_forward(cfg.with_(window=10), w, x), oracle.block_forward(cfg, w, x))


def test_sliding_window_decode_equals_prefill_bitwise(oracle):
    cfg = small_cfg(number=76, window=5)
    w, _ = block_weights(cfg)
    x, _ = activations(cfg, 1, 20)
    full = oracle.block_forward(cfg, w, x)
    kc = np.zeros((1, cfg.n_kv_heads, 20, cfg.head_dim), np.float32)
    vc = kc.copy()
    oracle.block_forward(cfg, w, x[:, :12], kc=kc, vc=vc)
    for p in range(12, 20):
        out = oracle.block_forward(cfg, w, x[:, p:p + 1], start=[p], kc=kc, vc=vc)
        assert np.array_equal(out[0, 0], full[0, p])


def test_decode_matches_fp64_library_composition(oracle):
    """Decode at position p equals row p of the full-sequence result ([GEN] Two phases)."""
    cfg = small_cfg(number=61)
    w, _ = block_weights(cfg)
    x, _ = activations(cfg, 1, 20)
    ref, _ = torch_block_f64(cfg, w, x)
    t_max = 32
    kc = np.full((1, cfg.n_kv_heads, t_max, cfg.head_dim), np.nan, np.float32)
    vc = kc.copy()
    oracle.block_forward(cfg, w, x[:, :16], kc=kc, vc=vc)
    for p in range(16, 20):
        out = oracle.block_forward(cfg, w, x[:, p:p + 1], start=[p], kc=kc, vc=vc)
        assert rel_err(out[0, 0], ref[0, p]) <= 1e-5
    assert np.isnan(kc[:, :, 20:]).all() and np.isnan(vc[:, :, 20:]).all()


def test_exact_decode_and_model_compositions(oracle):
    """The fp64 decode and model compositions (tests/exact.py, used to measure
    how far the method itself sits from the oracle at full size) agree with
    the oracle at tiny shapes: a decode step over a cache of earlier rows, with
    and without bf16 operands, and the bf16 model's last-row logits."""
    from tests.exact import decode_f64, model_f64
    import synth
    for dtype in ("f32", "bf16"):
        cfg = small_cfg(d=64, H=4, Hkv=2, f=192, number=62, dtype=dtype)
        w, _ = block_weights(cfg, gains="random")
        x, _ = activations(cfg, 3, 1)
        lens = np.array([5, 11, 1], np.int32)
        kc, _ = synth.normal(cfg.seed, 11, (3, 2, 16, 16), 1.0, dtype == "bf16")
        vc, _ = synth.normal(cfg.seed, 12, (3, 2, 16, 16), 1.0, dtype == "bf16")
        ref, inter = oracle.block_forward(cfg, w, x, start=lens, kc=kc.copy(), vc=vc.copy(), intermediates=True)
        got, ex = decode_f64(cfg, w, x, lens, kc, vc, bf16=dtype == "bf16")
        assert rel_err(got, ref) <= 1e-5, rel_err(got, ref)
        for key in ("q_pre", "k_pre", "att_pre", "act_pre"):
            assert rel_err(ex[key], inter[key]) <= 1e-5, key
    cfg = small_cfg(number=73, dtype="bf16")
    L, V, T = 2, 40, 7
    layers = [block_weights(cfg, layer=l, gains="random")[0] for l in range(L)]
    emb, _ = synth.normal(cfg.seed, 15, (V, cfg.d), 1.0, True)
    wu, _ = synth.normal(cfg.seed, 17, (cfg.d, V), 0.1, True)
    gf = synth.to_bf16(1.0 + synth.normal(cfg.seed, 16, (cfg.d,), 0.1, False)[0])[1]
    ids = synth.integers(cfg.seed, 14, (2, T), 0, V - 1)
    kcs = [np.zeros((2, cfg.n_kv_heads, T, cfg.head_dim), np.float32) for _ in range(L)]
    vcs = [a.copy() for a in kcs]
    logits, _ = oracle.model_forward(cfg, L, V, emb, layers, gf, wu, ids, kcs, vcs, rows=[T - 1])
    assert rel_err(logits, model_f64(cfg, layers, emb, gf, wu, ids)) <= 1e-5


def test_folded_norm_form_is_the_same_product(oracle):
    """The folded RMSNorm form of the exact evaluation (operand x * g, the row
    scale 1/rms(x) applied to the GEMM's products) is the oracle's block
    before any bf16 rounding, for every row folded or only a prefix; with bf16
    operands it moves only where the operand is rounded (the result stays
    within that rounding's reach of the oracle)."""
    cfg = small_cfg(d=64, H=4, Hkv=2, f=192, number=64)
    w, _ = block_weights(cfg, gains="random")
    x, _ = activations(cfg, 2, 9)
    ref = oracle.block_forward(cfg, w, x)
    for f1, f2 in ((9, 9), (0, 9), (4, 6)):
        got, _ = torch_block_f64(cfg, w, x, fold1=f1, fold2=f2)
        assert rel_err(got, ref) <= 1e-5, (f1, f2, rel_err(got, ref))
    plain, _ = torch_block_f64(cfg, w, x, bf16=True)
    folded, _ = torch_block_f64(cfg, w, x, bf16=True, fold1=9, fold2=9)
    assert not np.array_equal(plain, folded)
    assert rel_err(folded, plain) <= 2e-2


def test_prefix_invariance_bitwise(oracle):
    """[TIR] Code test: a prefix gives the same outputs as the full sequence.
    Exact here (the page asserts 1e-5)."""
    cfg = small_cfg(d=16, H=4, Hkv=2, f=48, number=62)
    w, _ = block_weights(cfg)
    x, _ = activations(cfg, 1, 5)
    full = oracle.block_forward(cfg, w, x)
    pre = oracle.block_forward(cfg, w, x[:, :3])
    assert np.array_equal(full[:, :3], pre)
    cfg = small_cfg(number=63)
    w, _ = block_weights(cfg)
    x, _ = activations(cfg, 2, 40)
    full = oracle.block_forward(cfg, w, x)
    for n in (1, 7, 16, 33):
        assert np.array_equal(full[:, :n], oracle.block_forward(cfg, w, x[:, :n]))


def test_decode_equals_prefill_bitwise(oracle):
    cfg = small_cfg(number=64)
    w, _ = block_weights(cfg)
    x, _ = activations(cfg, 3, 24)
    full = oracle.block_forward(cfg, w, x)
    kc = np.zeros((3, cfg.n_kv_heads, 24, cfg.head_dim), np.float32)
    vc = kc.copy()
    starts = np.array([5, 11, 17], np.int32)
    # each sequence prefilled to its own length, then one decode step each
    for b in range(3):
        kb, vb = kc[b:b + 1].copy(), vc[b:b + 1].copy()
        oracle.block_forward(cfg, w, x[b:b + 1, :starts[b]], kc=kb, vc=vb)
        kc[b], vc[b] = kb[0], vb[0]
    xd = np.stack([x[b, starts[b]] for b in range(3)])[:, None, :]
    out = oracle.block_forward(cfg, w, xd, start=starts, kc=kc, vc=vc)
    for b in range(3):
        assert np.array_equal(out[b, 0], full[b, starts[b]])


def test_selected_rows_equal_full_rows(oracle):
    cfg = small_cfg(number=65)
    w, _ = block_weights(cfg)
    x, _ = activations(cfg, 2, 30)
    full = oracle.block_forward(cfg, w, x)
    rows = [0, 7, 29, 13]
    sel = oracle.block_forward(cfg, w, x, rows=rows)
    assert np.array_equal(sel, full[:, rows])


def test_gqa_equals_mha_with_repeated_kv_bitwise(oracle):
    """GQA shares each KV head among H/Hkv consecutive query heads ([TIR] How it
    works; [MSA] 4.1): it must equal MHA whose Wk, Wv repeat each KV head."""
    for Hkv in (1, 2):
        cfg = small_cfg(H=4, Hkv=Hkv, number=66)
        w, _ = block_weights(cfg)
        x, _ = activations(cfg, 1, 12)
        dh, g = cfg.head_dim, cfg.n_heads // Hkv
        mha = dict(w)
        for n in ("wk", "wv"):
            cols = np.concatenate([np.arange(kv * dh, (kv + 1) * dh) for kv in range(Hkv) for _ in range(g)])
            mha[n] = np.ascontiguousarray(w[n][:, cols])
        cfg_m = small_cfg(H=4, Hkv=4, number=66)
        assert np.array_equal(oracle.block_forward(cfg, w, x), oracle.block_forward(cfg_m, mha, x))


def test_softmax_rows_sum_to_one(oracle):
    """[MSA] 1.3: softmax rows sum to 1; with V = ones every output is 1."""
    rng = np.random.default_rng(5)
    for n in (1, 2, 17, 300):
        q = rng.normal(size=16).astype(np.float32) * 3
        kc = rng.normal(size=(n, 16)).astype(np.float32)
        o = oracle.attend_row(q, kc, np.ones((n, 16), np.float32), n)
        assert np.max(np.abs(o - 1.0)) <= n * 2.0 ** -23 + 2.0 ** -22


def test_attention_closed_forms(oracle):
    rng = np.random.default_rng(6)
    kc = rng.normal(size=(9, 16)).astype(np.float32)
    vc = rng.normal(size=(9, 16)).astype(np.float32)
    # one key: the output is that key's value, exactly
    assert np.array_equal(oracle.attend_row(rng.normal(size=16), kc, vc, 1), vc[0])
    # q = 0: uniform weights, the output is the mean of the visible values
    for n in (2, 5, 9):
        o = oracle.attend_row(np.zeros(16, np.float32), kc, vc, n)
        assert np.allclose(o, vc[:n].astype(np.float64).mean(0), rtol=0, atol=2e-6)
    # masked keys beyond n_keys are never read (NaN there changes nothing)
    kn, vn = kc.copy(), vc.copy()
    kn[5:], vn[5:] = np.nan, np.nan
    q = rng.normal(size=16).astype(np.float32)
    assert np.array_equal(oracle.attend_row(q, kn, vn, 5), oracle.attend_row(q, kc, vc, 5))


def test_block_closed_forms(oracle):
    cfg = small_cfg(number=67)
    w, _ = block_weights(cfg)
    x, _ = activations(cfg, 1, 8)
    # Wo = W2 = 0: both sublayers add nothing, out = x bitwise
    z = dict(w, wo=np.zeros_like(w["wo"]), w2=np.zeros_like(w["w2"]))
    assert np.array_equal(oracle.block_forward(cfg, z, x), x)
    # W1 = 0: silu(0) = 0 so the MLP adds nothing, out = r bitwise
    z = dict(w, w1=np.zeros_like(w["w1"]))
    out, inter = oracle.block_forward(cfg, z, x, intermediates=True)
    assert np.array_equal(out, inter["r"]) and not np.any(inter["act"])
    # T = 1: attention returns v of the only token, so att = h Wv repeated per group
    out, inter = oracle.block_forward(cfg, w, x[:, :1], intermediates=True)
    h = oracle.rms_norm(x[0, :1], w["g_attn"], cfg.rms_eps)
    v = oracle.matmul(h, w["wv"]).reshape(cfg.n_kv_heads, cfg.head_dim)
    g = cfg.n_heads // cfg.n_kv_heads
    assert np.array_equal(inter["att"][0, 0].reshape(cfg.n_heads, cfg.head_dim), np.repeat(v, g, axis=0))


def test_rms_norm_closed_form(oracle):
    for c in (0.5, 3.0, -2.0, 1e-3):
        x = np.full((1, 64), c, np.float32)
        y = oracle.rms_norm(x, np.ones(64, np.float32), 1e-6)
        ref = c / np.sqrt(np.float64(c) ** 2 + 1e-6)
        assert np.allclose(y, ref, rtol=3e-7, atol=0)


def test_rope_properties(oracle):
    """[GEN] Positional encodings, RoPE: rotations of pairs, identity at position
    0, norms preserved, scores depend only on the offset n - m."""
    dh, base = 16, 10000.0
    c, s = oracle.rope_table(64, dh, base)
    i = np.arange(dh // 2)
    for t in (0, 1, 7, 63):
        a = t * np.power(base, -2.0 * i / dh)
        assert np.max(np.abs(c[t] - np.cos(a).astype(np.float32))) <= 6e-8
        assert np.max(np.abs(s[t] - np.sin(a).astype(np.float32))) <= 6e-8
    rng = np.random.default_rng(7)
    v = rng.normal(size=(4, 3, dh)).astype(np.float32)
    r0 = oracle.rope_apply(v, [0, 0, 0, 0], c, s)
    assert np.array_equal(r0, v)
    r = oracle.rope_apply(v, [1, 5, 30, 63], c, s)
    pn = lambda a: np.hypot(a[..., 0::2].astype(np.float64), a[..., 1::2].astype(np.float64))  # noqa: E731
    assert np.allclose(pn(r), pn(v), rtol=5e-7, atol=0)
    # <R_m q, R_n k> == <R_{m+delta} q, R_{n+delta} k>
    q, k = rng.normal(size=(1, 1, dh)).astype(np.float32), rng.normal(size=(1, 1, dh)).astype(np.float32)
    for m, n, delta in ((3, 9, 20), (0, 40, 11), (17, 2, 30)):
        s1 = float(np.dot(oracle.rope_apply(q, [m], c, s).ravel(), oracle.rope_apply(k, [n], c, s).ravel()))
        s2 = float(np.dot(oracle.rope_apply(q, [m + delta], c, s).ravel(),
                          oracle.rope_apply(k, [n + delta], c, s).ravel()))
        assert abs(s1 - s2) <= 2e-5 * (np.linalg.norm(q) * np.linalg.norm(k))
    # interleaved pairs: only components (2i, 2i+1) mix
    e = np.zeros((1, 1, dh), np.float32)
    e[0, 0, 2] = 1.0
    r = oracle.rope_apply(e, [5], c, s)[0, 0]
    assert np.count_nonzero(r) == 2 and r[2] == c[5, 1] and r[3] == s[5, 1]


def test_counters_match_flop_formulas(oracle):
    """Instrumented work equals the pages' formulas: 2 FLOPs per weight per token
    ([TIR] How it works, FLOPs per token) and a causal attention term of
    4 dh H T(T+1)/2, about half of the full 4 T d per token."""
    cfg = small_cfg(number=68)
    w, _ = block_weights(cfg)
    T = 16
    x, _ = activations(cfg, 1, T)
    cnt = O.Counters()
    oracle.block_forward(cfg, w, x, counters=cnt)
    n_blk = FM.block_matrix_params(cfg.d, cfg.n_heads, cfg.n_kv_heads, cfg.d_ff)
    assert n_blk == 12 * cfg.d ** 2 == 49152
    assert sum(int(np.prod(a.shape)) for k, a in w.items() if not k.startswith("g_")) == n_blk
    assert cnt.matmul_macs == T * n_blk
    dh, H = cfg.head_dim, cfg.n_heads
    assert cnt.qk_macs == cnt.pv_macs == H * dh * T * (T + 1) // 2
    assert 2 * (cnt.matmul_macs + cnt.qk_macs + cnt.pv_macs) == FM.block_prefill_flops_causal(
        1, T, cfg.d, H, cfg.n_kv_heads, cfg.d_ff)
    full = FM.block_prefill_flops_full(1, T, cfg.d, H, cfg.n_kv_heads, cfg.d_ff)
    assert full == T * FM.forward_flops_per_token(n_blk, 1, T, cfg.d)
    assert cnt.cache_values == T * 2 * cfg.n_kv_heads * dh


def test_kv_bytes_per_token_from_model_counters(oracle):
    """KV bytes per token = 2 L Hkv dh bytes ([TIR] How it works, KV cache)."""
    cfg = small_cfg(number=69)
    L, V, T = 2, 50, 6
    layers = [block_weights(cfg, layer=l)[0] for l in range(L)]
    import synth
    emb, _ = synth.normal(cfg.seed, 15, (V, cfg.d), 0.02, False)
    wu, _ = synth.normal(cfg.seed, 17, (cfg.d, V), 0.02, False)
    ids = synth.integers(cfg.seed, 14, (1, T), 0, V - 1)
    kcs = [np.zeros((1, cfg.n_kv_heads, 8, cfg.head_dim), np.float32) for _ in range(L)]
    vcs = [a.copy() for a in kcs]
    cnt = O.Counters()
    oracle.model_forward(cfg, L, V, emb, layers, np.ones(cfg.d, np.float32), wu, ids, kcs, vcs, counters=cnt)
    assert cnt.cache_values * 2 == T * FM.kv_bytes_per_token(L, cfg.n_kv_heads, cfg.head_dim, 2)
    assert FM.kv_bytes_per_token(32, 8, 128, 2) == 131072


def test_model_matches_fp64_composition(oracle):
    """Embed, L blocks, final norm, untied head, greedy argmax ([PID] The full model)."""
    cfg = small_cfg(number=70)
    L, V, T = 2, 40, 7
    import synth
    layers = [block_weights(cfg, layer=l, gains="random")[0] for l in range(L)]
    emb, _ = synth.normal(cfg.seed, 15, (V, cfg.d), 1.0, False)
    wu, _ = synth.normal(cfg.seed, 17, (cfg.d, V), 0.1, False)
    gf = 1.0 + synth.normal(cfg.seed, 16, (cfg.d,), 0.1, False)[0]
    ids = synth.integers(cfg.seed, 14, (2, T), 0, V - 1)
    kcs = [np.zeros((2, cfg.n_kv_heads, T, cfg.head_dim), np.float32) for _ in range(L)]
    vcs = [a.copy() for a in kcs]
    logits, nxt = oracle.model_forward(cfg, L, V, emb, layers, gf, wu, ids, kcs, vcs)
    x = emb[ids].astype(np.float64)
    for l in range(L):
        x, _ = torch_block_f64(cfg, layers[l], x)
    hn = F.rms_norm(torch.from_numpy(x), (cfg.d,), weight=torch.from_numpy(gf.astype(np.float64)),
                    eps=cfg.rms_eps).numpy()
    ref = hn @ wu.astype(np.float64)
    assert rel_err(logits, ref) <= 1e-5
    assert np.array_equal(nxt, np.argmax(logits[:, -1], axis=-1))


def test_bf16_model_matches_fp64_composition(oracle):
    """bf16 storage: block outputs handed to the next block and the final-norm
    rows are bf16 operands too ([TIR] Implementation notes)."""
    cfg = small_cfg(number=73, dtype="bf16")
    L, V, T = 2, 40, 7
    import synth
    layers = [block_weights(cfg, layer=l, gains="random")[0] for l in range(L)]
    emb, _ = synth.normal(cfg.seed, 15, (V, cfg.d), 1.0, True)
    wu, _ = synth.normal(cfg.seed, 17, (cfg.d, V), 0.1, True)
    gf = synth.to_bf16(1.0 + synth.normal(cfg.seed, 16, (cfg.d,), 0.1, False)[0])[1]
    ids = synth.integers(cfg.seed, 14, (2, T), 0, V - 1)
    kcs = [np.zeros((2, cfg.n_kv_heads, T, cfg.head_dim), np.float32) for _ in range(L)]
    vcs = [a.copy() for a in kcs]
    logits, _ = oracle.model_forward(cfg, L, V, emb, layers, gf, wu, ids, kcs, vcs)
    x = torch.from_numpy(emb[ids].astype(np.float64))
    for l in range(L):
        x = _bf16(torch.from_numpy(torch_block_f64(cfg, layers[l], x.numpy(), bf16=True)[0]))
    hn = _bf16(F.rms_norm(x, (cfg.d,), weight=torch.from_numpy(gf.astype(np.float64)), eps=cfg.rms_eps))
    ref = (hn @ torch.from_numpy(wu.astype(np.float64))).numpy()
    assert rel_err(logits, ref) <= 1e-5


def test_argmax_ties_take_lowest_index(oracle):
    cfg = small_cfg(number=71)
    V = 8
    w = block_weights(cfg)[0]
    # W_U with identical columns 2 and 5 that dominate: a tie broken to index 2
    wu = np.zeros((cfg.d, V), np.float32)
    wu[:, 2] = wu[:, 5] = 1.0
    emb = np.ones((V, cfg.d), np.float32)
    kcs = [np.zeros((1, cfg.n_kv_heads, 1, cfg.head_dim), np.float32)]
    z = dict(w, wo=np.zeros_like(w["wo"]), w2=np.zeros_like(w["w2"]))
    _, nxt = oracle.model_forward(cfg, 1, V, emb, [z], np.ones(cfg.d, np.float32), wu,
                                  np.array([[3]], np.int32), kcs, [kcs[0].copy()])
    assert nxt[0] == 2


def test_page_numbers():
    """Values the pages print, recomputed from the formula functions."""
    g = json.load(open(GOLDEN))
    e = g["gpt2_small_params"]
    assert FM.isclose_rel(FM.gpt2_params(**e["inputs"]), e["value_approx"], e["rel_tol"])
    assert FM.gpt2_params() == 124_318_464
    assert FM.isclose_rel(12 * 12 * 768 ** 2, g["gpt2_small_12Ld2"]["value_approx"], 0.001)
    e = g["exercise_params"]
    i = e["inputs"]
    assert 12 * i["L"] * i["d"] ** 2 + i["V"] * i["d"] == e["value"]
    e = g["llama2_70b_per_layer"]
    i = e["inputs"]
    dh = i["d"] // i["H"]
    att = 2 * i["d"] * i["H"] * dh + 2 * i["d"] * i["Hkv"] * dh
    mlp = 3 * i["d"] * i["f"]
    assert FM.isclose_rel(att, e["attention_approx"], e["rel_tol"])
    assert FM.isclose_rel(mlp, e["mlp_approx"], e["rel_tol"])
    tot = FM.model_params(i["L"], i["d"], i["H"], i["Hkv"], i["f"], i["V"])
    assert FM.isclose_rel(tot, e["total_approx"], e["rel_tol"]) and tot == 68_975_329_280
    assert FM.d_ff_swiglu(4096) == g["d_ff_4096"]["value"]
    for d, T, share in g["attention_share"]["rows"]:
        assert abs(FM.attention_share(d, T) - share) <= g["attention_share"]["abs_tol"]
    e = g["kv_cache_llama3_70b"]
    i = e["inputs"]
    mha = FM.kv_cache_bytes(i["L"], i["H"], i["d"] // i["H"], i["n"], i["bytes"])
    gqa = FM.kv_cache_bytes(i["L"], i["Hkv_gqa"], i["d"] // i["H"], i["n"], i["bytes"])
    assert FM.isclose_rel(mha, e["mha_approx_bytes"], 0.03)
    assert FM.isclose_rel(gqa, e["gqa_approx_bytes"], e["rel_tol"])
    e = g["decode_trace_llama3_8b"]
    i = e["inputs"]
    assert FM.isclose_rel(2 * i["d"] * i["d"] / 1e6, e["q_proj_mflop"], e["rel_tol"])
    assert FM.isclose_rel(i["d"] * i["d"] * i["bytes"] / 1e6, e["q_proj_mb"], e["rel_tol"])
    assert FM.isclose_rel(2 * i["d"] * i["kv_width"] / 1e6, e["k_proj_mflop"], e["rel_tol"])
    assert FM.isclose_rel(3 * 2 * i["d"] * i["f"] / 1e6, e["gate_up_down_mflop"], e["rel_tol"])
    assert FM.isclose_rel(2 * i["d"] * i["V"] / 1e9, e["lm_head_gflop"], e["rel_tol"])
    assert FM.isclose_rel(i["d"] * i["V"] * i["bytes"] / 1e9, e["lm_head_gb"], e["rel_tol"])


def test_thread_count_does_not_change_results(oracle, tmp_path):
    cfg = small_cfg(d=128, H=4, Hkv=2, f=256, number=72)
    w, _ = block_weights(cfg)
    x, _ = activations(cfg, 2, 70)
    here = oracle.block_forward(cfg, w, x)
    np.save(tmp_path / "here.npy", here)
    code = (
        "import numpy as np, sys; sys.path.insert(0, %r)\n"
        "import oracle as O\n"
        "from tests.inputs import block_weights, activations, small_cfg\n"
        "cfg = small_cfg(d=128, H=4, Hkv=2, f=256, number=72)\n"
        "w, _ = block_weights(cfg); x, _ = activations(cfg, 2, 70)\n"
        "o = O.Oracle(); assert o.threads() == 1\n"
        "print(int(np.array_equal(o.block_forward(cfg, w, x), np.load(%r))))\n"
    ) % (os.path.dirname(os.path.dirname(os.path.abspath(__file__))), str(tmp_path / "here.npy"))
    env = dict(os.environ, OMP_NUM_THREADS="1")
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, check=True)
    assert res.stdout.strip() == "1"
