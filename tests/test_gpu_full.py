"""Parity at the workloads' full sizes, in the launch configuration bench.py
times: the block output of both prefill workloads and of the decode step, the
whole KV cache written, and the two-layer model at the full model's widths.

Two bounds.  Sampled rows (first and last rows, tile borders, every decode
sequence) meet the stated bound max |err| <= 2e-2 rms(out) as it stands.  Over
every output value the bound also allows for the rounding of the bf16 output
itself, at most half a bf16 unit in the last place, i.e. 2^-8 |out|: over
millions of values a few of the largest outputs (|out| ~ 5 rms, where half a
unit is already 0.013 rms) carry that rounding on top of the bf16-operand
noise."""
import numpy as np
import pytest

import synth
from synth.configs import C2, C3, C4, C5, tensor_id
from tests.conftest import gpu_available
from tests.gpu_util import HALF_ULP, cache_ok, logits_ok, dev_weights, dev_x, stored_ok, to_dev, to_np, widen_cache
from tests.inputs import rel_err

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import transformer_decoder_block_rmsnorm_amd as tfb  # noqa: E402

TOL = 2e-2


def _prefill_full(oracle, cfg, rows):
    import torch
    tc = tfb.Config.of(cfg)
    w32, w = dev_weights(cfg)
    x32, x = dev_x(cfg, cfg.B, cfg.T)
    rope = tfb.rope_table_init(tc, cfg.t_max)
    dh = cfg.d // cfg.n_heads
    kc = torch.zeros((cfg.B, cfg.n_kv_heads, cfg.t_max, dh), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    out = torch.empty_like(x)
    ws = tfb.workspace(tc, cfg.B, cfg.T)
    tfb.block_prefill(tc, w, rope, x, out, cache=(kc, vc), ws=ws)
    torch.cuda.synchronize()
    okc = np.zeros((cfg.B, cfg.n_kv_heads, cfg.t_max, dh), np.float32)
    ovc = okc.copy()
    ref = oracle.block_forward(cfg, w32, x32, kc=okc, vc=ovc)
    got = to_np(out)
    assert rel_err(got[:, rows], ref[:, rows]) <= TOL, rel_err(got[:, rows], ref[:, rows])
    assert stored_ok(got, ref, TOL, HALF_ULP), rel_err(got, ref)
    assert cache_ok(cfg, widen_cache(kc), okc)
    assert cache_ok(cfg, widen_cache(vc), ovc)


def test_llama2_7b_block_prefill_full_size(oracle):
    """d=4096, H=Hkv=32, f=11008, B=1, T=2048 (the benchmark's headline shape)."""
    print("case: full-size 7B block prefill", flush=True)
    _prefill_full(oracle, C2, [0, 1, 2, 31, 32, 63, 64, 127, 128, 255, 256, 1000, 1023, 1024, 2046, 2047])


def test_gqa_long_context_block_prefill_full_size(oracle):
    """d=4096, H=32, Hkv=8, f=14336, base 5e5, B=2, T=8192."""
    print("case: full-size GQA long-context block prefill", flush=True)
    _prefill_full(oracle, C3, [0, 1, 31, 32, 63, 64, 127, 128, 4095, 4096, 8190, 8191])


def test_gqa_decode_step_full_size(oracle):
    """B=64 sequences, cache lengths uniform in [1024, 4096], one new token each."""
    import torch
    cfg = C4
    print("case: full-size GQA decode step", flush=True)
    tc = tfb.Config.of(cfg)
    dh = cfg.d // cfg.n_heads
    lens = synth.integers(cfg.seed, tensor_id("lens"), (cfg.B,), cfg.lens_lo, cfg.lens_hi)
    w32, w = dev_weights(cfg)
    x32, x = dev_x(cfg, cfg.B, 1)
    shape = (cfg.B, cfg.n_kv_heads, cfg.t_max, dh)
    rows = np.arange(cfg.t_max)[None, None, :, None]
    valid = rows < lens[:, None, None, None]
    host, dev = [], []
    for name in ("kc", "vc"):
        f, bits = synth.normal(cfg.seed, tensor_id(name), shape, 1.0, True)
        bits = np.where(valid, bits, np.uint16(0x7FC0))  # NaN beyond each sequence
        f = np.where(valid, f, np.float32(np.nan)).astype(np.float32)
        host.append(f)
        dev.append(to_dev(f, bits))
    pos = torch.from_numpy(lens).cuda()
    rope = tfb.rope_table_init(tc, cfg.t_max)
    out = torch.empty_like(x)
    ws = tfb.workspace(tc, cfg.B, 1)
    tfb.block_decode(tc, w, rope, x, out, tuple(dev), pos, int(lens.max()), ws=ws)
    torch.cuda.synchronize()
    ref = oracle.block_forward(cfg, w32, x32, start=lens, kc=host[0], vc=host[1])
    got = to_np(out)
    assert np.isfinite(got).all()
    assert rel_err(got, ref) <= TOL, rel_err(got, ref)
    gk = widen_cache(dev[0])
    for b in range(0, cfg.B, 7):
        assert cache_ok(cfg, gk[b, :, lens[b]], host[0][b, :, lens[b]])
        assert np.isnan(gk[b, :, lens[b] + 1:]).all()


def test_model_two_layers_full_widths(oracle):
    """The 32-layer model's widths (d=4096, Hkv=8, f=14336, V=32000), B=4,
    T=1024 prompt, with 2 layers so the oracle finishes: prefill logits of the
    last rows, then 3 greedy decode steps teacher-forced with the GPU's ids."""
    import torch
    cfg = C5
    L, V, B, T, steps = 2, cfg.vocab, cfg.B, cfg.T, 3
    print("case: 2-layer model at full widths", flush=True)
    tc = tfb.Config.of(cfg)
    layers32, layers = [], []
    for l in range(L):
        a, b = dev_weights(cfg, layer=l)
        layers32.append(a)
        layers.append(b)
    e32, eb = synth.normal(cfg.seed, tensor_id("embed"), (V, cfg.d), 0.02, True)
    u32, ub = synth.normal(cfg.seed, tensor_id("w_unembed"), (cfg.d, V), 0.02, True)
    g32 = np.ones(cfg.d, np.float32)
    gb, _ = synth.to_bf16(g32)
    h = tfb.ModelHandle(tc, layers, to_dev(e32, eb), to_dev(g32, gb), to_dev(u32, ub))
    t_max = T + steps + 1
    dh = cfg.d // cfg.n_heads
    caches = [(torch.zeros((B, cfg.n_kv_heads, t_max, dh), dtype=torch.bfloat16, device="cuda"),
               torch.zeros((B, cfg.n_kv_heads, t_max, dh), dtype=torch.bfloat16, device="cuda")) for _ in range(L)]
    rope = tfb.rope_table_init(tc, t_max)
    ids = synth.integers(cfg.seed, tensor_id("ids"), (B, T), 0, V - 1)
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    lg = torch.empty((B, 1, V), dtype=torch.float32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    tfb.model_forward(h, rope, torch.from_numpy(ids).cuda(), caches, lens, 0, logits=lg, last_only=True,
                      next_ids=nxt)
    torch.cuda.synchronize()
    okc = [np.zeros((B, cfg.n_kv_heads, t_max, dh), np.float32) for _ in range(L)]
    ovc = [a.copy() for a in okc]
    ref, _ = oracle.model_forward(cfg, L, V, e32, layers32, g32, u32, ids, okc, ovc, rows=[T - 1])
    got = lg.cpu().numpy()
    assert logits_ok(cfg, got, ref), rel_err(got, ref)
    cur = nxt.cpu().numpy()
    assert np.array_equal(cur, np.argmax(got[:, 0], axis=-1))
    for s in range(steps):
        ids1 = cur.reshape(B, 1).astype(np.int32)
        tfb.model_forward(h, rope, torch.from_numpy(ids1).cuda(), caches, lens, T + s, logits=lg, next_ids=nxt)
        torch.cuda.synchronize()
        r1, _ = oracle.model_forward(cfg, L, V, e32, layers32, g32, u32, ids1, okc, ovc,
                                     start=np.full(B, T + s, np.int32))
        g1 = lg.cpu().numpy()
        assert logits_ok(cfg, g1, r1), (s, rel_err(g1, r1))
        cur = nxt.cpu().numpy()
