"""GPU parity of the decoder block against the CPU oracle (same seeded inputs).

Tolerances: max |err| <= 1e-4 rms(oracle) for fp32 storage and 2e-2 rms for
bf16 storage with fp32 accumulation; cache placement and untouched rows are
checked bit for bit.
"""
import numpy as np
import pytest

from tests.conftest import gpu_available
from tests.gpu_util import cache_rows, check, check_cache, dev_weights, dev_x, new_cache, to_np, tol, widen_cache
from tests.inputs import rel_err, small_cfg
from synth.configs import C1

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import transformer_decoder_block_rmsnorm_amd as tfb  # noqa: E402


def _torch():
    import torch
    return torch


def run_prefill_decode(cfg, B, T0, steps, t_max, gains="ones", fold=0):
    """Prefill T0 tokens then `steps` decode steps on the GPU; returns outputs
    [B, T0+steps, d], the caches, and the inputs.  fold: the config's
    fold_norms."""
    torch = _torch()
    tc = tfb.Config.of(cfg, fold)
    w32, w = dev_weights(cfg, gains=gains)
    x32, x = dev_x(cfg, B, T0 + steps)
    rope = tfb.rope_table_init(tc, t_max)
    kc, vc = new_cache(cfg, B, t_max)
    out = torch.empty((B, T0, cfg.d), dtype=x.dtype, device="cuda")
    tfb.block_prefill(tc, w, rope, x[:, :T0].contiguous(), out, cache=(kc, vc))
    outs = [to_np(out)]
    for s in range(steps):
        pos = torch.full((B,), T0 + s, dtype=torch.int32, device="cuda")
        o1 = torch.empty((B, 1, cfg.d), dtype=x.dtype, device="cuda")
        tfb.block_decode(tc, w, rope, x[:, T0 + s:T0 + s + 1].contiguous(), o1, (kc, vc), pos, T0 + s)
        outs.append(to_np(o1))
    torch.cuda.synchronize()
    return np.concatenate(outs, axis=1), kc, vc, w32, x32


def check_against_oracle(oracle, cfg, B, T0, steps, t_max, gains="ones", fold=0):
    got, kc, vc, w32, x32 = run_prefill_decode(cfg, B, T0, steps, t_max, gains, fold)
    dh = cfg.d // cfg.n_heads
    okc = np.full((B, cfg.n_kv_heads, t_max, dh), np.nan, np.float32)
    ovc = okc.copy()
    ref, inter = oracle.block_forward(cfg, w32, x32, kc=okc, vc=ovc, intermediates=True)
    n = T0 + steps
    check("out", got, ref, tol(cfg))
    gk, gv = widen_cache(kc), widen_cache(vc)
    check_cache("k cache", cfg, gk[:, :, :n], cache_rows(inter["k_pre"], cfg.n_kv_heads))
    check_cache("v cache", cfg, gv[:, :, :n], cache_rows(inter["v_pre"], cfg.n_kv_heads))
    # rows never written keep their NaN sentinel, bit for bit
    assert np.isnan(gk[:, :, n:]).all() and np.isnan(gv[:, :, n:]).all()
    assert np.isfinite(gk[:, :, :n]).all() and np.isfinite(got).all()
    return got, ref


def test_tiny_fp32_block_prefill_then_decode(oracle):
    """The tiny fp32 workload: d=64, H=4, Hkv=2, f=192, T=16 then 4 decode steps."""
    print("case: tiny fp32 prefill 16 + 4 decode", flush=True)
    check_against_oracle(oracle, C1, 1, 16, 4, 32)


def test_fp32_random_gains_and_batch(oracle):
    cfg = small_cfg(d=128, H=4, Hkv=1, f=256, number=81)
    print("case: fp32 d=128 MQA B=3 T=37+3 random gains", flush=True)
    check_against_oracle(oracle, cfg, 3, 37, 3, 48, gains="random")


@pytest.mark.parametrize("d,H,Hkv,f", [
    (512, 2, 1, 256),   # dh = 256, the widest head the fp32 path takes
    (96, 4, 2, 64),     # dh = 24: not a multiple of the 64 lanes
])
def test_fp32_head_widths(oracle, d, H, Hkv, f):
    """fp32 storage runs the row-wise attention for any even head width up
    to 256: prefill then decode steps against the oracle."""
    cfg = small_cfg(d=d, H=H, Hkv=Hkv, f=f, number=84)
    print("case: fp32 head width", d // H, flush=True)
    check_against_oracle(oracle, cfg, 2, 70, 3, 80)


@pytest.mark.parametrize("shape", [
    dict(d=512, H=4, Hkv=2, f=1024, B=2, T0=300, steps=2),   # GQA, ragged rows (300 = 2*128 + 44)
    dict(d=256, H=2, Hkv=2, f=768, B=1, T0=129, steps=2),    # MHA, one row past a tile
    dict(d=512, H=8, Hkv=1, f=512, B=2, T0=70, steps=3),     # MQA, dh = 64
    dict(d=1024, H=8, Hkv=2, f=2048, B=1, T0=256, steps=1),  # full tiles
    # gate-up on 256x128 tiles with W1|W3 pairing (2048 rows, 2f = 4096: 128
    # tiles of 256x256 would leave half a round, 256 tiles of 256x128 fill one)
    dict(d=768, H=6, Hkv=2, f=2048, B=1, T0=2048, steps=1),
    dict(d=2048, H=32, Hkv=2, f=1024, B=2, T0=150, steps=2),  # 16 query heads per KV head, dh = 64
    dict(d=4096, H=32, Hkv=2, f=1024, B=1, T0=130, steps=2),  # 16 query heads per KV head, dh = 128
])
def test_bf16_block_prefill_then_decode(oracle, shape):
    cfg = small_cfg(d=shape["d"], H=shape["H"], Hkv=shape["Hkv"], f=shape["f"], dtype="bf16", number=82)
    print("case: bf16", shape, flush=True)
    check_against_oracle(oracle, cfg, shape["B"], shape["T0"], shape["steps"], shape["T0"] + shape["steps"] + 5)


@pytest.mark.parametrize("shape", [
    dict(d=512, H=4, Hkv=2, f=1024, B=2, T0=300, steps=2),    # 128x128 tiles, ragged last row tile
    dict(d=768, H=6, Hkv=2, f=2048, B=1, T0=2048, steps=1),   # gate-up on 256x128 tiles (W1|W3 pairs)
    dict(d=1024, H=8, Hkv=2, f=4096, B=1, T0=4096, steps=1),  # gate-up on 256x256 tiles
    # d = 320 is not a multiple of the 128-column tiles: the last column
    # tile of Wo (and of the gate-up's K range) ends past the row
    dict(d=320, H=5, Hkv=1, f=640, B=1, T0=300, steps=1),
])
def test_bf16_folded_norms_prefill_then_decode(oracle, shape):
    """fold_norms: RMSNorm2 folded into the Wo epilogue and the gate-up GEMM
    in prefill (the decode steps, 64 rows or fewer, run as before)."""
    cfg = small_cfg(d=shape["d"], H=shape["H"], Hkv=shape["Hkv"], f=shape["f"], dtype="bf16", number=83)
    print("case: bf16 folded norms", shape, flush=True)
    check_against_oracle(oracle, cfg, shape["B"], shape["T0"], shape["steps"], shape["T0"] + shape["steps"] + 5,
                         gains="random", fold=1)


@pytest.mark.parametrize("T0", [1, 2, 63, 64, 65, 127, 128, 129, 192])
def test_bf16_prefill_lengths_around_key_tiles(oracle, T0):
    """Prefill lengths at and around the 64-key tiles of the flash kernel:
    one tile, a partial second tile, whole tiles, and (with few workgroups)
    the two wave groups splitting one to four tiles, where the upper group
    may have none; every output and cache row against the oracle."""
    cfg = small_cfg(d=256, H=4, Hkv=1, f=512, dtype="bf16", number=131)
    print("case: bf16 prefill length", T0, flush=True)
    check_against_oracle(oracle, cfg, 2, T0, 1, T0 + 4)


@pytest.mark.parametrize("d,H,Hkv,B,T0,W", [
    (256, 4, 2, 80, 200, 0),    # dh 64, two heads per KV head: 4 x 80 x 2 = 640 blocks of 64 rows
    (256, 4, 2, 80, 200, 70),   # the same with a window
    (256, 2, 1, 160, 200, 0),   # dh 128: 4 x 160 = 640 blocks
    (512, 8, 2, 40, 201, 0),    # four heads per KV head: blocks of 32 rows, 7 x 40 x 2 = 560
])
def test_large_grid_prefill_one_wave_group_per_workgroup(oracle, d, H, Hkv, B, T0, W):
    """Grids larger than two workgroups per CU run the flash kernel with one
    wave group per workgroup (the long-context form, whose full-size test
    only checks sampled rows): every output row and cache row against the
    oracle, at ragged lengths, then one decode step."""
    cfg = small_cfg(d=d, H=H, Hkv=Hkv, f=2 * d, dtype="bf16", number=112, window=W)
    print("case: large-grid prefill", d, H, Hkv, B, T0, W, flush=True)
    check_against_oracle(oracle, cfg, B, T0, 1, T0 + 8)


def test_bf16_random_gains_rope_base_500k(oracle):
    cfg = small_cfg(d=512, H=4, Hkv=1, f=1536, dtype="bf16", base=500000.0, number=83)
    print("case: bf16 random gains base 5e5", flush=True)
    check_against_oracle(oracle, cfg, 2, 200, 2, 210, gains="random")


def test_prefill_without_cache_matches(oracle):
    torch = _torch()
    cfg = small_cfg(d=512, H=4, Hkv=2, f=1024, dtype="bf16", number=84)
    tc = tfb.Config.of(cfg)
    w32, w = dev_weights(cfg)
    x32, x = dev_x(cfg, 2, 150)
    rope = tfb.rope_table_init(tc, 150)
    out = torch.empty_like(x)
    tfb.block_prefill(tc, w, rope, x, out)
    torch.cuda.synchronize()
    check("out", to_np(out), oracle.block_forward(cfg, w32, x32), 2e-2)


def test_out_may_alias_x(oracle):
    torch = _torch()
    cfg = small_cfg(d=512, H=4, Hkv=2, f=1024, dtype="bf16", number=85)
    tc = tfb.Config.of(cfg)
    w32, w = dev_weights(cfg)
    x32, x = dev_x(cfg, 1, 64)
    rope = tfb.rope_table_init(tc, 64)
    tfb.block_prefill(tc, w, rope, x, x)
    torch.cuda.synchronize()
    check("out", to_np(x), oracle.block_forward(cfg, w32, x32), 2e-2)


def test_causal_mask_placement_bitwise():
    """Rows <= i must not change, bit for bit, when rows > i change."""
    torch = _torch()
    for cfg in (C1, small_cfg(d=512, H=4, Hkv=2, f=1024, dtype="bf16", number=86)):
        tc = tfb.Config.of(cfg)
        _, w = dev_weights(cfg)
        _, x = dev_x(cfg, 2, 200 if cfg.dtype == "bf16" else 16)
        T = x.shape[1]
        rope = tfb.rope_table_init(tc, T)
        o1 = torch.empty_like(x)
        tfb.block_prefill(tc, w, rope, x, o1)
        for i in (0, T // 3, T - 2):
            x2 = x.clone()
            x2[:, i + 1:] = 37.0
            o2 = torch.empty_like(x)
            tfb.block_prefill(tc, w, rope, x2, o2)
            torch.cuda.synchronize()
            assert torch.equal(o1[:, :i + 1], o2[:, :i + 1]), (cfg.dtype, i)
            assert not torch.equal(o1[:, i + 1:], o2[:, i + 1:])


def test_deterministic_repeat_bitwise():
    torch = _torch()
    cfg = small_cfg(d=512, H=4, Hkv=2, f=1024, dtype="bf16", number=87)
    tc = tfb.Config.of(cfg)
    _, w = dev_weights(cfg)
    _, x = dev_x(cfg, 2, 333)
    rope = tfb.rope_table_init(tc, 333)
    outs = []
    for _ in range(2):
        kc, vc = new_cache(cfg, 2, 333, 0.0)
        o = torch.empty_like(x)
        tfb.block_prefill(tc, w, rope, x, o, cache=(kc, vc))
        outs.append((o, kc, vc))
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


def test_gqa_equals_mha_with_repeated_kv():
    """GQA with Hkv KV heads equals MHA whose Wk and Wv repeat each KV head's
    columns H/Hkv times consecutively ([TIR] Code, the GQA index), bit for bit.
    128 rows: both run the tiled GEMMs without a k split, and the flash kernel
    splits every query's key tiles the same way for both head layouts."""
    torch = _torch()
    for dtype in ("f32", "bf16"):
        d, f = (64, 192) if dtype == "f32" else (512, 1024)
        cfg = small_cfg(d=d, H=4, Hkv=2, f=f, dtype=dtype, number=88)
        cfg_m = small_cfg(d=d, H=4, Hkv=4, f=f, dtype=dtype, number=88)
        _, w = dev_weights(cfg)
        _, x = dev_x(cfg, 1, 128)
        dh = d // 4
        cols = torch.cat([torch.arange(g * dh, (g + 1) * dh) for g in range(2) for _ in range(2)]).cuda()
        wm = dict(w, wk=w["wk"][:, cols].contiguous(), wv=w["wv"][:, cols].contiguous())
        outs = []
        for c, ww in ((cfg, w), (cfg_m, wm)):
            tc = tfb.Config.of(c)
            rope = tfb.rope_table_init(tc, 128)
            o = torch.empty_like(x)
            tfb.block_prefill(tc, ww, rope, x, o)
            outs.append(o)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), (dtype, (outs[0].float() - outs[1].float()).abs().max().item())


def test_decode_over_nan_tail_and_ragged_positions(oracle):
    """Sequences at different positions decode together; cache rows beyond
    pos[b] hold NaN and must never influence the result.  With few
    (sequence, KV head) pairs the attention kernel builds q and the new cache
    rows from the QKV partials, and the Wo GEMM merges the attention's chunk
    partials, so q and att (left in the workspace) and both appended rows are
    checked too."""
    torch = _torch()
    for cfg in (C1, small_cfg(d=512, H=4, Hkv=1, f=1024, dtype="bf16", number=89)):
        tc = tfb.Config.of(cfg)
        B, t_max = 3, 80
        w32, w = dev_weights(cfg)
        x32, x = dev_x(cfg, B, t_max)
        lens = [5, 33, 71]
        rope = tfb.rope_table_init(tc, t_max)
        kc, vc = new_cache(cfg, B, t_max)
        dh = cfg.d // cfg.n_heads
        okc = np.full((B, cfg.n_kv_heads, t_max, dh), np.nan, np.float32)
        ovc = okc.copy()
        for b in range(B):  # prefill each sequence to its own length
            kb, vb = new_cache(cfg, 1, t_max)
            ob = torch.empty((1, lens[b], cfg.d), dtype=x.dtype, device="cuda")
            tfb.block_prefill(tc, w, rope, x[b:b + 1, :lens[b]].contiguous(), ob, cache=(kb, vb))
            kc[b].copy_(kb[0])
            vc[b].copy_(vb[0])
            k1, v1 = okc[b:b + 1].copy(), ovc[b:b + 1].copy()
            oracle.block_forward(cfg, w32, x32[b:b + 1, :lens[b]], kc=k1, vc=v1)
            okc[b], ovc[b] = k1[0], v1[0]
        pos = torch.tensor(lens, dtype=torch.int32, device="cuda")
        xd = torch.stack([x[b, lens[b]] for b in range(B)])[:, None].contiguous()
        o = torch.empty_like(xd)
        ws = tfb.workspace(tc, B, 1)
        tfb.block_decode(tc, w, rope, xd, o, (kc, vc), pos, max(lens), ws=ws)
        torch.cuda.synchronize()
        xd32 = np.stack([x32[b, lens[b]] for b in range(B)])[:, None]
        ref, inter = oracle.block_forward(cfg, w32, xd32, start=np.array(lens, np.int32), kc=okc, vc=ovc,
                                          intermediates=True)
        got = to_np(o)
        assert np.isfinite(got).all()
        check("out", got, ref, tol(cfg))
        gk = widen_cache(kc)
        for b in range(B):
            assert np.isnan(gk[b, :, lens[b] + 1:]).all()
        check_cache("appended k rows", cfg, np.stack([gk[b, :, lens[b]] for b in range(B)]),
                    cache_rows(inter["k_pre"], cfg.n_kv_heads)[:, :, 0])
        gv = widen_cache(vc)
        check_cache("appended v rows", cfg, np.stack([gv[b, :, lens[b]] for b in range(B)]),
                    cache_rows(inter["v_pre"], cfg.n_kv_heads)[:, :, 0])
        q = to_np(tfb.workspace_view(tc, ws, B, 1, "q")).reshape(B, 1, cfg.d)
        check("q (after RoPE)", q, inter["q_pre"], tol(cfg))
        att = to_np(tfb.workspace_view(tc, ws, B, 1, "att"))
        check("att (head outputs)", att, inter["att_pre"], tol(cfg))


def test_kv_append_bit_exact(oracle):
    torch = _torch()
    for cfg in (C1, small_cfg(d=512, H=4, Hkv=2, f=1024, dtype="bf16", number=90)):
        tc = tfb.Config.of(cfg)
        B, t_max, n = 3, 40, 5
        dh = cfg.d // cfg.n_heads
        import synth
        kf, kb = synth.normal(cfg.seed, 11, (B, n, cfg.n_kv_heads, dh), 1.0, cfg.dtype == "bf16")
        vf, vb = synth.normal(cfg.seed, 12, (B, n, cfg.n_kv_heads, dh), 1.0, cfg.dtype == "bf16")
        from tests.gpu_util import to_dev
        k_new, v_new = to_dev(kf, kb), to_dev(vf, vb)
        start = np.array([0, 17, 35], np.int32)
        kc, vc = new_cache(cfg, B, t_max)
        tfb.kv_append(tc, (kc, vc), k_new, v_new, torch.from_numpy(start).cuda(), int(start.max()))
        torch.cuda.synchronize()
        okc = np.full((B, cfg.n_kv_heads, t_max, dh), np.nan, np.float32)
        ovc = okc.copy()
        oracle.kv_append(okc, ovc, kf, vf, start)
        g = widen_cache(kc)
        same = (g == okc) | (np.isnan(g) & np.isnan(okc))
        assert same.all()
        g = widen_cache(vc)
        assert ((g == ovc) | (np.isnan(g) & np.isnan(ovc))).all()


def test_kv_append_fp32_narrow_heads_bit_exact():
    """fp32 storage with a head width that is not a multiple of 4 (dh = 6):
    every value lands at cache[b, g, start[b] + t, e], nothing else changes.
    Each value encodes its own (b, t, g, e)."""
    torch = _torch()
    cfg = small_cfg(d=12, H=2, Hkv=1, f=16, number=92)
    tc = tfb.Config.of(cfg)
    B, n, Hkv, dh, t_max = 3, 4, 1, 6, 13
    b, t, g, e = np.meshgrid(np.arange(B), np.arange(n), np.arange(Hkv), np.arange(dh), indexing="ij")
    code = (1000 * b + 100 * t + 10 * g + e + 1).astype(np.float32)
    start = np.array([0, 5, 9], np.int32)
    kc, vc = new_cache(cfg, B, t_max, -7.0)
    tfb.kv_append(tc, (kc, vc), torch.from_numpy(code).cuda(), torch.from_numpy(-code).cuda(),
                  torch.from_numpy(start).cuda(), int(start.max()))
    torch.cuda.synchronize()
    want = np.full((B, Hkv, t_max, dh), -7.0, np.float32)
    want_v = want.copy()
    for bb in range(B):
        for tt in range(n):
            want[bb, :, start[bb] + tt] = code[bb, tt]
            want_v[bb, :, start[bb] + tt] = -code[bb, tt]
    assert np.array_equal(widen_cache(kc), want) and np.array_equal(widen_cache(vc), want_v)


def test_rope_table_matches_oracle(oracle):
    torch = _torch()
    for base, dh in ((10000.0, 16), (500000.0, 128), (10000.0, 64)):
        cfg = small_cfg(d=dh * 4, H=4, Hkv=2, f=64, base=base)
        tab = tfb.rope_table_init(tfb.Config.of(cfg), 4096)
        torch.cuda.synchronize()
        c, s = oracle.rope_table(4096, dh, base)
        g = tab.cpu().numpy()
        # fp64 angle rounded to fp32 on both sides: at most one ulp apart
        assert np.max(np.abs(g[..., 0] - c)) <= 6e-8 and np.max(np.abs(g[..., 1] - s)) <= 6e-8


@pytest.mark.parametrize("lens,d,H,Hkv", [
    ([700, 1500, 3000, 1], 512, 4, 1),      # several 512-key chunks, G = 4, a length-1 sequence
    ([40000], 256, 2, 2),                   # more chunks than the partial buffer holds: chunk growth
    ([5000, 2047], 512, 8, 2),              # dh = 64, G = 4
])
def test_decode_long_cache_chunks(oracle, lens, d, H, Hkv):
    """Decode against caches filled with seeded post-RoPE keys and values."""
    torch = _torch()
    import synth
    from tests.gpu_util import to_dev
    cfg = small_cfg(d=d, H=H, Hkv=Hkv, f=2 * d, dtype="bf16", base=500000.0, number=91)
    tc = tfb.Config.of(cfg)
    B, dh = len(lens), d // H
    t_max = max(lens) + 8
    shape = (B, Hkv, t_max, dh)
    kf, kb = synth.normal(cfg.seed, 11, shape, 1.0, True)
    vf, vb = synth.normal(cfg.seed, 12, shape, 1.0, True)
    rows = np.arange(t_max)[None, None, :, None]
    valid = rows < np.array(lens)[:, None, None, None]
    kb = np.where(valid, kb, np.uint16(0x7FC0))  # NaN beyond each sequence
    vb = np.where(valid, vb, np.uint16(0x7FC0))
    kf = np.where(valid, kf, np.nan).astype(np.float32)
    vf = np.where(valid, vf, np.nan).astype(np.float32)
    kc, vc = to_dev(kf, kb), to_dev(vf, vb)
    w32, w = dev_weights(cfg)
    x32, x = dev_x(cfg, B, 1)
    rope = tfb.rope_table_init(tc, t_max)
    pos = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o = torch.empty_like(x)
    print("case: decode lens", lens, flush=True)
    tfb.block_decode(tc, w, rope, x, o, (kc, vc), pos, max(lens))
    torch.cuda.synchronize()
    okc, ovc = kf.copy(), vf.copy()
    ref = oracle.block_forward(cfg, w32, x32, start=np.array(lens, np.int32), kc=okc, vc=ovc)
    got = to_np(o)
    assert np.isfinite(got).all()
    check("out", got, ref, 2e-2)


@pytest.mark.parametrize("B,d,H,Hkv,f", [
    (20, 512, 4, 2, 1024),     # 17-32 rows per weight stream: two 16-row tiles
    (40, 512, 8, 2, 1536),     # 33-48 rows: three 16-row tiles, dh = 64
    (64, 1024, 8, 8, 2048),    # the full 64 rows, 128-column weight blocks split along k
    (80, 512, 4, 2, 1024),     # more rows than a weight stream takes: the tiled GEMMs, one ragged 128-row tile
    (130, 256, 2, 1, 512),     # two row tiles, the second holding 2 rows; dh = 128, MQA
    (24, 2048, 16, 2, 1024),   # 8 query heads per KV head at dh = 128
    (100, 2048, 16, 2, 1024),  # the same heads through the tiled GEMMs, with fold_norms
])
def test_decode_batch_sizes(oracle, B, d, H, Hkv, f):
    """Decode of B sequences at spread positions: up to 64 rows the
    weight-streaming GEMMs take B rows (every row-tile count of the kernel),
    beyond that the tiled GEMMs with a ragged last row tile; all against the
    oracle."""
    torch = _torch()
    import synth
    from tests.gpu_util import to_dev
    cfg = small_cfg(d=d, H=H, Hkv=Hkv, f=f, dtype="bf16", base=500000.0, number=93)
    tc = tfb.Config.of(cfg, 1 if B == 100 else 0)
    dh = d // H
    lens = [int(v) for v in synth.integers(cfg.seed, 13, (B,), 1, 200)]
    t_max = max(lens) + 4
    shape = (B, Hkv, t_max, dh)
    kf, kb = synth.normal(cfg.seed, 11, shape, 1.0, True)
    vf, vb = synth.normal(cfg.seed, 12, shape, 1.0, True)
    kc, vc = to_dev(kf, kb), to_dev(vf, vb)
    w32, w = dev_weights(cfg)
    x32, x = dev_x(cfg, B, 1)
    rope = tfb.rope_table_init(tc, t_max)
    pos = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o = torch.empty_like(x)
    print("case: decode batch", B, d, H, Hkv, f, flush=True)
    tfb.block_decode(tc, w, rope, x, o, (kc, vc), pos, max(lens))
    torch.cuda.synchronize()
    okc, ovc = kf.copy(), vf.copy()
    ref, inter = oracle.block_forward(cfg, w32, x32, start=np.array(lens, np.int32), kc=okc, vc=ovc,
                                      intermediates=True)
    got = to_np(o)
    assert np.isfinite(got).all()
    check("out", got, ref, tol(cfg))
    gk, gv = widen_cache(kc), widen_cache(vc)
    check_cache("appended k rows", cfg, np.stack([gk[b, :, lens[b]] for b in range(B)]),
                cache_rows(inter["k_pre"], Hkv)[:, :, 0])
    check_cache("appended v rows", cfg, np.stack([gv[b, :, lens[b]] for b in range(B)]),
                cache_rows(inter["v_pre"], Hkv)[:, :, 0])


@pytest.mark.parametrize("dtype,chunks,fold", [("f32", [5, 7, 4], 0), ("bf16", [100, 37, 129, 1], 0),
                                              ("bf16", [64, 64, 64], 0), ("bf16", [100, 37, 129, 1], 1)])
def test_chunked_prefill_matches_full_prefill(oracle, dtype, chunks, fold):
    """Prefill in chunks at start positions 0, c0, c0+c1, ... into one cache
    (the causal diagonal shifts by the start position); fold: the config's
    fold_norms (chunks of more than 64 rows fold RMSNorm2)."""
    torch = _torch()
    d, f = (64, 192) if dtype == "f32" else (512, 1024)
    cfg = small_cfg(d=d, H=4, Hkv=2, f=f, dtype=dtype, number=97)
    tc = tfb.Config.of(cfg, fold)
    w32, w = dev_weights(cfg)
    T = sum(chunks)
    x32, x = dev_x(cfg, 2, T)
    t_max = T + 3
    rope = tfb.rope_table_init(tc, t_max)
    kc, vc = new_cache(cfg, 2, t_max)
    outs, s0 = [], 0
    print("case: chunked prefill", dtype, chunks, "fold_norms=%d" % fold, flush=True)
    for c in chunks:
        o = torch.empty((2, c, cfg.d), dtype=x.dtype, device="cuda")
        tfb.block_prefill(tc, w, rope, x[:, s0:s0 + c].contiguous(), o, start_pos=s0, cache=(kc, vc))
        outs.append(to_np(o))
        s0 += c
    torch.cuda.synchronize()
    got = np.concatenate(outs, axis=1)
    ref = oracle.block_forward(cfg, w32, x32)
    check("out", got, ref, tol(cfg))
    assert np.isnan(widen_cache(kc)[:, :, T:]).all()


# ---- sliding-window attention (pidoku "The Transformer", Sliding-window attention)
@pytest.mark.parametrize("dtype,d,H,Hkv,T,W", [
    ("f32", 64, 4, 2, 40, 7),
    ("bf16", 256, 4, 2, 200, 1),     # dh = 64; each query sees only itself
    ("bf16", 256, 4, 2, 200, 37),    # window edge inside tiles
    ("bf16", 512, 4, 1, 300, 128),   # dh = 128, MQA, window = two key tiles
    ("bf16", 512, 4, 4, 130, 500),   # window longer than the sequence
])
def test_sliding_window_prefill(oracle, dtype, d, H, Hkv, T, W):
    torch = _torch()
    cfg = small_cfg(d=d, H=H, Hkv=Hkv, f=2 * d, dtype=dtype, number=110, window=W)
    tc = tfb.Config.of(cfg)
    w32, w = dev_weights(cfg)
    x32, x = dev_x(cfg, 2, T)
    rope = tfb.rope_table_init(tc, T)
    kc, vc = new_cache(cfg, 2, T)
    out = torch.empty_like(x)
    print("case: window prefill", dtype, d, H, Hkv, T, W, flush=True)
    tfb.block_prefill(tc, w, rope, x, out, cache=(kc, vc))
    torch.cuda.synchronize()
    okc = np.zeros((2, Hkv, T, d // H), np.float32)
    ovc = okc.copy()
    ref, inter = oracle.block_forward(cfg, w32, x32, kc=okc, vc=ovc, intermediates=True)
    check("out", to_np(out), ref, tol(cfg))
    check_cache("k cache", cfg, widen_cache(kc), cache_rows(inter["k_pre"], Hkv))


def test_sliding_window_chunked_prefill_and_decode(oracle):
    """Chunks and decode steps past the window: rows below every query's
    window are NaN in the cache and must never be read."""
    torch = _torch()
    cfg = small_cfg(d=256, H=4, Hkv=2, f=512, dtype="bf16", number=111, window=50)
    tc = tfb.Config.of(cfg)
    w32, w = dev_weights(cfg)
    T, steps = 160, 4
    x32, x = dev_x(cfg, 2, T + steps)
    t_max = T + steps
    rope = tfb.rope_table_init(tc, t_max)
    kc, vc = new_cache(cfg, 2, t_max)
    print("case: window chunked prefill + decode", flush=True)
    o1 = torch.empty((2, 100, cfg.d), dtype=x.dtype, device="cuda")
    tfb.block_prefill(tc, w, rope, x[:, :100].contiguous(), o1, cache=(kc, vc))
    torch.cuda.synchronize()
    # poison rows 0..49: the chunk below starts at 100, so its earliest window starts at 51
    kc[:, :, :50] = float("nan")
    vc[:, :, :50] = float("nan")
    o2 = torch.empty((2, 60, cfg.d), dtype=x.dtype, device="cuda")
    tfb.block_prefill(tc, w, rope, x[:, 100:T].contiguous(), o2, start_pos=100, cache=(kc, vc))
    dec = []
    for s in range(steps):
        o = torch.empty((2, 1, cfg.d), dtype=x.dtype, device="cuda")
        pos = torch.full((2,), T + s, dtype=torch.int32, device="cuda")
        tfb.block_decode(tc, w, rope, x[:, T + s:T + s + 1].contiguous(), o, (kc, vc), pos, T + s)
        dec.append(to_np(o))
    torch.cuda.synchronize()
    got = np.concatenate([to_np(o1), to_np(o2)] + dec, axis=1)
    ref = oracle.block_forward(cfg, w32, x32)
    assert np.isfinite(got).all()
    check("out", got, ref, tol(cfg))


@pytest.mark.parametrize("lens,W", [([1100, 4000, 2500, 700], 1000), ([3000, 513], 4096), ([2048, 2049], 1)])
def test_sliding_window_decode_long_cache(oracle, lens, W):
    """Split-KV decode over the window of long caches (NaN below the window
    would poison the result if read)."""
    torch = _torch()
    import synth
    from tests.gpu_util import to_dev
    cfg = small_cfg(d=512, H=4, Hkv=1, f=1024, dtype="bf16", base=500000.0, number=112, window=W)
    tc = tfb.Config.of(cfg)
    B, dh = len(lens), cfg.head_dim
    t_max = max(lens) + 8
    shape = (B, 1, t_max, dh)
    kf, kb = synth.normal(cfg.seed, 11, shape, 1.0, True)
    vf, vb = synth.normal(cfg.seed, 12, shape, 1.0, True)
    rows = np.arange(t_max)[None, None, :, None]
    L = np.array(lens)[:, None, None, None]
    valid = (rows < L) & (rows >= L + 1 - W)  # the window of the new token at position len
    kb = np.where(valid, kb, np.uint16(0x7FC0))
    vb = np.where(valid, vb, np.uint16(0x7FC0))
    kf = np.where(valid, kf, np.nan).astype(np.float32)
    vf = np.where(valid, vf, np.nan).astype(np.float32)
    kc, vc = to_dev(kf, kb), to_dev(vf, vb)
    w32, w = dev_weights(cfg)
    x32, x = dev_x(cfg, B, 1)
    rope = tfb.rope_table_init(tc, t_max)
    pos = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o = torch.empty_like(x)
    print("case: window decode", lens, W, flush=True)
    tfb.block_decode(tc, w, rope, x, o, (kc, vc), pos, max(lens))
    torch.cuda.synchronize()
    okc, ovc = kf.copy(), vf.copy()
    ref = oracle.block_forward(cfg, w32, x32, start=np.array(lens, np.int32), kc=okc, vc=ovc)
    got = to_np(o)
    assert np.isfinite(got).all() and np.isfinite(ref).all()
    check("out", got, ref, 2e-2)


# ---- variable-length batched prefill (tirogla "Transformer block", Pitfalls:
# pad tokens must not be attended to in batched prefill)
@pytest.mark.parametrize("dtype,d,H,Hkv,W,fold", [("f32", 64, 4, 2, 0, 0), ("bf16", 512, 4, 2, 0, 0),
                                                   ("bf16", 256, 4, 1, 30, 0), ("bf16", 512, 4, 2, 0, 1)])
def test_varlen_prefill_matches_per_sequence(oracle, dtype, d, H, Hkv, W, fold):
    """Three right-padded sequences with their own starts and lengths (one
    empty) in one call; each real row must match that sequence alone (fold:
    the config's fold_norms)."""
    torch = _torch()
    from tests.gpu_util import to_dev
    cfg = small_cfg(d=d, H=H, Hkv=Hkv, f=2 * d, dtype=dtype, number=120, window=W)
    tc = tfb.Config.of(cfg, fold)
    w32, w = dev_weights(cfg)
    B, T = 3, 100
    starts, lens = np.array([0, 20, 64], np.int32), np.array([100, 37, 0], np.int32)
    t_max = int((starts + lens).max()) + 5
    dh = d // H
    xall32, xall = dev_x(cfg, B, int(starts.max()) + T)
    # earlier rows of each sequence: keys and values from the oracle, so both
    # sides start from the same cache
    okc = np.full((B, Hkv, t_max, dh), np.nan, np.float32)
    ovc = okc.copy()
    for b in range(B):
        if starts[b]:
            kb, vb = okc[b:b + 1].copy(), ovc[b:b + 1].copy()
            oracle.block_forward(cfg, w32, xall32[b:b + 1, :starts[b]], kc=kb, vc=vb)
            okc[b], ovc[b] = kb[0], vb[0]
    bits = None
    if dtype == "bf16":
        import synth
        bits = [synth.to_bf16(a)[0] for a in (okc, ovc)]
    kc = to_dev(okc, None if bits is None else bits[0])
    vc = to_dev(ovc, None if bits is None else bits[1])
    x32 = np.zeros((B, T, d), np.float32)
    for b in range(B):
        x32[b] = xall32[b, starts[b]:starts[b] + T]
    x = torch.stack([xall[b, starts[b]:starts[b] + T] for b in range(B)]).contiguous()
    rope = tfb.rope_table_init(tc, t_max)
    out = torch.empty_like(x)
    st = torch.from_numpy(starts).cuda()
    ln = torch.from_numpy(lens).cuda()
    print("case: varlen prefill", dtype, d, H, Hkv, W, flush=True)
    tfb.block_prefill_varlen(tc, w, rope, x, out, st, ln, int((starts + lens).max()), (kc, vc))
    torch.cuda.synchronize()
    got, gk = to_np(out), widen_cache(kc)
    for b in range(B):
        n = int(lens[b])
        kb, vb = okc[b:b + 1].copy(), ovc[b:b + 1].copy()
        if n:
            ref, inter = oracle.block_forward(cfg, w32, x32[b:b + 1, :n], start=[int(starts[b])], kc=kb, vc=vb,
                                              intermediates=True)
            check("out seq %d" % b, got[b, :n], ref[0], tol(cfg))
            s0 = int(starts[b])
            check_cache("k rows seq %d" % b, cfg, gk[b, :, s0:s0 + n], cache_rows(inter["k_pre"], Hkv)[0])
        # padding rows write nothing; earlier rows are untouched
        assert np.isnan(gk[b, :, int(starts[b] + lens[b]):]).all()
        assert np.array_equal(gk[b, :, :int(starts[b])], okc[b, :, :int(starts[b])])


# ---- paged KV cache (tirogla "Transformer block", Implementation notes: a
# cache allocated in fixed-size blocks per sequence)
@pytest.mark.parametrize("dtype,bs,W,fold", [("bf16", 16, 0, 0), ("bf16", 64, 0, 0), ("bf16", 256, 40, 0),
                                              ("f32", 8, 0, 0), ("bf16", 64, 0, 1)])
def test_paged_cache_matches_contiguous_bitwise(oracle, dtype, bs, W, fold):
    """Prefill in two chunks, then decode steps, through a block table that
    scatters each sequence over a shuffled pool: outputs and cached rows must
    equal the contiguous cache's bit for bit (only the addressing differs;
    fold: both with the config's fold_norms)."""
    torch = _torch()
    d, H, Hkv = (64, 4, 2) if dtype == "f32" else (256, 4, 2)
    cfg = small_cfg(d=d, H=H, Hkv=Hkv, f=2 * d, dtype=dtype, number=130, window=W)
    tc = tfb.Config.of(cfg, fold)
    w32, w = dev_weights(cfg)
    B, T1, T2, steps = 2, 100, 50, 3
    T = T1 + T2 + steps
    x32, x = dev_x(cfg, B, T)
    max_blocks = (T + bs - 1) // bs + 1
    t_max = max_blocks * bs
    n_blocks = B * max_blocks + 3
    perm = np.random.default_rng(bs).permutation(n_blocks)[:B * max_blocks].reshape(B, max_blocks)
    table = torch.from_numpy(perm.astype(np.int32)).cuda()
    dh = d // H
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kp = torch.full((n_blocks, Hkv, bs, dh), float("nan"), dtype=tdt, device="cuda")
    vp = kp.clone()
    kc, vc = new_cache(cfg, B, t_max)
    rope = tfb.rope_table_init(tc, t_max)
    print("case: paged", dtype, bs, W, "fold_norms=%d" % fold, flush=True)
    outs_c, outs_p = [], []
    for s0, n in ((0, T1), (T1, T2)):
        xi = x[:, s0:s0 + n].contiguous()
        oc, op = torch.empty_like(xi), torch.empty_like(xi)
        tfb.block_prefill(tc, w, rope, xi, oc, start_pos=s0, cache=(kc, vc))
        tfb.block_prefill_paged(tc, w, rope, xi, op, (kp, vp, table, bs), start_pos=s0)
        outs_c.append(oc)
        outs_p.append(op)
    for s in range(steps):
        p = T1 + T2 + s
        xi = x[:, p:p + 1].contiguous()
        oc, op = torch.empty_like(xi), torch.empty_like(xi)
        pos = torch.full((B,), p, dtype=torch.int32, device="cuda")
        tfb.block_decode(tc, w, rope, xi, oc, (kc, vc), pos, p)
        tfb.block_decode_paged(tc, w, rope, xi, op, (kp, vp, table, bs), pos, p)
        outs_c.append(oc)
        outs_p.append(op)
    torch.cuda.synchronize()
    got_c = np.concatenate([to_np(o) for o in outs_c], axis=1)
    got_p = np.concatenate([to_np(o) for o in outs_p], axis=1)
    assert np.array_equal(got_p, got_c)
    ref = oracle.block_forward(cfg, w32, x32)
    check("out", got_p, ref, tol(cfg))
    gk, gkp = widen_cache(kc), widen_cache(kp)
    gv, gvp = widen_cache(vc), widen_cache(vp)
    for b in range(B):
        for p in range(T):
            blk, r = perm[b, p // bs], p % bs
            assert np.array_equal(gkp[blk, :, r], gk[b, :, p]) and np.array_equal(gvp[blk, :, r], gv[b, :, p])
    # pool blocks no sequence owns are untouched
    free = np.setdiff1d(np.arange(n_blocks), perm.ravel())
    assert np.isnan(gkp[free]).all()


# ---- bounded sliding-window cache (pidoku "The Transformer", Sliding-window
# attention: with a window of W keys the KV cache is capped at W)
def _ring_run(cfg, x, chunks, steps, caches, paged=None):
    """Prefill in chunks then decode steps through one set of caches (either
    (k, v[, ring]) tuples or a paged tuple); returns the outputs."""
    torch = _torch()
    tc = tfb.Config.of(cfg)
    B = x.shape[0]
    T = sum(chunks) + steps
    rope = tfb.rope_table_init(tc, T)
    outs, s0 = [], 0
    for c in chunks:
        xi = x[:, s0:s0 + c].contiguous()
        o = torch.empty_like(xi)
        if paged is None:
            tfb.block_prefill(tc, caches["w"], rope, xi, o, start_pos=s0, cache=caches["kv"])
        else:
            tfb.block_prefill_paged(tc, caches["w"], rope, xi, o, paged, start_pos=s0)
        outs.append(o)
        s0 += c
    for s in range(steps):
        p = s0 + s
        xi = x[:, p:p + 1].contiguous()
        o = torch.empty_like(xi)
        pos = torch.full((B,), p, dtype=torch.int32, device="cuda")
        if paged is None:
            tfb.block_decode(tc, caches["w"], rope, xi, o, caches["kv"], pos, p)
        else:
            tfb.block_decode_paged(tc, caches["w"], rope, xi, o, paged, pos, p)
        outs.append(o)
    torch.cuda.synchronize()
    return np.concatenate([to_np(o) for o in outs], axis=1)


@pytest.mark.parametrize("dtype,d,H,Hkv,W,ring_rows,chunks,steps", [
    ("bf16", 256, 4, 2, 64, 64, [100], 160),          # ring of exactly W rows; decode to position 259 (> 4W)
    ("bf16", 256, 4, 2, 64, 64, [40, 70, 1, 30], 40),  # chunked prefill into the ring, a one-row chunk
    ("bf16", 512, 4, 1, 300, 300, [350], 400),         # dh 128, four heads per KV head, ring not a power of two
    ("bf16", 512, 4, 2, 100, 160, [90, 90], 100),      # ring longer than the window
    ("f32", 64, 4, 2, 7, 7, [20, 5], 30),              # fp32: row-wise attention over a 7-row ring
])
def test_ring_window_cache_matches_uncapped_bitwise(oracle, dtype, d, H, Hkv, W, ring_rows, chunks, steps):
    """A bounded window cache of ring_rows rows (position p in row p mod
    ring_rows) gives bit for bit the outputs of the same calls on an uncapped
    cache, far past 2W positions, and matches the oracle's full-cache
    computation."""
    torch = _torch()
    cfg = small_cfg(d=d, H=H, Hkv=Hkv, f=2 * d, dtype=dtype, base=500000.0, number=150, window=W)
    w32, w = dev_weights(cfg)
    B = 2
    T = sum(chunks) + steps
    x32, x = dev_x(cfg, B, T)
    print("case: ring cache", dtype, d, H, Hkv, W, ring_rows, chunks, steps, flush=True)
    kr, vr = new_cache(cfg, B, ring_rows)
    ku, vu = new_cache(cfg, B, T)
    got_r = _ring_run(cfg, x, chunks, steps, {"w": w, "kv": (kr, vr, True)})
    got_u = _ring_run(cfg, x, chunks, steps, {"w": w, "kv": (ku, vu)})
    assert np.array_equal(got_r, got_u)
    # the ring holds exactly the last ring_rows positions, each at its slot
    gr, gu = widen_cache(kr), widen_cache(ku)
    for p in range(T - ring_rows, T):
        assert np.array_equal(gr[:, :, p % ring_rows], gu[:, :, p])
    ref = oracle.block_forward(cfg, w32, x32)
    check("out", got_r, ref, tol(cfg))


@pytest.mark.parametrize("bs", [16, 64])
def test_paged_ring_window_cache_matches_uncapped_bitwise(bs):
    """A paged bounded window cache (ring over max_blocks * block_size slots)
    equals the contiguous uncapped cache bit for bit; pool blocks no sequence
    owns stay untouched."""
    torch = _torch()
    cfg = small_cfg(d=256, H=4, Hkv=2, f=512, dtype="bf16", base=500000.0, number=151, window=64)
    _, w = dev_weights(cfg)
    B, chunks, steps = 2, [70, 30], 120
    T = sum(chunks) + steps
    _, x = dev_x(cfg, B, T)
    max_blocks = 64 // bs
    n_blocks = B * max_blocks + 2
    perm = np.random.default_rng(bs).permutation(n_blocks)[:B * max_blocks].reshape(B, max_blocks)
    table = torch.from_numpy(perm.astype(np.int32)).cuda()
    kp = torch.full((n_blocks, 2, bs, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    vp = kp.clone()
    print("case: paged ring", bs, flush=True)
    got_p = _ring_run(cfg, x, chunks, steps, {"w": w}, paged=(kp, vp, table, bs, True))
    ku, vu = new_cache(cfg, B, T)
    got_u = _ring_run(cfg, x, chunks, steps, {"w": w, "kv": (ku, vu)})
    assert np.array_equal(got_p, got_u)
    free = np.setdiff1d(np.arange(n_blocks), perm.ravel())
    assert np.isnan(widen_cache(kp)[free]).all()


@pytest.mark.parametrize("fold", [0, 1])
def test_model_with_ring_window_caches_matches_uncapped_bitwise(fold):
    """The model (prefill, then greedy decode far past the window) on bounded
    window caches of W rows gives the logits and tokens of uncapped caches
    (fold: both with fold_norms; the 100-row prefill folds its norms and
    works in the ring's staging copy)."""
    import torch
    import synth
    from synth.configs import tensor_id
    from tests.test_gpu_model import model_inputs
    cfg = small_cfg(d=512, H=4, Hkv=2, f=1024, dtype="bf16", number=152, window=32)
    L, V, B, T, steps = 2, 1024, 2, 50, 80
    _, (ld, ed, gd, ud) = model_inputs(cfg, L, V)
    tc = tfb.Config.of(cfg, fold)
    h = tfb.ModelHandle(tc, ld, ed, gd, ud)
    rope = tfb.rope_table_init(tc, T + steps)
    ids = torch.from_numpy(synth.integers(cfg.seed, tensor_id("ids"), (B, T), 0, V - 1)).cuda()
    print("case: model ring caches, fold_norms=%d" % fold, flush=True)
    res = []
    for ring, rows in ((True, 32), (False, T + steps)):
        caches = [(torch.full((B, 2, rows, 128), float("nan"), dtype=torch.bfloat16, device="cuda"),
                   torch.full((B, 2, rows, 128), float("nan"), dtype=torch.bfloat16, device="cuda"), ring)
                  for _ in range(L)]
        lens = torch.zeros(B, dtype=torch.int32, device="cuda")
        nxt = torch.empty(B, dtype=torch.int32, device="cuda")
        lg = torch.empty((B, 1, V), dtype=torch.float32, device="cuda")
        out = []
        tfb.model_forward(h, rope, ids, caches, lens, 0, logits=lg, last_only=True, next_ids=nxt)
        out.append(lg.clone())
        for s in range(steps):
            tfb.model_forward(h, rope, nxt.view(B, 1), caches, lens, T + s, logits=lg, next_ids=nxt)
            out.append(lg.clone())
        torch.cuda.synchronize()
        res.append(torch.stack(out))
    assert torch.equal(res[0], res[1])


def test_kv_append_ring_slots():
    """Rows appended to a bounded window cache land at slots p mod t_max."""
    torch = _torch()
    cfg = small_cfg(d=512, H=4, Hkv=2, f=1024, dtype="bf16", number=153, window=8)
    tc = tfb.Config.of(cfg)
    B, n, t_max = 2, 5, 8
    import synth
    from tests.gpu_util import to_dev
    kf, kb = synth.normal(cfg.seed, 11, (B, n, 2, 128), 1.0, True)
    vf, vb = synth.normal(cfg.seed, 12, (B, n, 2, 128), 1.0, True)
    start = np.array([3, 30], np.int32)
    kc, vc = new_cache(cfg, B, t_max)
    tfb.kv_append(tc, (kc, vc, True), to_dev(kf, kb), to_dev(vf, vb), torch.from_numpy(start).cuda(), int(start.max()))
    torch.cuda.synchronize()
    gk, gv = widen_cache(kc), widen_cache(vc)
    for b in range(B):
        written = set()
        for t in range(n):
            slot = (start[b] + t) % t_max
            written.add(slot)
            assert np.array_equal(gk[b, :, slot], kf[b, t]) and np.array_equal(gv[b, :, slot], vf[b, t])
        for slot in set(range(t_max)) - written:
            assert np.isnan(gk[b, :, slot]).all()
