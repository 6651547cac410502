"""Benchmark of the decoder-block hot path on one MI355X.

Headline (`value`): block prefill TFLOP/s on the largest block-prefill
workload, the GQA long-context block (d=4096, H=32, Hkv=8, dh=128, f=14336,
RoPE base 5e5, B=2, T=8192, bf16 storage, fp32 accumulation, KV cache
written), algorithmic causal FLOP count; `roofline` is its dominant kernel,
the fused gate-up GEMM.  In the same run:
  - the Llama-2-7B-shaped block prefill (d=4096, H=Hkv=32, f=11008, B=1,
    T=2048) in TFLOP/s;
  - the GQA decode step (d=4096, H=32, Hkv=8, f=14336, B=64 sequences with
    cache lengths uniform in [1024, 4096]) in tokens/s, with the
    decode-attention kernel's and each weight-streaming GEMM's achieved HBM
    bandwidth;
  - the 32-layer model (B=4, prompt T=1024, V=32000): prefill TFLOP/s and
    128 greedy decode steps in tokens/s.
Inputs are synthetic and seeded, resident in HBM before timing starts.
Every timed leg first runs its warmup steps and then keeps stepping until at
least a second of warm work has run, so a short --warmup cannot leave the
timed steps on a cold clock.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--no-7b] [--no-model]
       python bench.py --copy-calibration   (a plain 1 GiB device copy, for
                                             scaling the HBM byte counters)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block prefill TFLOP/s + decode tok/s, as % of MFMA / HBM roofline on 1 GPU"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBPS = 8000.0      # HBM3E

# HBM traffic of the gate-up GEMM from rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
# with the sources of the kernel it was taken on (stale counters give null)
PMC_SUMMARY = os.path.join(ROOT, "profiles", "gateup_gemm_gqa_long_prefill_pmc.md")
GEMM_SOURCES = [os.path.join(ROOT, "transformer_decoder_block_rmsnorm_amd", "csrc", n)
                for n in ("gemm.hip", "epilogue.h", "common.h")]


# Algorithmic counts (2 FLOPs per multiply-add: tirogla "Transformer block",
# How it works; kirito-excalibur "The Transformer", 4. FLOP counting).
def block_matrix_params(d, H, Hkv, f):
    """Wq, Wk, Wv, Wo and the three SwiGLU matrices of one block."""
    dh = d // H
    return d * H * dh + 2 * d * Hkv * dh + H * dh * d + 3 * d * f


def prefill_flops(B, T, d, H, Hkv, f):
    """Weight products for every token plus causal attention: q.k and p.v over
    the T(T+1)/2 visible (query, key) pairs of each head."""
    dh = d // H
    return 2 * B * T * block_matrix_params(d, H, Hkv, f) + 4 * dh * H * B * T * (T + 1) // 2


def decode_attention_bytes(lens, Hkv, dh):
    """bf16 K and V rows 0..len_b (the new row included) of every sequence."""
    return sum((int(n) + 1) * Hkv * dh * 2 * 2 for n in lens)


def gemm_source_digest() -> str:
    h = hashlib.sha256()
    for p in GEMM_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """Bytes per launch from the committed counter summary, or None when the
    summary is missing or was taken on different kernel sources."""
    try:
        text = open(PMC_SUMMARY).read()
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    s = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    if not m or not s or s.group(1) != gemm_source_digest():
        return None
    return int(m.group(1))


def _dev_tensor(f32, bits):
    import numpy as np
    import torch
    if bits is not None:
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(f32).cuda()


MIN_WARM_SECONDS = 1.0  # set from --min-warm


def warm_up(step, warmup, min_seconds=None):
    """`warmup` untimed steps, then more until min_seconds of work have run."""
    import torch
    if min_seconds is None:
        min_seconds = MIN_WARM_SECONDS
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.time()
    while time.time() - t0 < min_seconds:
        for _ in range(4):
            step()
        torch.cuda.synchronize()


def block_inputs(cfg, B, T):
    from synth.inputs import activations, block_weights
    w32, bits = block_weights(cfg)
    w = {k: _dev_tensor(v, None if bits is None else bits[k]) for k, v in w32.items()}
    x32, xb = activations(cfg, B, T)
    return w32, w, x32, _dev_tensor(x32, xb)


def time_prefill(cfg, steps, warmup, fold=0):
    """fold: the config's fold_norms (RMSNorm2 folded into the Wo and gate-up
    GEMMs); the folded leg is timed without the per-stage pass."""
    import torch
    import transformer_decoder_block_rmsnorm_amd as tfb
    tc = tfb.Config.of(cfg, fold)
    B, T = cfg.B, cfg.T
    w32, w, x32, x = block_inputs(cfg, B, T)
    rope = tfb.rope_table_init(tc, cfg.t_max)
    kc = torch.zeros((B, cfg.n_kv_heads, cfg.t_max, tc.head_dim), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    out = torch.empty_like(x)
    ws = tfb.workspace(tc, B, T)

    def step():
        tfb.block_prefill(tc, w, rope, x, out, cache=(kc, vc), ws=ws)

    warm_up(step, warmup)
    # timed region: K steps; the dominant kernel (the fused gate-up GEMM) is
    # bracketed by HIP events on its launch stream
    tfb.profile_read()
    tfb.profile_stages(["gateup_gemm"])
    tfb.profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    tfb.profile_enable(False)
    ms = e0.elapsed_time(e1) / steps
    dominant = tfb.profile_read()
    if fold:
        flops = prefill_flops(B, T, cfg.d, cfg.n_heads, cfg.n_kv_heads, cfg.d_ff)
        return dict(ms=ms, flops=flops, dominant=dominant)
    # the same K steps with every launch bracketed: per-stage breakdown (the
    # event pairs add gaps between launches, so this pass is not the headline)
    tfb.profile_stages(None)
    tfb.profile_enable(True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    tfb.profile_enable(False)
    ms_all_events = e0.elapsed_time(e1) / steps
    stages = tfb.profile_read()
    flops = prefill_flops(B, T, cfg.d, cfg.n_heads, cfg.n_kv_heads, cfg.d_ff)
    return dict(ms=ms, ms_all_events=ms_all_events, flops=flops, stages=stages, dominant=dominant, w32=w32,
                x32=x32)


def time_decode(cfg, steps, warmup):
    import numpy as np
    import torch
    import synth
    import transformer_decoder_block_rmsnorm_amd as tfb
    from synth.configs import tensor_id
    tc = tfb.Config.of(cfg)
    B, dh = cfg.B, cfg.d // cfg.n_heads
    lens = synth.integers(cfg.seed, tensor_id("lens"), (B,), cfg.lens_lo, cfg.lens_hi)
    _, w, _, x = block_inputs(cfg, B, 1)
    shape = (B, cfg.n_kv_heads, cfg.t_max, dh)
    caches = []
    for name in ("kc", "vc"):
        _, bits = synth.normal(cfg.seed, tensor_id(name), shape, 1.0, True)
        rows = np.arange(cfg.t_max)[None, None, :, None]
        bits = np.where(rows < lens[:, None, None, None], bits, np.uint16(0))
        caches.append(_dev_tensor(None, bits))
    kc, vc = caches
    pos = torch.from_numpy(lens).cuda()
    rope = tfb.rope_table_init(tc, cfg.t_max)
    out = torch.empty_like(x)
    ws = tfb.workspace(tc, B, 1)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")  # > 256 MB Infinity Cache

    def step():
        tfb.block_decode(tc, w, rope, x, out, (kc, vc), pos, int(lens.max()), ws=ws)

    warm_up(step, warmup)
    # timed steps, nothing bracketed inside them (an event pair around a
    # short kernel adds several microseconds to a 0.26 ms step)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    total = 0.0
    for _ in range(steps):
        flush.fill_(1)  # evict the caches between steps; not timed
        torch.cuda.synchronize()
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        total += e0.elapsed_time(e1)
    ms = total / steps
    # the same steps with the attention kernel and its merge bracketed by
    # HIP events on their launch stream (the roofline entry)
    tfb.profile_read()
    tfb.profile_stages(["attention", "attention_combine"])
    for _ in range(steps):
        flush.fill_(1)
        torch.cuda.synchronize()
        tfb.profile_enable(True)
        step()
        torch.cuda.synchronize()
        tfb.profile_enable(False)
    dominant = tfb.profile_read()
    tfb.profile_stages(None)
    tfb.profile_enable(True)
    for _ in range(steps):
        flush.fill_(1)
        step()
    torch.cuda.synchronize()
    tfb.profile_enable(False)
    stages = tfb.profile_read()
    attn_bytes = decode_attention_bytes(lens, cfg.n_kv_heads, dh) + 2 * B * cfg.d * 2
    wbytes = 2 * block_matrix_params(cfg.d, cfg.n_heads, cfg.n_kv_heads, cfg.d_ff)
    return dict(ms=ms, stages=stages, dominant=dominant, attn_bytes=attn_bytes, weight_bytes=wbytes, lens=lens)


def decode_gemm_rates(cfg, stages):
    """Weight bytes of each decode GEMM (the bytes it must stream; the 64
    activation rows add <2%) over its bracketed time, reduce pass included."""
    d, H, Hkv, f = cfg.d, cfg.n_heads, cfg.n_kv_heads, cfg.d_ff
    dh = d // H
    wbytes = {"qkv_gemm": 2 * d * (H + 2 * Hkv) * dh, "wo_gemm": 2 * H * dh * d, "gateup_gemm": 2 * d * 2 * f,
              "w2_gemm": 2 * f * d}
    out = {}
    for k, b in wbytes.items():
        if k in stages and stages[k][1]:
            ms = stages[k][0] / stages[k][1]
            out[k] = {"weight_bytes": b, "ms": round(ms, 4), "GB_s": round(b / (ms * 1e-3) / 1e9, 1),
                      "frac": round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
    return out


def time_model(cfg, decode_steps, reps, fold=True):
    """The 32-layer model: prefill of the prompts (logits of the last rows,
    greedy next token), then decode_steps greedy steps with the growing cache.
    Weights are drawn N(0, 0.02) on the GPU (torch generator, seeded); the
    gains are 1.  With fold, the prefill is also timed with fold_norms (the
    RMSNorms that follow a GEMM folded into the GEMMs around them)."""
    import torch
    import transformer_decoder_block_rmsnorm_amd as tfb
    from synth.inputs import weight_shapes
    tc = tfb.Config.of(cfg)
    tc_fold = tfb.Config.of(cfg, 1)
    B, T, L, V, d = cfg.B, cfg.T, cfg.n_layers, cfg.vocab, cfg.d
    dh = d // cfg.n_heads
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed)

    def randn(shape):
        return (torch.randn(shape, generator=g, device="cuda") * cfg.w_sigma).to(torch.bfloat16)

    layers = []
    for _ in range(L):
        layers.append({n: (torch.ones(s, dtype=torch.bfloat16, device="cuda") if n.startswith("g_") else randn(s))
                       for n, s in weight_shapes(d, cfg.n_heads, cfg.n_kv_heads, cfg.d_ff).items()})
    embed, w_un = randn((V, d)), randn((d, V))
    g_final = torch.ones(d, dtype=torch.bfloat16, device="cuda")
    h = tfb.ModelHandle(tc, layers, embed, g_final, w_un)
    h_fold = tfb.ModelHandle(tc_fold, layers, embed, g_final, w_un) if fold else None
    caches = [(torch.zeros((B, cfg.n_kv_heads, cfg.t_max, dh), dtype=torch.bfloat16, device="cuda"),
               torch.zeros((B, cfg.n_kv_heads, cfg.t_max, dh), dtype=torch.bfloat16, device="cuda"))
              for _ in range(L)]
    rope = tfb.rope_table_init(tc, cfg.t_max)
    ids = torch.randint(0, V, (B, T), generator=g, device="cuda", dtype=torch.int32)
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    nxt = torch.empty((B, 1), dtype=torch.int32, device="cuda")
    ws_pre = tfb.workspace(tc, B, T, V)
    ws_pre_fold = tfb.workspace(tc_fold, B, T, V) if fold else None
    ws_dec = tfb.workspace(tc, B, 1, V)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def prefill(folded=False):
        lens.zero_()
        tfb.model_forward(h_fold if folded else h, rope, ids, caches, lens, 0, last_only=True, next_ids=nxt.view(B),
                          ws=ws_pre_fold if folded else ws_pre)

    def decode():
        for s in range(decode_steps):
            tfb.model_forward(h, rope, nxt, caches, lens, T + s, last_only=True, next_ids=nxt.view(B), ws=ws_dec)

    t0 = time.time()
    while True:
        prefill()
        decode()
        torch.cuda.synchronize()
        if time.time() - t0 >= MIN_WARM_SECONDS:
            break
    pre_ms, dec_ms, fold_ms = [], [], []
    for _ in range(reps):
        if fold:
            flush.fill_(1)
            torch.cuda.synchronize()
            e0.record()
            prefill(True)
            e1.record()
            torch.cuda.synchronize()
            fold_ms.append(e0.elapsed_time(e1))
        flush.fill_(1)
        torch.cuda.synchronize()
        e0.record()
        prefill()
        e1.record()
        torch.cuda.synchronize()
        pre_ms.append(e0.elapsed_time(e1))
        e0.record()
        decode()
        e1.record()
        torch.cuda.synchronize()
        dec_ms.append(e0.elapsed_time(e1))
    pre, dec = min(pre_ms), min(dec_ms)
    flops = L * prefill_flops(B, T, d, cfg.n_heads, cfg.n_kv_heads, cfg.d_ff) + 2 * B * d * V
    wbytes = 2 * (L * block_matrix_params(d, cfg.n_heads, cfg.n_kv_heads, cfg.d_ff) + d * V)
    kv = sum(L * decode_attention_bytes([T + s] * B, cfg.n_kv_heads, dh) for s in range(decode_steps))
    step_ms = dec / decode_steps
    folded = {}
    if fold:
        folded = {"prefill_folded_norms_ms": round(min(fold_ms), 3),
                  "prefill_folded_norms_tflops": round(flops / (min(fold_ms) * 1e-3) / 1e12, 2)}
    return {"workload": "32-layer GQA model: d=4096 H=32 Hkv=8 f=14336 V=32000 untied, B=4, prompt T=1024 "
                        "token ids uniform in [0, V), then %d greedy decode steps" % decode_steps,
            "prefill_ms": round(pre, 3), "prefill_tflops": round(flops / (pre * 1e-3) / 1e12, 2),
            "prefill_mfma_frac": round(flops / (pre * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            **folded,
            "decode_ms_per_step": round(step_ms, 4), "decode_tok_per_s": round(B / (step_ms * 1e-3), 1),
            "decode_hbm_frac": round((wbytes + kv / decode_steps) / (step_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "decode_bytes_per_step": int(wbytes + kv / decode_steps), "reps": reps,
            "note": "minimum over reps; the caches are flushed before each prefill; each decode step is one "
                    "tfb_model_forward call over all 32 layers"}


def time_tiny(cfg, reps):
    """The tiny fp32 block: prefill of T rows then single-token decode steps
    (launch-latency bound; microseconds only)."""
    import torch
    import transformer_decoder_block_rmsnorm_amd as tfb
    tc = tfb.Config.of(cfg)
    B, T, steps = cfg.B, cfg.T, cfg.decode_steps
    _, w, _, x = block_inputs(cfg, B, T + steps)
    rope = tfb.rope_table_init(tc, cfg.t_max)
    kc = torch.zeros((B, cfg.n_kv_heads, cfg.t_max, tc.head_dim), dtype=torch.float32, device="cuda")
    vc = torch.zeros_like(kc)
    xp = x[:, :T].contiguous()
    xd = [x[:, T + s:T + s + 1].contiguous() for s in range(steps)]
    out_p, out_d = torch.empty_like(xp), torch.empty_like(xd[0])
    pos = [torch.full((B,), T + s, dtype=torch.int32, device="cuda") for s in range(steps)]
    ws = tfb.workspace(tc, B, T)
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    pre, dec = [], []
    for _ in range(reps):
        torch.cuda.synchronize()
        e0.record()
        tfb.block_prefill(tc, w, rope, xp, out_p, cache=(kc, vc), ws=ws)
        e1.record()
        for s in range(steps):
            tfb.block_decode(tc, w, rope, xd[s], out_d, (kc, vc), pos[s], T + s, ws=ws)
        e2.record()
        torch.cuda.synchronize()
        pre.append(e0.elapsed_time(e1) * 1e3)
        dec.append(e1.elapsed_time(e2) * 1e3 / steps)
    pre.sort()
    dec.sort()
    return {"workload": "tiny fp32 block: d=64 H=4 Hkv=2 f=192, prefill T=16 then 4 decode steps",
            "prefill_us": round(pre[len(pre) // 2], 1), "decode_us_per_step": round(dec[len(dec) // 2], 1),
            "reps": reps, "note": "median; launch-latency bound, no roofline claim"}


def cpu_baseline(cfg, w32, x32, rows, min_seconds=10.0, max_passes=16):
    """The CPU oracle on a bounded prefix of the same block prefill, repeated
    until about min_seconds of work have run (at most max_passes passes)."""
    import oracle as O
    orc = O.Oracle()
    passes = 0
    t0 = time.time()
    while True:
        orc.block_forward(cfg, w32, x32[:, :rows])
        passes += 1
        dt = time.time() - t0
        if dt >= min_seconds or passes >= max_passes:
            break
    flops = passes * prefill_flops(cfg.B, rows, cfg.d, cfg.n_heads, cfg.n_kv_heads, cfg.d_ff)
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": orc.threads(), "kind": "oracle",
            "sample": "first %d of %d tokens of the same block prefill (B=%d, full widths), %d passes in %.1f s wall"
                      % (rows, cfg.T, cfg.B, passes, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-7b", action="store_true")
    ap.add_argument("--model-reps", type=int, default=3)
    ap.add_argument("--decode-only", action="store_true",
                    help="only the GQA decode step (for counter runs); prints the decode fields alone")
    ap.add_argument("--no-model", action="store_true")
    ap.add_argument("--no-fold", action="store_true", help="skip the folded-norm legs (profiling runs)")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--min-warm", type=float, default=1.0,
                    help="seconds of warm steps before each timed leg (after --warmup steps)")
    args = ap.parse_args()
    global MIN_WARM_SECONDS
    MIN_WARM_SECONDS = args.min_warm
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (requested --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    from synth.configs import C1, C2, C3, C4, C5
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.backends.cuda.matmul.allow_tf32 = False
    if args.copy_calibration:
        # one plain device copy kernel of known size per launch, three launches
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)
        return

    if args.decode_only:
        dec = time_decode(C4, args.steps, args.warmup)
        print(json.dumps({"decode_only": True, "tok_per_s": round(C4.B / (dec["ms"] * 1e-3), 1),
                          "ms_per_step": round(dec["ms"], 4), "attention_bytes": dec["attn_bytes"],
                          "weight_bytes": dec["weight_bytes"]}), flush=True)
        return
    def prefill_summary(cfg, pre, workload):
        """TFLOP/s of the block step and the roofline entry of its gate-up GEMM."""
        tflops = pre["flops"] / (pre["ms"] * 1e-3) / 1e12
        gms, gcalls = pre["dominant"]["gateup_gemm"]
        g_ms = gms / gcalls
        g_flops = 2 * cfg.B * cfg.T * cfg.d * 2 * cfg.d_ff
        roof = {"kernel": "gateup_gemm (fused W1|W3 GEMM + SiLU*up)", "bound": "mfma",
                "achieved": round(g_flops / (g_ms * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(g_flops / (g_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "launch_ms": round(g_ms, 4), "flops_per_launch": g_flops}
        stages = {k: round(v[0] / v[1], 4) for k, v in pre["stages"].items()}
        attn = 4 * (cfg.d // cfg.n_heads) * cfg.n_heads * cfg.B * cfg.T * (cfg.T + 1) // 2
        return tflops, roof, {"workload": workload, "tflops": round(tflops, 2),
                              "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4), "ms_per_step": round(pre["ms"], 4),
                              "ms_per_step_all_events": round(pre["ms_all_events"], 4),
                              "flops_per_step": pre["flops"], "stage_ms": stages,
                              "attention_tflops": round(attn / (stages["attention"] * 1e-3) / 1e12, 2)}

    long_workload = ("GQA long-context block prefill: d=4096 H=32 Hkv=8 dh=128 f=14336 RoPE base 5e5 B=2 T=8192, "
                     "KV cache written")
    pre = time_prefill(C3, args.steps, args.warmup)
    tflops, roof, long_summary = prefill_summary(C3, pre, long_workload)
    roof["traffic"] = measured_traffic()

    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(pre["ms"], 4),
        "ms_per_step_all_events": round(pre["ms_all_events"], 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": long_workload, "global_batch": C3.B, "seq_len": C3.T, "parallelism": "none"},
        "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "flops_per_step": pre["flops"],
        "roofline": roof,
        "prefill_stage_ms": long_summary["stage_ms"],
        "attention_tflops": long_summary["attention_tflops"],
    }
    def folded(cfg):
        """The same block step with fold_norms: RMSNorm2 folded into the Wo
        epilogue and the gate-up GEMM (not the headline: it moves where the
        GEMM operand is rounded to bf16)."""
        f = time_prefill(cfg, args.steps, args.warmup, fold=1)
        gms, gcalls = f["dominant"]["gateup_gemm"]
        return {"ms_per_step": round(f["ms"], 4), "tflops": round(f["flops"] / (f["ms"] * 1e-3) / 1e12, 2),
                "gateup_launch_ms": round(gms / gcalls, 4)}

    if not args.no_fold:
        result["prefill_folded_norms"] = {"long_context": folded(C3)}
    if not args.no_7b:
        pre7 = time_prefill(C2, args.steps, args.warmup)
        _, roof7, sum7 = prefill_summary(C2, pre7, "Llama-2-7B-shaped block prefill: d=4096 H=Hkv=32 dh=128 "
                                                   "f=11008 B=1 T=2048, KV cache written")
        sum7["gateup_roofline"] = roof7
        result["prefill_7b"] = sum7
        if not args.no_fold:
            result["prefill_folded_norms"]["7b"] = folded(C2)
    if not args.no_decode:
        dec = time_decode(C4, args.steps, args.warmup)
        ams, acalls = dec["dominant"]["attention"]
        cms, ccalls = dec["dominant"].get("attention_combine", (0.0, 1))
        k_ms = ams / acalls                        # the split-KV attention kernel
        m_ms = k_ms + (cms / ccalls if ccalls else 0.0)  # plus the merge of its chunk partials
        a_gbps = dec["attn_bytes"] / (k_ms * 1e-3) / 1e9
        am_gbps = dec["attn_bytes"] / (m_ms * 1e-3) / 1e9
        result["decode"] = {
            "workload": "GQA decode step: d=4096 H=32 Hkv=8 f=14336 B=64, cache lengths uniform in [1024, 4096], "
                        "caches flushed from Infinity Cache between steps",
            "tok_per_s": round(C4.B / (dec["ms"] * 1e-3), 1), "ms_per_step": round(dec["ms"], 4),
            "attention": {"kernel": "decode_attn_kernel (split-KV attention)", "bound": "hbm",
                          "achieved": round(a_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                          "frac": round(a_gbps / PEAK_HBM_GBPS, 4), "bytes_per_launch": dec["attn_bytes"],
                          "launch_ms": round(k_ms, 4)},
            "attention_with_merge": {"achieved": round(am_gbps, 1), "unit": "GB/s",
                                     "frac": round(am_gbps / PEAK_HBM_GBPS, 4), "ms": round(m_ms, 4)},
            "step_bytes": dec["attn_bytes"] + dec["weight_bytes"],
            "step_hbm_frac": round((dec["attn_bytes"] + dec["weight_bytes"]) / (dec["ms"] * 1e-3) / 1e9 /
                                   PEAK_HBM_GBPS, 4),
            "stage_ms": {k: round(v[0] / v[1], 4) for k, v in dec["stages"].items()},
            "gemm_hbm": decode_gemm_rates(C4, dec["stages"]),
        }
    if not args.no_model:
        result["model"] = time_model(C5, C5.decode_steps, max(1, args.model_reps), fold=not args.no_fold)
        result["tiny"] = time_tiny(C1, 21)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(C3, pre["w32"], pre["x32"], args.cpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
