"""Host logic of bench.py, on the CPU: the FLOP and byte counts its figures
are divided by, and its one-GPU contract.

The FLOP count of a prefill step must be the work the method does, so it is
checked against the oracle's instrumented multiply-adds ([TIR] "Transformer
block", How it works: 2 FLOPs per weight per token, and causal attention over
the T(T+1)/2 visible pairs of each head); the decode byte count against the
KV-cache size per token of the same page (2 Hkv dh values per layer).
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle as O
from oracle import formulas as FM
from synth.configs import C2, C3, C4
from tests.inputs import activations, block_weights, small_cfg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("shape", [
    dict(d=64, H=4, Hkv=2, f=192, B=1, T=16),   # GQA
    dict(d=32, H=4, Hkv=1, f=96, B=2, T=9),     # MQA, two sequences, odd length
    dict(d=48, H=3, Hkv=3, f=128, B=1, T=7),    # MHA
])
def test_prefill_flops_equal_the_oracle_counters(oracle, shape):
    cfg = small_cfg(d=shape["d"], H=shape["H"], Hkv=shape["Hkv"], f=shape["f"], number=90)
    B, T = shape["B"], shape["T"]
    w, _ = block_weights(cfg)
    x, _ = activations(cfg, B, T)
    cnt = O.Counters()
    oracle.block_forward(cfg, w, x, counters=cnt)
    macs = cnt.matmul_macs + cnt.qk_macs + cnt.pv_macs
    assert bench.prefill_flops(B, T, cfg.d, cfg.n_heads, cfg.n_kv_heads, cfg.d_ff) == 2 * macs


def test_prefill_flops_of_the_timed_workloads():
    # the long-context step's count is the one its bench line reports
    assert bench.prefill_flops(C3.B, C3.T, C3.d, C3.n_heads, C3.n_kv_heads, C3.d_ff) == 8246471426048
    for c in (C2, C3):
        assert bench.prefill_flops(c.B, c.T, c.d, c.n_heads, c.n_kv_heads, c.d_ff) == \
            FM.block_prefill_flops_causal(c.B, c.T, c.d, c.n_heads, c.n_kv_heads, c.d_ff)
    # Llama-2-7B's block: 4 d^2 attention weights and 3 d f MLP weights
    assert bench.block_matrix_params(4096, 32, 32, 11008) == 4 * 4096 ** 2 + 3 * 4096 * 11008


def test_decode_bytes_are_the_cache_rows_read():
    dh = C4.d // C4.n_heads
    lens = np.array([0, 1, 767, 768, 4095])
    got = bench.decode_attention_bytes(lens, C4.n_kv_heads, dh)
    per_token = FM.kv_bytes_per_token(1, C4.n_kv_heads, dh, 2)
    assert got == per_token * int((lens + 1).sum())


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    digest = bench.gemm_source_digest()
    good = tmp_path / "good.md"
    good.write_text("traffic_bytes_per_launch: 123456\nkernel_source_sha256: %s\n" % digest)
    stale = tmp_path / "stale.md"
    stale.write_text("traffic_bytes_per_launch: 123456\nkernel_source_sha256: %s\n" % ("0" * 64))
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(good))
    assert bench.measured_traffic() == 123456
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(stale))
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(tmp_path / "missing.md"))
    assert bench.measured_traffic() is None
