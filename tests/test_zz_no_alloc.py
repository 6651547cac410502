"""tfb_block_decode_noalloc: the allocation-free variant of tfb_block_decode
(for callers that cannot allocate device memory) against tfb_block_decode on
the same inputs, bit for bit, on two calls in a row, the second one smaller;
and its size limit."""
import numpy as np
import pytest

import synth
from tests.conftest import gpu_available
from tests.gpu_util import dev_weights, dev_x, to_dev
from tests.inputs import small_cfg
from synth.configs import C4

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import transformer_decoder_block_rmsnorm_amd as tfb  # noqa: E402


def _caches(cfg, B, t_max, lens, seed_off=0):
    """Seeded post-RoPE caches with NaN beyond each sequence's rows."""
    dh = cfg.d // cfg.n_heads
    shape = (B, cfg.n_kv_heads, t_max, dh)
    rows = np.arange(t_max)[None, None, :, None]
    valid = rows < np.asarray(lens)[:, None, None, None]
    out = []
    for tid in (11, 12):
        f, bits = synth.normal(cfg.seed + seed_off, tid, shape, 1.0, True)
        bits = np.where(valid, bits, np.uint16(0x7FC0))
        out.append(to_dev(np.where(valid, f, np.nan).astype(np.float32), bits))
    return out


def _pair(cfg, B, lens, t_max):
    """The same decode step through tfb_block_decode and through the
    allocation-free call, on separate copies of the caches."""
    import torch
    tc = tfb.Config.of(cfg)
    _, w = dev_weights(cfg)
    _, x = dev_x(cfg, B, 1)
    rope = tfb.rope_table_init(tc, t_max)
    kc, vc = _caches(cfg, B, t_max, lens)
    kc2, vc2 = kc.clone(), vc.clone()
    pos = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o1, o2 = torch.empty_like(x), torch.empty_like(x)
    tfb.block_decode(tc, w, rope, x, o1, (kc, vc), pos, max(lens))
    tfb.block_decode_noalloc(tc, w, rope, x, o2, (kc2, vc2), pos, max(lens))
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(o1, o2), (o1.float() - o2.float()).abs().max().item()
    assert torch.equal(torch.nan_to_num(kc), torch.nan_to_num(kc2))
    assert torch.equal(torch.nan_to_num(vc), torch.nan_to_num(vc2))


def test_noalloc_decode_equals_decode_twice_smaller_second():
    cfg = small_cfg(d=512, H=4, Hkv=2, f=1024, dtype="bf16", base=500000.0, number=140)
    print("case: noalloc small, B=5 then B=3", flush=True)
    _pair(cfg, 5, [700, 33, 1, 1500, 260], 1600)
    _pair(cfg, 3, [12, 5, 90], 100)


def test_noalloc_decode_full_size_then_smaller():
    """The GQA decode step (B=64, d=4096, f=14336, cache lengths in [1024, 4096]),
    then 16 sequences."""
    print("case: noalloc full size B=64 then B=16", flush=True)
    lens = [int(v) for v in synth.integers(C4.seed, 13, (64,), 1024, 4096)]
    _pair(C4, 64, lens, C4.t_max)
    _pair(C4, 16, lens[:16], C4.t_max)


def test_noalloc_rejects_calls_beyond_its_scratch():
    """Past the static array's size the call returns TFB_ERR_WORKSPACE and
    launches nothing (the output keeps its sentinel)."""
    import torch
    # 16 query heads per KV head (the split-KV kernel, whose chunk partials
    # grow with the cache length): 40010 rows need ~43 MB of partials
    cfg = small_cfg(d=4096, H=32, Hkv=2, f=512, dtype="bf16", number=141)
    tc = tfb.Config.of(cfg)
    B, t_max = 64, 40010
    _, w = dev_weights(cfg)
    _, x = dev_x(cfg, B, 1)
    rope = tfb.rope_table_init(tc, t_max)
    kc = torch.zeros((B, 2, t_max, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.full_like(x, 7.0)
    with pytest.raises(tfb.TfbError) as e:
        tfb.block_decode_noalloc(tc, w, rope, x, out, (kc, vc), pos, t_max - 1)
    assert e.value.code == -5
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    assert tfb.noalloc_scratch_bytes() == 32 << 20
