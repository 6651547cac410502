"""GPU parity of the model path (embedding, L blocks, final RMSNorm, untied LM
head, greedy next token) against the CPU oracle, in prefill and decode.

Decode steps are teacher-forced: the token fed at each step is the GPU's own
greedy choice, and the oracle is given the same ids, so a near-tie argmax
cannot make the two sides diverge."""
import numpy as np
import pytest

import synth
from synth.configs import tensor_id
from tests.conftest import gpu_available
from tests.gpu_util import cache_rows, check, dev_weights, to_dev, to_np, tol
from tests.inputs import rel_err, small_cfg

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import transformer_decoder_block_rmsnorm_amd as tfb  # noqa: E402


def model_inputs(cfg, L, V):
    bf = cfg.dtype == "bf16"
    layers32, layers = [], []
    for l in range(L):
        w32, w = dev_weights(cfg, layer=l, gains="random")
        layers32.append(w32)
        layers.append(w)
    emb32, embb = synth.normal(cfg.seed, tensor_id("embed"), (V, cfg.d), 1.0, bf)
    wu32, wub = synth.normal(cfg.seed, tensor_id("w_unembed"), (cfg.d, V), 0.02, bf)
    gf = 1.0 + synth.normal(cfg.seed, tensor_id("g_final"), (cfg.d,), 0.1, False)[0]
    if bf:
        gfb, gf32 = synth.to_bf16(gf)
    else:
        gfb, gf32 = None, gf.astype(np.float32)
    return (layers32, emb32, gf32, wu32), (layers, to_dev(emb32, embb), to_dev(gf32, gfb), to_dev(wu32, wub))


@pytest.mark.parametrize("dtype,d,H,Hkv,f,L,V,B,T,steps,fold", [
    ("f32", 64, 4, 2, 192, 2, 100, 2, 12, 3, 0),
    ("bf16", 512, 4, 2, 1024, 2, 1024, 2, 40, 3, 0),
    ("bf16", 256, 2, 1, 512, 3, 512, 3, 70, 2, 0),
    # RMSNorms folded into the GEMMs around them (prefill: 80 and 210 rows)
    ("bf16", 512, 4, 2, 1024, 2, 1024, 2, 40, 3, 1),
    ("bf16", 256, 2, 1, 512, 3, 512, 3, 70, 2, 1),
    # widths that end inside a column tile (W2 folds the next RMSNorm1 there)
    ("bf16", 320, 5, 1, 640, 2, 512, 2, 50, 2, 1),
])
def test_model_prefill_then_greedy_decode(oracle, dtype, d, H, Hkv, f, L, V, B, T, steps, fold):
    import torch
    cfg = small_cfg(d=d, H=H, Hkv=Hkv, f=f, dtype=dtype, base=500000.0, number=95)
    print("case: model", dtype, d, L, V, B, T, steps, "fold_norms=%d" % fold, flush=True)
    (l32, e32, g32, u32), (ld, ed, gd, ud) = model_inputs(cfg, L, V)
    tc = tfb.Config.of(cfg, fold)
    h = tfb.ModelHandle(tc, ld, ed, gd, ud)
    t_max = T + steps + 2
    dh = d // H
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    caches = [(torch.full((B, Hkv, t_max, dh), float("nan"), dtype=tdt, device="cuda"),
               torch.full((B, Hkv, t_max, dh), float("nan"), dtype=tdt, device="cuda")) for _ in range(L)]
    rope = tfb.rope_table_init(tc, t_max)
    ids = synth.integers(cfg.seed, tensor_id("ids"), (B, T), 0, V - 1)
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    logits = torch.empty((B, T, V), dtype=torch.float32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    tfb.model_forward(h, rope, torch.from_numpy(ids).cuda(), caches, lens, 0, logits=logits, next_ids=nxt)
    torch.cuda.synchronize()
    okc = [np.full((B, Hkv, t_max, dh), np.nan, np.float32) for _ in range(L)]
    ovc = [a.copy() for a in okc]
    ref, ref_next, kpre, _ = oracle.model_forward(cfg, L, V, e32, l32, g32, u32, ids, okc, ovc, kv_pre=True)
    got = logits.cpu().numpy()
    check("prefill logits (all rows)", got, ref, tol(cfg))
    g_next = nxt.cpu().numpy()
    assert np.array_equal(g_next, np.argmax(got[:, -1], axis=-1))
    assert lens.cpu().numpy().tolist() == [T] * B
    # every layer's cache rows 0..T-1 hold the oracle's keys; rows beyond stay NaN
    for l in range(L):
        gk = to_np(caches[l][0])
        check("layer %d k cache" % l, gk[:, :, :T], cache_rows(kpre[l], Hkv), tol(cfg))
        assert np.isnan(gk[:, :, T:]).all()

    cur = g_next.copy()
    for s in range(steps):
        pos = T + s
        ids1 = cur.reshape(B, 1).astype(np.int32)
        lg1 = torch.empty((B, 1, V), dtype=torch.float32, device="cuda")
        tfb.model_forward(h, rope, torch.from_numpy(ids1).cuda(), caches, lens, pos, logits=lg1, next_ids=nxt)
        torch.cuda.synchronize()
        r1, _ = oracle.model_forward(cfg, L, V, e32, l32, g32, u32, ids1, okc, ovc,
                                     start=np.full(B, pos, np.int32))
        g1 = lg1.cpu().numpy()
        check("decode step %d logits" % s, g1, r1, tol(cfg))
        cur = nxt.cpu().numpy()
        assert np.array_equal(cur, np.argmax(g1[:, -1], axis=-1))
        assert lens.cpu().numpy().tolist() == [pos + 1] * B


def test_model_last_only_and_next_ids_only(oracle):
    import torch
    cfg = small_cfg(d=512, H=4, Hkv=2, f=1024, dtype="bf16", number=96)
    L, V, B, T = 2, 1024, 2, 33
    (l32, e32, g32, u32), (ld, ed, gd, ud) = model_inputs(cfg, L, V)
    tc = tfb.Config.of(cfg)
    h = tfb.ModelHandle(tc, ld, ed, gd, ud)
    dh = cfg.d // cfg.n_heads
    ids = synth.integers(cfg.seed, tensor_id("ids"), (B, T), 0, V - 1)
    okc = [np.zeros((B, cfg.n_kv_heads, T, dh), np.float32) for _ in range(L)]
    ovc = [a.copy() for a in okc]
    ref, ref_next = oracle.model_forward(cfg, L, V, e32, l32, g32, u32, ids, okc, ovc, rows=[T - 1])
    for mode in ("last_only", "next_only"):
        caches = [(torch.zeros((B, cfg.n_kv_heads, T, dh), dtype=torch.bfloat16, device="cuda"),
                   torch.zeros((B, cfg.n_kv_heads, T, dh), dtype=torch.bfloat16, device="cuda")) for _ in range(L)]
        rope = tfb.rope_table_init(tc, T)
        lens = torch.zeros(B, dtype=torch.int32, device="cuda")
        nxt = torch.empty(B, dtype=torch.int32, device="cuda")
        lg = torch.empty((B, 1, V), dtype=torch.float32, device="cuda") if mode == "last_only" else None
        tfb.model_forward(h, rope, torch.from_numpy(ids).cuda(), caches, lens, 0, logits=lg, last_only=True,
                          next_ids=nxt)
        torch.cuda.synchronize()
        if lg is not None:
            got = lg.cpu().numpy()
            check("last-row logits", got, ref, tol(cfg))
            assert np.array_equal(nxt.cpu().numpy(), np.argmax(got[:, -1], axis=-1))
        # the oracle's greedy choice agrees unless its top two logits nearly tie
        top2 = np.sort(ref[:, -1], axis=-1)[:, -2:]
        margin = (top2[:, 1] - top2[:, 0]) / np.sqrt(np.mean(ref ** 2))
        agree = nxt.cpu().numpy() == ref_next
        assert np.all(agree | (margin < 0.05))


def test_model_all_row_logits_with_large_vocabulary(oracle):
    """Logits for every row of a short prompt (B*T <= 64 rows, so the LM head
    runs the weight-streaming GEMM over all rows) with a vocabulary much wider
    than the block's GEMMs: the head's split-k partials need their own share
    of the workspace."""
    import torch
    cfg = small_cfg(d=512, H=4, Hkv=2, f=1024, dtype="bf16", number=99)
    L, V, B, T = 2, 32000, 2, 16
    print("case: all-row logits, V", V, "rows", B * T, flush=True)
    (l32, e32, g32, u32), (ld, ed, gd, ud) = model_inputs(cfg, L, V)
    tc = tfb.Config.of(cfg)
    h = tfb.ModelHandle(tc, ld, ed, gd, ud)
    dh = cfg.d // cfg.n_heads
    caches = [(torch.zeros((B, cfg.n_kv_heads, T, dh), dtype=torch.bfloat16, device="cuda"),
               torch.zeros((B, cfg.n_kv_heads, T, dh), dtype=torch.bfloat16, device="cuda")) for _ in range(L)]
    rope = tfb.rope_table_init(tc, T)
    ids = synth.integers(cfg.seed, tensor_id("ids"), (B, T), 0, V - 1)
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    lg = torch.empty((B, T, V), dtype=torch.float32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    tfb.model_forward(h, rope, torch.from_numpy(ids).cuda(), caches, lens, 0, logits=lg, next_ids=nxt)
    torch.cuda.synchronize()
    okc = [np.zeros((B, cfg.n_kv_heads, T, dh), np.float32) for _ in range(L)]
    ovc = [a.copy() for a in okc]
    ref, _ = oracle.model_forward(cfg, L, V, e32, l32, g32, u32, ids, okc, ovc)
    got = lg.cpu().numpy()
    check("logits (all rows)", got, ref, tol(cfg))
    assert np.array_equal(nxt.cpu().numpy(), np.argmax(got[:, -1], axis=-1))
    assert lens.cpu().numpy().tolist() == [T] * B


def test_decode_step_replays_from_a_hip_graph():
    """One decode step of the model recorded into a HIP graph and replayed:
    the library allocates nothing and never synchronises inside the call, and
    the position of each sequence lives in the device-side lens, so each
    replay is the next decode step.  Every replay (with eager work and a
    synchronisation between replays) must give the eager step's logits and
    greedy token bit for bit.  The eager steps use the same host bound; at
    this size it yields the same launches as the per-step bound that the
    oracle-checked decode test uses."""
    import torch
    cfg = small_cfg(d=512, H=4, Hkv=2, f=1024, dtype="bf16", number=97)
    L, V, B, T, steps = 2, 1024, 3, 37, 4
    print("case: graph replay of a decode step", L, V, B, T, steps, flush=True)
    _, (ld, ed, gd, ud) = model_inputs(cfg, L, V)
    tc = tfb.Config.of(cfg)
    h = tfb.ModelHandle(tc, ld, ed, gd, ud)
    t_max = T + steps + 3
    bound = t_max - 2  # a host bound of max(lens) valid for every step
    dh = cfg.d // cfg.n_heads
    caches = [(torch.zeros((B, cfg.n_kv_heads, t_max, dh), dtype=torch.bfloat16, device="cuda"),
               torch.zeros((B, cfg.n_kv_heads, t_max, dh), dtype=torch.bfloat16, device="cuda")) for _ in range(L)]
    rope = tfb.rope_table_init(tc, t_max)
    ids = torch.from_numpy(synth.integers(cfg.seed, tensor_id("ids"), (B, T), 0, V - 1)).cuda()
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    lg = torch.empty((B, 1, V), dtype=torch.float32, device="cuda")
    ws_pre = tfb.workspace(tc, B, T, V)
    ws_dec = tfb.workspace(tc, B, 1, V)

    def prefill():
        lens.zero_()
        tfb.model_forward(h, rope, ids, caches, lens, 0, last_only=True, next_ids=nxt, ws=ws_pre)

    def step():
        tfb.model_forward(h, rope, nxt.view(B, 1), caches, lens, bound, logits=lg, last_only=True, next_ids=nxt,
                          ws=ws_dec)

    prefill()
    ref = []
    for _ in range(steps):
        step()
        ref.append((lg.clone(), nxt.clone()))
    torch.cuda.synchronize()

    prefill()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    prefill()  # capture ran nothing; start again from the prompt all the same
    torch.cuda.synchronize()
    for s in range(steps):
        graph.replay()
        got_l, got_i = lg.clone(), nxt.clone()
        _ = (got_l * 2.0).sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(got_l, ref[s][0]), s
        assert torch.equal(got_i, ref[s][1]), s
        assert lens.cpu().numpy().tolist() == [T + s + 1] * B


@pytest.mark.parametrize("V,cols,expected", [
    (9024, [6001, 37, 4100, 9023], 37),   # tied columns in different threads, waves and 4-column groups
    (9024, [9023, 9020, 9022], 9020),     # a tie inside one 4-column group of one thread
    (128, [127, 64, 65], 64),
])
def test_greedy_next_token_ties_take_lowest_index(V, cols, expected):
    """Greedy decoding breaks ties toward the lowest index (the oracle pin of
    the same rule builds the same model).  Zero Wo and W2 make the block the
    identity on its input, an embedding of ones and unit gains then give the
    final hidden row of ones, and W_U has identical dominant columns: those
    logits are exactly d, every other one is 0."""
    import torch
    cfg = small_cfg(d=256, H=2, Hkv=1, f=512, dtype="bf16", number=98)
    B, T = 2, 3
    print("case: argmax ties", V, cols, flush=True)
    _, w = dev_weights(cfg, layer=0, gains="ones")
    w = dict(w, wo=torch.zeros_like(w["wo"]), w2=torch.zeros_like(w["w2"]))
    emb = torch.ones((V, cfg.d), dtype=torch.bfloat16, device="cuda")
    wu = torch.zeros((cfg.d, V), dtype=torch.bfloat16, device="cuda")
    for c in cols:
        wu[:, c] = 1.0
    gf = torch.ones(cfg.d, dtype=torch.bfloat16, device="cuda")
    tc = tfb.Config.of(cfg)
    h = tfb.ModelHandle(tc, [w], emb, gf, wu)
    dh = cfg.d // cfg.n_heads
    caches = [(torch.zeros((B, cfg.n_kv_heads, T, dh), dtype=torch.bfloat16, device="cuda"),
               torch.zeros((B, cfg.n_kv_heads, T, dh), dtype=torch.bfloat16, device="cuda"))]
    rope = tfb.rope_table_init(tc, T)
    ids = torch.randint(0, V, (B, T), dtype=torch.int32, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    nxt = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    lg = torch.empty((B, 1, V), dtype=torch.float32, device="cuda")
    tfb.model_forward(h, rope, ids, caches, lens, 0, logits=lg, last_only=True, next_ids=nxt)
    torch.cuda.synchronize()
    got = lg.cpu().numpy()[:, 0]
    assert np.all(got[:, cols] == float(cfg.d)), got[:, cols]
    assert np.count_nonzero(got) == B * len(cols)
    assert nxt.cpu().numpy().tolist() == [expected] * B
