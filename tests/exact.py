"""An exact evaluation of the method: an fp64 composition of PyTorch library
routines (rms_norm, matmul, complex rotation, scaled_dot_product_attention),
written from the pages independently of the oracle and of the HIP path.

It pins the oracle at tiny shapes (tests/test_oracle_pins.py).  At full size
it measures how far the method itself, computed exactly with bf16 operands
rounded at the same places as the oracle, sits from the fp32 oracle: the
distance any implementation of the method has to be allowed.

Page short names: [TIR] tirogla "Transformer block", [GEN] thegeniusblogs
"The Transformer Architecture".
"""
import numpy as np
import torch
import torch.nn.functional as F


# --------------------------------------------------------------------------
# An independent fp64 composition out of PyTorch library routines (rms_norm,
# matmul, complex rotation, scaled_dot_product_attention with is_causal, silu).
# With bf16=True every GEMM operand is rounded to bf16 by torch's own
# conversion where the pages' precision rule puts it ([TIR] Implementation
# notes: bf16 GEMMs with fp32 accumulation, softmax and norms in fp32).
# --------------------------------------------------------------------------
def _bf16(a):
    return a.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def _norm_operand(v, g, eps, rb, fold_rows):
    """The GEMM operand of an RMSNorm over the last axis of v [B, T, d] and the
    scale of each row of the GEMM's products.  Rows t < fold_rows take the
    folded form, where the row scale 1/rms(v) is applied to the products
    instead of the operand: operand rb(v * g), scale 1/rms(v).  The other rows
    take rb(rms_norm(v) * g) and scale 1.  Both are the same product before
    rounding (row m of (s v * g) W is s ((v * g) W)); only where the operand is
    rounded to bf16 differs."""
    d = v.shape[-1]
    plain = rb(F.rms_norm(v, (d,), weight=g, eps=eps))
    if not fold_rows:
        return plain, None
    rows = (torch.arange(v.shape[1]) < fold_rows)[None, :, None]
    s = torch.rsqrt(v.pow(2).mean(-1, keepdim=True) + eps)
    return torch.where(rows, rb(v * g), plain), torch.where(rows, s, torch.ones_like(s))


def torch_block_f64(cfg, w, x, start=0, bf16=False, window=0, fold1=0, fold2=0):
    """fold1, fold2: rows (token index t < fold) whose RMSNorm 1 / 2 takes the
    folded form of _norm_operand."""
    d, H, Hkv = cfg.d, cfg.n_heads, cfg.n_kv_heads
    dh = d // H
    rb = _bf16 if bf16 else (lambda a: a)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))  # noqa: E731
    X = t(x)
    B, T, _ = X.shape
    h, s1 = _norm_operand(X, t(w["g_attn"]), cfg.rms_eps, rb, fold1)
    sc1 = (lambda a: a) if s1 is None else (lambda a: a * s1)  # noqa: E731
    q = sc1(h @ t(w["wq"])).reshape(B, T, H, dh)
    k = sc1(h @ t(w["wk"])).reshape(B, T, Hkv, dh)
    v = sc1(h @ t(w["wv"])).reshape(B, T, Hkv, dh)
    pos = torch.arange(start, start + T, dtype=torch.float64)
    theta = torch.tensor([cfg.rope_base ** (-2.0 * i / dh) for i in range(dh // 2)], dtype=torch.float64)
    rot = torch.polar(torch.ones(T, dh // 2, dtype=torch.float64), pos[:, None] * theta[None, :])

    def rope(a):
        c = torch.view_as_complex(a.reshape(*a.shape[:-1], dh // 2, 2).contiguous())
        return torch.view_as_real(c * rot[None, :, None, :]).reshape(a.shape)

    pre = {"q_pre": rope(q).reshape(B, T, H * dh).numpy(), "k_pre": rope(k).reshape(B, T, Hkv * dh).numpy(),
           "v_pre": v.reshape(B, T, Hkv * dh).numpy()}
    q, k, v = rb(rope(q)), rb(rope(k)), rb(v)
    g = H // Hkv
    K = k.repeat_interleave(g, dim=2).transpose(1, 2)
    V = v.repeat_interleave(g, dim=2).transpose(1, 2)
    if window:
        # band mask: key j visible to query i iff i - window < j <= i
        i = torch.arange(T)[:, None]
        j = torch.arange(T)[None, :]
        band = (j <= i) & (j > i - window)
        o = F.scaled_dot_product_attention(q.transpose(1, 2), K, V, attn_mask=band)
    else:
        o = F.scaled_dot_product_attention(q.transpose(1, 2), K, V, is_causal=True)
    o = o.transpose(1, 2).reshape(B, T, H * dh)
    pre["att_pre"] = o.numpy()
    o = rb(o)
    r = X + o @ t(w["wo"])
    h2, s2 = _norm_operand(r, t(w["g_mlp"]), cfg.rms_eps, rb, fold2)
    sc2 = (lambda a: a) if s2 is None else (lambda a: a * s2)  # noqa: E731
    act = F.silu(sc2(h2 @ t(w["w1"]))) * sc2(h2 @ t(w["w3"]))
    pre["act_pre"] = act.numpy()
    act = rb(act)
    return (r + act @ t(w["w2"])).numpy(), {"q": q.reshape(B, T, H * dh).numpy(), "att": o.numpy(),
                                            "r": r.numpy(), "act": act.numpy(), **pre}


def decode_f64(cfg, w, x, lens, kc, vc, bf16=True):
    """One decode step of B sequences ([GEN] KV cache and inference math, two
    phases): x [B, 1, d] at positions lens[b], caches [B, Hkv, >=len, dh] whose
    rows 0..lens[b]-1 hold earlier keys and values.  Returns (out [B, 1, d],
    intermediates as torch_block_f64, rows of the new token)."""
    d, H, Hkv = cfg.d, cfg.n_heads, cfg.n_kv_heads
    dh = d // H
    rb = _bf16 if bf16 else (lambda a: a)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))  # noqa: E731
    X = t(x)[:, 0]
    B = X.shape[0]
    h = rb(F.rms_norm(X, (d,), weight=t(w["g_attn"]), eps=cfg.rms_eps))
    q = (h @ t(w["wq"])).reshape(B, H, dh)
    k = (h @ t(w["wk"])).reshape(B, Hkv, dh)
    v = (h @ t(w["wv"])).reshape(B, Hkv, dh)
    theta = torch.tensor([cfg.rope_base ** (-2.0 * i / dh) for i in range(dh // 2)], dtype=torch.float64)
    pos = torch.tensor(np.asarray(lens, np.float64))
    rot = torch.polar(torch.ones(B, dh // 2, dtype=torch.float64), pos[:, None] * theta[None, :])

    def rope(a):
        c = torch.view_as_complex(a.reshape(*a.shape[:-1], dh // 2, 2).contiguous())
        return torch.view_as_real(c * rot[:, None, :]).reshape(a.shape)

    pre = {"q_pre": rope(q).reshape(B, 1, H * dh).numpy(), "k_pre": rope(k).reshape(B, 1, Hkv * dh).numpy(),
           "v_pre": v.reshape(B, 1, Hkv * dh).numpy()}
    q, k, v = rb(rope(q)), rb(rope(k)), rb(v)
    g = H // Hkv
    o = torch.empty(B, H, dh, dtype=torch.float64)
    for b in range(B):
        n = int(lens[b])
        K = torch.cat([t(kc[b, :, :n]), k[b][:, None]], dim=1).repeat_interleave(g, dim=0)
        V = torch.cat([t(vc[b, :, :n]), v[b][:, None]], dim=1).repeat_interleave(g, dim=0)
        o[b] = F.scaled_dot_product_attention(q[b][:, None], K, V)[:, 0]
    o = o.reshape(B, H * dh)
    pre["att_pre"] = o[:, None].numpy()
    o = rb(o)
    r = X + o @ t(w["wo"])
    h2 = rb(F.rms_norm(r, (d,), weight=t(w["g_mlp"]), eps=cfg.rms_eps))
    act = F.silu(h2 @ t(w["w1"])) * (h2 @ t(w["w3"]))
    pre["act_pre"] = act[:, None].numpy()
    act = rb(act)
    out = r + act @ t(w["w2"])
    return out[:, None].numpy(), {"q": q.reshape(B, 1, H * dh).numpy(), "att": o[:, None].numpy(),
                                  "r": r[:, None].numpy(), "act": act[:, None].numpy(), **pre}


def model_f64(cfg, layers, embed, g_final, w_unembed, ids, bf16=True, kv=False, fold_rows=0):
    """Logits of the last row of each sequence: embed, L blocks (outputs handed
    on as bf16 activations), final RMSNorm, untied head.  With kv, also each
    layer's k (after RoPE) and v before bf16 storage, [B, T, Hkv*dh].
    fold_rows: rows t < fold_rows take the folded form of every RMSNorm that
    follows a GEMM (RMSNorm 2, and RMSNorm 1 after the first layer)."""
    rb = _bf16 if bf16 else (lambda a: a)
    x = torch.from_numpy(embed[ids].astype(np.float64))
    ks, vs = [], []
    for l, w in enumerate(layers):
        y, inter = torch_block_f64(cfg, w, x.numpy(), bf16=bf16, fold1=fold_rows if l else 0, fold2=fold_rows)
        ks.append(inter["k_pre"])
        vs.append(inter["v_pre"])
        x = rb(torch.from_numpy(y))
    hn = rb(F.rms_norm(x[:, -1:], (cfg.d,), weight=torch.from_numpy(np.asarray(g_final, np.float64)),
                       eps=cfg.rms_eps))
    logits = (hn @ torch.from_numpy(np.asarray(w_unembed, np.float64))).numpy()
    return (logits, ks, vs) if kv else logits


def stored_bf16(a):
    """fp64 values rounded to bf16 (through fp32), as a bf16 tensor stores them."""
    return torch.from_numpy(np.asarray(a, np.float64)).float().bfloat16().double().numpy()
