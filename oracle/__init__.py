"""ORACLE — test infrastructure, not part of the product.

Python access (ctypes + numpy) to the plain scalar fp32 CPU oracle in
``oracle.c``.  Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg may import this package; the GPU library never does.

Every array handed over is float32 (bf16 inputs arrive already widened, exactly,
by ``synth``); caches are ``[B, Hkv, t_max, dh]`` float32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import formulas  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O3", "-march=x86-64-v3", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared"]
_lib = None


def build(src: str | None = None, out: str | None = None, extra: list[str] | None = None) -> str:
    """Compile oracle.c (always recompiles).  ``extra`` adds -D flags for
    planted-mistake builds used by the tests."""
    src = src or os.path.join(_HERE, "oracle.c")
    out = out or _SO
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, *(extra or []), src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


class _Cfg(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("gemm_bf16", ctypes.c_int32), ("window", ctypes.c_int32)]


class _W(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("g_attn", "g_mlp", "wq", "wk", "wv", "wo", "w1", "w3", "w2")]


class Counters(ctypes.Structure):
    _fields_ = [("matmul_macs", ctypes.c_int64), ("qk_macs", ctypes.c_int64), ("pv_macs", ctypes.c_int64),
                ("cache_values", ctypes.c_int64)]


INTER_NAMES = ("q", "att", "r", "act", "q_pre", "att_pre", "act_pre", "k_pre", "v_pre")


class _Inter(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in INTER_NAMES]


WEIGHT_NAMES = ("g_attn", "g_mlp", "wq", "wk", "wv", "wo", "w1", "w3", "w2")
_VP = ctypes.c_void_p


def load(path: str | None = None):
    """Load (building if absent) an oracle shared library."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    so = path or _SO
    if not os.path.exists(so):
        build(out=so)
    lib = ctypes.CDLL(so)
    lib.o_rms_norm.argtypes = [_VP, _VP, ctypes.c_int64, ctypes.c_int, ctypes.c_float, _VP]
    lib.o_matmul.argtypes = [_VP, _VP, ctypes.c_int64, ctypes.c_int, ctypes.c_int, _VP, _VP]
    lib.o_rope_table.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double, _VP, _VP]
    lib.o_rope_apply.argtypes = [_VP, ctypes.c_int64, ctypes.c_int, ctypes.c_int, _VP, _VP, _VP]
    lib.o_attend_row.argtypes = [_VP, _VP, _VP, ctypes.c_int, ctypes.c_int, _VP]
    lib.o_attend_row_range.argtypes = [_VP, _VP, _VP, ctypes.c_int, ctypes.c_int, ctypes.c_int, _VP]
    lib.o_window_first_key.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.o_window_first_key.restype = ctypes.c_int
    lib.o_block_forward.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_W), _VP, _VP, ctypes.c_int, _VP,
                                    ctypes.c_int, ctypes.c_int, _VP, _VP, _VP, ctypes.c_int, _VP, ctypes.c_int,
                                    _VP, ctypes.POINTER(_Inter), ctypes.POINTER(Counters)]
    lib.o_block_forward.restype = ctypes.c_int
    lib.o_kv_append.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _VP, _VP, _VP,
                                ctypes.c_int, _VP, _VP]
    lib.o_kv_append.restype = ctypes.c_int
    lib.o_model_forward.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int, ctypes.c_int, _VP, ctypes.POINTER(_W), _VP,
                                    _VP, _VP, _VP, ctypes.c_int, _VP, ctypes.c_int, ctypes.c_int, _VP,
                                    ctypes.POINTER(_VP), ctypes.POINTER(_VP), ctypes.c_int, _VP, ctypes.c_int, _VP,
                                    _VP, _VP, _VP, ctypes.POINTER(Counters)]
    lib.o_model_forward.restype = ctypes.c_int
    lib.o_omp_threads.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


class Oracle:
    """Thin numpy front end over one oracle library (default: the real one)."""

    def __init__(self, path: str | None = None):
        self.lib = load(path)

    # ---- helpers -------------------------------------------------------
    @staticmethod
    def _f32(a):
        return np.ascontiguousarray(a, dtype=np.float32)

    @staticmethod
    def _p(a):
        return None if a is None else a.ctypes.data_as(_VP)

    @staticmethod
    def _cfg(cfg) -> _Cfg:
        # bf16 storage: GEMM operands are rounded to bf16 (tirogla "Transformer
        # block", Implementation notes: bf16 GEMMs with fp32 accumulation)
        return _Cfg(cfg.d, cfg.n_heads, cfg.n_kv_heads, cfg.d // cfg.n_heads, cfg.d_ff, cfg.rope_base, cfg.rms_eps,
                    1 if cfg.dtype == "bf16" else 0, int(getattr(cfg, "window", 0)))

    def _weights(self, w: dict):
        arrs = {n: self._f32(w[n]) for n in WEIGHT_NAMES}
        return _W(*[self._p(arrs[n]) for n in WEIGHT_NAMES]), arrs

    def threads(self) -> int:
        return int(self.lib.o_omp_threads())

    # ---- primitives ----------------------------------------------------
    def rms_norm(self, x, g, eps):
        x = self._f32(x)
        g = self._f32(g)
        y = np.empty_like(x)
        d = x.shape[-1]
        self.lib.o_rms_norm(self._p(x), self._p(g), x.size // d, d, eps, self._p(y))
        return y

    def matmul(self, x, w):
        x = self._f32(x)
        w = self._f32(w)
        t, k = x.shape
        n = w.shape[1]
        y = np.empty((t, n), np.float32)
        self.lib.o_matmul(self._p(x), self._p(w), t, k, n, self._p(y), None)
        return y

    def rope_table(self, t_max: int, dh: int, base: float):
        c = np.empty((t_max, dh // 2), np.float32)
        s = np.empty((t_max, dh // 2), np.float32)
        self.lib.o_rope_table(t_max, dh, float(base), self._p(c), self._p(s))
        return c, s

    def rope_apply(self, v, pos, cos_tab, sin_tab):
        """v: [rows, heads, dh] rotated in a copy at positions pos[rows]."""
        v = self._f32(v).copy()
        rows, heads, dh = v.shape
        pos = np.ascontiguousarray(pos, np.int32)
        self.lib.o_rope_apply(self._p(v), rows, heads, dh, self._p(pos), self._p(self._f32(cos_tab)),
                              self._p(self._f32(sin_tab)))
        return v

    def attend_row(self, q, kc, vc, n_keys, first_key=None):
        """Attention of one query over keys [first_key, n_keys) (default: from 0)."""
        q, kc, vc = self._f32(q), self._f32(kc), self._f32(vc)
        dh = q.shape[-1]
        o = np.empty(dh, np.float32)
        if first_key is None:
            self.lib.o_attend_row(self._p(q), self._p(kc), self._p(vc), n_keys, dh, self._p(o))
        else:
            self.lib.o_attend_row_range(self._p(q), self._p(kc), self._p(vc), first_key, n_keys, dh, self._p(o))
        return o

    def window_first_key(self, p: int, window: int) -> int:
        return int(self.lib.o_window_first_key(p, window))

    # ---- block ---------------------------------------------------------
    def block_forward(self, cfg, w: dict, x, start=None, kc=None, vc=None, rows=None, rope=None,
                      intermediates=False, counters: Counters | None = None):
        """x: [B, T, d].  Returns out [B, R, d] (and a dict of intermediates).
        kc / vc (float32 [B, Hkv, t_max, dh]) are updated in place."""
        x = self._f32(x)
        B, T, d = x.shape
        dh = cfg.d // cfg.n_heads
        t_max = kc.shape[2] if kc is not None else T
        if rope is None:
            rope = self.rope_table(max(t_max, T), dh, cfg.rope_base)
        cos_tab, sin_tab = (self._f32(a) for a in rope)
        rows_a = None if rows is None else np.ascontiguousarray(rows, np.int32)
        R = T if rows_a is None else len(rows_a)
        out = np.empty((B, R, d), np.float32)
        st = None if start is None else np.ascontiguousarray(start, np.int32)
        if kc is not None:
            assert kc.dtype == np.float32 and kc.flags.c_contiguous and vc.flags.c_contiguous
        inter = _Inter()
        got = {}
        if intermediates:
            # q, att, act: the operands as handed on; *_pre: the same values
            # before bf16 rounding; k_pre, v_pre: every row, [B, T, Hkv*dh]
            qd, kvd = cfg.n_heads * dh, cfg.n_kv_heads * dh
            shapes = {"q": (B, R, qd), "att": (B, R, qd), "r": (B, R, d), "act": (B, R, cfg.d_ff),
                      "k_pre": (B, T, kvd), "v_pre": (B, T, kvd)}
            for k in ("q", "att", "act"):
                shapes[k + "_pre"] = shapes[k]
            got = {k: np.empty(shapes[k], np.float32) for k in INTER_NAMES}
            inter = _Inter(*[self._p(got[k]) for k in INTER_NAMES])
        cw, keep = self._weights(w)
        cnt = counters if counters is not None else Counters()
        rc = self.lib.o_block_forward(ctypes.byref(self._cfg(cfg)), ctypes.byref(cw), self._p(cos_tab),
                                      self._p(sin_tab), cos_tab.shape[0], self._p(x), B, T, self._p(st),
                                      self._p(kc), self._p(vc), t_max, self._p(rows_a), R, self._p(out),
                                      ctypes.byref(inter), ctypes.byref(cnt))
        if rc != 0:
            raise ValueError("oracle block_forward failed with %d" % rc)
        del keep
        return (out, got) if intermediates else out

    def kv_append(self, kc, vc, k_new, v_new, start):
        B, Hkv, t_max, dh = kc.shape
        k_new, v_new = self._f32(k_new), self._f32(v_new)
        n = k_new.shape[1]
        st = np.ascontiguousarray(start, np.int32)
        rc = self.lib.o_kv_append(B, Hkv, dh, t_max, self._p(k_new), self._p(v_new), self._p(st), n, self._p(kc),
                                  self._p(vc))
        if rc != 0:
            raise ValueError("oracle kv_append failed with %d" % rc)

    # ---- model ---------------------------------------------------------
    def model_forward(self, cfg, n_layers, vocab, embed, layers: list, g_final, w_unembed, ids, kcs, vcs,
                      start=None, rows=None, rope=None, counters: Counters | None = None, kv_pre=False):
        """Returns (logits [B, R, V], next_ids [B]); with kv_pre also the lists
        of each layer's k and v before bf16 storage ([B, T, Hkv*dh] each)."""
        ids = np.ascontiguousarray(ids, np.int32)
        B, T = ids.shape
        t_max = kcs[0].shape[2]
        dh = cfg.d // cfg.n_heads
        if rope is None:
            rope = self.rope_table(t_max, dh, cfg.rope_base)
        cos_tab, sin_tab = (self._f32(a) for a in rope)
        embed, g_final, w_unembed = self._f32(embed), self._f32(g_final), self._f32(w_unembed)
        lw = (_W * n_layers)()
        keep = []
        for i, w in enumerate(layers):
            cw, arrs = self._weights(w)
            lw[i] = cw
            keep.append(arrs)
        kp = (_VP * n_layers)(*[self._p(a) for a in kcs])
        vp = (_VP * n_layers)(*[self._p(a) for a in vcs])
        rows_a = None if rows is None else np.ascontiguousarray(rows, np.int32)
        R = T if rows_a is None else len(rows_a)
        logits = np.empty((B, R, vocab), np.float32)
        nxt = np.empty(B, np.int32)
        st = None if start is None else np.ascontiguousarray(start, np.int32)
        cnt = counters if counters is not None else Counters()
        kpre = vpre = None
        kpp = vpp = None
        if kv_pre:
            kvd = cfg.n_kv_heads * dh
            kpre = [np.empty((B, T, kvd), np.float32) for _ in range(n_layers)]
            vpre = [np.empty((B, T, kvd), np.float32) for _ in range(n_layers)]
            kpp = (_VP * n_layers)(*[self._p(a) for a in kpre])
            vpp = (_VP * n_layers)(*[self._p(a) for a in vpre])
        rc = self.lib.o_model_forward(ctypes.byref(self._cfg(cfg)), n_layers, vocab, self._p(embed), lw,
                                      self._p(g_final), self._p(w_unembed), self._p(cos_tab), self._p(sin_tab),
                                      cos_tab.shape[0], self._p(ids), B, T, self._p(st), kp, vp, t_max,
                                      self._p(rows_a), R, self._p(logits), self._p(nxt), kpp, vpp, ctypes.byref(cnt))
        if rc != 0:
            raise ValueError("oracle model_forward failed with %d" % rc)
        return (logits, nxt, kpre, vpre) if kv_pre else (logits, nxt)
