"""Python binding of libtfb.so (include/tfb.h): argument marshalling only.

Every step of the decoder block runs in the library's HIP kernels; torch is
used here for device memory and the current stream.  Importing works without
a GPU, but calling into the library requires the built ``libtfb.so`` and
raises ``RuntimeError`` when it is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtfb.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "tfb.h")

TFB_F32, TFB_BF16 = 0, 1
STATUS = {0: "TFB_OK", -1: "TFB_ERR_NULL", -2: "TFB_ERR_SHAPE", -3: "TFB_ERR_DTYPE", -4: "TFB_ERR_ALIGN",
          -5: "TFB_ERR_WORKSPACE", -6: "TFB_ERR_CACHE_OVERFLOW", -7: "TFB_ERR_HIP", -8: "TFB_ERR_UNSUPPORTED"}
EXPORTS = ("tfb_workspace_bytes", "tfb_rope_table_init", "tfb_block_prefill", "tfb_block_decode", "tfb_kv_append",
           "tfb_model_forward", "tfb_block_prefill_varlen", "tfb_block_prefill_paged", "tfb_block_decode_paged",
           "tfb_status_string", "tfb_version", "tfb_profile_enable", "tfb_profile_read",
           "tfb_profile_stages", "tfb_profile_stage_name", "tfb_workspace_view",
           "tfb_block_decode_noalloc", "tfb_noalloc_scratch_bytes")
VIEWS = {"q": 0, "att": 1, "r": 2, "act": 3}

_VP = ctypes.c_void_p


class BlockConfig(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int32), ("window", ctypes.c_int32),
                ("fold_norms", ctypes.c_int32)]


class BlockWeights(ctypes.Structure):
    _fields_ = [(n, _VP) for n in ("g_attn", "g_mlp", "wq", "wk", "wv", "wo", "w1", "w3", "w2")]


class KVCache(ctypes.Structure):
    _fields_ = [("k", _VP), ("v", _VP), ("batch", ctypes.c_int32), ("t_max", ctypes.c_int32),
                ("ring", ctypes.c_int32)]


class PagedKVCache(ctypes.Structure):
    _fields_ = [("k", _VP), ("v", _VP), ("block_table", _VP), ("batch", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32), ("n_blocks", ctypes.c_int32),
                ("ring", ctypes.c_int32)]


class Model(ctypes.Structure):
    _fields_ = [("blk", BlockConfig), ("n_layers", ctypes.c_int32), ("vocab", ctypes.c_int32), ("embed", _VP),
                ("layers", ctypes.POINTER(BlockWeights)), ("g_final", _VP), ("w_unembed", _VP)]


WEIGHT_NAMES = ("g_attn", "g_mlp", "wq", "wk", "wv", "wo", "w1", "w3", "w2")


class TfbError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__("%s failed: %s (%d)" % (where, STATUS.get(code, "?"), code))
        self.code = code


_lib = None


def lib():
    """The loaded libtfb.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libtfb.so is not built (run __graft_entry__.build()); there is no fallback")
        L = ctypes.CDLL(LIB_PATH)
        L.tfb_workspace_bytes.argtypes = [ctypes.POINTER(BlockConfig), ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32]
        L.tfb_workspace_bytes.restype = ctypes.c_size_t
        L.tfb_workspace_view.argtypes = [ctypes.POINTER(BlockConfig), ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
        L.tfb_workspace_view.restype = ctypes.c_int
        L.tfb_rope_table_init.argtypes = [ctypes.POINTER(BlockConfig), ctypes.c_int32, _VP, _VP]
        L.tfb_block_prefill.argtypes = [ctypes.POINTER(BlockConfig), ctypes.POINTER(BlockWeights), _VP,
                                        ctypes.c_int32, _VP, _VP, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.POINTER(KVCache), _VP, ctypes.c_size_t, _VP]
        L.tfb_block_prefill_paged.argtypes = [ctypes.POINTER(BlockConfig), ctypes.POINTER(BlockWeights), _VP,
                                              ctypes.c_int32, _VP, _VP, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.POINTER(PagedKVCache), _VP, ctypes.c_size_t, _VP]
        L.tfb_block_decode_paged.argtypes = [ctypes.POINTER(BlockConfig), ctypes.POINTER(BlockWeights), _VP,
                                             ctypes.c_int32, _VP, _VP, ctypes.c_int32, ctypes.POINTER(PagedKVCache),
                                             _VP, ctypes.c_int32, _VP, ctypes.c_size_t, _VP]
        L.tfb_block_prefill_varlen.argtypes = [ctypes.POINTER(BlockConfig), ctypes.POINTER(BlockWeights), _VP,
                                               ctypes.c_int32, _VP, _VP, ctypes.c_int32, ctypes.c_int32, _VP, _VP,
                                               ctypes.c_int32, ctypes.POINTER(KVCache), _VP, ctypes.c_size_t, _VP]
        L.tfb_block_decode.argtypes = [ctypes.POINTER(BlockConfig), ctypes.POINTER(BlockWeights), _VP,
                                       ctypes.c_int32, _VP, _VP, ctypes.c_int32, ctypes.POINTER(KVCache), _VP,
                                       ctypes.c_int32, _VP, ctypes.c_size_t, _VP]
        L.tfb_block_decode_noalloc.argtypes = [ctypes.POINTER(BlockConfig), ctypes.POINTER(BlockWeights), _VP,
                                               ctypes.c_int32, _VP, _VP, ctypes.c_int32, ctypes.POINTER(KVCache), _VP,
                                               ctypes.c_int32, _VP]
        L.tfb_block_decode_noalloc.restype = ctypes.c_int
        L.tfb_noalloc_scratch_bytes.restype = ctypes.c_size_t
        L.tfb_kv_append.argtypes = [ctypes.POINTER(BlockConfig), ctypes.POINTER(KVCache), _VP, _VP, _VP,
                                    ctypes.c_int32, ctypes.c_int32, _VP]
        L.tfb_model_forward.argtypes = [ctypes.POINTER(Model), _VP, ctypes.c_int32, _VP, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.POINTER(KVCache), _VP, ctypes.c_int32, _VP,
                                        ctypes.c_int32, _VP, _VP, ctypes.c_size_t, _VP]
        for f in ("tfb_rope_table_init", "tfb_block_prefill", "tfb_block_decode", "tfb_kv_append",
                  "tfb_model_forward", "tfb_block_prefill_varlen", "tfb_block_prefill_paged",
                  "tfb_block_decode_paged"):
            getattr(L, f).restype = ctypes.c_int
        L.tfb_status_string.argtypes = [ctypes.c_int]
        L.tfb_status_string.restype = ctypes.c_char_p
        L.tfb_version.restype = ctypes.c_int32
        L.tfb_profile_enable.argtypes = [ctypes.c_int32]
        L.tfb_profile_enable.restype = ctypes.c_int
        L.tfb_profile_stages.argtypes = [ctypes.c_uint32]
        L.tfb_profile_stages.restype = ctypes.c_int
        L.tfb_profile_read.argtypes = [_VP, _VP, ctypes.c_int32]
        L.tfb_profile_read.restype = ctypes.c_int32
        L.tfb_profile_stage_name.argtypes = [ctypes.c_int32]
        L.tfb_profile_stage_name.restype = ctypes.c_char_p
        _lib = L
    return _lib


# ---------------------------------------------------------------------------
# torch-side helpers (device memory and streams only)
# ---------------------------------------------------------------------------
def _ptr(t):
    return None if t is None else _VP(t.data_ptr())


def _stream():
    import torch
    return _VP(torch.cuda.current_stream().cuda_stream)


def _check(rc: int, where: str):
    if rc != 0:
        raise TfbError(rc, where)


@dataclass
class Config:
    d: int
    n_heads: int
    n_kv_heads: int
    d_ff: int
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    dtype: str = "bf16"
    window: int = 0  # sliding-window attention: keys per query (0 = full causal)
    fold_norms: int = 0  # fold RMSNorms that follow a GEMM into the GEMMs around them (bf16, > 64 rows)

    @property
    def head_dim(self) -> int:
        return self.d // self.n_heads

    def c(self) -> BlockConfig:
        return BlockConfig(self.d, self.n_heads, self.n_kv_heads, self.head_dim, self.d_ff, self.rope_base,
                           self.rms_eps, TFB_BF16 if self.dtype == "bf16" else TFB_F32, self.window,
                           self.fold_norms)

    @staticmethod
    def of(obj, fold_norms: int = 0) -> "Config":
        return Config(obj.d, obj.n_heads, obj.n_kv_heads, obj.d_ff, obj.rope_base, obj.rms_eps, obj.dtype,
                      int(getattr(obj, "window", 0)), fold_norms)


def weights_struct(w: dict) -> BlockWeights:
    return BlockWeights(*[_VP(w[n].data_ptr()) for n in WEIGHT_NAMES])


def cache_struct(k, v, ring: bool = False) -> KVCache:
    """k, v: [B, Hkv, t_max, dh]; ring: a bounded window cache holding the last
    t_max positions (position p in row p mod t_max)."""
    return KVCache(_VP(k.data_ptr()), _VP(v.data_ptr()), k.shape[0], k.shape[2], 1 if ring else 0)


def workspace_bytes(cfg: Config, B: int, T: int, vocab: int = 0) -> int:
    return int(lib().tfb_workspace_bytes(ctypes.byref(cfg.c()), B, T, vocab))


def workspace(cfg: Config, B: int, T: int, vocab: int = 0, device="cuda"):
    import torch
    n = workspace_bytes(cfg, B, T, vocab)
    if n == 0:
        raise TfbError(-2, "tfb_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def workspace_view(cfg: Config, ws, B: int, T: int, name: str, vocab: int = 0):
    """A tensor view (no copy) of an intermediate the last block call left in
    the workspace ``ws``: q [B, H, T, dh], att [B, T, H*dh], r [B, T, d]
    (fp32) or act [B, T, f]."""
    import torch
    off = ctypes.c_size_t(0)
    _check(lib().tfb_workspace_view(ctypes.byref(cfg.c()), B, T, vocab, VIEWS[name], ctypes.byref(off)),
           "tfb_workspace_view")
    dh = cfg.head_dim
    shape = {"q": (B, cfg.n_heads, T, dh), "att": (B, T, cfg.n_heads * dh), "r": (B, T, cfg.d),
             "act": (B, T, cfg.d_ff)}[name]
    dt = torch.float32 if (name == "r" or cfg.dtype != "bf16") else torch.bfloat16
    n = 1
    for v in shape:
        n *= v
    nbytes = n * (4 if dt == torch.float32 else 2)
    return ws[off.value:off.value + nbytes].view(dt).view(shape)


def rope_table_init(cfg: Config, t_max: int, table=None):
    import torch
    if table is None:
        table = torch.empty((t_max, cfg.head_dim // 2, 2), dtype=torch.float32, device="cuda")
    _check(lib().tfb_rope_table_init(ctypes.byref(cfg.c()), t_max, _ptr(table), _stream()), "tfb_rope_table_init")
    return table


def block_prefill(cfg: Config, w: dict, rope, x, out, start_pos: int = 0, cache=None, ws=None):
    """x, out: [B, T, d] device tensors; cache: (k, v) tensors [B, Hkv, t_max, dh] or None."""
    B, T, _ = x.shape
    if ws is None:
        ws = workspace(cfg, B, T)
    kv = None if cache is None else ctypes.byref(cache_struct(*cache))
    ws_n = ws.numel() * ws.element_size()
    _check(lib().tfb_block_prefill(ctypes.byref(cfg.c()), ctypes.byref(weights_struct(w)), _ptr(rope),
                                   rope.shape[0], _ptr(x), _ptr(out), B, T, start_pos, kv, _ptr(ws), ws_n,
                                   _stream()), "tfb_block_prefill")
    return out


def block_prefill_varlen(cfg: Config, w: dict, rope, x, out, start, lens, max_end: int, cache, ws=None):
    """Right-padded batched prefill: sequence b has lens[b] real rows at positions
    start[b] + t.  start, lens: int32 [B] device tensors; max_end >= max(start + lens)."""
    B, T, _ = x.shape
    if ws is None:
        ws = workspace(cfg, B, T)
    kv = ctypes.byref(cache_struct(*cache))
    ws_n = ws.numel() * ws.element_size()
    _check(lib().tfb_block_prefill_varlen(ctypes.byref(cfg.c()), ctypes.byref(weights_struct(w)), _ptr(rope),
                                          rope.shape[0], _ptr(x), _ptr(out), B, T, _ptr(start), _ptr(lens), max_end,
                                          kv, _ptr(ws), ws_n, _stream()), "tfb_block_prefill_varlen")
    return out


def paged_cache_struct(k, v, table, block_size: int, ring: bool = False) -> PagedKVCache:
    """k, v: pools [n_blocks, Hkv, block_size, dh]; table: int32 [B, max_blocks] device tensor."""
    return PagedKVCache(_VP(k.data_ptr()), _VP(v.data_ptr()), _VP(table.data_ptr()), table.shape[0], block_size,
                        table.shape[1], k.shape[0], 1 if ring else 0)


def block_prefill_paged(cfg: Config, w: dict, rope, x, out, paged, start_pos: int = 0, ws=None):
    """paged: (k_pool, v_pool, block_table, block_size)."""
    B, T, _ = x.shape
    if ws is None:
        ws = workspace(cfg, B, T)
    pc = paged_cache_struct(*paged)
    ws_n = ws.numel() * ws.element_size()
    _check(lib().tfb_block_prefill_paged(ctypes.byref(cfg.c()), ctypes.byref(weights_struct(w)), _ptr(rope),
                                         rope.shape[0], _ptr(x), _ptr(out), B, T, start_pos, ctypes.byref(pc),
                                         _ptr(ws), ws_n, _stream()), "tfb_block_prefill_paged")
    return out


def block_decode_paged(cfg: Config, w: dict, rope, x, out, paged, pos, max_pos: int, ws=None):
    B = x.shape[0]
    if ws is None:
        ws = workspace(cfg, B, 1)
    pc = paged_cache_struct(*paged)
    ws_n = ws.numel() * ws.element_size()
    _check(lib().tfb_block_decode_paged(ctypes.byref(cfg.c()), ctypes.byref(weights_struct(w)), _ptr(rope),
                                        rope.shape[0], _ptr(x), _ptr(out), B, ctypes.byref(pc), _ptr(pos), max_pos,
                                        _ptr(ws), ws_n, _stream()), "tfb_block_decode_paged")
    return out


def block_decode(cfg: Config, w: dict, rope, x, out, cache, pos, h_max_pos: int, ws=None):
    """x, out: [B, 1, d]; cache: (k, v); pos: int32 [B] device tensor."""
    B = x.shape[0]
    if ws is None:
        ws = workspace(cfg, B, 1)
    ws_n = ws.numel() * ws.element_size()
    _check(lib().tfb_block_decode(ctypes.byref(cfg.c()), ctypes.byref(weights_struct(w)), _ptr(rope),
                                  rope.shape[0], _ptr(x), _ptr(out), B, ctypes.byref(cache_struct(*cache)),
                                  _ptr(pos), h_max_pos, _ptr(ws), ws_n, _stream()), "tfb_block_decode")
    return out


def block_decode_noalloc(cfg: Config, w: dict, rope, x, out, cache, pos, h_max_pos: int):
    """tfb_block_decode with the library's static scratch as workspace (no
    allocation anywhere in the call)."""
    B = x.shape[0]
    _check(lib().tfb_block_decode_noalloc(ctypes.byref(cfg.c()), ctypes.byref(weights_struct(w)), _ptr(rope),
                                          rope.shape[0], _ptr(x), _ptr(out), B, ctypes.byref(cache_struct(*cache)),
                                          _ptr(pos), h_max_pos, _stream()), "tfb_block_decode_noalloc")
    return out


def noalloc_scratch_bytes() -> int:
    return int(lib().tfb_noalloc_scratch_bytes())


def kv_append(cfg: Config, cache, k_new, v_new, start, h_max_start: int):
    n_new = k_new.shape[1]
    _check(lib().tfb_kv_append(ctypes.byref(cfg.c()), ctypes.byref(cache_struct(*cache)), _ptr(k_new),
                               _ptr(v_new), _ptr(start), n_new, h_max_start, _stream()), "tfb_kv_append")


class ModelHandle:
    """Keeps the ctypes structs of a model alive across calls."""

    def __init__(self, cfg: Config, layers: list, embed, g_final, w_unembed):
        self.cfg = cfg
        self.vocab = embed.shape[0]
        self._layers = (BlockWeights * len(layers))(*[weights_struct(w) for w in layers])
        self._tensors = (layers, embed, g_final, w_unembed)
        self.m = Model(cfg.c(), len(layers), self.vocab, _VP(embed.data_ptr()), self._layers,
                       _VP(g_final.data_ptr()), _VP(w_unembed.data_ptr()))


def model_forward(h: ModelHandle, rope, ids, caches: list, lens, h_max_len: int, logits=None, last_only=False,
                  next_ids=None, ws=None):
    B, T = ids.shape
    if ws is None:
        ws = workspace(h.cfg, B, T, h.vocab)
    kv = (KVCache * len(caches))(*[cache_struct(*c) for c in caches])
    ws_n = ws.numel() * ws.element_size()
    _check(lib().tfb_model_forward(ctypes.byref(h.m), _ptr(rope), rope.shape[0], _ptr(ids), B, T, kv, _ptr(lens),
                                   h_max_len, _ptr(logits), 1 if last_only else 0, _ptr(next_ids), _ptr(ws), ws_n,
                                   _stream()), "tfb_model_forward")


def profile_enable(on: bool = True):
    _check(lib().tfb_profile_enable(1 if on else 0), "tfb_profile_enable")


def profile_stages(names=None):
    """Stages bracketed while profiling: an iterable of stage names, or None for all."""
    L = lib()
    if names is None:
        mask = 0xFFFFFFFF
    else:
        index = {}
        for k in range(32):
            n = L.tfb_profile_stage_name(k)
            if n:
                index[n.decode()] = k
        mask = 0
        for n in names:
            if n not in index:
                raise ValueError("unknown stage %r" % n)
            mask |= 1 << index[n]
    _check(L.tfb_profile_stages(ctypes.c_uint32(mask)), "tfb_profile_stages")


def profile_read() -> dict:
    """{stage name: (total ms, launches)} for the launches recorded since the last read."""
    L = lib()
    cap = 64
    ms = (ctypes.c_float * cap)()
    calls = (ctypes.c_int32 * cap)()
    n = min(cap, L.tfb_profile_read(ms, calls, cap))  # one read: it also clears the records
    return {L.tfb_profile_stage_name(i).decode(): (ms[i], calls[i]) for i in range(n) if calls[i]}
