"""Helpers for the GPU tests: move seeded inputs to the device and run the
library through its C ABI.  The CPU oracle is called from the tests."""
from __future__ import annotations

import numpy as np

import transformer_decoder_block_rmsnorm_amd as tfb
from tests.inputs import activations, block_weights

BF16_TOL = 2e-2
F32_TOL = 1e-4


def torch_dtype(cfg):
    import torch
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def to_dev(f32: np.ndarray, bits: np.ndarray | None, dev="cuda"):
    import torch
    if bits is not None:
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(dev)


def dev_weights(cfg, layer=None, gains="ones"):
    w32, bits = block_weights(cfg, layer=layer, gains=gains)
    w = {k: to_dev(v, None if bits is None else bits[k]) for k, v in w32.items()}
    return w32, w


def dev_x(cfg, B, T, name="x"):
    x32, bits = activations(cfg, B, T, name)
    return x32, to_dev(x32, bits)


def to_np(t) -> np.ndarray:
    return t.float().cpu().numpy()


def folded_rows(cfg, M: int, T: int, fold: int) -> int:
    """Rows per sequence whose RMSNorms that follow a GEMM the library folds
    into the GEMMs around them (config fold_norms): every row of a bf16 call
    over more rows than its weight-streaming GEMMs take (64), else none."""
    return T if fold and cfg.dtype == "bf16" and M > 64 else 0


def tol(cfg) -> float:
    return BF16_TOL if cfg.dtype == "bf16" else F32_TOL


def check(name: str, got, ref, bound: float) -> float:
    """The stated bound, as written: max |got - ref| <= bound * rms(ref) over
    every value.  Prints the measured figure so every run records it."""
    from tests.inputs import rel_err
    e = rel_err(got, ref)
    print("  %-28s max|err|/rms = %.4g  (bound %.0e)" % (name, e, bound), flush=True)
    assert e <= bound, (name, e, bound)
    return e


class Checks:
    """Runs several bound checks, printing each measured figure, and fails
    at the end with every one that missed (one GPU run reports them all)."""

    def __init__(self):
        self.failed = []

    def __call__(self, name: str, got, ref, bound: float) -> float:
        from tests.inputs import rel_err
        e = rel_err(got, ref)
        print("  %-28s max|err|/rms = %.4g  (bound %.0e)" % (name, e, bound), flush=True)
        if not e <= bound:
            self.failed.append((name, e, bound))
        return e

    def against_floor(self, name: str, got, ref, exact, bound: float, sigma_slack: float = 1.1) -> float:
        """The bound, or the exact evaluation's own distance from the oracle
        where that is larger.  exact: the same quantity from the fp64
        evaluation of the method (bf16 operands rounded where the oracle
        rounds them, stored like the GPU stores it).  Limit on the largest
        error: max(bound, e_max + 2 sigma) of the exact evaluation's error (a
        maximum over many values moves by a fraction of sigma between two
        draws); the GPU's error sigma must also stay within sigma_slack of the
        exact evaluation's."""
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        exact = np.asarray(exact, np.float64)
        r = np.sqrt(np.mean(ref * ref))
        eg, ee = (got - ref) / r, (exact - ref) / r
        gmax, emax, gs, es = np.abs(eg).max(), np.abs(ee).max(), eg.std(), ee.std()
        limit = max(bound, emax + 2 * es)
        print("  %-28s max|err|/rms = %.4g sigma %.3g | exact method: max %.4g sigma %.3g | limit %.4g" % (
            name, gmax, gs, emax, es, limit), flush=True)
        if not gmax <= limit:
            self.failed.append((name, gmax, limit))
        if not gs <= sigma_slack * max(es, 1e-3 * bound):
            self.failed.append((name + " sigma", gs, es))
        return gmax

    def flips(self, name: str, got, ref_rounded):
        """Reported, not bounded: the share of bf16 values that differ from the
        oracle's bf16 operand (the two sides rounded slightly different fp32
        values to neighbouring bf16 values)."""
        _, n = bf16_gap(got, ref_rounded)
        frac = n / max(1, np.asarray(got).size)
        print("  %-28s bf16 values differing from the oracle's operand: %d (%.3g%%)" % (name, n, 100 * frac),
              flush=True)

    def done(self):
        assert not self.failed, self.failed


def bf16_gap(got, ref):
    """(largest gap in bf16 steps, number of values not bitwise equal); the
    steps are counted through zero, so -tiny and +tiny are close."""
    def ordered(x):
        u = np.asarray(x, np.float32).view(np.uint32).astype(np.int64)
        assert not np.any(u & 0xFFFF), "values must be bf16"
        m = (u >> 16) & 0x7FFF
        return np.where(u >> 31, -m, m)
    diff = np.abs(ordered(got) - ordered(ref))
    return int(diff.max(initial=0)), int(np.count_nonzero(diff))


def check_cache(name: str, cfg, got, ref_pre):
    """Cache rows against the oracle's k or v as computed, before any bf16
    storage (the oracle's *_pre intermediates): the stored row carries only
    its own rounding plus the compute difference."""
    return check(name, got, ref_pre, tol(cfg))


def cache_rows(pre, Hkv: int) -> np.ndarray:
    """[B, T, Hkv*dh] rows of k or v -> the cache layout [B, Hkv, T, dh]."""
    B, T, kvd = pre.shape
    return np.ascontiguousarray(pre.reshape(B, T, Hkv, kvd // Hkv).transpose(0, 2, 1, 3))


def new_cache(cfg, B, t_max, fill=float("nan")):
    import torch
    k = torch.full((B, cfg.n_kv_heads, t_max, cfg.d // cfg.n_heads), fill, dtype=torch_dtype(cfg), device="cuda")
    return k, k.clone()


def widen_cache(t) -> np.ndarray:
    return np.ascontiguousarray(to_np(t), dtype=np.float32)
