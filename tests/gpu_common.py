"""Shared set-up of the GPU parity tests: one copy of each drafter's weights per process, the
oracle and the GPU library fed the same seeded inputs, and the parity measures."""
from __future__ import annotations

import sys
import time

import numpy as np

import dflash_inputs as di


def say(*a):
    print("[gpu-test]", *a, file=sys.stderr, flush=True)


_GEOM = ("layers", "hidden", "heads", "kv_heads", "head_dim", "intermediate", "n_taps", "vocab", "body_fmt", "fc_fmt",
         "head_fmt", "weight_std", "norm_mean", "norm_std", "conv_group", "conv_kernel", "conv_std")


def drafter_key(cfg: di.Config):
    """Workloads that share a drafter (same weight seed and shapes) share its weights."""
    return (cfg.weight_seed or cfg.seed,) + tuple(getattr(cfg, n) for n in _GEOM)


_WEIGHTS: dict = {}


def weights_for(cfg: di.Config) -> dict:
    key = drafter_key(cfg)
    if key not in _WEIGHTS:
        if len(_WEIGHTS) >= 2:
            _WEIGHTS.pop(next(iter(_WEIGHTS)))
        t = time.time()
        _WEIGHTS[key] = di.make_weights(cfg)
        say(f"weights of {cfg.key}: {time.time() - t:.1f} s")
    return _WEIGHTS[key]


def logits_parity(got: np.ndarray, ref: np.ndarray):
    """max |dlogit| / max |logit| and the share of rows whose top-1 agrees (lowest index on ties,
    numpy's argmax rule, on both sides)."""
    got = got.reshape(-1, got.shape[-1]).astype(np.float64)
    ref = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    rel = float(np.abs(got - ref).max() / np.abs(ref).max())
    top1 = float(np.mean(got.argmax(axis=1) == ref.argmax(axis=1)))
    return rel, top1


def cache_match(got, want, dtype=np.float32, max_frac=1e-3):
    """K/V rows read back against the oracle's: equal, except that a few elements may sit one
    unit in the last place of `dtype` away.  Each row element is the single f32 rounding of an
    f64-evaluated sum (f16 after that for an f16 cache); the GPU adds the f64 terms in another
    order than the oracle, so where the exact value lies within that order's f64 error of a
    rounding boundary (sums with heavy cancellation) the two round to neighbouring values: one
    element of one cache in a sweep of 2000 random drafters did.  Returns the count of such
    elements."""
    ints = {np.dtype(np.float32): (np.int32, 31), np.dtype(np.float16): (np.int16, 15)}[np.dtype(dtype)]
    g = np.ascontiguousarray(np.asarray(got, np.float32).astype(dtype)).view(ints[0]).astype(np.int64)
    w = np.ascontiguousarray(np.asarray(want, np.float32).astype(dtype)).view(ints[0]).astype(np.int64)
    mag = (1 << ints[1]) - 1
    og = np.where(g < 0, -(g & mag), g)  # sign-magnitude -> ordered integers (+0 and -0 meet)
    ow = np.where(w < 0, -(w & mag), w)
    dist = np.abs(og - ow)
    assert dist.max(initial=0) <= 1, f"cache rows differ by {dist.max()} units in the last place"
    n = int((dist > 0).sum())
    assert n <= max_frac * dist.size, f"{n} of {dist.size} cache elements one unit apart"
    return n


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))
