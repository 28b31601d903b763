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


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))
