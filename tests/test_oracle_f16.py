"""Pins of the f16 K/V cache (an f16 cache is the pages' throughput variant of the f32 one:
cortiq-engine dflash.rs keeps f32 rows; this variant stores each element rounded to IEEE
binary16): the oracle's rounding against numpy's float16 conversion on edge values and random
bit patterns, the cache it holds against the f32 cache rounded by numpy, and the block against
transformers' layers over the f16-rounded context."""
import numpy as np
import torch

import dflash_inputs as di
import oracle
import test_oracle_model as TM
from hf_reference import HFDrafter

SHARP2 = TM.SHARP.replace(key="tiny_f32_sharp_2l", layers=2, seed=2003)


def _rel(a, b):
    return float(np.abs(a.astype(np.float64) - b).max() / np.abs(b).max())


def test_round_f16_against_numpy():
    edges = np.array([0.0, -0.0, 1.0, 65504.0, 65519.996, 65520.0, 1e6, -65520.0, 2.0 ** -24, 2.0 ** -25,
                      3 * 2.0 ** -26, 2.0 ** -25 * 1.0000001, 2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -11),
                      1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 1 + 2.0 ** -11 + 2.0 ** -20, np.inf, -np.inf],
                     np.float32)
    r = np.random.default_rng(7)
    bits = r.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    exps = (bits >> 23) & 0xFF
    bits = bits[(exps >= 100) & (exps <= 145)]  # around the binary16 range, subnormals to overflow
    x = np.concatenate([edges, bits.view(np.float32)])
    with np.errstate(over="ignore"):  # the overflow to infinity is part of the check
        want = x.astype(np.float16).astype(np.float64)
    np.testing.assert_array_equal(oracle.round_f16(x), want)


def test_f16_cache_holds_the_rounded_rows():
    for cfg in (SHARP2, TM.QTINY):
        w = di.make_weights(cfg)
        taps = di.make_taps(cfg, 0, 0, cfg.ctx)
        m32 = oracle.Model(cfg, w, max_ctx=cfg.ctx + 64)
        m16 = oracle.Model(cfg.replace(kv_f16=True), w, max_ctx=cfg.ctx + 64)
        for m in (m32, m16):
            assert m.append(0, 0, taps) == 0
        for li in range(cfg.layers):
            k32, v32 = m32.read_kv(li, 0, 0, cfg.ctx)
            k16, v16 = m16.read_kv(li, 0, 0, cfg.ctx)
            np.testing.assert_array_equal(k16, k32.astype(np.float16).astype(np.float32))
            np.testing.assert_array_equal(v16, v32.astype(np.float16).astype(np.float32))


def test_f16_cache_block_matches_transformers():
    cfg = SHARP2
    first = 77
    w = di.make_weights(cfg)
    taps = di.make_taps(cfg, 0, first, cfg.ctx)
    m16 = oracle.Model(cfg.replace(kv_f16=True), w, max_ctx=cfg.ctx + 64)
    m32 = oracle.Model(cfg, w, max_ctx=cfg.ctx + 64)
    for m in (m16, m32):
        assert m.append(0, first, taps) == 0
    hf = HFDrafter(cfg, w)
    kv = [(k.to(torch.float16).double(), v.to(torch.float16).double()) for k, v in hf.context_kv(taps, first)]
    for bi, anchor in enumerate([first + cfg.ctx, first + cfg.ctx - 11]):
        h = di.make_block_input(cfg, 0, bi)
        got = m16.block_forward([0], [anchor], h[None])[0]
        n = anchor - first
        ref = hf.block_logits([(k[:, :, :n], v[:, :, :n]) for k, v in kv], anchor, h)
        # two f32 layers: the f64 evaluations agree to f32 rounding (~2e-7 here), far inside the
        # f16 rounding's own effect on the logits (~8e-6), so a cache kept in f32 would fail
        assert _rel(got, ref) < 1e-6
        assert _rel(m32.block_forward([0], [anchor], h[None])[0], got) > 3e-6
