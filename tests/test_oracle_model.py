"""Pins of the oracle's drafter as a whole: its forward against transformers' Qwen3 layers
(an independent library implementation of the same layer), and the context bookkeeping of
the pages (cortiq-engine dflash.rs, Drafter::queue_context / truncate / reset /
settle_rows, Drafter::block) as invariants."""
import numpy as np
import pytest

import dflash_inputs as di
import oracle

from hf_reference import HFDrafter

TINY = di.CONFIGS["tiny_f32"]
# the tiny drafter with norm weights near 1 and unit taps, so attention is far from flat
SHARP = TINY.replace(key="tiny_f32_sharp", norm_mean=1.0, taps_std=1.0, emb_std=1.0, seed=2001)
# a shrunken quantized drafter: every quantized path, two layers
QTINY = di.Config("q_tiny", 2, 256, 4, 2, 64, 512, 2, 1024, 8, 40, di.Q4_32, di.Q8_32, di.Q8_32, seed=2002)


def _setup(cfg, ctx=None, max_ctx=None, first=0):
    w = di.make_weights(cfg)
    m = oracle.Model(cfg, w, max_ctx=max_ctx or (cfg.ctx + 64))
    n = cfg.ctx if ctx is None else ctx
    taps = di.make_taps(cfg, 0, first, n)
    assert m.append(0, first, taps) == 0
    return w, m, taps


def _rel(a, b):
    return float(np.abs(a.astype(np.float64) - b).max() / np.abs(b).max())


@pytest.mark.parametrize("cfg", [TINY, SHARP, QTINY], ids=lambda c: c.key)
def test_forward_matches_transformers_qwen3_layers(cfg):
    first = 1000  # positions are absolute: the context need not start at 0
    w, m, taps = _setup(cfg, first=first)
    hf = HFDrafter(cfg, w)
    kv = hf.context_kv(taps, first)
    # the context the oracle holds equals the library's K and V of the same rows
    for li in range(cfg.layers):
        k, v = m.read_kv(li, 0, 0, cfg.ctx)
        kr = kv[li][0][0].permute(1, 0, 2).numpy()
        vr = kv[li][1][0].permute(1, 0, 2).numpy()
        tol = 1e-5 if cfg.body_fmt == di.F32 else 3e-3
        assert _rel(k, kr) < tol and _rel(v, vr) < tol
    for bi, anchor in enumerate([first + cfg.ctx, first + cfg.ctx - 5, first + cfg.ctx + 9]):
        h = di.make_block_input(cfg, 0, bi)
        got = m.block_forward([0], [anchor], h[None])[0]
        n = min(anchor, first + cfg.ctx) - first
        kv_a = [(k[:, :, :n], v[:, :, :n]) for k, v in kv]
        ref = hf.block_logits(kv_a, anchor, h)
        if cfg.body_fmt == di.F32:
            assert _rel(got, ref) < 2e-5
        else:
            assert _rel(got, ref) < 2e-3
            assert np.mean(got.argmax(1) == ref.argmax(1)) >= 0.99


def test_anchor_row_vs_draft_rows_non_causal():
    """Changing a later block row changes an earlier row's logits (no causal mask)."""
    _, m, _ = _setup(SHARP)
    h = di.make_block_input(SHARP, 0, 0)
    a = m.block_forward([0], [SHARP.ctx], h[None])[0]
    h2 = h.copy()
    h2[6] += 0.5
    b = m.block_forward([0], [SHARP.ctx], h2[None])[0]
    assert np.abs(a[2] - b[2]).max() > 1e-4 * np.abs(a).max()


def test_context_past_the_anchor_is_not_read():
    w, m, taps = _setup(SHARP)
    h = di.make_block_input(SHARP, 0, 3)
    a = m.block_forward([0], [40], h[None])[0]
    # rewrite positions 40.. with other rows: a block anchored at 40 must not see them
    assert m.append(0, 40, di.make_taps(SHARP, 7, 0, 24)) == 0
    b = m.block_forward([0], [40], h[None])[0]
    assert np.array_equal(a, b)
    # but one anchored later does
    c = m.block_forward([0], [64], h[None])[0]
    assert not np.array_equal(a, c)


def test_append_chunking_truncate_and_reset():
    cfg = QTINY
    w = di.make_weights(cfg)
    taps = di.make_taps(cfg, 0, 0, 40)
    m1 = oracle.Model(cfg, w, max_ctx=64)
    assert m1.append(0, 0, taps) == 0
    m2 = oracle.Model(cfg, w, max_ctx=64)
    for a, b in [(0, 13), (13, 14), (14, 40)]:
        assert m2.append(0, a, taps[a:b]) == 0
    for li in range(cfg.layers):
        assert all(np.array_equal(x, y) for x, y in zip(m1.read_kv(li, 0, 0, 40), m2.read_kv(li, 0, 0, 40)))
    # truncate then re-append the same rows == never truncated
    assert m2.truncate(0, 25) == 0 and m2.span(0) == (0, 25)
    assert m2.append(0, 25, taps[25:]) == 0
    for li in range(cfg.layers):
        assert all(np.array_equal(x, y) for x, y in zip(m1.read_kv(li, 0, 0, 40), m2.read_kv(li, 0, 0, 40)))
    # a position inside the span replaces it and what follows
    assert m2.append(0, 30, taps[10:12]) == 0 and m2.span(0) == (0, 32)
    # a gap starts over at the new position; so does a position before the first
    assert m2.append(0, 50, taps[:3]) == 0 and m2.span(0) == (50, 53)
    assert m2.append(0, 49, taps[:2]) == 0 and m2.span(0) == (49, 51)
    # K of a row depends on its taps and absolute position only
    k_new, _ = m2.read_kv(0, 0, 0, 2)
    m3 = oracle.Model(cfg, w, max_ctx=64)
    assert m3.append(0, 49, taps[:2]) == 0
    assert np.array_equal(k_new, m3.read_kv(0, 0, 0, 2)[0])
    # capacity: refused and nothing changes
    assert m2.append(0, 51, di.make_taps(cfg, 0, 0, 63)) == -2 and m2.span(0) == (49, 51)
    assert m2.reset(0) == 0 and m2.span(0) == (0, 0)
    assert m2.truncate(0, 5) == 0 and m2.span(0) == (0, 0)


def test_block_leaves_context_unchanged_and_sequences_are_independent():
    cfg = QTINY.replace(n_seqs=2)
    w = di.make_weights(cfg)
    m = oracle.Model(cfg, w, max_ctx=64, max_seqs=2)
    t0, t1 = di.make_taps(cfg, 0, 0, 40), di.make_taps(cfg, 1, 0, 33)
    assert m.append(0, 0, t0) == 0 and m.append(1, 100, t1) == 0
    before = [m.read_kv(li, s, 0, 33) for li in range(cfg.layers) for s in range(2)]
    h = np.stack([di.make_block_input(cfg, 0, 0), di.make_block_input(cfg, 1, 0)])
    both = m.block_forward([0, 1], [40, 133], h)
    after = [m.read_kv(li, s, 0, 33) for li in range(cfg.layers) for s in range(2)]
    assert all(np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) for a, b in zip(before, after))
    one = m.block_forward([1], [133], h[1:])
    assert np.array_equal(both[1], one[0])
    swapped = m.block_forward([1, 0], [133, 40], h[::-1].copy())
    assert np.array_equal(swapped[1], both[0])
    # bad arguments are refused
    with pytest.raises(ValueError):
        m.block_forward([0, 0], [40, 40], np.concatenate([h[:1], h[:1]]))
