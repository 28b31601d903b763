"""Pins of the per-layer attention options of the drafter (cortiq-engine dflash.rs: Geometry
window / windows / no_rope with window_of and rotary; Drafter::settle_rows dropping the rows
that fell out of a window; Drafter::block's per-row window mask) and of the head shortlist the
device block takes (Drafter::block_dev: the head's first rows).

The windowed and unrotated forward is checked against transformers' Qwen3 layers with an
explicit additive mask and identity rotary embeddings, with the context slice and the dropped
row counts worked out here by hand from the pages' rules."""
import numpy as np

import dflash_inputs as di
import oracle
import test_oracle_model as TM
from hf_reference import HFDrafter


def _rel(a, b):
    return float(np.abs(a.astype(np.float64) - b).max() / np.abs(b).max())


def _model(cfg, w, windows=None, rotary=None, max_ctx=None):
    m = oracle.Model(cfg, w, max_ctx=max_ctx or (cfg.ctx + 64))
    assert m.set_layer_options(windows, rotary) == 0
    return m


def _hf_inputs(cfg, kv, first, end, dropped, windows, anchor):
    """The context slice and per-row masks of every layer, from Drafter::block's rule:
    base = first + dropped, hi = max(min(anchor, end), base), lo = base or, under a window w,
    clamp(anchor + 1 - w, base, hi); row r sees positions >= anchor + r + 1 - w."""
    B = cfg.block
    kv_a, masks = [], []
    for li in range(cfg.layers):
        w = windows[li]
        base = first + dropped[li]
        hi = max(min(anchor, end), base)
        lo = base if w == 0 else min(max(anchor + 1 - w, base), hi)
        k, v = kv[li]
        kv_a.append((k[:, :, lo - first:hi - first], v[:, :, lo - first:hi - first]))
        if w == 0:
            masks.append(None)
        else:
            pos = lo + np.arange(hi - lo)
            masks.append(pos[None, :] < (anchor + np.arange(B) + 1 - w)[:, None])
    return kv_a, masks


def _check(cfg, got, ref):
    if cfg.body_fmt == di.F32:
        assert _rel(got, ref) < 2e-5
    else:
        assert _rel(got, ref) < 2e-3
        assert np.mean(got.argmax(1) == ref.argmax(1)) >= 0.99


# two f32 layers with sharp attention: the options of one layer reach the next unquantized, so
# the comparison holds to f32 rounding (a quantized drafter amplifies a one-ulp difference at an
# int8 code into ~1% of the logits, which would hide a small mistake)
SHARP2 = TM.SHARP.replace(key="tiny_f32_sharp_2l", layers=2, seed=2003)


def test_windows_and_no_rope_match_transformers():
    # (drafter, windows, rotary, dropped after one append of the whole context, by hand)
    cases = [
        # one layer: window 10 of 64 rows; 64 > 2*10 keeps the last 10, so 54 dropped
        (TM.SHARP, [10], [0], [54]),
        # layer 0 a window of 12 (64 > 24: 52 dropped), layer 1 all rows and no rotary
        (SHARP2, [12, 0], [1, 0], [52, 0]),
        # layer 0 all rows and no rotary, layer 1 a window of 40 (64 <= 80: nothing dropped)
        (SHARP2, [0, 40], [0, 1], [0, 0]),
    ]
    for cfg, windows, rotary, dropped in cases:
        first = 300
        w = di.make_weights(cfg)
        m = _model(cfg, w, windows, rotary)
        taps = di.make_taps(cfg, 0, first, cfg.ctx)
        assert m.append(0, first, taps) == 0
        assert [m.dropped(0, li) for li in range(cfg.layers)] == dropped
        hf = HFDrafter(cfg, w)
        kv = hf.context_kv(taps, first, rotary=rotary)
        plain = _model(cfg, w)
        assert plain.append(0, first, taps) == 0
        end = first + cfg.ctx
        # at the end, inside the context (the window reaches back into the dropped rows), past it
        for bi, anchor in enumerate([end, end - 3, end + 5, end - 30, end - 55]):
            h = di.make_block_input(cfg, 0, bi)
            got = m.block_forward([0], [anchor], h[None])[0]
            kv_a, masks = _hf_inputs(cfg, kv, first, end, dropped, windows, anchor)
            ref = hf.block_logits(kv_a, anchor, h, masks=masks, rotary=rotary)
            _check(cfg, got, ref)
            # the options change the result well beyond the tolerance (the pin has teeth)
            other = plain.block_forward([0], [anchor], h[None])[0]
            assert _rel(other, got) > 1e-2


def test_window_drop_bookkeeping():
    cfg = TM.QTINY
    w = di.make_weights(cfg)
    windows = [4, 0]
    m = _model(cfg, w, windows)
    taps = di.make_taps(cfg, 0, 0, 64)
    # a layer holding more than twice its window keeps the last window's worth (settle_rows)
    assert m.append(0, 0, taps[:10]) == 0
    assert (m.dropped(0, 0), m.dropped(0, 1)) == (6, 0)  # 10 > 8: keep 4
    assert m.append(0, 10, taps[10:13]) == 0
    assert m.dropped(0, 0) == 6  # holds 7 <= 8
    assert m.append(0, 13, taps[13:15]) == 0
    assert m.dropped(0, 0) == 11  # holds 9 > 8: keep 4
    # truncate clips the dropped rows to what it keeps
    assert m.truncate(0, 8) == 0
    assert m.dropped(0, 0) == 8 and m.span(0) == (0, 8)
    hf = HFDrafter(cfg, w)
    kv = hf.context_kv(taps[:12], 0)
    h = di.make_block_input(cfg, 0, 0)
    # layer 0 holds none of positions 0..7 now: its block attends to itself only
    got = m.block_forward([0], [8], h[None])[0]
    kv_a, masks = _hf_inputs(cfg, kv, 0, 8, [8, 0], windows, 8)
    assert kv_a[0][0].shape[2] == 0 and kv_a[1][0].shape[2] == 8
    _check(cfg, got, hf.block_logits(kv_a, 8, h, masks=masks))
    # rows appended again after the truncation are held; the dropped ones stay dropped
    assert m.append(0, 8, taps[8:12]) == 0
    assert m.dropped(0, 0) == 8  # holds 4
    got = m.block_forward([0], [10], h[None])[0]
    kv_a, masks = _hf_inputs(cfg, kv, 0, 12, [8, 0], windows, 10)
    assert kv_a[0][0].shape[2] == 2  # positions 8, 9 (the window would start at 7)
    _check(cfg, got, hf.block_logits(kv_a, 10, h, masks=masks))
    # appending in pieces or at once drops different rows, but a block at the end reads the
    # same window either way
    m2 = _model(cfg, w, windows)
    assert m2.append(0, 0, taps[:12]) == 0
    assert m2.dropped(0, 0) == 8
    m3 = _model(cfg, w, windows)
    for p in range(0, 12, 3):
        assert m3.append(0, p, taps[p:p + 3]) == 0
    assert m3.dropped(0, 0) == 5  # 9 > 8 after the third piece: keep 4; then holds 7
    np.testing.assert_array_equal(m2.block_forward([0], [12], h[None]), m3.block_forward([0], [12], h[None]))
    # a gap starts over: nothing dropped; so does a reset
    assert m3.append(0, 100, taps[:5]) == 0
    assert m3.dropped(0, 0) == 0 and m3.span(0) == (100, 105)
    assert m2.reset(0) == 0 and m2.dropped(0, 0) == 0
    # the options are fixed once rows are held
    assert m3.set_layer_options([0, 0]) == -1
    assert _model(cfg, w).set_layer_options([-1, 0]) == -1


def test_no_rope_everywhere_is_position_free():
    cfg = TM.QTINY
    w = di.make_weights(cfg)
    taps = di.make_taps(cfg, 0, 0, cfg.ctx)
    h = di.make_block_input(cfg, 0, 0)
    out = {}
    for rot in (0, 1):
        for first, gap in ((0, 0), (777, 0), (0, 50)):
            m = _model(cfg, w, rotary=[rot] * cfg.layers)
            assert m.append(0, first, taps) == 0
            out[rot, first, gap] = m.block_forward([0], [first + cfg.ctx + gap], h[None])[0]
    # without rotary positions neither where the rows sit nor how far the block is from the
    # context matters; with them the distance does
    np.testing.assert_array_equal(out[0, 0, 0], out[0, 777, 0])
    np.testing.assert_array_equal(out[0, 0, 0], out[0, 0, 50])
    assert _rel(out[1, 0, 50], out[1, 0, 0]) > 1e-2


def test_shortlist_head_is_a_prefix():
    for cfg in (TM.SHARP, TM.QTINY):
        w = di.make_weights(cfg)
        m = _model(cfg, w)
        assert m.append(0, 0, di.make_taps(cfg, 0, 0, cfg.ctx)) == 0
        h = di.make_block_input(cfg, 0, 1)
        full = m.block_forward([0], [cfg.ctx], h[None])
        for n in (16, cfg.vocab // 4, cfg.vocab):
            np.testing.assert_array_equal(m.block_forward([0], [cfg.ctx], h[None], head_rows=n), full[..., :n])


def test_block_cut_to_its_first_rows_matches_transformers():
    """The device block may run only the anchor and the next rows (gpu_wgpu/dflash_dev.rs,
    Dev::block): those rows are then the whole block, attention among them included."""
    cfg = SHARP2
    first = 40
    w = di.make_weights(cfg)
    m = oracle.Model(cfg, w, max_ctx=cfg.ctx + 64, max_seqs=2)
    taps = di.make_taps(cfg, 0, first, cfg.ctx)
    for s in (0, 1):  # two sequences of one call, the same context
        assert m.append(s, first, taps) == 0
    hf = HFDrafter(cfg, w)
    kv = hf.context_kv(taps, first)
    h = np.stack([di.make_block_input(cfg, 0, 3), di.make_block_input(cfg, 0, 4)])
    full = m.block_forward([0, 1], [first + cfg.ctx] * 2, h)
    for b in (2, 5, cfg.block):
        got = m.block_forward([0, 1], [first + cfg.ctx] * 2, np.ascontiguousarray(h[:, :b]))
        assert got.shape == (2, b, cfg.vocab)
        for s in (0, 1):
            _check(cfg, got[s], hf.block_logits(kv, first + cfg.ctx, h[s, :b]))
        if b < cfg.block:  # the later mask rows shape the earlier ones: cutting them changes those
            assert _rel(got, full[:, :b]) > 1e-3
        else:
            np.testing.assert_array_equal(got, full)
