"""Per-layer windows, layers without rotary positions, the rows a window drops, and the head
shortlist (cortiq-engine dflash.rs: Geometry window / windows / no_rope, Drafter::settle_rows,
Drafter::block; Drafter::block_dev for the shortlist): the GPU library through its C ABI
against the oracle on the same seeded inputs.

The pages give no window values for these workloads; the windows below are chosen to cover
the cases the rule has: a window inside the context, one longer than the context, one so short
that most block rows see no context row at all, dropped rows reached by an anchor inside the
context, and sequences of one call with different ranges.  Bar as for the plain block: logits
max |d| <= 2e-3 * max |logit| (1e-5 for the f32 drafter) and top-1 agreement >= 99.9%; the
dropped-row counts are integers and must be equal."""
import numpy as np
import pytest

import dflash_inputs as di
import oracle
from gpu_common import logits_parity, say, weights_for

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SHARP2 = di.CONFIGS["tiny_f32"].replace(key="tiny_f32_sharp_2l", layers=2, norm_mean=1.0, taps_std=1.0,
                                        emb_std=1.0, seed=2003)
QTINY = di.Config("q_tiny", 2, 256, 4, 2, 64, 512, 2, 1024, 8, 40, di.Q4_32, di.Q8_32, di.Q8_32, seed=2002)
Q8B = di.CONFIGS["qwen3_8b"]


def _pair(cfg, windows, rotary, max_ctx, n_seqs=1):
    from block_draft_model_dflash_amd import Drafter

    w = weights_for(cfg)
    om = oracle.Model(cfg, w, max_ctx=max_ctx, max_seqs=n_seqs)
    gm = Drafter(cfg, w, max_ctx=max_ctx, max_seqs=n_seqs)
    assert om.set_layer_options(windows, rotary) == 0
    gm.set_layer_options(windows, rotary)
    return om, gm


def _append(cfg, om, gm, seq, pos, n, chunk=4096):
    for p0 in range(0, n, chunk):
        k = min(chunk, n - p0)
        taps = di.make_taps(cfg, seq, pos + p0, k)
        assert om.append(seq, pos + p0, taps) == 0
        gm.append(seq, pos + p0, taps)
    for li in range(cfg.layers):
        assert gm.dropped(seq, li) == om.dropped(seq, li), (seq, li)
    assert gm.span(seq) == om.span(seq)


def _block(cfg, om, gm, seqs, anchors, index, tol, head_rows=None):
    h = np.stack([di.make_block_input(cfg, s, index) for s in seqs])
    say(f"{cfg.key}: windowed block seqs={list(seqs)} anchors={list(anchors)} head_rows={head_rows}")
    got = gm.block_forward(list(seqs), list(anchors), h, head_rows=head_rows)
    torch.cuda.synchronize()
    ref = om.block_forward(list(seqs), list(anchors), h, head_rows=head_rows)
    rel, top1 = logits_parity(got.cpu().numpy(), ref)
    say(f"{cfg.key}: rel {rel:.3e} top1 {top1:.4f}")
    assert rel <= tol and top1 >= 0.999
    return got


def test_windows_f32_drafter():
    cfg = SHARP2
    om, gm = _pair(cfg, [10, 0], [1, 0], cfg.ctx + 64)
    _append(cfg, om, gm, 0, 100, cfg.ctx)
    assert om.dropped(0, 0) == 54  # 64 rows held > 2 * 10: the last 10 kept
    end = 100 + cfg.ctx
    for i, anchor in enumerate([end, end - 3, end + 5, end - 30, 50]):
        _block(cfg, om, gm, (0,), (anchor,), i, 1e-5)


def test_windows_quantized_sequences_appends_and_truncation():
    cfg = QTINY.replace(n_seqs=3)
    windows, rotary = [12, 5], [0, 1]
    om, gm = _pair(cfg, windows, rotary, 200, n_seqs=3)
    _append(cfg, om, gm, 0, 0, 37)  # two tiles and a ragged tail
    _append(cfg, om, gm, 1, 500, 21)
    _append(cfg, om, gm, 2, 0, 70)
    # one call, three ranges: at the end, inside the context, and far past it
    _block(cfg, om, gm, (0, 1, 2), (37, 515, 90), 0, 2e-3)
    _block(cfg, om, gm, (2, 0), (60, 30), 1, 2e-3)
    # rows arriving a few at a time drop incrementally
    for step in range(4):
        _append(cfg, om, gm, 0, 37 + 5 * step, 5)
        _block(cfg, om, gm, (0, 2), (42 + 5 * step, 70), 2 + step, 2e-3)
    # a truncation behind a window: the dropped rows stay unread
    for m in (om, gm):
        m.truncate(0, 30)
    assert [gm.dropped(0, li) for li in range(cfg.layers)] == [om.dropped(0, li) for li in range(cfg.layers)]
    _block(cfg, om, gm, (0,), (30,), 7, 2e-3)
    _append(cfg, om, gm, 0, 30, 6)
    _block(cfg, om, gm, (0, 1), (33, 521), 8, 2e-3)


@pytest.mark.timeout(600)
def test_windows_qwen3_8b_shaped_and_shortlist():
    """The 8B-shaped drafter at its full size with mixed layer options, and its head over the
    first 65536 rows (the device block's default shortlist)."""
    cfg = Q8B
    windows, rotary = [1000, 0, 4096, 64, 0], [1, 0, 1, 1, 0]
    om, gm = _pair(cfg, windows, rotary, cfg.ctx + 64)
    _append(cfg, om, gm, 0, 0, cfg.ctx)
    assert [om.dropped(0, li) for li in range(cfg.layers)] == [3096, 0, 0, 4032, 0]
    full = _block(cfg, om, gm, (0,), (cfg.ctx,), 0, 2e-3)
    _block(cfg, om, gm, (0,), (cfg.ctx - 700,), 1, 2e-3)
    short = _block(cfg, om, gm, (0,), (cfg.ctx,), 0, 2e-3, head_rows=65536)
    torch.cuda.synchronize()
    # the shortlist is the same product over fewer rows
    assert torch.equal(short, full[..., :65536])


def test_shortlist_and_option_errors():
    from block_draft_model_dflash_amd import DFlashError

    cfg = QTINY
    om, gm = _pair(cfg, None, None, cfg.ctx + 64)
    _append(cfg, om, gm, 0, 0, cfg.ctx)
    full = _block(cfg, om, gm, (0,), (cfg.ctx,), 0, 2e-3)
    for n in (16, 256, cfg.vocab):
        short = _block(cfg, om, gm, (0,), (cfg.ctx,), 0, 2e-3, head_rows=n)
        torch.cuda.synchronize()
        assert torch.equal(short, full[..., :n])
    h = di.make_block_input(cfg, 0, 0)[None]
    for n in (0, 8, 24 + cfg.vocab, 100):
        with pytest.raises(DFlashError):
            gm.block_forward([0], [cfg.ctx], h, head_rows=n)
    # options are fixed while context is held; nothing changes on a refused call
    with pytest.raises(DFlashError):
        gm.set_layer_options([4, 4], None)
    gm.reset(0)
    with pytest.raises(DFlashError):
        gm.set_layer_options([4, -1], None)
    assert [gm.dropped(0, li) for li in range(cfg.layers)] == [0, 0]


def _cut_block(cfg, om, gm, seqs, anchors, index, rows, tol, head_rows=None):
    h = np.ascontiguousarray(np.stack([di.make_block_input(cfg, s, index) for s in seqs])[:, :rows])
    say(f"{cfg.key}: block cut to {rows} rows, seqs={list(seqs)} head_rows={head_rows}")
    got = gm.block_forward(list(seqs), list(anchors), h, head_rows=head_rows)
    torch.cuda.synchronize()
    ref = om.block_forward(list(seqs), list(anchors), h, head_rows=head_rows)
    assert got.shape == ref.shape
    rel, top1 = logits_parity(got.cpu().numpy(), ref)
    say(f"{cfg.key}: rel {rel:.3e} top1 {top1:.4f}")
    assert rel <= tol and top1 >= 0.999


def test_block_cut_to_its_first_rows():
    """The device block's cut (gpu_wgpu/dflash_dev.rs, Dev::block): the anchor and the next
    rows only, several sequences in one call and with windows on."""
    from block_draft_model_dflash_amd import DFlashError

    cfg = QTINY.replace(n_seqs=3)
    om, gm = _pair(cfg, [12, 0], None, 200, n_seqs=3)
    _append(cfg, om, gm, 0, 0, 37)
    _append(cfg, om, gm, 1, 500, 21)
    _append(cfg, om, gm, 2, 0, 70)
    for rows in (1, 5, 8):
        _cut_block(cfg, om, gm, (0, 1, 2), (37, 521, 70), rows, rows, 2e-3)
    _cut_block(cfg, om, gm, (2,), (70,), 3, 4, 2e-3, head_rows=32)
    h = np.zeros((1, 9, cfg.hidden), np.float32)  # more rows than the block holds
    with pytest.raises(DFlashError):
        gm.block_forward([0], [37], h)


@pytest.mark.timeout(600)
def test_block_cut_qwen3_8b_shaped():
    cfg = Q8B
    om, gm = _pair(cfg, None, None, cfg.ctx + 64)
    _append(cfg, om, gm, 0, 0, cfg.ctx)
    _cut_block(cfg, om, gm, (0,), (cfg.ctx,), 0, 8, 2e-3)
    _cut_block(cfg, om, gm, (0,), (cfg.ctx,), 1, 8, 2e-3, head_rows=65536)
