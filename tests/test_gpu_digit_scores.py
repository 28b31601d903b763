"""Attention scored from int8 digit splits of the queries and keys (dflash_set_score_mode,
DFLASH_SCORES_DIGITS) against the oracle, which scores in f64, on the cases the default mode
leaves to the f64 kernel (contexts under 16384 rows): small contexts with ragged tiles, several
sequences of different ranges in one call, windows and unrotated layers, truncation, blocks cut
to fewer rows with a head shortlist, an f16 cache, and the 8B-shaped drafter; and the default
mode's switch at 16384 context rows a call.  Both modes give the correctly rounded f32 of the exact
attention sums, so they are held to the same bar as every block: logits max |d| <= 2e-3 * max
|logit| and top-1 agreement >= 99.9%."""
import numpy as np
import pytest

import dflash_inputs as di
import oracle
from gpu_common import logits_parity, say, weights_for

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SMALL = di.CONFIGS["small_q"]  # head_dim 128, four q heads per kv head
SMALL2 = SMALL.replace(key="small_q_2l", layers=2, seed=2011)
Q8B = di.CONFIGS["qwen3_8b"]


def _pair(cfg, max_ctx, n_seqs=1, windows=None, rotary=None, mode=None):
    from block_draft_model_dflash_amd import DFLASH_SCORES_DIGITS, Drafter

    w = weights_for(cfg)
    om = oracle.Model(cfg, w, max_ctx=max_ctx, max_seqs=n_seqs)
    gm = Drafter(cfg, w, max_ctx=max_ctx, max_seqs=n_seqs)
    if windows is not None or rotary is not None:
        assert om.set_layer_options(windows, rotary) == 0
        gm.set_layer_options(windows, rotary)
    gm.set_score_mode(DFLASH_SCORES_DIGITS if mode is None else mode)
    return om, gm


def _append(cfg, om, gm, seq, pos, n, chunk=4096):
    for p0 in range(0, n, chunk):
        k = min(chunk, n - p0)
        taps = di.make_taps(cfg, seq, pos + p0, k)
        assert om.append(seq, pos + p0, taps) == 0
        gm.append(seq, pos + p0, taps)
    assert gm.span(seq) == om.span(seq)


def _block(cfg, om, gm, seqs, anchors, index, tol=2e-3, ref=None):
    h = np.stack([di.make_block_input(cfg, s, index) for s in seqs])
    say(f"{cfg.key}: digit-scored block seqs={list(seqs)} anchors={list(anchors)}")
    got = gm.block_forward(list(seqs), list(anchors), h)
    torch.cuda.synchronize()
    if ref is None:
        ref = om.block_forward(list(seqs), list(anchors), h)
    rel, top1 = logits_parity(got.cpu().numpy(), ref)
    say(f"{cfg.key}: rel {rel:.3e} top1 {top1:.4f} identical {bool(np.array_equal(got.cpu().numpy(), ref))}")
    assert rel <= tol and top1 >= 0.999
    return got, ref


@pytest.mark.timeout(300)
def test_digit_scores_small_drafter_blocks():
    """512 context rows (8 chunks of 64 keys, 4 tiles each), 32 blocks."""
    cfg = SMALL
    om, gm = _pair(cfg, cfg.ctx + 64)
    _append(cfg, om, gm, 0, 0, cfg.ctx)
    from block_draft_model_dflash_amd import DFLASH_SCORES_AUTO, DFLASH_SCORES_DIGITS

    assert gm.last_scores() == DFLASH_SCORES_AUTO  # no block yet
    for i in range(32):
        _block(cfg, om, gm, (0,), (cfg.ctx,), i)
    assert gm.last_scores() == DFLASH_SCORES_DIGITS


def test_digit_scores_sequences_windows_truncation():
    """Three sequences with ragged contexts in one call, a window on layer 0 and an unrotated
    layer 1, anchors inside and past the context, one before the first position (no context
    row), appends arriving a few rows at a time and a truncation."""
    cfg = SMALL2.replace(n_seqs=3)
    om, gm = _pair(cfg, 400, n_seqs=3, windows=[40, 0], rotary=[1, 0])
    _append(cfg, om, gm, 0, 0, 37)    # two tiles and a ragged tail
    _append(cfg, om, gm, 1, 500, 21)  # starts at 500
    _append(cfg, om, gm, 2, 0, 300)
    _block(cfg, om, gm, (0, 1, 2), (37, 515, 300), 0)
    _block(cfg, om, gm, (2, 0), (150, 30), 1)
    _block(cfg, om, gm, (1,), (400,), 2)  # an anchor before the first position
    for step in range(3):
        _append(cfg, om, gm, 0, 37 + 5 * step, 5)
        _block(cfg, om, gm, (0, 2), (42 + 5 * step, 300), 3 + step)
    for m in (om, gm):
        m.truncate(2, 90)
    _block(cfg, om, gm, (2, 1), (90, 521), 6)


def test_digit_scores_cut_blocks_and_shortlist():
    """Blocks cut to their first rows (fewer query rows than the 16 of a tile) and a head
    shortlist, two sequences."""
    cfg = SMALL.replace(n_seqs=2)
    om, gm = _pair(cfg, 300, n_seqs=2)
    _append(cfg, om, gm, 0, 0, 120)
    _append(cfg, om, gm, 1, 40, 61)
    for rows, head_rows in ((1, None), (5, 512), (8, None), (15, 16)):
        h = np.ascontiguousarray(np.stack([di.make_block_input(cfg, s, rows) for s in (0, 1)])[:, :rows])
        say(f"{cfg.key}: digit-scored cut block rows={rows} head_rows={head_rows}")
        got = gm.block_forward([0, 1], [120, 101], h, head_rows=head_rows)
        torch.cuda.synchronize()
        ref = om.block_forward([0, 1], [120, 101], h, head_rows=head_rows)
        assert got.shape == ref.shape
        rel, top1 = logits_parity(got.cpu().numpy(), ref)
        say(f"{cfg.key}: rel {rel:.3e} top1 {top1:.4f}")
        assert rel <= 2e-3 and top1 >= 0.999


def test_digit_scores_f16_cache():
    """Digits of the f16 values the cache holds, two sequences."""
    cfg = SMALL.replace(key="small_q_f16", kv_f16=True, n_seqs=2)
    om, gm = _pair(cfg, 400, n_seqs=2)
    _append(cfg, om, gm, 0, 0, 200)
    _append(cfg, om, gm, 1, 300, 77)
    _block(cfg, om, gm, (0, 1), (200, 377), 0)
    _block(cfg, om, gm, (1,), (377,), 1)


@pytest.mark.timeout(600)
def test_digit_and_f64_scores_8b_shaped():
    """The 8B-shaped drafter at 4096 context rows: the same blocks scored both ways, each
    against the oracle."""
    from block_draft_model_dflash_amd import DFLASH_SCORES_DIGITS, DFLASH_SCORES_F64

    cfg = Q8B
    om, gm = _pair(cfg, cfg.ctx + 64, mode=DFLASH_SCORES_F64)
    _append(cfg, om, gm, 0, 0, cfg.ctx)
    same = 0
    for i in range(4):
        anchor = cfg.ctx - 3 * i
        gm.set_score_mode(DFLASH_SCORES_F64)
        a, ref = _block(cfg, om, gm, (0,), (anchor,), i)
        a = a.clone()
        gm.set_score_mode(DFLASH_SCORES_DIGITS)
        assert gm.last_scores() == DFLASH_SCORES_F64
        b, _ = _block(cfg, om, gm, (0,), (anchor,), i, ref=ref)
        assert gm.last_scores() == DFLASH_SCORES_DIGITS
        same += int(torch.equal(a, b))
    say(f"{cfg.key}: {same} of 4 blocks bit-identical between the two score modes")


@pytest.mark.timeout(600)
def test_ragged_sequences_8b_shaped_both_modes():
    """The 8B-shaped drafter with four sequences of 8192, 3000, 100 and 0 context rows in one
    call (the longest sets the chunk size and count; the others' chunks past their rows, and every
    chunk of the empty one, do nothing), then three of them with anchors inside their contexts:
    f64 and digit scores each against the oracle."""
    from block_draft_model_dflash_amd import DFLASH_SCORES_DIGITS, DFLASH_SCORES_F64

    cfg = Q8B.replace(n_seqs=4)
    om, gm = _pair(cfg, 8192 + 64, n_seqs=4, mode=DFLASH_SCORES_F64)
    for seq, n in ((0, 8192), (1, 3000), (2, 100)):
        _append(cfg, om, gm, seq, 0, n)
    for i, (seqs, anchors) in enumerate((((0, 1, 2, 3), (8192, 3000, 100, 0)), ((2, 0, 1), (64, 5000, 2999)))):
        gm.set_score_mode(DFLASH_SCORES_F64)
        _, ref = _block(cfg, om, gm, seqs, anchors, i)
        gm.set_score_mode(DFLASH_SCORES_DIGITS)
        _block(cfg, om, gm, seqs, anchors, i, ref=ref)


@pytest.mark.timeout(300)
def test_default_mode_switches_at_16384_call_rows():
    """The default mode scores a call with digits from 16384 context rows, counted over the
    call's sequences: one sequence at 16383 / 16384 rows, then two whose rows add up to 16383 /
    16384.  Each block's logits equal those of the same block with that mode forced (the same
    kernels on the same inputs, with no atomics: bit for bit), and `last_scores` reports it."""
    from block_draft_model_dflash_amd import (DFLASH_SCORES_AUTO, DFLASH_SCORES_DIGITS, DFLASH_SCORES_F64,
                                              Drafter)

    cfg = SMALL.replace(n_seqs=2)
    gm = Drafter(cfg, weights_for(cfg), max_ctx=16400, max_seqs=2)
    for seq, n in ((0, 16384), (1, 8192)):
        for p0 in range(0, n, 4096):
            gm.append(seq, p0, di.make_taps(cfg, seq, p0, 4096))
    cases = [((0,), (16383,), DFLASH_SCORES_F64), ((0,), (16384,), DFLASH_SCORES_DIGITS),
             ((0, 1), (8192, 8191), DFLASH_SCORES_F64), ((0, 1), (8192, 8192), DFLASH_SCORES_DIGITS)]
    for i, (seqs, anchors, want) in enumerate(cases):
        h = np.stack([di.make_block_input(cfg, s, i) for s in seqs])
        say(f"{cfg.key}: default score mode, seqs={list(seqs)} anchors={list(anchors)}")
        gm.set_score_mode(DFLASH_SCORES_AUTO)
        auto = gm.block_forward(list(seqs), list(anchors), h).clone()
        assert gm.last_scores() == want
        gm.set_score_mode(want)
        forced = gm.block_forward(list(seqs), list(anchors), h)
        torch.cuda.synchronize()
        assert gm.last_scores() == want
        assert torch.equal(auto, forced)
    gm.close()


def test_score_mode_refused_where_the_geometry_cannot_take_it():
    from block_draft_model_dflash_amd import DFLASH_SCORES_DIGITS, DFlashError, Drafter

    cfg = di.CONFIGS["tiny_f32"]  # head_dim 64
    gm = Drafter(cfg, weights_for(cfg), max_ctx=128, max_seqs=1)
    with pytest.raises(DFlashError):
        gm.set_score_mode(DFLASH_SCORES_DIGITS)
    with pytest.raises(DFlashError):
        gm.set_score_mode(7)
    gm.close()
