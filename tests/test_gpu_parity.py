"""Whole-path parity through the C ABI: context append (K/V cache) and block logits of the GPU
library against the CPU oracle on the same seeded inputs.

Bar (the drafter's stated tolerance): logits max |d| <= 2e-3 * max |logit| and top-1 agreement
>= 99.9% of rows; the K/V cache is held to the same relative bound.  The f32 workload has no
quantizer, so it is held to 1e-5, the f32 rounding of a few layers."""
import numpy as np
import pytest

import dflash_inputs as di
import oracle
from gpu_common import logits_parity, rel_err, say, weights_for

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TINY = di.CONFIGS["tiny_f32"]
SHARP = TINY.replace(key="tiny_f32_sharp", norm_mean=1.0, taps_std=1.0, emb_std=1.0, seed=2001)
QTINY = di.Config("q_tiny", 2, 256, 4, 2, 64, 512, 2, 1024, 8, 40, di.Q4_32, di.Q8_32, di.Q8_32, seed=2002)
SMALL = di.CONFIGS["small_q"]
Q8B = di.CONFIGS["qwen3_8b"]
LONG = di.CONFIGS["qwen3_8b_long"]
BATCH = di.CONFIGS["qwen3_8b_batch8"]


def _scores(name):
    import block_draft_model_dflash_amd as D

    return getattr(D, "DFLASH_SCORES_" + name)


def _pair(cfg, ctx, max_ctx, n_seqs=1, first=0, chunk=4096):
    from block_draft_model_dflash_amd import Drafter

    w = weights_for(cfg)
    om = oracle.Model(cfg, w, max_ctx=max_ctx, max_seqs=n_seqs)
    say(f"{cfg.key}: create on the GPU")
    gm = Drafter(cfg, w, max_ctx=max_ctx, max_seqs=n_seqs)
    for s in range(n_seqs):
        for p0 in range(0, ctx, chunk):
            n = min(chunk, ctx - p0)
            taps = di.make_taps(cfg, s, first + p0, n)
            say(f"{cfg.key}: append rows {p0}..{p0 + n} of sequence {s}")
            assert om.append(s, first + p0, taps) == 0
            gm.append(s, first + p0, taps)
            torch.cuda.synchronize()
    return w, om, gm


def _kv_check(cfg, om, gm, seq, rows, tol):
    for li in range(cfg.layers):
        for r0, n in rows:
            ko, vo = om.read_kv(li, seq, r0, n)
            kg, vg = gm.read_kv(li, seq, r0, n)
            torch.cuda.synchronize()
            ek, ev = rel_err(kg.cpu().numpy(), ko), rel_err(vg.cpu().numpy(), vo)
            assert ek <= tol and ev <= tol, (li, r0, ek, ev)


class Pooled:
    """Parity over every row of every block evaluated on a workload: max |dlogit| over all of
    them against max |logit| over all of them, and the share of rows whose top-1 agrees (lowest
    index on ties on both sides); blocks bit-identical to the oracle are counted too."""

    def __init__(self, key):
        self.key, self.diff, self.ref, self.agree, self.rows, self.blocks, self.equal = key, 0.0, 0.0, 0, 0, 0, 0

    def add(self, got, ref):
        got = np.asarray(got, np.float32).reshape(-1, got.shape[-1])
        ref = np.asarray(ref, np.float32).reshape(-1, ref.shape[-1])
        self.diff = max(self.diff, float(np.abs(got.astype(np.float64) - ref).max()))
        self.ref = max(self.ref, float(np.abs(ref).max()))
        self.agree += int((got.argmax(axis=1) == ref.argmax(axis=1)).sum())
        self.rows += got.shape[0]
        self.blocks += 1
        self.equal += int(np.array_equal(got, ref))

    def check(self, tol, top1_min, rows_min):
        rel, top1 = self.diff / self.ref, self.agree / self.rows
        say(f"{self.key}: {self.blocks} blocks, {self.rows} rows: max|d| / max|logit| {rel:.3e}, top-1 "
            f"{self.agree}/{self.rows}, {self.equal} blocks bit-identical")
        assert self.rows >= rows_min, (self.key, self.rows)
        assert rel <= tol, (self.key, rel)
        assert top1 >= top1_min, (self.key, top1)


def _blocks(cfg, om, gm, cases, tol, top1_min):
    rels, agree = [], []
    for seqs, anchors, index in cases:
        h = np.stack([di.make_block_input(cfg, s, index) for s in seqs])
        say(f"{cfg.key}: block seqs={list(seqs)} anchors={list(anchors)}")
        got = gm.block_forward(list(seqs), list(anchors), h)
        torch.cuda.synchronize()
        ref = om.block_forward(list(seqs), list(anchors), h)
        rel, top1 = logits_parity(got.cpu().numpy(), ref)
        say(f"{cfg.key}: rel {rel:.3e} top1 {top1:.4f}")
        rels.append(rel)
        agree.append(top1)
        assert rel <= tol
    assert np.mean(agree) >= top1_min


@pytest.mark.parametrize("cfg", [TINY, SHARP], ids=lambda c: c.key)
def test_f32_drafter(cfg):
    _, om, gm = _pair(cfg, cfg.ctx, cfg.ctx + 64, first=100)
    _kv_check(cfg, om, gm, 0, [(0, cfg.ctx)], 1e-5)
    cases = [((0,), (100 + cfg.ctx,), 0), ((0,), (100 + cfg.ctx - 9,), 1), ((0,), (100 + cfg.ctx + 5,), 2),
             ((0,), (50,), 3)]  # an anchor before the first position: no context at all
    _blocks(cfg, om, gm, cases, 1e-5, 1.0)


def test_quantized_small_two_sequences_ragged():
    cfg = QTINY.replace(n_seqs=2)
    _, om, gm = _pair(cfg, 37, 100, n_seqs=2)  # 37 rows: two tiles and a ragged tail
    for m in (om, gm):
        m.append(1, 500, di.make_taps(cfg, 1, 500, 21))  # a gap: sequence 1 starts over at 500
    _kv_check(cfg, om, gm, 0, [(0, 37)], 2e-3)
    _kv_check(cfg, om, gm, 1, [(0, 21)], 2e-3)
    _blocks(cfg, om, gm, [((0, 1), (37, 521), 0), ((1, 0), (510, 30), 1), ((1,), (600, ), 2)], 2e-3, 0.999)


def test_append_chunking_truncate_and_empty_on_gpu():
    """Rows are independent: any chunking gives the same cache bits; truncate + re-append is
    a no-op; n = 0 only moves the bookkeeping."""
    from block_draft_model_dflash_amd import Drafter

    cfg = QTINY
    w = weights_for(cfg)
    taps = di.make_taps(cfg, 0, 0, 300)
    a = Drafter(cfg, w, max_ctx=320)
    a.append(0, 0, taps)
    b = Drafter(cfg, w, max_ctx=320)
    for c0, c1 in [(0, 1), (1, 129), (129, 130), (130, 300)]:
        b.append(0, c0, taps[c0:c1])
    b.truncate(0, 200)
    assert b.span(0) == (0, 200)
    b.append(0, 200, taps[200:])
    b.append(0, 300, np.zeros((0, cfg.tap_width), np.float32))
    assert b.span(0) == (0, 300)
    for li in range(cfg.layers):
        ka, va = a.read_kv(li, 0, 0, 300)
        kb, vb = b.read_kv(li, 0, 0, 300)
        torch.cuda.synchronize()
        assert torch.equal(ka, kb) and torch.equal(va, vb)
    from block_draft_model_dflash_amd import DFlashError

    with pytest.raises(DFlashError):
        b.append(0, 290, di.make_taps(cfg, 0, 0, 40))  # 330 rows > 320
    assert b.span(0) == (0, 300)


def _scale_blocks(cfg, om, gm, pooled, seqs, anchors, index):
    h = np.stack([di.make_block_input(cfg, s, index) for s in seqs])
    got = gm.block_forward(list(seqs), list(anchors), h)
    torch.cuda.synchronize()
    ref = om.block_forward(list(seqs), list(anchors), h)
    pooled.add(got.cpu().numpy(), ref)


@pytest.mark.timeout(300)
def test_tiny_f32_drafter_128_blocks():
    """The tiny f32 workload as its measurement states it: context positions 0..63, 128 blocks
    anchored at 64, each with its own anchor row.  No quantizer: held to 1e-5."""
    cfg = TINY
    _, om, gm = _pair(cfg, cfg.ctx, cfg.ctx + 64)
    pooled = Pooled(cfg.key)
    for i in range(128):
        _scale_blocks(cfg, om, gm, pooled, (0,), (cfg.ctx,), i)
    pooled.check(1e-5, 1.0, 1024)


@pytest.mark.timeout(300)
def test_small_quantized_drafter():
    """The small quantized workload: 512 context rows, 64 blocks of 16 rows (1024 rows)."""
    cfg = SMALL
    _, om, gm = _pair(cfg, cfg.ctx, cfg.ctx + 64)
    _kv_check(cfg, om, gm, 0, [(0, 64), (448, 64)], 2e-3)
    pooled = Pooled(cfg.key)
    for i in range(64):
        _scale_blocks(cfg, om, gm, pooled, (0,), (cfg.ctx,), i)
    pooled.check(2e-3, 0.999, 1024)


@pytest.mark.timeout(600)
def test_qwen3_8b_shaped_drafter():
    """The 8B-shaped drafter at its full size: 4096 context rows, 64 blocks of 16 rows (1024
    rows), 151936 logits each."""
    cfg = Q8B
    _, om, gm = _pair(cfg, cfg.ctx, cfg.ctx + 64)
    _kv_check(cfg, om, gm, 0, [(0, 32), (2000, 16), (4064, 32)], 2e-3)
    pooled = Pooled(cfg.key)
    for i in range(64):
        _scale_blocks(cfg, om, gm, pooled, (0,), (cfg.ctx,), i)
        if i % 16 == 15:
            say(f"{cfg.key}: {i + 1} blocks")
    pooled.check(2e-3, 0.999, 1024)
    assert gm.last_scores() == _scores("F64")  # 4096 context rows: the default scores in f64


@pytest.mark.timeout(900)
def test_long_context_append_then_block():
    """The long-context workload at its full size: a 32768-row context, then 64 steps of 16 new
    context rows appended and a block anchored after them (the step the benchmark times)."""
    cfg = LONG
    steps = 64
    _, om, gm = _pair(cfg, cfg.ctx, cfg.ctx + steps * cfg.append_per_block + 64)
    _kv_check(cfg, om, gm, 0, [(0, 16), (20000, 16), (32752, 16)], 2e-3)
    pooled = Pooled(cfg.key)
    for step in range(steps):
        p = cfg.ctx + step * cfg.append_per_block
        taps = di.make_taps(cfg, 0, p, cfg.append_per_block)
        assert om.append(0, p, taps) == 0
        gm.append(0, p, taps)
        if step % 16 == 0:
            _kv_check(cfg, om, gm, 0, [(p, cfg.append_per_block)], 2e-3)
        _scale_blocks(cfg, om, gm, pooled, (0,), (p + cfg.append_per_block,), step)
        assert gm.last_scores() == _scores("DIGITS")  # over 16384 context rows: digit scores
        if step % 16 == 15:
            say(f"{cfg.key}: {step + 1} steps")
    pooled.check(2e-3, 0.999, 1024)


@pytest.mark.timeout(900)
def test_eight_sequences_batched():
    """The batched workload at its full size: 8 sequences of 8192 context rows, 8 forwards of
    one 16-row block each in one call (128 rows through every matrix; 1024 rows in all), then a
    subset of the sequences, out of order and with other anchors."""
    cfg = BATCH
    _, om, gm = _pair(cfg, cfg.ctx, cfg.ctx + 64, n_seqs=cfg.n_seqs)
    _kv_check(cfg, om, gm, 7, [(0, 16), (8176, 16)], 2e-3)
    seqs = tuple(range(cfg.n_seqs))
    pooled = Pooled(cfg.key)
    for i in range(8):
        _scale_blocks(cfg, om, gm, pooled, seqs, (cfg.ctx,) * cfg.n_seqs, i)
        assert gm.last_scores() == _scores("DIGITS")  # 65536 context rows in the call
        say(f"{cfg.key}: {i + 1} forwards")
    pooled.check(2e-3, 0.999, 1024)
    _blocks(cfg, om, gm, [((5, 2, 7), (cfg.ctx, cfg.ctx - 100, 4000), 8)], 2e-3, 0.999)
