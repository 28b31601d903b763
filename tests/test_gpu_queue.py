"""The deferred context queue (cortiq-engine dflash.rs: Drafter::queue_context, settle,
push_context; PENDING_ROWS and CONTEXT_CHUNK): the GPU library through its C ABI against the
oracle, driven through the same calls on the same seeded rows.  Spans, waiting-row counts and
dropped-row counts are integers and must be equal; the cache read back matches the oracle's
up to isolated last-place differences (gpu_common.cache_match; rows are settled by the same
arithmetic whenever they settle); logits are held to the
drafter's bar, max |d| <= 2e-3 * max |logit| and top-1 agreement >= 99.9%."""
import numpy as np
import pytest

import dflash_inputs as di
import oracle
from gpu_common import cache_match, logits_parity, say, weights_for

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

QTINY = di.Config("q_tiny", 2, 256, 4, 2, 64, 512, 2, 1024, 8, 40, di.Q4_32, di.Q8_32, di.Q8_32, seed=2002,
                  pending_rows=100)
Q8B = di.CONFIGS["qwen3_8b"].replace(pending_rows=512)


def _pair(cfg, max_ctx, n_seqs=1, windows=None):
    from block_draft_model_dflash_amd import Drafter

    w = weights_for(cfg)
    om, gm = oracle.Model(cfg, w, max_ctx=max_ctx, max_seqs=n_seqs), Drafter(cfg, w, max_ctx=max_ctx, max_seqs=n_seqs)
    if windows is not None:
        assert om.set_layer_options(windows) == 0
        gm.set_layer_options(windows)
    return om, gm


def _same_state(cfg, om, gm, seq):
    assert gm.span(seq) == om.span(seq)
    assert gm.pending(seq) == om.pending(seq)
    assert [gm.dropped(seq, li) for li in range(cfg.layers)] == [om.dropped(seq, li) for li in range(cfg.layers)]


def _both(cfg, om, gm, op, seq, *a):
    if op == "queue":
        pos, taps = a
        assert om.queue(seq, pos, taps) == 0
        gm.queue(seq, pos, taps)
    elif op == "truncate":
        assert om.truncate(seq, a[0]) == 0
        gm.truncate(seq, a[0])
    elif op == "settle":
        assert om.settle(seq) == 0
        gm.settle(seq)
    _same_state(cfg, om, gm, seq)


def _kv_equal(cfg, om, gm, seq, r0, n):
    for li in range(cfg.layers):
        ko, vo = om.read_kv(li, seq, r0, n)
        kg, vg = gm.read_kv(li, seq, r0, n)
        torch.cuda.synchronize()
        cache_match(kg.cpu().numpy(), ko)
        cache_match(vg.cpu().numpy(), vo)


def _block(cfg, om, gm, seqs, anchors, index):
    h = np.stack([di.make_block_input(cfg, s, index) for s in seqs])
    say(f"{cfg.key}: block after queued rows, seqs={list(seqs)} anchors={list(anchors)}")
    got = gm.block_forward(list(seqs), list(anchors), h)
    torch.cuda.synchronize()
    ref = om.block_forward(list(seqs), list(anchors), h)
    rel, top1 = logits_parity(got.cpu().numpy(), ref)
    say(f"{cfg.key}: rel {rel:.3e} top1 {top1:.4f}")
    assert rel <= 2e-3 and top1 >= 0.999
    for s in seqs:  # the block settled what waited
        assert gm.pending(s) == 0 == om.pending(s)


def test_queue_settle_truncate_and_the_ring():
    cfg = QTINY.replace(n_seqs=2)
    om, gm = _pair(cfg, 400, n_seqs=2)
    taps = di.make_taps(cfg, 0, 0, 400)
    # counts as worked out from the pages' rules: 70 wait; 140 > 100 settles 64; ...
    _both(cfg, om, gm, "queue", 0, 0, taps[:70])
    _both(cfg, om, gm, "queue", 0, 70, taps[70:140])
    assert gm.pending(0) == 76
    _both(cfg, om, gm, "queue", 0, 140, taps[140:170])
    _both(cfg, om, gm, "truncate", 0, 150)
    _both(cfg, om, gm, "queue", 0, 150, taps[150:260])  # the ring wraps around
    _both(cfg, om, gm, "queue", 0, 200, taps[200:230])  # into the waiting rows
    _both(cfg, om, gm, "queue", 1, 1000, di.make_taps(cfg, 1, 1000, 30))
    _block(cfg, om, gm, (0, 1), (230, 1030), 0)
    _kv_equal(cfg, om, gm, 0, 0, 230)
    _both(cfg, om, gm, "queue", 0, 230, taps[230:300])
    _both(cfg, om, gm, "settle", 0)
    _kv_equal(cfg, om, gm, 0, 200, 100)
    # a gap starts over and forgets what waits
    _both(cfg, om, gm, "queue", 0, 230, taps[230:250])
    _both(cfg, om, gm, "queue", 0, 900, taps[:10])
    _block(cfg, om, gm, (0,), (910,), 1)


def test_queue_with_windows():
    cfg = QTINY.replace(pending_rows=20)
    om, gm = _pair(cfg, 200, windows=[30, 0])
    taps = di.make_taps(cfg, 0, 0, 200)
    _both(cfg, om, gm, "queue", 0, 0, taps[:84])
    assert gm.dropped(0, 0) == 34 and gm.pending(0) == 20
    _both(cfg, om, gm, "settle", 0)
    for p in range(84, 164, 16):  # a block after every 16 rows, as a decode would
        _both(cfg, om, gm, "queue", 0, p, taps[p:p + 16])
        _block(cfg, om, gm, (0,), (p + 16,), p)


@pytest.mark.timeout(600)
def test_queue_qwen3_8b_shaped():
    """The 8B-shaped drafter with the pages' 512 waiting rows: 4096 rows prefilled, then 16-row
    pieces queued, settled by the pages' rule (576 > 512: one 64-row chunk) and by a block."""
    cfg = Q8B
    om, gm = _pair(cfg, cfg.ctx + 1024)
    for p0 in range(0, cfg.ctx, 2048):
        taps = di.make_taps(cfg, 0, p0, 2048)
        _both(cfg, om, gm, "queue", 0, p0, taps)
    _both(cfg, om, gm, "settle", 0)
    for i in range(36):
        p = cfg.ctx + 16 * i
        _both(cfg, om, gm, "queue", 0, p, di.make_taps(cfg, 0, p, 16))
    assert gm.pending(0) == 576 - 64
    _kv_equal(cfg, om, gm, 0, cfg.ctx, 64)
    _block(cfg, om, gm, (0,), (cfg.ctx + 576,), 0)
