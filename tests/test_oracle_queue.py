"""Pins of the deferred context queue (cortiq-engine dflash.rs: Drafter::queue_context, settle,
push_context, next_position / span, truncate; PENDING_ROWS and CONTEXT_CHUNK): the counts of
waiting and settled rows worked out by hand from the pages' rules, deferral leaving the cache
and the block unchanged (rows are independent), and the one place where it shows: the rows a
window drops are decided at each settle."""
import numpy as np

import dflash_inputs as di
import oracle
import test_oracle_model as TM

CFG = TM.QTINY.replace(key="q_tiny_queue", pending_rows=100)


def _state(m, seq=0):
    return m.span(seq), m.pending(seq)


def test_queue_counts_by_hand():
    w = di.make_weights(CFG)
    m = oracle.Model(CFG, w, max_ctx=400)
    taps = di.make_taps(CFG, 0, 0, 400)
    assert m.queue(0, 0, taps[:70]) == 0
    assert _state(m) == ((0, 70), 70)  # waiting rows count in the span
    assert m.queue(0, 70, taps[70:140]) == 0
    assert _state(m) == ((0, 140), 76)  # 140 > 100: the oldest 64 (one chunk) settled
    assert m.queue(0, 140, taps[140:170]) == 0
    assert _state(m) == ((0, 170), 42)  # 106 > 100: one more chunk
    # a truncation reaches into the waiting rows: the settled ones stay
    assert m.truncate(0, 150) == 0
    assert _state(m) == ((0, 150), 22)
    assert m.truncate(0, 100) == 0
    assert _state(m) == ((0, 100), 0)
    # a position inside the waiting rows replaces them and what follows
    assert m.queue(0, 100, taps[100:130]) == 0
    assert m.queue(0, 110, taps[110:120]) == 0
    assert _state(m) == ((0, 120), 20)
    assert m.settle(0) == 0
    assert _state(m) == ((0, 120), 0)
    # a gap starts over: nothing waits
    assert m.queue(0, 500, taps[:10]) == 0
    assert _state(m) == ((500, 510), 10)
    # the capacity counts the waiting rows
    assert m.queue(0, 510, taps[:391]) == -2
    assert _state(m) == ((500, 510), 10)


def test_deferral_leaves_the_cache_and_the_block_unchanged():
    w = di.make_weights(CFG)
    taps = di.make_taps(CFG, 0, 0, 250)
    now = oracle.Model(CFG, w, max_ctx=400)
    later = oracle.Model(CFG, w, max_ctx=400)
    assert now.append(0, 0, taps) == 0
    for a, b in ((0, 33), (33, 160), (160, 161), (161, 250)):
        assert later.queue(0, a, taps[a:b]) == 0
    assert later.pending(0) > 0
    h = di.make_block_input(CFG, 0, 0)
    # the block settles what waits, then reads it
    np.testing.assert_array_equal(later.block_forward([0], [250], h[None]), now.block_forward([0], [250], h[None]))
    assert later.pending(0) == 0
    for li in range(CFG.layers):
        for a, b in zip(now.read_kv(li, 0, 0, 250), later.read_kv(li, 0, 0, 250)):
            np.testing.assert_array_equal(a, b)


def test_window_drops_follow_the_settles():
    """A window of 30 and at most 20 waiting rows: 84 rows queued at once settle 64 (held 64 > 60:
    34 dropped), the last 20 wait; settling them leaves 50 held <= 60, nothing more dropped.
    Pushing them (queue, then settle) does the same.  With no rows allowed to wait the 84 rows
    settle together: 84 > 60, 54 dropped."""
    cfg = CFG.replace(pending_rows=20)
    w = di.make_weights(cfg)
    taps = di.make_taps(cfg, 0, 0, 84)
    q = oracle.Model(cfg, w, max_ctx=200)
    r = oracle.Model(cfg, w, max_ctx=200)
    p = oracle.Model(cfg.replace(pending_rows=0), w, max_ctx=200)
    for m in (q, r, p):
        assert m.set_layer_options([30, 0]) == 0
    assert q.queue(0, 0, taps) == 0
    assert (q.dropped(0, 0), q.pending(0)) == (34, 20)
    assert q.settle(0) == 0
    assert (q.dropped(0, 0), q.dropped(0, 1), q.span(0)) == (34, 0, (0, 84))
    assert r.append(0, 0, taps) == 0
    assert (r.dropped(0, 0), r.pending(0)) == (34, 0)
    assert p.append(0, 0, taps) == 0
    assert p.dropped(0, 0) == 54
