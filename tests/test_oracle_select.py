"""Pins of the oracle's candidate selection (cortiq-engine dflash.rs: top_k and
Drafter::select_with): the pages' own worked example of top_k, a brute-force order, and
properties of the greedy re-scoring that hold whatever the numbers."""
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "top_k_pages_example.txt")


def _golden():
    lines = [ln for ln in open(GOLDEN).read().splitlines() if ln and not ln.startswith("#")]
    x = np.array([float(v) for v in lines[0].split(":")[1].split()], np.float32)
    cases = []
    for ln in lines[1:]:
        head, body = ln.split(":")
        pairs = [p.split() for p in body.split("|")]
        cases.append((int(head.split("=")[1]), [(float(v), int(i)) for v, i in pairs]))
    return x, cases


def test_top_k_pages_worked_example():
    x, cases = _golden()
    assert len(cases) == 2
    for k, want in cases:
        vals, idx = oracle.top_k(x, k)
        assert [(float(v), int(i)) for v, i in zip(vals, idx)] == want


def test_top_k_is_the_head_of_the_value_then_index_order():
    rng = np.random.default_rng(7)
    for n, k in [(1, 1), (50, 7), (1000, 16), (4099, 32)]:
        x = rng.integers(-20, 20, n).astype(np.float32) / 4  # many equal values
        vals, idx = oracle.top_k(x, k)
        order = sorted(range(n), key=lambda i: (-float(x[i]), i))[:k]
        assert list(idx) == order
        assert np.array_equal(vals, x[order])


def _case(rng, rows=6, width=300, rank=8, vocab=300, top=5):
    logits = rng.standard_normal((rows, width)).astype(np.float32)
    hp = rng.standard_normal((rows, rank)).astype(np.float32)
    pred = (rng.standard_normal((vocab, rank)) * 0.5).astype(np.float16)
    succ = (rng.standard_normal((vocab, rank)) * 0.5).astype(np.float16)
    return logits, hp, pred, succ, top


def test_select_reduces_to_top_1():
    rng = np.random.default_rng(8)
    logits, hp, pred, succ, top = _case(rng)
    # one candidate: nothing to re-score
    chosen, plain = oracle.select(logits, hp, pred, succ, 1, 3)
    assert np.array_equal(chosen, plain)
    assert np.array_equal(plain, logits.argmax(axis=1))
    # zero codebooks: the score is the logit
    z = np.zeros_like(pred)
    chosen, plain = oracle.select(logits, hp, z, z, top, 3)
    assert np.array_equal(chosen, plain)
    # equal logits and zero codebooks: equal scores, the first candidate (earlier index) stays
    tied = (rng.integers(0, 3, logits.shape)).astype(np.float32)
    chosen, plain = oracle.select(tied, hp, z, z, top, 3)
    assert np.array_equal(chosen, plain)
    assert np.array_equal(plain, tied.argmax(axis=1))


def test_select_chooses_among_the_candidates_and_follows_the_chain():
    rng = np.random.default_rng(9)
    logits, hp, pred, succ, top = _case(rng)
    chosen, plain = oracle.select(logits, hp, pred, succ, top, 11)
    for j in range(logits.shape[0]):
        _, idx = oracle.top_k(logits[j], top)
        assert chosen[j] in idx and plain[j] == idx[0]
    # a successor row that outweighs every logit gap wins wherever it is a candidate
    big = succ.copy()
    tok = int(oracle.top_k(logits[2], top)[1][top - 1])  # row 2's last candidate
    rank = hp.shape[1]
    pred1 = np.ones_like(pred)
    hp1 = np.ones_like(hp)
    big[:] = 0
    big[tok] = np.float16(100.0 / rank)
    chosen, _ = oracle.select(logits, hp1, pred1, big, top, 11)
    assert chosen[2] == tok
    # the predecessor of row j is row j-1's choice: pred rows of every other token are ignored
    pred2 = np.zeros_like(pred)
    pred2[11] = pred[11]
    c_all, _ = oracle.select(logits[:1], hp[:1], pred, succ, top, 11)
    c_one, _ = oracle.select(logits[:1], hp[:1], pred2, succ, top, 11)
    assert np.array_equal(c_all, c_one)


def test_select_brute_force_small():
    """Small cases against an f32 loop in the pages' order (sum of the products from r = 0, then
    the logit added; the first largest score wins)."""
    rng = np.random.default_rng(10)
    for _ in range(5):
        logits, hp, pred, succ, top = _case(rng, rows=4, width=40, rank=6, vocab=40, top=4)
        chosen, plain = oracle.select(logits, hp, pred, succ, top, 5)
        prev = 5
        for j in range(4):
            order = sorted(range(40), key=lambda i: (-float(logits[j, i]), i))[:top]
            assert plain[j] == order[0]
            pc = [np.float32(np.float32(pred[prev, r]) * hp[j, r]) for r in range(6)]
            best, pick = -np.inf, order[0]
            for t in order:
                acc = np.float32(0)
                for r in range(6):
                    acc = np.float32(acc + np.float32(pc[r] * np.float32(succ[t, r])))
                score = np.float32(logits[j, t] + acc)
                if score > best:
                    best, pick = score, t
            assert chosen[j] == pick
            prev = pick
