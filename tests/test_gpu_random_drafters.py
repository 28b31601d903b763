"""Seeded random drafters and random call sequences, the GPU library through its C ABI against
the oracle: shapes (hidden, heads, head_dim, intermediate, taps, vocab, block rows, sequences),
formats (f32 or Q4_32/Q8_32), row convolutions, the f16 cache, waiting rows, per-layer windows
and unrotated layers drawn per case; then appends, queued rows, truncations, settles and blocks
(cut or whole, with or without a shortlist) at random anchors; three in four drafters whose geometry
allows it (head_dim 128, four q heads per kv head) score attention from int8 digits.  Integer state (spans, waiting
and dropped rows) must be equal after every call, the cache read back equal but for isolated
one-unit-in-the-last-place elements (gpu_common.cache_match), and logits within
max |d| <= 2e-3 * max |logit| (1e-5 for f32 drafters) with top-1 >= 99.9% over a case."""
import os

import numpy as np
import pytest

import dflash_inputs as di
import oracle
from gpu_common import cache_match, logits_parity, say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

# 200 cases in the regular suite (about 20 s); DFLASH_RANDOM_CASES asks for a longer sweep
N_CASES = int(os.environ.get("DFLASH_RANDOM_CASES", "200"))


def _case(seed: int):
    r = np.random.default_rng(seed)
    H = int(r.choice([256, 512]))
    heads, kvh = [(4, 2), (8, 2), (4, 4), (8, 1)][r.integers(4)]
    hd = int(r.choice([64, 128]))
    quant = bool(r.integers(2))
    B = int(r.choice([2, 4, 8, 16]))
    n_seqs = int(r.integers(1, 4))
    conv = bool(r.integers(2))
    gs, kn = (0, 0)
    if conv:  # kernel projections of 2*kn*H/gs rows, a multiple of 16
        gs, kn = [(16, 1), (16, 4), (32, 2), (64, 4), (32, 4)][r.integers(5)]
    cfg = di.Config(f"rand{seed}", int(r.integers(1, 3)), H, heads, kvh, hd, int(r.choice([512, 768])),
                    int(r.integers(1, 4)), int(r.choice([1024, 2048])), B, 0,
                    di.Q4_32 if quant else di.F32, di.Q8_32 if quant else di.F32, di.Q8_32 if quant else di.F32,
                    n_seqs=n_seqs, norm_mean=1.0, taps_std=1.0, emb_std=1.0 if not quant else 0.02, seed=3000 + seed,
                    conv_group=gs, conv_kernel=kn, conv_std=0.02 if not quant else 0.0025,
                    kv_f16=bool(r.integers(2)), pending_rows=int(r.choice([0, 20, 64])))
    windows = [int(r.choice([0, 0, 5, 17, 40])) for _ in range(cfg.layers)]
    rotary = [int(r.integers(4) > 0) for _ in range(cfg.layers)]
    return cfg, windows, rotary, r


@pytest.mark.timeout(900)
@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_drafter_and_calls(seed):
    from block_draft_model_dflash_amd import Drafter

    cfg, windows, rotary, r = _case(seed)
    say(f"case {seed}: {cfg} windows={windows} rotary={rotary}")
    w = di.make_weights(cfg)
    max_ctx = 260
    om = oracle.Model(cfg, w, max_ctx=max_ctx, max_seqs=cfg.n_seqs)
    gm = Drafter(cfg, w, max_ctx=max_ctx, max_seqs=cfg.n_seqs)
    assert om.set_layer_options(windows, rotary) == 0
    gm.set_layer_options(windows, rotary)
    if cfg.head_dim == 128 and cfg.heads == 4 * cfg.kv_heads and seed % 4 != 0:
        from block_draft_model_dflash_amd import DFLASH_SCORES_DIGITS

        say(f"case {seed}: scores from int8 digits")
        gm.set_score_mode(DFLASH_SCORES_DIGITS)  # three in four of the cases whose geometry can take them
    tol = 1e-5 if cfg.body_fmt == di.F32 else 2e-3
    agree = []

    def same():
        for s in range(cfg.n_seqs):
            assert gm.span(s) == om.span(s), s
            assert gm.pending(s) == om.pending(s), s
            assert [gm.dropped(s, li) for li in range(cfg.layers)] == [om.dropped(s, li) for li in range(cfg.layers)]

    for step in range(20):
        op = r.choice(["append", "queue", "queue", "truncate", "settle", "block", "block", "block"])
        s = int(r.integers(cfg.n_seqs))
        first, end = om.span(s)
        if op in ("append", "queue"):
            pos = int(end if r.integers(5) else r.integers(first, end + 1) if end > first else end)
            if r.integers(8) == 0:
                pos = end + int(r.integers(1, 20))  # a gap: starts over
            n = int(r.integers(0, 70))
            if pos + n - (first if first <= pos <= end else pos) > max_ctx:
                continue
            taps = di.make_taps(cfg, s, pos, n)
            assert getattr(om, op)(s, pos, taps) == 0
            getattr(gm, op)(s, pos, taps)
        elif op == "truncate":
            pos = int(r.integers(first, end + 1))
            assert om.truncate(s, pos) == 0
            gm.truncate(s, pos)
        elif op == "settle":
            assert om.settle(s) == 0
            gm.settle(s)
        else:
            k = int(r.integers(1, cfg.n_seqs + 1))
            seqs = [int(x) for x in r.permutation(cfg.n_seqs)[:k]]
            anchors = []
            for q in seqs:
                f, e = om.span(q)
                anchors.append(int(max(0, e + int(r.integers(-30, 10)))))
            rows = cfg.block if r.integers(3) else int(r.integers(1, cfg.block + 1))
            head_rows = None if r.integers(3) else 16 * int(r.integers(1, cfg.vocab // 16 + 1))
            h = np.ascontiguousarray(np.stack([di.make_block_input(cfg, q, step) for q in seqs])[:, :rows])
            say(f"case {seed} step {step}: block seqs={seqs} anchors={anchors} rows={rows} head_rows={head_rows}")
            got = gm.block_forward(seqs, anchors, h, head_rows=head_rows)
            torch.cuda.synchronize()
            ref = om.block_forward(seqs, anchors, h, head_rows=head_rows)
            rel, top1 = logits_parity(got.cpu().numpy(), ref)
            say(f"case {seed} step {step}: rel {rel:.3e} top1 {top1:.4f}")
            assert rel <= tol, (seed, step, rel)
            agree.append(top1)
        same()
    for s in range(cfg.n_seqs):
        assert om.settle(s) == 0
        gm.settle(s)
        first, end = om.span(s)
        n = end - first
        if n:
            for li in range(cfg.layers):
                ko, vo = om.read_kv(li, s, 0, n)
                kg, vg = gm.read_kv(li, s, 0, n)
                torch.cuda.synchronize()
                dt = np.float16 if cfg.kv_f16 else np.float32
                cache_match(kg.cpu().numpy(), ko, dt)
                cache_match(vg.cpu().numpy(), vo, dt)
    if agree:
        assert np.mean(agree) >= 0.999
