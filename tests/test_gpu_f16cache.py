"""The f16 K/V cache (each element the f32 value rounded to binary16; half the cache bytes):
the GPU library through its C ABI against the oracle on the same seeded inputs.  The cache
read back must equal the oracle's bit for bit (the same f32 values rounded the same way);
logits are held to the drafter's bar, max |d| <= 2e-3 * max |logit| (1e-5 for the f32
drafter) and top-1 agreement >= 99.9%."""
import numpy as np
import pytest

import dflash_inputs as di
import oracle
from gpu_common import cache_match, logits_parity, say, weights_for

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SHARP2 = di.CONFIGS["tiny_f32"].replace(key="tiny_f32_sharp_2l", layers=2, norm_mean=1.0, taps_std=1.0,
                                        emb_std=1.0, seed=2003, kv_f16=True)
QTINY = di.Config("q_tiny", 2, 256, 4, 2, 64, 512, 2, 1024, 8, 40, di.Q4_32, di.Q8_32, di.Q8_32, seed=2002,
                  kv_f16=True)
LONG = di.CONFIGS["qwen3_8b_long"].replace(kv_f16=True)


def _pair(cfg, max_ctx, n_seqs=1):
    from block_draft_model_dflash_amd import Drafter

    w = weights_for(cfg)
    return oracle.Model(cfg, w, max_ctx=max_ctx, max_seqs=n_seqs), Drafter(cfg, w, max_ctx=max_ctx, max_seqs=n_seqs)


def _append(cfg, om, gm, seq, pos, n, chunk=4096):
    for p0 in range(0, n, chunk):
        k = min(chunk, n - p0)
        taps = di.make_taps(cfg, seq, pos + p0, k)
        assert om.append(seq, pos + p0, taps) == 0
        gm.append(seq, pos + p0, taps)


def _kv_equal(cfg, om, gm, seq, r0, n):
    for li in range(cfg.layers):
        ko, vo = om.read_kv(li, seq, r0, n)
        kg, vg = gm.read_kv(li, seq, r0, n)
        torch.cuda.synchronize()
        cache_match(kg.cpu().numpy(), ko, np.float16)
        cache_match(vg.cpu().numpy(), vo, np.float16)


def _block(cfg, om, gm, seqs, anchors, index, tol):
    h = np.stack([di.make_block_input(cfg, s, index) for s in seqs])
    say(f"{cfg.key}: f16 cache block seqs={list(seqs)} anchors={list(anchors)}")
    got = gm.block_forward(list(seqs), list(anchors), h)
    torch.cuda.synchronize()
    ref = om.block_forward(list(seqs), list(anchors), h)
    rel, top1 = logits_parity(got.cpu().numpy(), ref)
    say(f"{cfg.key}: rel {rel:.3e} top1 {top1:.4f}")
    assert rel <= tol and top1 >= 0.999


def test_f16_cache_f32_drafter():
    cfg = SHARP2
    om, gm = _pair(cfg, cfg.ctx + 64)
    _append(cfg, om, gm, 0, 100, cfg.ctx)
    _kv_equal(cfg, om, gm, 0, 0, cfg.ctx)
    for i, anchor in enumerate([100 + cfg.ctx, 100 + cfg.ctx - 9]):
        _block(cfg, om, gm, (0,), (anchor,), i, 1e-5)


def test_f16_cache_quantized_sequences():
    cfg = QTINY.replace(n_seqs=2)
    om, gm = _pair(cfg, 120, n_seqs=2)
    _append(cfg, om, gm, 0, 0, 37)
    _append(cfg, om, gm, 1, 300, 50)
    _kv_equal(cfg, om, gm, 1, 0, 50)
    _block(cfg, om, gm, (0, 1), (37, 350), 0, 2e-3)


@pytest.mark.timeout(900)
def test_f16_cache_long_context():
    """The long-context workload with an f16 cache: 32768 context rows, then 16 appended rows
    and a block anchored after them."""
    cfg = LONG
    om, gm = _pair(cfg, cfg.ctx + 64)
    _append(cfg, om, gm, 0, 0, cfg.ctx)
    _kv_equal(cfg, om, gm, 0, 32752, 16)
    p = cfg.ctx
    _append(cfg, om, gm, 0, p, cfg.append_per_block)
    _kv_equal(cfg, om, gm, 0, p, cfg.append_per_block)
    _block(cfg, om, gm, (0,), (p + cfg.append_per_block,), 0, 2e-3)
