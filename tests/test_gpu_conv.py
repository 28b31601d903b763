"""Row convolutions around the attention and the MLP (cortiq-engine dflash.rs: Drafter::conv_in,
Drafter::conv; the device block's dflash_conv): the GPU library through its C ABI against the
oracle on the same seeded inputs.

The workloads declare no convolutions and the pages give no conv_group / conv_kernel for them;
these drafters take 16 columns a group and 4 offsets (kernel projections of 2*4*H/16 rows,
coded like the FC), with static kernels near the identity.  Bar as for the plain block: logits
max |d| <= 2e-3 * max |logit| (1e-5 for the f32 drafter) and top-1 agreement >= 99.9%."""
import numpy as np
import pytest

import dflash_inputs as di
import oracle
from gpu_common import logits_parity, say, weights_for

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

CONV2 = di.CONFIGS["tiny_f32"].replace(key="tiny_f32_conv", layers=2, norm_mean=1.0, taps_std=1.0, emb_std=1.0,
                                       conv_group=16, conv_kernel=4, conv_std=0.02, seed=2004)
QCONV = di.Config("q_tiny_conv", 2, 256, 4, 2, 64, 512, 2, 1024, 8, 40, di.Q4_32, di.Q8_32, di.Q8_32, seed=2005,
                  conv_group=16, conv_kernel=4)
Q8B_CONV = di.CONFIGS["qwen3_8b"].replace(key="qwen3_8b_conv", conv_group=16, conv_kernel=4)


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


def _block(cfg, om, gm, seqs, anchors, index, tol):
    h = np.stack([di.make_block_input(cfg, s, index) for s in seqs])
    say(f"{cfg.key}: conv block seqs={list(seqs)} anchors={list(anchors)}")
    got = gm.block_forward(list(seqs), list(anchors), h)
    torch.cuda.synchronize()
    ref = om.block_forward(list(seqs), list(anchors), h)
    rel, top1 = logits_parity(got.cpu().numpy(), ref)
    say(f"{cfg.key}: rel {rel:.3e} top1 {top1:.4f}")
    assert rel <= tol and top1 >= 0.999


def test_conv_f32_drafter():
    cfg = CONV2
    om, gm = _pair(cfg, cfg.ctx + 64)
    _append(cfg, om, gm, 0, 100, cfg.ctx)
    for i, anchor in enumerate([100 + cfg.ctx, 100 + cfg.ctx - 9, 50]):
        _block(cfg, om, gm, (0,), (anchor,), i, 1e-5)


def test_conv_quantized_sequences_share_tiles():
    """Blocks of 8 rows: two sequences share each 16-row tile, and the convolution must not
    reach across from one into the other."""
    cfg = QCONV.replace(n_seqs=3)
    om, gm = _pair(cfg, 120, n_seqs=3)
    _append(cfg, om, gm, 0, 0, 37)
    _append(cfg, om, gm, 1, 300, 21)
    _append(cfg, om, gm, 2, 0, 64)
    _block(cfg, om, gm, (0, 1, 2), (37, 321, 64), 0, 2e-3)
    _block(cfg, om, gm, (2, 0), (40, 37), 1, 2e-3)
    # with per-layer windows and an unrotated layer as well
    om2, gm2 = _pair(cfg, 120, n_seqs=3)
    assert om2.set_layer_options([9, 0], [1, 0]) == 0
    gm2.set_layer_options([9, 0], [1, 0])
    _append(cfg, om2, gm2, 0, 0, 37)
    _block(cfg, om2, gm2, (0,), (37,), 2, 2e-3)


@pytest.mark.timeout(600)
def test_conv_qwen3_8b_shaped():
    cfg = Q8B_CONV
    om, gm = _pair(cfg, cfg.ctx + 64)
    _append(cfg, om, gm, 0, 0, cfg.ctx)
    _block(cfg, om, gm, (0,), (cfg.ctx,), 0, 2e-3)
    _block(cfg, om, gm, (0,), (cfg.ctx - 300,), 1, 2e-3)
