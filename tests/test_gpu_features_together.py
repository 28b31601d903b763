"""Every optional part of the drafter at once -- row convolutions, an f16 K/V cache, per-layer
windows and an unrotated layer, the deferred queue, blocks cut to fewer rows and a head
shortlist -- on a quantized drafter with two sequences, the GPU library through its C ABI
against the oracle driven through the same calls.  Integer state (spans, waiting rows, dropped
rows) must be equal; logits are held to max |d| <= 2e-3 * max |logit| and top-1 >= 99.9%."""
import numpy as np
import pytest

import dflash_inputs as di
import oracle
from gpu_common import cache_match, logits_parity, say, weights_for

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

CFG = di.Config("q_tiny_all", 2, 256, 4, 2, 64, 512, 2, 1024, 8, 40, di.Q4_32, di.Q8_32, di.Q8_32, seed=2006,
                n_seqs=2, conv_group=16, conv_kernel=4, kv_f16=True, pending_rows=50)


def test_all_optional_parts_together():
    from block_draft_model_dflash_amd import Drafter

    cfg = CFG
    w = weights_for(cfg)
    om = oracle.Model(cfg, w, max_ctx=300, max_seqs=2)
    gm = Drafter(cfg, w, max_ctx=300, max_seqs=2)
    assert om.set_layer_options([12, 0], [1, 0]) == 0
    gm.set_layer_options([12, 0], [1, 0])
    taps = [di.make_taps(cfg, s, 0, 200) for s in range(2)]

    def same():
        for s in range(2):
            assert gm.span(s) == om.span(s) and gm.pending(s) == om.pending(s)
            assert [gm.dropped(s, li) for li in range(2)] == [om.dropped(s, li) for li in range(2)]

    def block(seqs, anchors, index, rows, head_rows=None):
        h = np.ascontiguousarray(np.stack([di.make_block_input(cfg, s, index) for s in seqs])[:, :rows])
        say(f"all parts: seqs={seqs} anchors={anchors} rows={rows} head_rows={head_rows}")
        got = gm.block_forward(list(seqs), list(anchors), h, head_rows=head_rows)
        torch.cuda.synchronize()
        ref = om.block_forward(list(seqs), list(anchors), h, head_rows=head_rows)
        rel, top1 = logits_parity(got.cpu().numpy(), ref)
        say(f"all parts: rel {rel:.3e} top1 {top1:.4f}")
        assert rel <= 2e-3 and top1 >= 0.999

    for s, pieces in ((0, [(0, 30), (30, 90), (90, 97)]), (1, [(0, 64), (64, 70)])):
        for a, b in pieces:
            assert om.queue(s, a, taps[s][a:b]) == 0
            gm.queue(s, a, taps[s][a:b])
            same()
    block((0, 1), (97, 70), 0, 8)
    same()
    block((1, 0), (60, 97), 1, 5, head_rows=256)
    for m in (om, gm):
        m.truncate(0, 80)
    same()
    for a in range(80, 120, 8):
        assert om.queue(0, a, taps[0][a:a + 8]) == 0
        gm.queue(0, a, taps[0][a:a + 8])
        same()
        block((0,), (a + 8,), a, 8)
    for li in range(2):
        for s in range(2):
            n = gm.span(s)[1]
            ko, vo = om.read_kv(li, s, 0, n)
            kg, vg = gm.read_kv(li, s, 0, n)
            torch.cuda.synchronize()
            dt = np.float16 if cfg.kv_f16 else np.float32
            cache_match(kg.cpu().numpy(), ko, dt)
            cache_match(vg.cpu().numpy(), vo, dt)
