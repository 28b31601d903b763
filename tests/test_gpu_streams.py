"""One drafter driven from two streams in turn.  Appends and blocks share the drafter's workspace
(activations, partial sums, the cache), so a call on a new stream must wait for the work still in
flight on the old one; the logits then equal the oracle's on every block."""
import pytest

import dflash_inputs as di
import oracle
from gpu_common import logits_parity, say, weights_for

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

QTINY = di.Config("q_tiny", 2, 256, 4, 2, 64, 512, 2, 1024, 8, 40, di.Q4_32, di.Q8_32, di.Q8_32, seed=2002)


def test_append_and_block_alternate_between_two_streams():
    from block_draft_model_dflash_amd import Drafter

    cfg = QTINY
    w = weights_for(cfg)
    om = oracle.Model(cfg, w, max_ctx=320)
    gm = Drafter(cfg, w, max_ctx=320)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    got, want = [], []
    pos = 0
    for step in range(8):
        n = 17 + 5 * step  # ragged appends: the cache grows while blocks read it
        taps = di.make_taps(cfg, 0, pos, n)
        assert om.append(0, pos, taps) == 0
        a, b = (s1, s2) if step % 2 == 0 else (s2, s1)
        say(f"streams: step {step}, append {n} rows at {pos}")
        with torch.cuda.stream(a):
            gm.append(0, pos, taps)
        pos += n
        h = di.make_block_input(cfg, 0, step)[None]
        with torch.cuda.stream(b):
            got.append(gm.block_forward([0], [pos], h))
        want.append(om.block_forward([0], [pos], h))
    torch.cuda.synchronize()
    for step, (g, r) in enumerate(zip(got, want)):
        rel, top1 = logits_parity(g.cpu().numpy(), r)
        say(f"streams: block {step} rel {rel:.3e} top1 {top1:.3f}")
        assert rel <= 2e-3 and top1 == 1.0, (step, rel, top1)
