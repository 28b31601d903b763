"""Pins of the drafter's row convolutions (cortiq-engine dflash.rs: Drafter::conv_in and
Drafter::conv, the Conv of each layer's attention and MLP, Geometry conv_group / conv_kernel).

The convolution step is pinned against torch's depthwise conv1d (the static kernels, and
dynamic kernels constant over the rows), against where each input may reach (causal over the
block's rows, kn rows back, a dynamic kernel only within its column group and row), and the
whole drafter against transformers' Qwen3 layers with the convolutions inserted around the
attention and the MLP, and against the plain layer when the convolutions are the identity."""
import numpy as np
import torch
import torch.nn.functional as F

import dflash_inputs as di
import oracle
import test_oracle_model as TM
from hf_reference import HFDrafter

GS, KN = 16, 4
# two f32 layers with sharp attention and row convolutions (16 columns a group, 4 offsets)
CONV2 = TM.SHARP.replace(key="tiny_f32_conv", layers=2, conv_group=GS, conv_kernel=KN, conv_std=0.02, seed=2004)
# the quantized twin: Q8_32 kernel projections, A8_32 activations
QCONV = TM.QTINY.replace(key="q_tiny_conv", conv_group=GS, conv_kernel=KN, seed=2005)


def _rel(a, b):
    return float(np.abs(a.astype(np.float64) - b).max() / np.abs(b).max())


def _inputs(rows=11, hidden=64, seed=0):
    r = np.random.default_rng(seed)
    x = r.standard_normal((rows, hidden)).astype(np.float32)
    base = r.standard_normal((2, KN, hidden)).astype(np.float32)
    d = r.standard_normal((rows, 2 * KN * hidden // GS)).astype(np.float32)
    return x, base, d


def _conv1d(x, kern):
    """torch's depthwise causal conv1d over the rows: y[r][i] = sum_o kern[o][i] x[r-o][i]."""
    xt = torch.from_numpy(x.astype(np.float64)).T[None]  # [1][H][rows]
    w = torch.from_numpy(kern[::-1].copy().astype(np.float64)).T[:, None, :]  # [H][1][kn], last tap = offset 0
    y = F.conv1d(F.pad(xt, (kern.shape[0] - 1, 0)), w, groups=x.shape[1])
    return y[0].T.numpy()


def test_row_conv_against_torch_conv1d():
    x, base, d = _inputs()
    rows, H = x.shape
    for stage in (0, 1):
        # static kernels only
        got = oracle.row_conv(x, GS, KN, stage, base, np.zeros_like(d))
        np.testing.assert_allclose(got, _conv1d(x, base[stage]), rtol=1e-6, atol=1e-6)
        # dynamic kernels the same in every row: the convolution with their sum
        dd = np.tile(d[:1], (rows, 1))
        got = oracle.row_conv(x, GS, KN, stage, base, dd)
        dk = dd[0].reshape(2, KN, H // GS)[stage].repeat(GS, axis=1)
        np.testing.assert_allclose(got, _conv1d(x, base[stage] + dk), rtol=1e-6, atol=1e-5)
    # a one-hot static kernel and no dynamic part: a plain shift of the rows
    for o in range(KN):
        b1 = np.zeros_like(base)
        b1[:, o] = 1
        got = oracle.row_conv(x, GS, KN, 1, b1, np.zeros_like(d))
        want = np.zeros_like(x)
        want[o:] = x[:rows - o]
        np.testing.assert_array_equal(got, want)


def test_row_conv_reach():
    x, base, d = _inputs()
    rows, H = x.shape
    ref = oracle.row_conv(x, GS, KN, 0, base, d)
    # an input row reaches itself and the kn - 1 rows after it, nothing before
    for j in (0, 5, rows - 1):
        x2 = x.copy()
        x2[j] += 1
        changed = np.abs(oracle.row_conv(x2, GS, KN, 0, base, d) - ref).max(axis=1) > 0
        assert list(np.nonzero(changed)[0]) == list(range(j, min(rows, j + KN)))
    # a dynamic kernel reaches its own row and column group only, and only in its stage
    for stage in (0, 1):
        for o, g in ((0, 0), (2, 3), (KN - 1, H // GS - 1)):
            d2 = d.copy()
            d2[6, (stage * KN + o) * (H // GS) + g] += 1
            diff = np.abs(oracle.row_conv(x, GS, KN, 0, base, d2) - ref) > 0
            if stage == 1:
                assert not diff.any()
            else:
                rr, cc = np.nonzero(diff)
                assert set(rr) == {6} and set(cc // GS) == {g}


def _with_identity_convs(cfg, w):
    """kn = 1, static kernels 1, kernel projections 0: both stages are the identity."""
    c1 = cfg.replace(conv_kernel=1)
    w1 = dict(w)
    w1["layers"] = []
    for lw in w["layers"]:
        lw = dict(lw)
        for name in ("attn_kp", "mlp_kp"):
            rows = c1.conv_rows
            codes, scales = di.quantize_rows(np.zeros((rows, cfg.hidden), np.float32), cfg.fc_fmt)
            lw[name] = {"fmt": cfg.fc_fmt, "rows": rows, "cols": cfg.hidden, "codes": codes, "scales": scales}
        lw["attn_base"] = np.ones((2, 1, cfg.hidden), np.float32)
        lw["mlp_base"] = np.ones((2, 1, cfg.hidden), np.float32)
        w1["layers"].append(lw)
    return c1, w1


def test_identity_convolutions_give_the_plain_layer():
    for cfg in (CONV2, QCONV):
        plain_cfg = cfg.replace(conv_kernel=0)
        w = di.make_weights(plain_cfg)
        c1, w1 = _with_identity_convs(cfg, w)
        taps = di.make_taps(cfg, 0, 0, cfg.ctx)
        h = di.make_block_input(cfg, 0, 0)
        outs = []
        for c, ww in ((plain_cfg, w), (c1, w1)):
            m = oracle.Model(c, ww, max_ctx=cfg.ctx + 64)
            assert m.append(0, 0, taps) == 0
            outs.append(m.block_forward([0], [cfg.ctx], h[None]))
        np.testing.assert_array_equal(outs[0], outs[1])


def test_convolutions_match_transformers():
    first = 200
    for cfg in (CONV2, QCONV):
        w = di.make_weights(cfg)
        m = oracle.Model(cfg, w, max_ctx=cfg.ctx + 64)
        taps = di.make_taps(cfg, 0, first, cfg.ctx)
        assert m.append(0, first, taps) == 0
        plain = oracle.Model(cfg.replace(conv_kernel=0), w, max_ctx=cfg.ctx + 64)
        assert plain.append(0, first, taps) == 0
        hf = HFDrafter(cfg, w)
        kv = hf.context_kv(taps, first)
        for bi, anchor in enumerate([first + cfg.ctx, first + cfg.ctx - 7]):
            h = di.make_block_input(cfg, 0, bi)
            got = m.block_forward([0], [anchor], h[None])[0]
            n = anchor - first
            ref = hf.block_logits([(k[:, :, :n], v[:, :, :n]) for k, v in kv], anchor, h)
            if cfg.body_fmt == di.F32:
                assert _rel(got, ref) < 2e-5
            else:
                assert _rel(got, ref) < 2e-3
                assert np.mean(got.argmax(1) == ref.argmax(1)) >= 0.99
            # the convolutions change the result well beyond the tolerance
            assert _rel(plain.block_forward([0], [anchor], h[None])[0], got) > 1e-2
