"""Pins of the oracle's unit steps against things other than itself: IEEE decoding by numpy,
library routines (torch's rms_norm / scaled_dot_product_attention / silu, transformers'
Qwen3 rotary helpers, numpy's dense matmul), closed forms, invariants and brute force."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import dflash_inputs as di
import oracle


# ---- f16 scales ---------------------------------------------------------------------------


def test_f16_decode_matches_numpy_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


# ---- inv_freq -----------------------------------------------------------------------------


@pytest.mark.parametrize("hd", [64, 128])
def test_inv_freq_against_transformers_definition(hd):
    from transformers.models.qwen3.modeling_qwen3 import Qwen3Config, Qwen3RotaryEmbedding

    theta = 1.0e6
    cfg = Qwen3Config(hidden_size=hd * 2, num_attention_heads=2, num_key_value_heads=1, head_dim=hd,
                      rope_theta=theta, rope_parameters={"rope_type": "default", "rope_theta": theta})
    hf = Qwen3RotaryEmbedding(cfg).inv_freq.double().numpy()
    got = oracle.inv_freq(theta, hd).astype(np.float64)
    # transformers evaluates the power in f32: agree to a couple of f32 ulps
    assert np.allclose(got, hf, rtol=3e-7, atol=0)
    # closed form: a geometric sequence from 1 with ratio theta^(-2/hd)
    assert got[0] == 1.0
    ratio = theta ** (-2.0 / hd)
    assert np.allclose(got[1:] / got[:-1], ratio, rtol=2e-7)


# ---- RMSNorm ------------------------------------------------------------------------------


@pytest.mark.parametrize("n", [64, 128, 4096])
def test_rmsnorm_against_torch(n):
    rng = np.random.default_rng(n)
    x = (rng.standard_normal((7, n)) * rng.uniform(0.01, 10, (7, 1))).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(n)).astype(np.float32)
    got = oracle.rmsnorm(x, w, 1e-6).astype(np.float64)
    ref = F.rms_norm(torch.from_numpy(x).double(), (n,), torch.from_numpy(w).double(), eps=1e-6).numpy()
    assert np.allclose(got, ref, rtol=2e-6, atol=1e-7)


def test_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(5)
    n = 256
    x = rng.standard_normal((3, n)).astype(np.float32)
    ones = np.ones(n, np.float32)
    y = oracle.rmsnorm(x, ones, 1e-6).astype(np.float64)
    ms = (x.astype(np.float64) ** 2).mean(axis=1)
    assert np.allclose(np.sqrt((y ** 2).mean(axis=1)), np.sqrt(ms / (ms + 1e-6)), rtol=1e-6)
    y2 = oracle.rmsnorm(x * np.float32(37.0), ones, 1e-6).astype(np.float64)
    assert np.allclose(y, y2, rtol=1e-5, atol=1e-6)
    # eps matters only for tiny rows: a zero row stays zero
    assert np.all(oracle.rmsnorm(np.zeros((1, n), np.float32), ones, 1e-6) == 0)


# ---- RoPE ---------------------------------------------------------------------------------


@pytest.mark.parametrize("pos", [0, 1, 17, 4095, 32800])
def test_rope_against_transformers_rotate_half(pos):
    from transformers.models.qwen3.modeling_qwen3 import apply_rotary_pos_emb

    hd, heads = 128, 3
    rng = np.random.default_rng(pos)
    x = rng.standard_normal((heads, hd)).astype(np.float32)
    inv = oracle.inv_freq(1e6, hd)
    got = oracle.rope(x, pos, inv).astype(np.float64)
    ang = (np.float32(pos) * inv).astype(np.float64)  # the f32 product, then f64 cos/sin
    emb = np.concatenate([ang, ang])
    cos = torch.from_numpy(np.cos(emb))[None, None]  # [batch, seq, hd]
    sin = torch.from_numpy(np.sin(emb))[None, None]
    t = torch.from_numpy(x).double()[None, :, None, :]
    ref, _ = apply_rotary_pos_emb(t, t, cos, sin)
    assert np.allclose(got, ref[0, :, 0].numpy(), rtol=1e-6, atol=1e-6)


def test_rope_invariants():
    hd = 64
    rng = np.random.default_rng(3)
    inv = oracle.inv_freq(1e6, hd)
    x = rng.standard_normal((4, hd)).astype(np.float32)
    # position 0 is the identity
    assert np.array_equal(oracle.rope(x, 0, inv), x)
    # each (i, i + hd/2) pair keeps its norm
    y = oracle.rope(x, 12345, inv).astype(np.float64)
    xd = x.astype(np.float64)
    pair = lambda a: a[:, : hd // 2] ** 2 + a[:, hd // 2:] ** 2  # noqa: E731
    assert np.allclose(pair(y), pair(xd), rtol=1e-5)
    # relative: <R(p)q, R(p')k> depends on p - p' only
    q, k = x[0:1], x[1:2]
    d1 = float(np.dot(oracle.rope(q, 10, inv)[0].astype(np.float64), oracle.rope(k, 3, inv)[0]))
    d2 = float(np.dot(oracle.rope(q, 107, inv)[0].astype(np.float64), oracle.rope(k, 100, inv)[0]))
    assert abs(d1 - d2) < 1e-4 * (1 + abs(d1))
    # R(p) then R(-p) gives back x
    z = oracle.rope(oracle.rope(x, 50, inv), -50, inv)
    assert np.allclose(z, x, rtol=1e-5, atol=1e-6)


# ---- A8_32 activation quantizer -----------------------------------------------------------


def test_quant_act_nearest_code_brute_force():
    rng = np.random.default_rng(11)
    # groups of very different magnitudes, so a scale shared across groups would fail
    x = (rng.standard_normal((5, 256)) * np.repeat(10.0 ** rng.uniform(-4, 3, (5, 8)), 32, axis=1)).astype(np.float32)
    q, d = oracle.quant_act(x)
    amax = np.abs(x.reshape(5, 8, 32)).max(axis=2)
    assert np.array_equal(d, (amax / np.float32(127)).astype(np.float32))
    codes = np.arange(-127, 128)
    xd = x.astype(np.float64).reshape(5, 8, 32)
    dd = d.astype(np.float64)[:, :, None, None]
    # every element's code is the nearest of all 255 codes (up to exact ties)
    err = np.abs(xd[..., None] - dd * codes[None, None, None, :])
    best = codes[np.argmin(err, axis=-1)]
    qq = q.reshape(5, 8, 32)
    near_tie = np.abs(np.abs(xd / dd[..., 0] - np.trunc(xd / dd[..., 0])) - 0.5) < 1e-4
    assert np.array_equal(qq[~near_tie], best[~near_tie])
    # error bound and extremes
    assert np.all(np.abs(xd - dd[..., 0] * qq) <= dd[..., 0] * (0.5 + 1e-5))
    i = np.argmax(np.abs(xd), axis=2)
    top = np.take_along_axis(qq, i[..., None], axis=2)[..., 0]
    assert np.all(np.abs(top) == 127)


def test_quant_act_zero_group_and_ties():
    x = np.zeros((1, 64), np.float32)
    x[0, 32:] = np.linspace(-1, 1, 32, dtype=np.float32)
    q, d = oracle.quant_act(x)
    assert d[0, 0] == 0 and np.all(q[0, :32] == 0)
    assert d[0, 1] == np.float32(1.0) / np.float32(127)
    # x * (127/amax) landing on k + 1/2 exactly rounds to the even neighbour
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 127.0
    x[0, 1] = 2.5
    x[0, 2] = 3.5
    x[0, 3] = -2.5
    q, d = oracle.quant_act(x)
    assert d[0, 0] == 1.0 and list(q[0, :4]) == [127, 2, 4, -2]


# ---- quantized matrices -------------------------------------------------------------------


def test_canonical_formats_by_hand():
    # byte 0x21 holds column 0 = 1 (low nibble) and column 1 = 2 (high); 0xF8 holds -8 and -1
    codes = np.zeros((1, 16), np.uint8)
    codes[0, 0], codes[0, 1] = 0x21, 0xF8
    scales = np.array([[1.0]], np.float16)
    w = di.dequantize_rows(codes, scales, di.Q4_32, 32)
    assert list(w[0, :4]) == [1.0, 2.0, -8.0, -1.0]
    xq = np.zeros((1, 32), np.int8)
    xq[0, :4] = [1, 10, 100, 3]
    mat = {"fmt": di.Q4_32, "rows": 1, "cols": 32, "codes": codes, "scales": scales}
    assert oracle.group_sums(mat, xq)[0, 0, 0] == 1 + 20 - 800 - 3


@pytest.mark.parametrize("fmt", [di.Q4_32, di.Q8_32])
def test_weight_coding_round_trip(fmt):
    rng = np.random.default_rng(fmt)
    w = (rng.standard_normal((40, 256)) * 0.02).astype(np.float32)
    w[3, 64:96] = 0  # an all-zero group
    codes, scales = di.quantize_rows(w, fmt)
    back = di.dequantize_rows(codes, scales, fmt, 256)
    d = scales.astype(np.float64).repeat(32, axis=1)
    assert np.all(np.abs(back - w) <= d * 0.5 + 1e-12)
    assert np.all(back[3, 64:96] == 0)


@pytest.mark.parametrize("fmt", [di.Q4_32, di.Q8_32])
def test_quantized_matmul_against_dense(fmt):
    rng = np.random.default_rng(20 + fmt)
    rows, cols, m = 48, 320, 5
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    codes, scales = di.quantize_rows(w, fmt)
    mat = {"fmt": fmt, "rows": rows, "cols": cols, "codes": codes, "scales": scales}
    x = rng.standard_normal((m, cols)).astype(np.float32)
    xq, dx = oracle.quant_act(x)
    y = oracle.matmul_q(mat, xq, dx).astype(np.float64)
    wd = di.dequantize_rows(codes, scales, fmt, cols)
    xd = xq.astype(np.float64) * dx.astype(np.float64).repeat(32, axis=1)
    ref = xd @ wd.T
    bound = np.abs(xd) @ np.abs(wd).T
    assert np.all(np.abs(y - ref) <= 1e-6 * bound + 1e-30)
    # and close to the unquantized product (quantization error only)
    full = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.abs(y - full).max() < 0.2 * np.abs(full).max()
    # integer group sums by brute force
    s = oracle.group_sums(mat, xq).astype(np.int64)
    qw = np.rint(wd / scales.astype(np.float64).repeat(32, axis=1)).astype(np.int64)
    ref_s = np.einsum("mgk,rgk->mrg", xq.astype(np.int64).reshape(m, cols // 32, 32), qw.reshape(rows, cols // 32, 32))
    assert np.array_equal(s, ref_s)


def test_f32_matmul_against_numpy():
    rng = np.random.default_rng(7)
    w = rng.standard_normal((33, 96)).astype(np.float32)
    x = rng.standard_normal((4, 96)).astype(np.float32)
    y = oracle.matmul_f32(w, x)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.allclose(y, ref, rtol=1e-6, atol=1e-6)


# ---- attention ----------------------------------------------------------------------------


def test_attention_against_torch_sdpa():
    rng = np.random.default_rng(9)
    nq, nk, hd = 6, 75, 64
    q = rng.standard_normal((nq, hd)).astype(np.float32)
    k = rng.standard_normal((nk, hd)).astype(np.float32)
    v = rng.standard_normal((nk, hd)).astype(np.float32)
    scale = float(np.float32(hd) ** np.float32(-0.5))
    y, p = oracle.attend(q, k, v, scale, want_p=True)
    t = lambda a: torch.from_numpy(a).double()[None, None]  # noqa: E731
    ref = F.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale)[0, 0].numpy()
    assert np.allclose(y, ref, rtol=1e-6, atol=1e-6)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(10)
    hd = 32
    q = rng.standard_normal((3, hd)).astype(np.float32)
    k = rng.standard_normal((1, hd)).astype(np.float32)
    v = rng.standard_normal((1, hd)).astype(np.float32)
    assert np.allclose(oracle.attend(q, k, v, 0.2), np.repeat(v, 3, axis=0), atol=1e-7)
    k4 = np.repeat(k, 4, axis=0)
    v4 = rng.standard_normal((4, hd)).astype(np.float32)
    assert np.allclose(oracle.attend(q, k4, v4, 0.2), np.repeat(v4.astype(np.float64).mean(0, keepdims=True), 3, 0), atol=1e-6)
    # permuting the keys (with their values) changes nothing
    k = rng.standard_normal((40, hd)).astype(np.float32)
    v = rng.standard_normal((40, hd)).astype(np.float32)
    perm = rng.permutation(40)
    assert np.allclose(oracle.attend(q, k, v, 0.3), oracle.attend(q, k[perm], v[perm], 0.3), atol=1e-6)
    # the online-softmax merge of two halves equals the whole
    def part(kk, vv):
        s = (q.astype(np.float64) @ kk.astype(np.float64).T) * 0.3
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        return m, e.sum(axis=1, keepdims=True), e @ vv.astype(np.float64)
    m1, l1, a1 = part(k[:17], v[:17])
    m2, l2, a2 = part(k[17:], v[17:])
    mm = np.maximum(m1, m2)
    merged = (a1 * np.exp(m1 - mm) + a2 * np.exp(m2 - mm)) / (l1 * np.exp(m1 - mm) + l2 * np.exp(m2 - mm))
    assert np.allclose(oracle.attend(q, k, v, 0.3), merged, atol=1e-6)


def test_silu_against_torch():
    rng = np.random.default_rng(12)
    g = (rng.standard_normal(1000) * 6).astype(np.float32)
    u = rng.standard_normal(1000).astype(np.float32)
    a = oracle.silu_mul(g, u)
    ref = (F.silu(torch.from_numpy(g).double()) * torch.from_numpy(u).double()).numpy()
    assert np.allclose(a, ref, rtol=2e-7, atol=1e-30)
    z = oracle.silu_mul(np.array([0.0, 40.0, -40.0], np.float32), np.ones(3, np.float32))
    assert z[0] == 0 and abs(z[1] - 40) < 1e-5 and abs(z[2]) < 1e-15
