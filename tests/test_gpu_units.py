"""GPU unit parity through the C ABI: the activation quantizer and the quantized product's
integer accumulators are bit-exact against the oracle on identical inputs; the product itself
agrees to its f32 rounding bound."""
import numpy as np
import pytest

import block_draft_model_dflash_amd as D
import dflash_inputs as di
import oracle
from gpu_common import say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _st():
    return torch.cuda.current_stream().cuda_stream


def _acts(rng, rows, cols):
    x = rng.standard_normal((rows, cols)) * np.repeat(10.0 ** rng.uniform(-3, 2, (rows, cols // 32)), 32, axis=1)
    x = x.astype(np.float32)
    if cols >= 64:
        x[0, 32:64] = 0.0  # a zero group
    x[-1, :4] = [127.0, 2.5, -3.5, 0.5]  # exact ties under d = 1
    x[-1, 4:32] = 0.0
    return x


@pytest.mark.parametrize("rows,cols", [(1, 32), (7, 256), (16, 4096), (130, 2048), (3, 20480)])
def test_quant_act_bit_exact(rows, cols):
    say(f"quant_act rows={rows} cols={cols}")
    rng = np.random.default_rng(rows * 7 + cols)
    x = _acts(rng, rows, cols)
    q, d = oracle.quant_act(x)
    gq = torch.empty((rows, cols), dtype=torch.int8, device="cuda")
    gd = torch.empty((rows, cols // 32), dtype=torch.float32, device="cuda")
    gx = _dev(x)  # held: a temporary's memory could be handed to the next allocation
    D.dflash_quant_act(gx.data_ptr(), rows, cols, gq.data_ptr(), gd.data_ptr(), _st())
    torch.cuda.synchronize()
    assert np.array_equal(gq.cpu().numpy(), q)
    assert np.array_equal(gd.cpu().numpy(), d)


def _matrix(rng, fmt, rows, cols, full_range=True):
    """Codes over the whole range the decoder accepts (-8..7 / -128..127) and positive scales."""
    scales = (rng.uniform(0.5, 2.0, (rows, cols // 32)) * 0.01).astype(np.float16)
    if fmt == di.Q4_32:
        codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    else:
        codes = rng.integers(-128 if full_range else -127, 128, (rows, cols), dtype=np.int16).astype(np.int8)
    return {"fmt": fmt, "rows": rows, "cols": cols, "codes": codes, "scales": scales}


def _packed(mat):
    n = D.dflash_packed_bytes(mat["fmt"], mat["rows"], mat["cols"])
    p = torch.empty(n, dtype=torch.uint8, device="cuda")
    c, s = _dev(mat["codes"]), _dev(mat["scales"])
    D.dflash_pack(mat["fmt"], mat["rows"], mat["cols"], c.data_ptr(), s.data_ptr(), p.data_ptr(), _st())
    torch.cuda.synchronize()
    return p


SHAPES = [(16, 128, 1), (48, 384, 5), (64, 256, 16), (32, 512, 33), (16, 128, 128), (80, 1024, 100)]
# K long enough for several activation chunks in LDS, the last one ragged (16, 48 and 128 rows)
GEMM_SHAPES = SHAPES + [(64, 4608, 16), (48, 2560, 40), (32, 1152, 128)]


@pytest.mark.parametrize("fmt", [di.Q4_32, di.Q8_32], ids=["q4", "q8"])
@pytest.mark.parametrize("rows,cols,m", SHAPES)
def test_group_sums_bit_exact(fmt, rows, cols, m):
    say(f"group_sums fmt={fmt} rows={rows} cols={cols} m={m}")
    rng = np.random.default_rng(rows + cols + m + fmt)
    mat = _matrix(rng, fmt, rows, cols)
    xq = rng.integers(-127, 128, (m, cols), dtype=np.int16).astype(np.int8)
    ref = oracle.group_sums(mat, xq)
    p = _packed(mat)
    scratch = torch.empty(D.dflash_gemm_scratch_bytes(rows, cols, m, 1), dtype=torch.uint8, device="cuda")
    sums = torch.empty((m, rows, cols // 32), dtype=torch.int32, device="cuda")
    gx = _dev(xq)
    D.dflash_group_sums(fmt, p.data_ptr(), rows, cols, gx.data_ptr(), m, sums.data_ptr(), scratch.data_ptr(), _st())
    torch.cuda.synchronize()
    assert np.array_equal(sums.cpu().numpy(), ref)


@pytest.mark.parametrize("fmt", [di.Q4_32, di.Q8_32], ids=["q4", "q8"])
@pytest.mark.parametrize("rows,cols,m", GEMM_SHAPES)
@pytest.mark.parametrize("splits", [0, 1, 2, 8])
def test_gemm_correctly_rounded(fmt, rows, cols, m, splits):
    _check_gemm(fmt, rows, cols, m, splits)


def _check_gemm(fmt, rows, cols, m, splits):
    """The product is the f32 rounding of its exact value, as the oracle's f64 evaluation: equal
    to the oracle's f32 except where the two f64 sums straddle a rounding boundary (rare), and
    never more than one ulp apart."""
    say(f"gemm fmt={fmt} rows={rows} cols={cols} m={m} splits={splits}")
    rng = np.random.default_rng(rows * 3 + cols + m + fmt + splits)
    mat = _matrix(rng, fmt, rows, cols)
    x = _acts(rng, m, cols)
    xq, dx = oracle.quant_act(x)
    ref = oracle.matmul_q(mat, xq, dx).astype(np.float64)
    # bound of the f32 accumulation: (groups + 2) ulps of sum |d_w d_x s_g|
    s = oracle.group_sums(mat, xq).astype(np.float64)
    dw = mat["scales"].astype(np.float64)
    mag = np.einsum("mrg,rg,mg->mr", np.abs(s), dw, dx.astype(np.float64))
    tol = (cols // 32 + 2) * 2.0 ** -23 * mag + 1e-30
    p = _packed(mat)
    scratch = torch.empty(D.dflash_gemm_scratch_bytes(rows, cols, m, splits), dtype=torch.uint8, device="cuda")
    y = torch.empty((m, rows), dtype=torch.float32, device="cuda")
    gx, gd = _dev(xq), _dev(dx)
    D.dflash_gemm(fmt, p.data_ptr(), rows, cols, gx.data_ptr(), gd.data_ptr(), m, y.data_ptr(), splits,
                  scratch.data_ptr(), _st())
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(err <= tol), float((err / tol).max())
    ref32 = ref.astype(np.float32)
    ulp = np.spacing(np.abs(ref32)).astype(np.float64)
    assert np.all(err <= ulp)
    assert np.mean(got == ref32) >= 0.999


# The production loops' integer accumulators, bit for bit: with every weight scale and activation
# scale 1.0 each rescale term d_w * d_x * s_g is the group sum s_g itself, every f64 partial sum is
# an integer below 2^53, and the f32 output below 2^24 is exact, so the product must equal the sum
# over groups of the oracle's integer group sums exactly.  One case per path the product takes:
# the K-split kernel (16 rows, few n-tiles), one and two k-waves per n-tile, eight n-tiles a
# workgroup (16 rows, more than 1024 n-tiles; the head's K) and the row kernel (more than 16 rows).
UNIT_SHAPES = [(96, 4096, 16, 0), (96, 4096, 16, 8), (48, 2560, 16, 1), (64, 4608, 16, 2), (16400, 1024, 16, 0),
               (65600, 4096, 16, 0), (96, 4096, 48, 0), (80, 1024, 128, 0), (2048, 512, 100, 0)]


@pytest.mark.parametrize("fmt", [di.Q4_32, di.Q8_32], ids=["q4", "q8"])
@pytest.mark.parametrize("rows,cols,m,splits", UNIT_SHAPES)
def test_gemm_integer_accumulators_exact(fmt, rows, cols, m, splits):
    say(f"gemm unit scales fmt={fmt} rows={rows} cols={cols} m={m} splits={splits}")
    rng = np.random.default_rng(rows + 5 * cols + m + fmt + splits)
    mat = _matrix(rng, fmt, rows, cols)
    mat["scales"] = np.ones_like(mat["scales"])
    xq = rng.integers(-127, 128, (m, cols), dtype=np.int16).astype(np.int8)
    want = oracle.group_sums(mat, xq).astype(np.int64).sum(axis=2)
    assert np.abs(want).max() < 2 ** 24  # exact in f32
    p = _packed(mat)
    scratch = torch.empty(D.dflash_gemm_scratch_bytes(rows, cols, m, splits), dtype=torch.uint8, device="cuda")
    y = torch.empty((m, rows), dtype=torch.float32, device="cuda")
    gx, gd = _dev(xq), _dev(np.ones((m, cols // 32), np.float32))
    D.dflash_gemm(fmt, p.data_ptr(), rows, cols, gx.data_ptr(), gd.data_ptr(), m, y.data_ptr(), splits,
                  scratch.data_ptr(), _st())
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.int64), want)


# thousands of n-tiles with 16 activation rows: workgroups of eight n-tiles (ragged: 1025 tiles
# are not a whole number of eight-tile blocks)
@pytest.mark.parametrize("fmt", [di.Q4_32, di.Q8_32], ids=["q4", "q8"])
# (65600 rows: 4100 n-tiles, more than four rounds of the grid, the head's K)
@pytest.mark.parametrize("rows,cols,m", [(16400, 2048, 16), (16400, 4096, 3), (65600, 4096, 16), (65600, 4096, 5)])
def test_gemm_many_tiles(fmt, rows, cols, m):
    _check_gemm(fmt, rows, cols, m, 0)


GEMM_CASES = int(__import__("os").environ.get("DFLASH_GEMM_CASES", "100"))


@pytest.mark.parametrize("seed", range(GEMM_CASES))
def test_gemm_random_shapes(seed):
    """Seeded random products: 16..4096 weight rows, 128..6144 columns, 1..128 activation rows,
    either format, any of the layouts (splits 0 = chosen from the shape, 1, 2, 8); the bar of
    the fixed shapes above (one ulp at most, 99.9% equal to the oracle's f32)."""
    r = np.random.default_rng(90_000 + seed)
    rows = 16 * int(r.integers(1, 257))
    cols = 128 * int(r.integers(1, 49))
    m = int(r.integers(1, 17)) if r.integers(2) else int(r.integers(17, 129))
    while m > 1 and rows * cols * m > 400_000_000:  # keep the oracle's share to a few seconds
        m //= 2
    fmt = di.Q4_32 if r.integers(2) else di.Q8_32
    splits = int(r.choice([0, 1, 2, 8]))
    _check_gemm(fmt, rows, cols, m, splits)
