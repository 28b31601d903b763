"""Candidate selection on the GPU (cortiq-engine dflash.rs: top_k, Drafter::select_with) against
the oracle: the top-k lists bit for bit (values and indices, ties included), and the chosen
tokens of the greedy re-scoring.  Inputs come from the seeded generators or from the oracle."""
import numpy as np
import pytest

import dflash_inputs as di
import oracle
from gpu_common import say, weights_for

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _st():
    return torch.cuda.current_stream().cuda_stream


def _gpu_top_k(x: np.ndarray, k: int, ld: int | None = None):
    import block_draft_model_dflash_amd as D

    rows, width = x.shape
    ld = ld or width
    buf = np.zeros((rows, ld), np.float32)
    buf[:, :width] = x
    gx = torch.from_numpy(buf).cuda()
    vals = torch.empty((rows, k), dtype=torch.float32, device="cuda")
    idx = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    scratch = torch.empty(D.dflash_top_k_scratch_bytes(rows, width, k), dtype=torch.uint8, device="cuda")
    D.dflash_top_k(gx.data_ptr(), rows, width, ld, k, vals.data_ptr(), idx.data_ptr(), scratch.data_ptr(), _st())
    torch.cuda.synchronize()
    return vals.cpu().numpy(), idx.cpu().numpy()


@pytest.mark.parametrize("width,k,ld", [(6, 3, 6), (100, 1, 128), (4096, 16, 4096), (4097, 16, 4100),
                                        (151936, 16, 151936), (151936, 64, 151936), (40000, 64, 40001)])
def test_top_k_matches_the_oracle(width, k, ld):
    rng = np.random.default_rng(width + k)
    rows = 5
    say(f"top_k width={width} k={k}")
    x = rng.standard_normal((rows, width)).astype(np.float32)
    x[1] = rng.integers(-3, 4, width).astype(np.float32)  # a row of many equal values
    x[2, :] = 1.0  # every value equal: the first k indices
    # the largest values crowded into few threads of one workgroup (the first 16 of every 256
    # indices of the first chunk): more candidates than one sort holds
    i = np.arange(min(width, 4096))
    x[3, i[(i % 256) < 16]] += 10.0
    x[4, ::7] = -0.0  # -0 ties with +0 (and with the other zeros)
    x[4, 3::7] = 0.0
    vals, idx = _gpu_top_k(x, k, ld)
    for r in range(rows):
        ov, oi = oracle.top_k(x[r], k)
        assert np.array_equal(idx[r], oi), r
        assert np.array_equal(vals[r], ov), r


def test_top_k_pages_example_on_gpu():
    x = np.array([[0.5, 2.0, -1.0, 2.0, 3.5, 0.0]], np.float32)
    vals, idx = _gpu_top_k(x, 3)
    assert list(idx[0]) == [4, 1, 3] and list(vals[0]) == [3.5, 2.0, 2.0]


def _gpu_select(logits, hp, pred, succ, top, anchor, ld=None, width=None):
    """logits [rows][ld or its width]: each row's first `width` entries (all, by default) count."""
    import block_draft_model_dflash_amd as D

    rows, width = logits.shape[0], width or logits.shape[1]
    vocab, rank = pred.shape
    gl = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
    gh = torch.from_numpy(np.ascontiguousarray(hp, np.float32)).cuda()
    gp = torch.from_numpy(np.ascontiguousarray(pred, np.float16).view(np.int16)).cuda()
    gs = torch.from_numpy(np.ascontiguousarray(succ, np.float16).view(np.int16)).cuda()
    chosen = torch.empty(rows, dtype=torch.int32, device="cuda")
    plain = torch.empty(rows, dtype=torch.int32, device="cuda")
    scratch = torch.empty(D.dflash_select_scratch_bytes(rows, width, top), dtype=torch.uint8, device="cuda")
    D.dflash_select(gl.data_ptr(), rows, width, ld or width, gh.data_ptr(), rank, gp.data_ptr(), gs.data_ptr(), vocab,
                    top, anchor, chosen.data_ptr(), plain.data_ptr(), scratch.data_ptr(), _st())
    torch.cuda.synchronize()
    return chosen.cpu().numpy(), plain.cpu().numpy()


# scores for every predecessor option with the rows' tables in LDS (the first four), and the
# sequential kernel when the tables exceed LDS (rank 4096 with 40 candidates)
@pytest.mark.parametrize("rows,vocab,rank,top", [(7, 1000, 32, 8), (15, 151936, 128, 16), (3, 50, 5, 50),
                                                 (15, 40000, 128, 64), (2, 100, 4096, 40)])
def test_select_matches_the_oracle(rows, vocab, rank, top):
    rng = np.random.default_rng(rows * 7 + rank)
    say(f"select rows={rows} vocab={vocab} rank={rank} top={top}")
    logits = rng.standard_normal((rows, vocab)).astype(np.float32)
    hp = rng.standard_normal((rows, rank)).astype(np.float32)
    pred = (rng.standard_normal((vocab, rank)) * 0.3).astype(np.float16)
    succ = (rng.standard_normal((vocab, rank)) * 0.3).astype(np.float16)
    chosen, plain = _gpu_select(logits, hp, pred, succ, top, 17 % vocab)
    oc, op = oracle.select(logits, hp, pred, succ, top, 17 % vocab)
    assert np.array_equal(plain, op)
    assert np.array_equal(chosen, oc)
    # the re-scoring changes some choices here, so the test exercises it
    if rows >= 7:
        assert (chosen != plain).any()


@pytest.mark.timeout(600)
def test_selection_chain_of_the_8b_drafter():
    """The whole chain on the 8B-shaped drafter: GPU block (final hidden rows) -> A8 -> selector
    projection (Q8_32 GEMM) -> GPU selection, against the same chain in the oracle: the chosen
    draft tokens agree."""
    import block_draft_model_dflash_amd as D
    from block_draft_model_dflash_amd import Drafter

    cfg = di.CONFIGS["qwen3_8b"].replace(ctx=512)
    w = weights_for(cfg)
    sel = di.make_selector(cfg)
    rank, top, anchor_tok = sel["rank"], 16, 1234
    om = oracle.Model(cfg, w, max_ctx=cfg.ctx + 64)
    gm = Drafter(cfg, w, max_ctx=cfg.ctx + 64)
    taps = di.make_taps(cfg, 0, 0, cfg.ctx)
    assert om.append(0, 0, taps) == 0
    gm.append(0, 0, taps)
    h = di.make_block_input(cfg, 0, 0)[None]
    # oracle chain
    hid = om.block_hidden([0], [cfg.ctx], h).reshape(cfg.block, cfg.hidden)[1:]
    logits = om.block_forward([0], [cfg.ctx], h).reshape(cfg.block, cfg.vocab)[1:]
    hp = oracle.matmul(sel["sel"], hid)
    oc, op = oracle.select(logits, hp, sel["pred"], sel["succ"], top, anchor_tok)
    # GPU chain
    ghid = gm.block_hidden([0], [cfg.ctx], h).reshape(cfg.block, cfg.hidden)[1:].contiguous()
    glog = gm.block_forward([0], [cfg.ctx], h).reshape(cfg.block, cfg.vocab)
    n = cfg.block - 1
    gq = torch.empty((n, cfg.hidden), dtype=torch.int8, device="cuda")
    gd = torch.empty((n, cfg.hidden // 32), dtype=torch.float32, device="cuda")
    D.dflash_quant_act(ghid.data_ptr(), n, cfg.hidden, gq.data_ptr(), gd.data_ptr(), _st())
    packed = torch.empty(D.dflash_packed_bytes(cfg.head_fmt, rank, cfg.hidden), dtype=torch.uint8, device="cuda")
    codes = torch.from_numpy(sel["sel"]["codes"].view(np.uint8)).cuda()
    scales = torch.from_numpy(sel["sel"]["scales"].view(np.uint16)).cuda()
    D.dflash_pack(cfg.head_fmt, rank, cfg.hidden, codes.data_ptr(), scales.data_ptr(), packed.data_ptr(), _st())
    ghp = torch.empty((n, rank), dtype=torch.float32, device="cuda")
    scr = torch.empty(D.dflash_gemm_scratch_bytes(rank, cfg.hidden, n, 0), dtype=torch.uint8, device="cuda")
    D.dflash_gemm(cfg.head_fmt, packed.data_ptr(), rank, cfg.hidden, gq.data_ptr(), gd.data_ptr(), n,
                  ghp.data_ptr(), 0, scr.data_ptr(), _st())
    gp = torch.from_numpy(sel["pred"].view(np.int16)).cuda()
    gs = torch.from_numpy(sel["succ"].view(np.int16)).cuda()
    chosen = torch.empty(n, dtype=torch.int32, device="cuda")
    plain = torch.empty(n, dtype=torch.int32, device="cuda")
    ss = torch.empty(D.dflash_select_scratch_bytes(n, cfg.vocab, top), dtype=torch.uint8, device="cuda")
    D.dflash_select(glog.data_ptr() + cfg.vocab * 4, n, cfg.vocab, cfg.vocab, ghp.data_ptr(), rank, gp.data_ptr(),
                    gs.data_ptr(), cfg.vocab, top, anchor_tok, chosen.data_ptr(), plain.data_ptr(), ss.data_ptr(),
                    _st())
    torch.cuda.synchronize()
    say(f"chosen {chosen.cpu().numpy().tolist()} plain {plain.cpu().numpy().tolist()}")
    assert np.array_equal(plain.cpu().numpy(), op)
    assert np.array_equal(chosen.cpu().numpy(), oc)


# random widths, k, strides and value mixes; DFLASH_TOPK_CASES asks for a longer sweep
TOPK_CASES = int(__import__("os").environ.get("DFLASH_TOPK_CASES", "60"))


@pytest.mark.parametrize("seed", range(TOPK_CASES))
def test_top_k_random_shapes(seed):
    """Seeded random shapes: width 1..160000, k 1..min(64, width), a row stride past the width,
    and rows drawn from five mixes (normal, a few integer values with many ties, one constant,
    maxima crowded into one corner of a chunk, signed zeros among small values).  Indices must
    equal the oracle's, ties included, and values compare equal to it and to the entries they
    index (a -0 entry ties with +0 and comes back as +0, which compares equal)."""
    r = np.random.default_rng(50_000 + seed)
    width = int(r.choice([int(r.integers(1, 300)), int(r.integers(300, 20000)), int(r.integers(20000, 160000))]))
    k = int(r.integers(1, min(64, width) + 1))
    ld = width + int(r.choice([0, 0, 1, 7, 64]))
    rows = int(r.integers(1, 6))
    x = np.empty((rows, width), np.float32)
    for row in range(rows):
        mix = int(r.integers(5))
        if mix == 0:
            x[row] = r.standard_normal(width)
        elif mix == 1:
            x[row] = r.integers(-2, 3, width)
        elif mix == 2:
            x[row] = np.float32(r.standard_normal())
        elif mix == 3:
            x[row] = r.standard_normal(width)
            lo = int(r.integers(0, width))
            x[row, lo:lo + int(r.integers(1, 300))] += 50.0
        else:
            x[row] = np.round(r.standard_normal(width), 1) * (r.random(width) < 0.5)
            x[row, r.random(width) < 0.3] = -0.0
    say(f"top_k random seed={seed} rows={rows} width={width} k={k} ld={ld}")
    vals, idx = _gpu_top_k(x, k, ld)
    for row in range(rows):
        ov, oi = oracle.top_k(x[row], k)
        assert np.array_equal(idx[row], oi), (seed, row)
        assert np.array_equal(vals[row], ov), (seed, row)
        assert np.array_equal(vals[row], x[row, idx[row]]), (seed, row)


SELECT_CASES = int(__import__("os").environ.get("DFLASH_SELECT_CASES", "40"))


@pytest.mark.parametrize("seed", range(SELECT_CASES))
def test_select_random_shapes(seed):
    """Seeded random selector problems: 1..16 rows, vocab 2..60000 (width up to the vocab, a row
    stride past it), rank 1..512 (now and then 4096, the sequential kernel), top 1..min(64,
    width), any anchor; logits sometimes with many ties, codebooks sometimes all zero (the
    re-scoring then keeps each row's own top token).  Chosen and plain tokens must equal the
    oracle's."""
    r = np.random.default_rng(70_000 + seed)
    rows = int(r.integers(1, 17))
    vocab = int(r.choice([int(r.integers(2, 200)), int(r.integers(200, 5000)), int(r.integers(5000, 60000))]))
    width = int(r.integers(1, vocab + 1)) if r.integers(4) == 0 else vocab
    ld = width + int(r.choice([0, 0, 3]))
    rank = 4096 if r.integers(12) == 0 else int(r.integers(1, 513))
    top = int(r.integers(1, min(64, width) + 1))
    anchor = int(r.integers(0, vocab))
    logits = r.standard_normal((rows, width)).astype(np.float32)
    if r.integers(3) == 0:
        logits = np.round(logits * 2).astype(np.float32)  # many equal logits
    hp = r.standard_normal((rows, rank)).astype(np.float32)
    scale = 0.0 if r.integers(6) == 0 else float(r.choice([0.05, 0.3, 1.0]))
    pred = (r.standard_normal((vocab, rank)) * scale).astype(np.float16)
    succ = (r.standard_normal((vocab, rank)) * scale).astype(np.float16)
    say(f"select random seed={seed} rows={rows} vocab={vocab} width={width} ld={ld} rank={rank} top={top}")
    buf = np.zeros((rows, ld), np.float32)
    buf[:, :width] = logits
    chosen, plain = _gpu_select(buf, hp, pred, succ, top, anchor, ld=ld, width=width)
    oc, op = oracle.select(logits, hp, pred, succ, top, anchor)
    assert np.array_equal(plain, op), seed
    assert np.array_equal(chosen, oc), seed
    if scale == 0.0:
        assert np.array_equal(chosen, plain), seed
