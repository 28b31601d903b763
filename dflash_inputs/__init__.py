"""Seeded synthetic inputs for the DFlash 2 block drafter: geometries, weights and rows.

This module is shared by the CPU oracle (``oracle/``) and the GPU path
(``block_draft_model_dflash_amd``); it holds none of the forward pass's
arithmetic.  It only draws numbers and stores them in the canonical formats
both sides decode on their own:

* ``F32``   -- row-major float32 ``[rows][cols]``.
* ``Q4_32`` -- per output row and group of 32 input columns one float16 scale
  ``d`` and 32 four-bit two's-complement codes ``q``; the weight is
  ``float(d) * q``.  Codes plane ``uint8 [rows][cols/2]`` with column ``2j``
  in the low nibble of byte ``j`` and ``2j+1`` in the high nibble; scales
  plane ``float16 [rows][cols/32]``.
* ``Q8_32`` -- the same with int8 codes ``int8 [rows][cols]``.

The pages (cortiq-engine ``gpu_wgpu/dflash_dev.rs``, ``kind_of``) name a
four-bit tiled and an eight-bit format without giving their bytes, so the
layouts above are this project's contract.  Turning the drawn float weights
into those codes is the sidecar converter's job on the pages (``cortiq
convert --dflash-sidecar``, named in the module header of ``dflash.rs``), not
part of the drafter's forward pass, which is why it lives here as data
preparation: ``amax`` of the group, ``d = f16(amax / qmax)``,
``q = clip(rint(w / d), -qmax, qmax)`` with ``qmax`` 7 (Q4) or 127 (Q8).

Every draw comes from ``numpy.random.Generator(PCG64)`` keyed by a
``SeedSequence([seed, stream, index])`` so each tensor, each context chunk and
each block input is reproducible on its own, on any machine.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

F32, Q4_32, Q8_32 = 0, 1, 2
FMT_NAMES = {F32: "f32", Q4_32: "q4_32", Q8_32: "q8_32"}

# stream ids of SeedSequence([seed, stream, index])
_S_WEIGHT, _S_NORM, _S_TAPS, _S_ANCHOR, _S_MASK, _S_SELECTOR, _S_CONV = 1, 2, 3, 4, 5, 6, 7


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload: the drafter's geometry plus how its inputs look."""

    key: str
    layers: int
    hidden: int
    heads: int
    kv_heads: int
    head_dim: int
    intermediate: int
    n_taps: int
    vocab: int
    block: int
    ctx: int  # context rows held before the first block (per sequence)
    body_fmt: int
    fc_fmt: int
    head_fmt: int
    n_seqs: int = 1
    append_per_block: int = 0  # rows appended before each block (long-context workload)
    rope_theta: float = 1.0e6
    eps: float = 1.0e-6
    weight_std: float = 0.02
    norm_mean: float = 1.0  # norm weights are norm_mean + N(0, norm_std)
    norm_std: float = 0.02
    taps_std: float = 1.0
    emb_std: float = 0.02
    seed: int = 1000
    weight_seed: int = 0  # seed of the weights when they are another workload's drafter (0: seed)
    # row convolutions around attention and the MLP (0: none, the plain Qwen3 layer): columns
    # per kernel group, offsets per kernel, and the spread of the kernel projections' weights
    conv_group: int = 0
    conv_kernel: int = 0
    conv_std: float = 0.0025
    kv_f16: bool = False  # the K/V cache holds f16 elements instead of f32
    pending_rows: int = 0  # context rows that may wait unsettled (0: every row settles at once)

    @property
    def tap_width(self) -> int:
        return self.n_taps * self.hidden

    @property
    def q_dim(self) -> int:
        return self.heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.kv_heads * self.head_dim

    @property
    def conv_rows(self) -> int:
        """Rows of a kernel projection: two stages x offsets x groups."""
        return 2 * self.conv_kernel * (self.hidden // self.conv_group) if self.conv_kernel else 0

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# The five workloads: sizes as their descriptions state, inputs as drawn below.
CONFIGS = {
    # tiny, unquantized: every weight and input N(0, 0.02), norm weights included
    "tiny_f32": Config("tiny_f32", 1, 256, 4, 2, 64, 768, 3, 4096, 8, 64,
                       F32, F32, F32, norm_mean=0.0, norm_std=0.02, taps_std=0.02, seed=1001),
    "small_q": Config("small_q", 1, 2048, 16, 4, 128, 6144, 4, 32768, 16, 512,
                      Q4_32, Q8_32, Q8_32, seed=1002),
    "qwen3_8b": Config("qwen3_8b", 5, 4096, 32, 8, 128, 12288, 5, 151936, 16, 4096,
                       Q4_32, Q8_32, Q8_32, seed=1003),
    # the same 8B-shaped drafter (its weights drawn from seed 1003) over other contexts
    "qwen3_8b_long": Config("qwen3_8b_long", 5, 4096, 32, 8, 128, 12288, 5, 151936, 16, 32768,
                            Q4_32, Q8_32, Q8_32, append_per_block=16, seed=1004, weight_seed=1003),
    "qwen3_8b_batch8": Config("qwen3_8b_batch8", 5, 4096, 32, 8, 128, 12288, 5, 151936, 16, 8192,
                              Q4_32, Q8_32, Q8_32, n_seqs=8, seed=1005, weight_seed=1003),
}
CONFIG_ORDER = ["tiny_f32", "small_q", "qwen3_8b", "qwen3_8b_long", "qwen3_8b_batch8"]


def shrink(cfg: Config, **kw) -> Config:
    """A smaller twin of a workload (same formats and distributions)."""
    return cfg.replace(**kw)


def _rng(seed: int, stream: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, index])))


# ---------------------------------------------------------------------------------------------
# weight preparation (the converter's job on the pages, not the forward pass)


def quantize_rows(w: np.ndarray, fmt: int):
    """Float weights [rows][cols] -> (codes, scales) in the canonical format ``fmt``."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if fmt == F32:
        return w, None
    rows, cols = w.shape
    assert cols % 32 == 0, "quantized matrices need cols % 32 == 0"
    qmax = 7 if fmt == Q4_32 else 127
    g = w.reshape(rows, cols // 32, 32)
    amax = np.abs(g).max(axis=2)
    d16 = (amax / np.float32(qmax)).astype(np.float16)
    d32 = d16.astype(np.float32)
    safe = np.where(d32 == 0, np.float32(1), d32)
    q = np.rint(g / safe[:, :, None])
    q = np.clip(q, -qmax, qmax)
    q[d32 == 0] = 0
    q = q.astype(np.int8).reshape(rows, cols)
    if fmt == Q8_32:
        return q, d16
    nib = (q.astype(np.uint8) & np.uint8(0x0F))
    codes = nib[:, 0::2] | (nib[:, 1::2] << np.uint8(4))
    return np.ascontiguousarray(codes), d16


def dequantize_rows(codes: np.ndarray, scales, fmt: int, cols: int) -> np.ndarray:
    """Canonical format -> float64 weights (a plain decode, used by tests and brute force)."""
    if fmt == F32:
        return np.asarray(codes, dtype=np.float64)
    rows = codes.shape[0]
    if fmt == Q8_32:
        q = codes.astype(np.int64)
    else:
        lo = (codes & 0x0F).astype(np.int64)
        hi = (codes >> 4).astype(np.int64)
        lo = np.where(lo >= 8, lo - 16, lo)
        hi = np.where(hi >= 8, hi - 16, hi)
        q = np.empty((rows, cols), dtype=np.int64)
        q[:, 0::2] = lo
        q[:, 1::2] = hi
    d = scales.astype(np.float64).repeat(32, axis=1)
    return q.astype(np.float64) * d


def _draw_matrix(cfg: Config, index: int, rows: int, cols: int, fmt: int, chunk_rows: int = 8192,
                 std: float | None = None):
    """N(0, weight_std) [rows][cols] drawn in row chunks (each chunk its own stream), then coded."""
    codes_parts, scale_parts = [], []
    for c0 in range(0, rows, chunk_rows):
        n = min(chunk_rows, rows - c0)
        r = _rng(cfg.weight_seed or cfg.seed, _S_WEIGHT, index * 100003 + c0 // chunk_rows)
        w = r.standard_normal((n, cols), dtype=np.float32) * np.float32(cfg.weight_std if std is None else std)
        c, s = quantize_rows(w, fmt)
        codes_parts.append(c)
        if s is not None:
            scale_parts.append(s)
    codes = np.concatenate(codes_parts, axis=0) if len(codes_parts) > 1 else codes_parts[0]
    scales = (np.concatenate(scale_parts, axis=0) if len(scale_parts) > 1 else scale_parts[0]) if scale_parts else None
    return {"fmt": fmt, "rows": rows, "cols": cols, "codes": codes, "scales": scales}


def _norm_vec(cfg: Config, index: int, n: int) -> np.ndarray:
    r = _rng(cfg.weight_seed or cfg.seed, _S_NORM, index)
    return (np.float32(cfg.norm_mean) + r.standard_normal(n, dtype=np.float32) * np.float32(cfg.norm_std)).astype(np.float32)


MATRIX_NAMES = ["q", "k", "v", "o", "gate", "up", "down"]
CONV_NAMES = ["attn_kp", "mlp_kp"]  # kernel projections of the attention and MLP convolutions
NORM_NAMES = ["in_norm", "post_norm", "q_norm", "k_norm"]


def make_weights(cfg: Config, threads: int | None = None) -> dict:
    """All weights of a drafter, canonical formats, as numpy arrays.

    ``{"fc": mat, "head": mat, "hidden_norm": f32[H], "norm": f32[H],
       "layers": [{"q": mat, ..., "in_norm": f32[H], "q_norm": f32[hd], ...}]}``
    where ``mat`` is ``{"fmt", "rows", "cols", "codes", "scales"}``.
    """
    H, I, hd = cfg.hidden, cfg.intermediate, cfg.head_dim
    shapes = {"q": (cfg.q_dim, H), "k": (cfg.kv_dim, H), "v": (cfg.kv_dim, H), "o": (H, cfg.q_dim),
              "gate": (I, H), "up": (I, H), "down": (H, I)}
    jobs = {("fc",): (0, H, cfg.tap_width, cfg.fc_fmt), ("head",): (1, cfg.vocab, H, cfg.head_fmt)}
    for li in range(cfg.layers):
        for mi, name in enumerate(MATRIX_NAMES):
            rows, cols = shapes[name]
            jobs[(li, name)] = (10 + li * 16 + mi, rows, cols, cfg.body_fmt)
    threads = threads or min(8, os.cpu_count() or 1)
    with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
        futs = {k: ex.submit(_draw_matrix, cfg, *v) for k, v in jobs.items()}
        mats = {k: f.result() for k, f in futs.items()}
    out = {"fc": mats[("fc",)], "head": mats[("head",)],
           "hidden_norm": _norm_vec(cfg, 0, H), "norm": _norm_vec(cfg, 1, H), "layers": []}
    for li in range(cfg.layers):
        layer = {name: mats[(li, name)] for name in MATRIX_NAMES}
        layer["in_norm"] = _norm_vec(cfg, 10 + li * 8 + 0, H)
        layer["post_norm"] = _norm_vec(cfg, 10 + li * 8 + 1, H)
        layer["q_norm"] = _norm_vec(cfg, 10 + li * 8 + 2, hd)
        layer["k_norm"] = _norm_vec(cfg, 10 + li * 8 + 3, hd)
        out["layers"].append(layer)
    return add_conv_weights(cfg, out, threads) if cfg.conv_kernel else out


def add_conv_weights(cfg: Config, weights: dict, threads: int | None = None) -> dict:
    """The drafter's weights with its row convolutions' drawn in (a copy of the layer dicts; the
    other arrays are shared): per layer the kernel projections ``attn_kp`` / ``mlp_kp``, coded
    like the FC (Q8_32, or f32 unquantized), and the static kernels ``attn_base`` / ``mlp_base``."""
    H = cfg.hidden
    jobs = {(li, name): (10 + li * 16 + 8 + ci, cfg.conv_rows, H, cfg.fc_fmt, 8192, cfg.conv_std)
            for li in range(cfg.layers) for ci, name in enumerate(CONV_NAMES)}
    threads = threads or min(8, os.cpu_count() or 1)
    with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
        futs = {k: ex.submit(_draw_matrix, cfg, *v) for k, v in jobs.items()}
        mats = {k: f.result() for k, f in futs.items()}
    out = dict(weights)
    out["layers"] = []
    for li, lw in enumerate(weights["layers"]):
        layer = dict(lw)
        for ci, name in enumerate(CONV_NAMES):
            layer[name] = mats[(li, name)]
            layer[name.replace("_kp", "_base")] = _conv_base(cfg, li * 2 + ci)
        out["layers"].append(layer)
    return out


def _conv_base(cfg: Config, index: int) -> np.ndarray:
    """A convolution's static kernels [stage][offset][hidden]: 1 at offset 0 (the row itself) and
    0 further back, plus N(0, weight_std), so each stage starts near the identity."""
    r = _rng(cfg.weight_seed or cfg.seed, _S_CONV, index)
    b = r.standard_normal((2, cfg.conv_kernel, cfg.hidden), dtype=np.float32) * np.float32(cfg.weight_std)
    b[:, 0, :] += np.float32(1)
    return np.ascontiguousarray(b)


# ---------------------------------------------------------------------------------------------
# rows


def make_taps(cfg: Config, seq: int, pos0: int, n: int) -> np.ndarray:
    """Context rows (the target's tapped layer outputs joined) of positions pos0 .. pos0+n-1.

    Drawn per 64-position chunk so any span of positions is reproducible on its own.
    """
    out = np.empty((n, cfg.tap_width), dtype=np.float32)
    p, i = pos0, 0
    while i < n:
        c = p // 64
        off = p - c * 64
        take = min(64 - off, n - i)
        r = _rng(cfg.seed, _S_TAPS, seq * 1_000_003 + c)
        block = r.standard_normal((64, cfg.tap_width), dtype=np.float32) * np.float32(cfg.taps_std)
        out[i:i + take] = block[off:off + take]
        i += take
        p += take
    return out


def make_block_input(cfg: Config, seq: int, index: int) -> np.ndarray:
    """Block rows [anchor, MASK, ..., MASK] as embeddings: row 0 the anchor token's (fresh per
    block), rows 1.. the mask token's (one vector per drafter), each N(0, emb_std)."""
    a = _rng(cfg.seed, _S_ANCHOR, seq * 1_000_003 + index).standard_normal(cfg.hidden, dtype=np.float32)
    m = _rng(cfg.weight_seed or cfg.seed, _S_MASK, 0).standard_normal(cfg.hidden, dtype=np.float32)
    h = np.empty((cfg.block, cfg.hidden), dtype=np.float32)
    h[0] = a * np.float32(cfg.emb_std)
    h[1:] = m * np.float32(cfg.emb_std)
    return h


def make_selector(cfg: Config, rank: int = 128, book_std: float = 0.1) -> dict:
    """The candidate selector's tensors (the pages give no rank or top count for these workloads;
    rank 128 is this project's choice): the hidden projection [rank][hidden] N(0, weight_std)
    coded like the head, and the predecessor and successor codebooks, f16 [vocab][rank]
    N(0, book_std)."""
    sel = _draw_matrix(cfg, 10_000, rank, cfg.hidden, cfg.head_fmt)
    r = _rng(cfg.weight_seed or cfg.seed, _S_SELECTOR, 0)
    pred = (r.standard_normal((cfg.vocab, rank), dtype=np.float32) * book_std).astype(np.float16)
    succ = (r.standard_normal((cfg.vocab, rank), dtype=np.float32) * book_std).astype(np.float16)
    return {"sel": sel, "pred": pred, "succ": succ, "rank": rank}


def algorithmic_bytes(cfg: Config, ctx_rows: int | None = None) -> dict:
    """Bytes one block must move (weights once in their stored format, the context's K/V rows
    read in f32, the logits written), and for an append of ``append_per_block`` rows the FC and
    every layer's Wk, Wv, the taps read and the K/V rows written."""
    def mbytes(rows, cols, fmt):
        if fmt == F32:
            return rows * cols * 4
        per = 18 if fmt == Q4_32 else 34
        return rows * (cols // 32) * per
    H, I = cfg.hidden, cfg.intermediate
    body = cfg.layers * (mbytes(cfg.q_dim + 2 * cfg.kv_dim, H, cfg.body_fmt) + mbytes(H, cfg.q_dim, cfg.body_fmt)
                         + mbytes(2 * I, H, cfg.body_fmt) + mbytes(H, I, cfg.body_fmt))
    head = mbytes(cfg.vocab, H, cfg.head_fmt)
    n_ctx = cfg.ctx if ctx_rows is None else ctx_rows
    kv = cfg.n_seqs * n_ctx * cfg.layers * 2 * cfg.kv_dim * 4
    logits = cfg.n_seqs * cfg.block * cfg.vocab * 4
    out = {"body": body, "head": head, "kv": kv, "logits": logits}
    if cfg.append_per_block:
        n = cfg.append_per_block * cfg.n_seqs
        out["append_fc"] = mbytes(H, cfg.tap_width, cfg.fc_fmt)
        out["append_kv_w"] = cfg.layers * mbytes(2 * cfg.kv_dim, H, cfg.body_fmt)
        out["append_taps"] = n * cfg.tap_width * 4
        out["append_kv_write"] = n * cfg.layers * 2 * cfg.kv_dim * 4
    out["total"] = sum(out.values())
    return out
