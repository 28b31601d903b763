"""CPU oracle of the DFlash 2 block drafter -- TEST INFRASTRUCTURE ONLY.

Python marshalling over ``dflash_oracle.c`` (plain C, f64 inside each step).  Only
``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package; the GPU library never does, and this package imports nothing from it.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dflash_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F32, Q4_32, Q8_32 = 0, 1, 2


def build(src: str = SRC, out: str = LIB, opt: str = "-O3") -> str:
    """Compile the oracle: gcc, no fast-math, fp-contract off (every expression rounded as
    written), OpenMP for the independent output rows."""
    cmd = ["gcc", opt, "-mavx2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-I", HERE, "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(out + ".tmp", out)
    return out


class og_geometry(C.Structure):
    _fields_ = [("rope_theta", C.c_double), ("eps", C.c_double)] + [
        (n, C.c_int32) for n in ("layers", "hidden", "heads", "kv_heads", "head_dim", "intermediate", "vocab",
                                 "block", "n_taps", "body_fmt", "fc_fmt", "head_fmt", "max_seqs", "max_ctx",
                                 "conv_group", "conv_kernel", "conv_fmt", "kv_f16", "pending_rows")]


class og_matrix(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p)]


class og_layer(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("in_norm", "post_norm", "q_norm", "k_norm")] + [
        (n, og_matrix) for n in ("q", "k", "v", "o", "gate", "up", "down", "attn_kp", "mlp_kp")] + [
        ("attn_base", C.c_void_p), ("mlp_base", C.c_void_p)]


class og_weights(C.Structure):
    _fields_ = [("fc", og_matrix), ("head", og_matrix), ("hidden_norm", C.c_void_p), ("norm", C.c_void_p),
                ("layer", C.POINTER(og_layer))]


_lib = None


def use_library(path: str | None) -> None:
    """Load the oracle from another build of its source (``None``: the default build).  The
    pin tests use this to run against deliberately broken copies."""
    global _lib
    _lib = None
    lib(path)


def lib(path: str | None = None):
    global _lib
    if _lib is None:
        path = path or LIB
        if path == LIB and not os.path.exists(LIB):
            build()
        L = C.CDLL(path)
        vp, i32, i64, f32, f64 = C.c_void_p, C.c_int, C.c_int64, C.c_float, C.c_double
        sig = {
            "og_set_threads": (None, [i32]), "og_get_threads": (i32, []),
            "og_f16_to_f64": (f64, [C.c_uint16]),
            "og_round_f16": (f64, [f32]),
            "og_inv_freq": (None, [f64, i32, vp]),
            "og_rmsnorm_row": (None, [vp, vp, i32, f32, vp]),
            "og_rope_head": (None, [vp, i32, i64, vp]),
            "og_quant_act_row": (None, [vp, i32, vp, vp]),
            "og_matmul_q": (None, [i32, og_matrix, i32, i32, vp, vp, i32, vp]),
            "og_group_sums": (None, [i32, og_matrix, i32, i32, vp, i32, vp]),
            "og_matmul_f32": (None, [vp, i32, i32, vp, i32, vp]),
            "og_attend": (None, [vp, i32, vp, vp, i32, i32, f32, vp, vp]),
            "og_silu_mul": (None, [vp, vp, i32, vp]),
            "og_row_conv": (None, [vp, i32, i32, i32, i32, i32, vp, vp, vp]),
            "og_create": (vp, [C.POINTER(og_geometry), C.POINTER(og_weights)]),
            "og_destroy": (None, [vp]),
            "og_ctx_append": (i32, [vp, i32, i64, vp, i32]),
            "og_ctx_truncate": (i32, [vp, i32, i64]),
            "og_ctx_queue": (i32, [vp, i32, i64, vp, i32]),
            "og_ctx_settle": (i32, [vp, i32]),
            "og_pending": (i64, [vp, i32]),
            "og_ctx_reset": (i32, [vp, i32]),
            "og_ctx_span": (i32, [vp, i32, C.POINTER(C.c_int64), C.POINTER(C.c_int64)]),
            "og_read_kv": (i32, [vp, i32, i32, i32, i32, vp, vp]),
            "og_block_forward": (i32, [vp, i32, vp, vp, vp, vp]),
            "og_block_forward_rows": (i32, [vp, i32, vp, vp, vp, i32, i32, vp]),
            "og_set_layer_options": (i32, [vp, vp, vp]),
            "og_dropped": (i64, [vp, i32, i32]),
            "og_block_hidden": (i32, [vp, i32, vp, vp, vp, vp]),
            "og_top_k": (None, [vp, i32, i32, vp, vp]),
            "og_select": (None, [vp, i32, i32, i32, vp, i32, vp, vp, i32, i32, vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        L.og_set_threads(default_threads())
        _lib = L
    return _lib


def default_threads() -> int:
    """Threads the oracle runs on: DFLASH_ORACLE_THREADS if set, else the host's CPU share for
    this process -- OMP_NUM_THREADS where the host sets it (a machine whose cores are shared among
    several GPUs gives one GPU's process that many), else the cores this process may run on."""
    for var in ("DFLASH_ORACLE_THREADS", "OMP_NUM_THREADS"):
        v = os.environ.get(var, "").strip()
        if v.isdigit() and int(v) > 0:
            return int(v)
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def set_threads(n: int) -> None:
    lib().og_set_threads(int(n))


def threads() -> int:
    return lib().og_get_threads()


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- unit steps --------------------------------------------------------------------------


def f16_to_f64(bits: int) -> float:
    return lib().og_f16_to_f64(int(bits))


def round_f16(x) -> np.ndarray:
    """Each f32 value rounded to binary16 (ties to even), returned as f64."""
    x = np.asarray(x, np.float32).ravel()
    L = lib()
    return np.array([L.og_round_f16(float(v)) for v in x], np.float64)


def inv_freq(theta: float, head_dim: int) -> np.ndarray:
    out = np.empty(head_dim // 2, np.float32)
    lib().og_inv_freq(theta, head_dim, _p(out))
    return out


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of each row of x (last axis = len(w))."""
    x = _c(x, np.float32)
    w = _c(w, np.float32)
    n = w.shape[0]
    flat = x.reshape(-1, n)
    out = np.empty_like(flat)
    for i in range(flat.shape[0]):
        lib().og_rmsnorm_row(_p(flat[i]), _p(w), n, eps, _p(out[i]))
    return out.reshape(x.shape)


def rope(x: np.ndarray, pos: int, inv: np.ndarray) -> np.ndarray:
    """Rotate every head (last axis = head_dim) of x to position pos."""
    x = _c(x, np.float32).copy()
    hd = x.shape[-1]
    flat = x.reshape(-1, hd)
    inv = _c(inv, np.float32)
    for i in range(flat.shape[0]):
        lib().og_rope_head(_p(flat[i]), hd, int(pos), _p(inv))
    return flat.reshape(x.shape)


def quant_act(x: np.ndarray):
    """A8_32 of each row: (codes int8 [..., n], scales f32 [..., n/32])."""
    x = _c(x, np.float32)
    n = x.shape[-1]
    flat = x.reshape(-1, n)
    q = np.empty(flat.shape, np.int8)
    d = np.empty((flat.shape[0], n // 32), np.float32)
    for i in range(flat.shape[0]):
        lib().og_quant_act_row(_p(flat[i]), n, _p(q[i]), _p(d[i]))
    return q.reshape(x.shape), d.reshape(x.shape[:-1] + (n // 32,))


def _mat(m: dict) -> og_matrix:
    return og_matrix(m["codes"].ctypes.data, None if m["scales"] is None else m["scales"].ctypes.data)


def matmul_q(mat: dict, xq: np.ndarray, dx: np.ndarray) -> np.ndarray:
    xq = _c(xq, np.int8)
    dx = _c(dx, np.float32)
    m = xq.shape[0]
    y = np.empty((m, mat["rows"]), np.float32)
    lib().og_matmul_q(mat["fmt"], _mat(mat), mat["rows"], mat["cols"], _p(xq), _p(dx), m, _p(y))
    return y


def group_sums(mat: dict, xq: np.ndarray) -> np.ndarray:
    xq = _c(xq, np.int8)
    m = xq.shape[0]
    s = np.empty((m, mat["rows"], mat["cols"] // 32), np.int32)
    lib().og_group_sums(mat["fmt"], _mat(mat), mat["rows"], mat["cols"], _p(xq), m, _p(s))
    return s


def matmul_f32(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    w = _c(w, np.float32)
    x = _c(x, np.float32)
    y = np.empty((x.shape[0], w.shape[0]), np.float32)
    lib().og_matmul_f32(_p(w), w.shape[0], w.shape[1], _p(x), x.shape[0], _p(y))
    return y


def matmul(mat: dict, x: np.ndarray) -> np.ndarray:
    """MM(W, x) as the forward uses it: A8_32 of x first for a quantized W."""
    if mat["fmt"] == F32:
        return matmul_f32(mat["codes"], x)
    q, d = quant_act(x)
    return matmul_q(mat, q, d)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, want_p: bool = False):
    q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
    nq, hd = q.shape
    nk = k.shape[0]
    y = np.empty((nq, hd), np.float32)
    p = np.empty((nq, nk), np.float64) if want_p else None
    lib().og_attend(_p(q), nq, _p(k), _p(v), nk, hd, scale, _p(y), _p(p))
    return (y, p) if want_p else y


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g, u = _c(g, np.float32), _c(u, np.float32)
    a = np.empty_like(g)
    lib().og_silu_mul(_p(g), _p(u), g.size, _p(a))
    return a


def row_conv(x: np.ndarray, gs: int, kn: int, stage: int, base: np.ndarray, d: np.ndarray) -> np.ndarray:
    """One stage of the grouped causal row convolution over the rows x [rows][hidden]: base
    [2][kn][hidden], d [rows][2*kn*hidden/gs] (dflash.rs Drafter::conv)."""
    x, base, d = _c(x, np.float32), _c(base, np.float32), _c(d, np.float32)
    rows, hidden = x.shape
    if base.shape != (2, kn, hidden) or d.shape != (rows, 2 * kn * (hidden // gs)) or hidden % gs:
        raise ValueError("row_conv: shapes")
    y = np.empty_like(x)
    lib().og_row_conv(_p(x), rows, hidden, gs, kn, stage, _p(base), _p(d), _p(y))
    return y


def top_k(x: np.ndarray, k: int):
    """dflash.rs top_k: the k largest of x with their indices, largest first (earlier index first
    among equal values)."""
    x = _c(x, np.float32).ravel()
    if not 1 <= k <= x.size:
        raise ValueError("k outside [1, len(x)]")
    vals = np.empty(k, np.float32)
    idx = np.empty(k, np.int32)
    lib().og_top_k(_p(x), x.size, k, _p(vals), _p(idx))
    return vals, idx


def select(logits: np.ndarray, hp: np.ndarray, pred: np.ndarray, succ: np.ndarray, top: int, anchor: int):
    """dflash.rs Drafter::select_with over logits [rows][width] (the draft rows), the selector's
    rows hp [rows][rank] and the f16 codebooks [vocab][rank]: (chosen tokens, each row's top)."""
    logits = _c(logits, np.float32)
    hp = _c(hp, np.float32)
    pred = _c(pred, np.float16).view(np.uint16)
    succ = _c(succ, np.float16).view(np.uint16)
    rows, width = logits.shape
    rank = hp.shape[1]
    if hp.shape[0] != rows or pred.shape[1] != rank or succ.shape != pred.shape or not 1 <= top <= width:
        raise ValueError("select: shapes")
    if not 0 <= anchor < pred.shape[0]:
        raise ValueError("select: anchor token outside the codebooks")
    chosen = np.empty(rows, np.int32)
    plain = np.empty(rows, np.int32)
    lib().og_select(_p(logits), rows, width, width, _p(hp), rank, _p(pred), _p(succ), top, anchor, _p(chosen),
                    _p(plain))
    return chosen, plain


# ---- the drafter --------------------------------------------------------------------------


class Model:
    """The oracle drafter over canonical numpy weights (``dflash_inputs.make_weights``)."""

    def __init__(self, cfg, weights: dict, max_ctx: int | None = None, max_seqs: int | None = None):
        self.cfg = cfg
        self.w = weights  # keep the arrays alive
        g = og_geometry()
        g.rope_theta, g.eps = cfg.rope_theta, cfg.eps
        for n in ("layers", "hidden", "heads", "kv_heads", "head_dim", "intermediate", "vocab", "block", "n_taps",
                  "body_fmt", "fc_fmt", "head_fmt"):
            setattr(g, n, getattr(cfg, n))
        g.conv_group, g.conv_kernel, g.conv_fmt = cfg.conv_group, cfg.conv_kernel, cfg.fc_fmt
        g.kv_f16 = int(cfg.kv_f16)
        g.pending_rows = int(cfg.pending_rows)
        g.max_seqs = max_seqs if max_seqs is not None else cfg.n_seqs
        g.max_ctx = max_ctx if max_ctx is not None else cfg.ctx + 64 * max(1, cfg.append_per_block)
        self.geometry = g
        layers = (og_layer * cfg.layers)()
        for i, lw in enumerate(weights["layers"]):
            L = layers[i]
            for n in ("in_norm", "post_norm", "q_norm", "k_norm"):
                setattr(L, n, lw[n].ctypes.data)
            for n in ("q", "k", "v", "o", "gate", "up", "down"):
                setattr(L, n, _mat(lw[n]))
            if cfg.conv_kernel:
                for n in ("attn_kp", "mlp_kp"):
                    setattr(L, n, _mat(lw[n]))
                L.attn_base, L.mlp_base = lw["attn_base"].ctypes.data, lw["mlp_base"].ctypes.data
        self._layers = layers
        W = og_weights()
        W.fc, W.head = _mat(weights["fc"]), _mat(weights["head"])
        W.hidden_norm, W.norm = weights["hidden_norm"].ctypes.data, weights["norm"].ctypes.data
        W.layer = C.cast(layers, C.POINTER(og_layer))
        self._W = W
        self.h = lib().og_create(C.byref(g), C.byref(W))
        if not self.h:
            raise ValueError("oracle rejected the geometry")

    def close(self):
        if self.h:
            lib().og_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def append(self, seq: int, pos: int, taps: np.ndarray) -> int:
        taps = _c(taps, np.float32)
        n = taps.shape[0] if taps.ndim == 2 else 0
        return lib().og_ctx_append(self.h, seq, pos, _p(taps) if n else None, n)

    def queue(self, seq: int, pos: int, taps: np.ndarray) -> int:
        taps = _c(taps, np.float32)
        n = taps.shape[0] if taps.ndim == 2 else 0
        return lib().og_ctx_queue(self.h, seq, pos, _p(taps) if n else None, n)

    def settle(self, seq: int) -> int:
        return lib().og_ctx_settle(self.h, seq)

    def pending(self, seq: int) -> int:
        return int(lib().og_pending(self.h, seq))

    def truncate(self, seq: int, pos: int) -> int:
        return lib().og_ctx_truncate(self.h, seq, pos)

    def reset(self, seq: int) -> int:
        return lib().og_ctx_reset(self.h, seq)

    def span(self, seq: int):
        a, b = C.c_int64(), C.c_int64()
        rc = lib().og_ctx_span(self.h, seq, C.byref(a), C.byref(b))
        if rc:
            raise ValueError(rc)
        return a.value, b.value

    def read_kv(self, layer: int, seq: int, row0: int, n: int):
        c = self.cfg
        k = np.empty((n, c.kv_heads, c.head_dim), np.float32)
        v = np.empty_like(k)
        rc = lib().og_read_kv(self.h, layer, seq, row0, n, _p(k), _p(v))
        if rc:
            raise ValueError(rc)
        return k, v

    def set_layer_options(self, windows=None, rotary=None) -> int:
        """Per-layer windows (0: all positions) and rotary flags (0: no rotary position), before
        any context row is held (dflash.rs Geometry::window_of / rotary)."""
        L = self.cfg.layers
        w = None if windows is None else np.ascontiguousarray(np.broadcast_to(np.asarray(windows, np.int32), (L,)))
        r = None if rotary is None else np.ascontiguousarray(np.broadcast_to(np.asarray(rotary, np.int32), (L,)))
        self._opts = (w, r)
        return lib().og_set_layer_options(self.h, _p(w), _p(r))

    def dropped(self, seq: int, layer: int) -> int:
        return int(lib().og_dropped(self.h, seq, layer))

    def block_forward(self, seqs, anchors, h: np.ndarray, head_rows: int | None = None) -> np.ndarray:
        """Logits of every block row; with head_rows, over the head's first head_rows rows only.
        h [seqs][rows][hidden]: fewer rows than the block's cut it to those rows."""
        seqs = np.asarray(seqs, np.int32)
        anchors = np.asarray(anchors, np.int64)
        h = _c(h, np.float32)
        rows = h.shape[1]
        n = self.cfg.vocab if head_rows is None else int(head_rows)
        out = np.empty((len(seqs), rows, n), np.float32)
        rc = lib().og_block_forward_rows(self.h, len(seqs), _p(seqs), _p(anchors), _p(h), rows, n, _p(out))
        if rc:
            raise ValueError(rc)
        return out

    def block_hidden(self, seqs, anchors, h: np.ndarray) -> np.ndarray:
        seqs = np.asarray(seqs, np.int32)
        anchors = np.asarray(anchors, np.int64)
        h = _c(h, np.float32)
        out = np.empty((len(seqs), self.cfg.block, self.cfg.hidden), np.float32)
        rc = lib().og_block_hidden(self.h, len(seqs), _p(seqs), _p(anchors), _p(h), _p(out))
        if rc:
            raise ValueError(rc)
        return out
