"""MI355X (gfx950) DFlash 2 block drafter.

``libdflash.so`` (HIP kernels + the C ABI of ``include/dflash.h``) does all the work; this
module only marshals arguments to it through ctypes, under the same names.  PyTorch appears
only in :class:`Drafter`, for device memory and the current stream.  There is no other code
path: without the built library every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdflash.so")

DFLASH_OK, DFLASH_EINVAL, DFLASH_ECAPACITY, DFLASH_EHIP, DFLASH_ENOTSUP = 0, -1, -2, -3, -4
DFLASH_F32, DFLASH_Q4_32, DFLASH_Q8_32 = 0, 1, 2

EXPORTS = [
    "dflash_workspace_bytes", "dflash_create", "dflash_set_stream", "dflash_ctx_append", "dflash_ctx_truncate",
    "dflash_ctx_reset", "dflash_ctx_span", "dflash_block_forward", "dflash_block_hidden", "dflash_last_error",
    "dflash_destroy", "dflash_quant_act", "dflash_packed_bytes", "dflash_pack", "dflash_gemm_scratch_bytes",
    "dflash_gemm", "dflash_group_sums", "dflash_read_kv", "dflash_time_stage", "dflash_read_timing",
    "dflash_top_k_scratch_bytes", "dflash_top_k", "dflash_select_scratch_bytes", "dflash_select",
    "dflash_set_layer_options", "dflash_ctx_dropped", "dflash_block_forward_rows", "dflash_ctx_queue",
    "dflash_ctx_settle", "dflash_ctx_pending", "dflash_top_k_noalloc", "dflash_set_score_mode",
    "dflash_last_scores",
]
DFLASH_SCORES_AUTO, DFLASH_SCORES_F64, DFLASH_SCORES_DIGITS = 0, 1, 2
(DFLASH_STAGE_HEAD, DFLASH_STAGE_QKV, DFLASH_STAGE_ATTENTION, DFLASH_STAGE_O, DFLASH_STAGE_GATE_UP, DFLASH_STAGE_DOWN,
 DFLASH_STAGE_BLOCK, DFLASH_STAGE_APPEND, DFLASH_STAGE_ATTN_CHUNKS) = range(9)


class dflash_geometry(C.Structure):
    _fields_ = [("rope_theta", C.c_double), ("eps", C.c_double)] + [
        (n, C.c_int32) for n in ("layers", "hidden", "heads", "kv_heads", "head_dim", "intermediate", "vocab",
                                 "block", "n_taps", "body_fmt", "fc_fmt", "head_fmt", "max_seqs", "max_ctx",
                                 "conv_group", "conv_kernel", "conv_fmt", "kv_f16", "pending_rows")]


class dflash_matrix(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p)]


class dflash_layer_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("in_norm", "post_norm", "q_norm", "k_norm")] + [
        (n, dflash_matrix) for n in ("q", "k", "v", "o", "gate", "up", "down", "attn_kp", "mlp_kp")] + [
        ("attn_base", C.c_void_p), ("mlp_base", C.c_void_p)]


class dflash_weights(C.Structure):
    _fields_ = [("fc", dflash_matrix), ("head", dflash_matrix), ("hidden_norm", C.c_void_p), ("norm", C.c_void_p),
                ("layer", C.POINTER(dflash_layer_weights))]


class DFlashError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dflash error {code}: {msg}")
        self.code = code


_lib = None


def lib():
    """The loaded library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (__graft_entry__.build())")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        G, W = C.POINTER(dflash_geometry), C.POINTER(dflash_weights)
        sig = {
            "dflash_workspace_bytes": (i32, [G, C.POINTER(sz)]),
            "dflash_create": (i32, [G, W, vp, sz, vp, C.POINTER(vp)]),
            "dflash_set_stream": (i32, [vp, vp]),
            "dflash_ctx_append": (i32, [vp, i32, i64, vp, i32]),
            "dflash_ctx_truncate": (i32, [vp, i32, i64]),
            "dflash_ctx_queue": (i32, [vp, i32, i64, vp, i32]),
            "dflash_ctx_settle": (i32, [vp, i32]),
            "dflash_ctx_pending": (i32, [vp, i32, C.POINTER(i64)]),
            "dflash_ctx_reset": (i32, [vp, i32]),
            "dflash_ctx_span": (i32, [vp, i32, C.POINTER(i64), C.POINTER(i64)]),
            "dflash_block_forward": (i32, [vp, i32, vp, vp, vp, vp]),
            "dflash_block_forward_rows": (i32, [vp, i32, vp, vp, vp, i32, i32, vp]),
            "dflash_set_layer_options": (i32, [vp, vp, vp]),
            "dflash_set_score_mode": (i32, [vp, i32]),
            "dflash_last_scores": (i32, [vp, C.POINTER(C.c_int32)]),
            "dflash_ctx_dropped": (i32, [vp, i32, i32, C.POINTER(i64)]),
            "dflash_block_hidden": (i32, [vp, i32, vp, vp, vp, vp]),
            "dflash_last_error": (C.c_char_p, [vp]),
            "dflash_destroy": (None, [vp]),
            "dflash_quant_act": (i32, [vp, i32, i32, vp, vp, vp]),
            "dflash_packed_bytes": (i32, [i32, i32, i32, C.POINTER(sz)]),
            "dflash_pack": (i32, [i32, i32, i32, dflash_matrix, vp, vp]),
            "dflash_gemm_scratch_bytes": (i32, [i32, i32, i32, i32, C.POINTER(sz)]),
            "dflash_gemm": (i32, [i32, vp, i32, i32, vp, vp, i32, vp, i32, vp, vp]),
            "dflash_group_sums": (i32, [i32, vp, i32, i32, vp, i32, vp, vp, vp]),
            "dflash_read_kv": (i32, [vp, i32, i32, i32, i32, vp, vp]),
            "dflash_time_stage": (i32, [vp, i32]),
            "dflash_read_timing": (i32, [vp, i32, C.POINTER(C.c_double), C.POINTER(i64)]),
            "dflash_top_k_scratch_bytes": (i32, [i32, i32, i32, C.POINTER(sz)]),
            "dflash_top_k": (i32, [vp, i32, i32, i32, i32, vp, vp, vp, vp]),
            "dflash_top_k_noalloc": (i32, [vp, i32, i32, i32, i32, vp, vp, vp]),
            "dflash_select_scratch_bytes": (i32, [i32, i32, i32, C.POINTER(sz)]),
            "dflash_select": (i32, [vp, i32, i32, i32, vp, i32, vp, vp, i32, i32, i32, vp, vp, vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int, ctx=None) -> int:
    if rc != DFLASH_OK:
        msg = lib().dflash_last_error(ctx)
        raise DFlashError(rc, msg.decode() if msg else "")
    return rc


# ---- the C ABI under its own names (pointers are ints: device addresses or host buffers) ----


def dflash_workspace_bytes(g: dflash_geometry) -> int:
    n = C.c_size_t()
    _check(lib().dflash_workspace_bytes(C.byref(g), C.byref(n)))
    return n.value


def dflash_create(g: dflash_geometry, w: dflash_weights, workspace: int, nbytes: int, stream: int):
    out = C.c_void_p()
    _check(lib().dflash_create(C.byref(g), C.byref(w), workspace, nbytes, stream, C.byref(out)))
    return out


def dflash_set_stream(ctx, stream: int) -> int:
    return _check(lib().dflash_set_stream(ctx, stream), ctx)


def dflash_ctx_append(ctx, seq: int, pos: int, taps: int, n: int) -> int:
    return _check(lib().dflash_ctx_append(ctx, seq, pos, taps, n), ctx)


def dflash_ctx_queue(ctx, seq: int, pos: int, taps: int, n: int) -> int:
    return _check(lib().dflash_ctx_queue(ctx, seq, pos, taps, n), ctx)


def dflash_ctx_settle(ctx, seq: int) -> int:
    return _check(lib().dflash_ctx_settle(ctx, seq), ctx)


def dflash_ctx_pending(ctx, seq: int) -> int:
    n = C.c_int64()
    _check(lib().dflash_ctx_pending(ctx, seq, C.byref(n)), ctx)
    return n.value


def dflash_ctx_truncate(ctx, seq: int, pos: int) -> int:
    return _check(lib().dflash_ctx_truncate(ctx, seq, pos), ctx)


def dflash_ctx_reset(ctx, seq: int) -> int:
    return _check(lib().dflash_ctx_reset(ctx, seq), ctx)


def dflash_ctx_span(ctx, seq: int):
    a, b = C.c_int64(), C.c_int64()
    _check(lib().dflash_ctx_span(ctx, seq, C.byref(a), C.byref(b)), ctx)
    return a.value, b.value


def _host_arrays(seqs, anchors):
    n = len(seqs)
    s = (C.c_int32 * n)(*[int(x) for x in seqs])
    a = (C.c_int64 * n)(*[int(x) for x in anchors])
    return n, s, a


def dflash_block_forward(ctx, seqs, anchors, h: int, logits: int) -> int:
    n, s, a = _host_arrays(seqs, anchors)
    return _check(lib().dflash_block_forward(ctx, n, C.cast(s, C.c_void_p), C.cast(a, C.c_void_p), h, logits), ctx)


def dflash_block_forward_rows(ctx, seqs, anchors, h: int, block_rows: int, head_rows: int, logits: int) -> int:
    n, s, a = _host_arrays(seqs, anchors)
    return _check(lib().dflash_block_forward_rows(ctx, n, C.cast(s, C.c_void_p), C.cast(a, C.c_void_p), h,
                                                  int(block_rows), int(head_rows), logits), ctx)


def dflash_set_layer_options(ctx, windows=None, rotary=None) -> int:
    """windows / rotary: host sequences of one int per layer, or None for the defaults."""
    w = None if windows is None else (C.c_int32 * len(windows))(*[int(x) for x in windows])
    r = None if rotary is None else (C.c_int32 * len(rotary))(*[int(x) for x in rotary])
    return _check(lib().dflash_set_layer_options(ctx, None if w is None else C.cast(w, C.c_void_p),
                                                 None if r is None else C.cast(r, C.c_void_p)), ctx)


def dflash_set_score_mode(ctx, mode: int) -> int:
    """DFLASH_SCORES_AUTO, DFLASH_SCORES_F64 or DFLASH_SCORES_DIGITS (include/dflash.h)."""
    return _check(lib().dflash_set_score_mode(ctx, int(mode)), ctx)


def dflash_last_scores(ctx) -> int:
    """What the last block call scored with: DFLASH_SCORES_F64 or _DIGITS (_AUTO before one)."""
    m = C.c_int32()
    _check(lib().dflash_last_scores(ctx, C.byref(m)), ctx)
    return m.value


def dflash_ctx_dropped(ctx, seq: int, layer: int) -> int:
    d = C.c_int64()
    _check(lib().dflash_ctx_dropped(ctx, seq, layer, C.byref(d)), ctx)
    return d.value


def dflash_block_hidden(ctx, seqs, anchors, h: int, hidden: int) -> int:
    n, s, a = _host_arrays(seqs, anchors)
    return _check(lib().dflash_block_hidden(ctx, n, C.cast(s, C.c_void_p), C.cast(a, C.c_void_p), h, hidden), ctx)


def dflash_last_error(ctx=None) -> str:
    m = lib().dflash_last_error(ctx)
    return m.decode() if m else ""


def dflash_destroy(ctx) -> None:
    lib().dflash_destroy(ctx)


def dflash_quant_act(x: int, rows: int, cols: int, q: int, d: int, stream: int) -> int:
    return _check(lib().dflash_quant_act(x, rows, cols, q, d, stream))


def dflash_packed_bytes(fmt: int, rows: int, cols: int) -> int:
    n = C.c_size_t()
    _check(lib().dflash_packed_bytes(fmt, rows, cols, C.byref(n)))
    return n.value


def dflash_pack(fmt: int, rows: int, cols: int, codes: int, scales: int, packed: int, stream: int) -> int:
    return _check(lib().dflash_pack(fmt, rows, cols, dflash_matrix(codes, scales), packed, stream))


def dflash_gemm_scratch_bytes(rows: int, cols: int, m: int, splits: int) -> int:
    n = C.c_size_t()
    _check(lib().dflash_gemm_scratch_bytes(rows, cols, m, splits, C.byref(n)))
    return n.value


def dflash_gemm(fmt, packed, rows, cols, xq, dx, m, y, splits, scratch, stream) -> int:
    return _check(lib().dflash_gemm(fmt, packed, rows, cols, xq, dx, m, y, splits, scratch, stream))


def dflash_group_sums(fmt, packed, rows, cols, xq, m, sums, scratch, stream) -> int:
    return _check(lib().dflash_group_sums(fmt, packed, rows, cols, xq, m, sums, scratch, stream))


def dflash_read_kv(ctx, layer: int, seq: int, row0: int, n: int, k: int, v: int) -> int:
    return _check(lib().dflash_read_kv(ctx, layer, seq, row0, n, k, v), ctx)


def dflash_time_stage(ctx, stage: int) -> int:
    return _check(lib().dflash_time_stage(ctx, stage), ctx)


def dflash_read_timing(ctx, stage: int):
    """(summed milliseconds, number of timed launches) of one stage since its last read."""
    ms, n = C.c_double(), C.c_int64()
    _check(lib().dflash_read_timing(ctx, stage, C.byref(ms), C.byref(n)), ctx)
    return ms.value, n.value


def dflash_top_k_scratch_bytes(rows: int, width: int, k: int) -> int:
    n = C.c_size_t()
    _check(lib().dflash_top_k_scratch_bytes(rows, width, k, C.byref(n)))
    return n.value


def dflash_top_k(x: int, rows: int, width: int, ld: int, k: int, vals: int, idx: int, scratch: int, stream) -> int:
    return _check(lib().dflash_top_k(x, rows, width, ld, k, vals, idx, scratch, stream))


def dflash_top_k_noalloc(x: int, rows: int, width: int, ld: int, k: int, vals: int, idx: int, stream) -> int:
    return _check(lib().dflash_top_k_noalloc(x, rows, width, ld, k, vals, idx, stream))


def dflash_select_scratch_bytes(rows: int, width: int, top: int) -> int:
    n = C.c_size_t()
    _check(lib().dflash_select_scratch_bytes(rows, width, top, C.byref(n)))
    return n.value


def dflash_select(logits: int, rows: int, width: int, ld: int, hp: int, rank: int, pred: int, succ: int, vocab: int,
                  top: int, anchor: int, chosen: int, plain: int, scratch: int, stream) -> int:
    return _check(lib().dflash_select(logits, rows, width, ld, hp, rank, pred, succ, vocab, top, anchor, chosen, plain,
                                      scratch, stream))


from .drafter import Drafter  # noqa: E402,F401  (torch-backed convenience wrapper)
