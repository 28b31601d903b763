"""A torch-backed handle on one ``dflash_ctx``: torch allocates the workspace, the outputs and
provides the current stream; every computation is a call into ``libdflash.so``."""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import (dflash_block_forward, dflash_block_forward_rows, dflash_block_hidden, dflash_create,
               dflash_ctx_append, dflash_ctx_dropped, dflash_ctx_pending, dflash_ctx_queue, dflash_ctx_reset,
               dflash_ctx_settle, dflash_ctx_span, dflash_ctx_truncate,
               dflash_destroy, dflash_geometry, dflash_last_scores, dflash_layer_weights, dflash_matrix,
               dflash_read_kv,
               dflash_set_layer_options, dflash_set_score_mode, dflash_set_stream, dflash_weights,
               dflash_workspace_bytes)

GEOMETRY_FIELDS = ("layers", "hidden", "heads", "kv_heads", "head_dim", "intermediate", "vocab", "block", "n_taps",
                   "body_fmt", "fc_fmt", "head_fmt")


def geometry(spec, max_ctx: int, max_seqs: int) -> dflash_geometry:
    """dflash_geometry from any object with the geometry's attribute names."""
    g = dflash_geometry()
    g.rope_theta = float(spec.rope_theta)
    g.eps = float(spec.eps)
    for n in GEOMETRY_FIELDS:
        setattr(g, n, int(getattr(spec, n)))
    g.max_ctx = int(max_ctx)
    g.max_seqs = int(max_seqs)
    # row convolutions (absent: none); their kernel projections are coded like the FC
    g.conv_group = int(getattr(spec, "conv_group", 0))
    g.conv_kernel = int(getattr(spec, "conv_kernel", 0))
    g.conv_fmt = int(getattr(spec, "conv_fmt", spec.fc_fmt))
    g.kv_f16 = int(bool(getattr(spec, "kv_f16", False)))
    g.pending_rows = int(getattr(spec, "pending_rows", 0))
    return g


def _stream(torch):
    return torch.cuda.current_stream().cuda_stream


class Drafter:
    """The drafter on the current GPU.  ``weights`` holds canonical matrices
    (``{"fmt", "rows", "cols", "codes", "scales"}`` with numpy or torch arrays) and norm
    vectors, as ``dflash_inputs.make_weights`` draws them."""

    def __init__(self, spec, weights: dict, max_ctx: int, max_seqs: int = 1, device: str = "cuda"):
        import torch

        self.torch = torch
        self.device = torch.device(device)
        self.spec = spec
        self.g = geometry(spec, max_ctx, max_seqs)
        keep = []

        def dev(a):
            t = a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))
            t = t.to(self.device).contiguous()
            keep.append(t)
            return t.data_ptr()

        def mat(m) -> dflash_matrix:
            return dflash_matrix(dev(m["codes"]), None if m["scales"] is None else dev(m["scales"]))

        layers = (dflash_layer_weights * spec.layers)()
        for i, lw in enumerate(weights["layers"]):
            L = layers[i]
            for n in ("in_norm", "post_norm", "q_norm", "k_norm"):
                setattr(L, n, dev(lw[n]))
            for n in ("q", "k", "v", "o", "gate", "up", "down"):
                setattr(L, n, mat(lw[n]))
            if self.g.conv_kernel:
                L.attn_kp, L.mlp_kp = mat(lw["attn_kp"]), mat(lw["mlp_kp"])
                L.attn_base, L.mlp_base = dev(lw["attn_base"]), dev(lw["mlp_base"])
        W = dflash_weights()
        W.fc, W.head = mat(weights["fc"]), mat(weights["head"])
        W.hidden_norm, W.norm = dev(weights["hidden_norm"]), dev(weights["norm"])
        W.layer = C.cast(layers, C.POINTER(dflash_layer_weights))
        self.nbytes = dflash_workspace_bytes(self.g)
        self.workspace = torch.empty(self.nbytes, dtype=torch.uint8, device=self.device)
        self.ctx = dflash_create(self.g, W, self.workspace.data_ptr(), self.nbytes, _stream(torch))
        del keep  # dflash_create waited for the repack: the canonical copies can go

    # -- context ---------------------------------------------------------------------------
    def append(self, seq: int, pos: int, taps) -> None:
        t = self._f32(taps)
        n = t.shape[0] if t.dim() == 2 else 0
        self._sync_stream()
        dflash_ctx_append(self.ctx, seq, pos, t.data_ptr() if n else None, n)
        self._last_inputs = t

    def set_layer_options(self, windows=None, rotary=None) -> None:
        L = self.g.layers
        as_list = lambda x: None if x is None else [int(v) for v in np.broadcast_to(np.asarray(x), (L,))]
        dflash_set_layer_options(self.ctx, as_list(windows), as_list(rotary))

    def set_score_mode(self, mode: int) -> None:
        """How attention scores context keys: DFLASH_SCORES_AUTO, _F64 or _DIGITS."""
        dflash_set_score_mode(self.ctx, mode)

    def last_scores(self) -> int:
        """What the last block call scored with (DFLASH_SCORES_F64 or _DIGITS)."""
        return dflash_last_scores(self.ctx)

    def dropped(self, seq: int, layer: int) -> int:
        return dflash_ctx_dropped(self.ctx, seq, layer)

    def queue(self, seq: int, pos: int, taps) -> None:
        """Context rows that wait until a block reads them or more than pending_rows wait."""
        t = self._f32(taps)
        n = t.shape[0] if t.dim() == 2 else 0
        self._sync_stream()
        dflash_ctx_queue(self.ctx, seq, pos, t.data_ptr() if n else None, n)
        self._last_inputs = t

    def settle(self, seq: int) -> None:
        self._sync_stream()
        dflash_ctx_settle(self.ctx, seq)

    def pending(self, seq: int) -> int:
        return dflash_ctx_pending(self.ctx, seq)

    def truncate(self, seq: int, pos: int) -> None:
        dflash_ctx_truncate(self.ctx, seq, pos)

    def reset(self, seq: int) -> None:
        dflash_ctx_reset(self.ctx, seq)

    def span(self, seq: int):
        return dflash_ctx_span(self.ctx, seq)

    def read_kv(self, layer: int, seq: int, row0: int, n: int):
        torch = self.torch
        k = torch.empty((n, self.g.kv_heads, self.g.head_dim), dtype=torch.float32, device=self.device)
        v = torch.empty_like(k)
        self._sync_stream()
        dflash_read_kv(self.ctx, layer, seq, row0, n, k.data_ptr(), v.data_ptr())
        return k, v

    # -- blocks ----------------------------------------------------------------------------
    def block_forward(self, seqs, anchors, h, out=None, head_rows=None):
        """Logits of every block row, over the head's first head_rows rows when given.  h is
        [seqs][rows][hidden]: fewer rows than the block's cut the block to those rows."""
        torch = self.torch
        t = self._f32(h)
        rows = t.shape[1]
        n = self.g.vocab if head_rows is None else int(head_rows)
        if out is None:
            out = torch.empty((len(seqs), rows, n), dtype=torch.float32, device=self.device)
        self._sync_stream()
        if head_rows is None and rows == self.g.block:
            dflash_block_forward(self.ctx, seqs, anchors, t.data_ptr(), out.data_ptr())
        else:
            dflash_block_forward_rows(self.ctx, seqs, anchors, t.data_ptr(), rows, n, out.data_ptr())
        self._last_inputs = t
        return out

    def block_hidden(self, seqs, anchors, h):
        torch = self.torch
        t = self._f32(h)
        out = torch.empty((len(seqs), self.g.block, self.g.hidden), dtype=torch.float32, device=self.device)
        self._sync_stream()
        dflash_block_hidden(self.ctx, seqs, anchors, t.data_ptr(), out.data_ptr())
        self._last_inputs = t
        return out

    def close(self):
        if getattr(self, "ctx", None):
            dflash_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- plumbing --------------------------------------------------------------------------
    def _f32(self, a):
        torch = self.torch
        t = a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        return t.to(device=self.device, dtype=torch.float32).contiguous()

    def _sync_stream(self):
        dflash_set_stream(self.ctx, _stream(self.torch))
