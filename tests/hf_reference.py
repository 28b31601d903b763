"""An independent reference for pinning the oracle's whole forward: transformers' Qwen3
decoder layers (the library's own RMSNorm, projections, q/k norms, rotate-half RoPE, GQA
attention and SwiGLU MLP) in float64.

The drafter's layer is a Qwen3 decoder layer whose keys and values are the context's
(computed from ``t`` by the layer's own k/v projections, k-norm and rotation) followed by the
block's own rows, with no causal mask (cortiq-engine dflash.rs, module header and
Drafter::block).  The context goes in as the layer's KV cache and the mask is all zeros.
For quantized drafters every linear layer's input is fake-quantized to A8_32 by a
forward pre-hook and the weights are the decoded codes.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

import dflash_inputs as di


def _a8_fake(x: torch.Tensor) -> torch.Tensor:
    """A8_32 quantize-dequantize in the contract's f32 arithmetic (pinned on its own by the
    brute-force nearest-code test)."""
    shp = x.shape
    x32 = x.to(torch.float32).reshape(-1, shp[-1] // 32, 32)
    amax = x32.abs().amax(dim=-1, keepdim=True)
    d = amax / 127.0
    inv = 127.0 / amax
    q = torch.clamp(torch.round(x32 * inv), -127, 127)
    q = torch.where(amax == 0, torch.zeros_like(q), q)
    d = torch.where(amax == 0, torch.zeros_like(d), d)
    return (q.double() * d.double()).reshape(shp).to(x.dtype)


def _inv_freq(theta: float, hd: int) -> np.ndarray:
    return np.array([theta ** (-(2.0 * i) / hd) for i in range(hd // 2)], dtype=np.float64).astype(np.float32)


def _cos_sin(positions, inv):
    ang = (np.asarray(positions, np.float32)[:, None] * inv[None, :]).astype(np.float64)
    emb = np.concatenate([ang, ang], axis=1)
    return torch.from_numpy(np.cos(emb))[None], torch.from_numpy(np.sin(emb))[None]


def _w(mat: dict) -> torch.Tensor:
    return torch.from_numpy(di.dequantize_rows(mat["codes"], mat["scales"], mat["fmt"], mat["cols"]))


def _row_conv_torch(x: torch.Tensor, base: torch.Tensor, d: torch.Tensor, stage: int, gs: int) -> torch.Tensor:
    """One stage of the drafter's row convolution on x [B][H] (float64), written with torch ops:
    for every offset o, the rows shifted down by o (zeros shifted in), times the static kernel
    plus the rows' dynamic kernels expanded over their column groups."""
    B, H = x.shape
    kn = base.shape[1]
    dk = d.view(B, 2, kn, H // gs)[:, stage].repeat_interleave(gs, dim=-1)  # [B][kn][H]
    y = torch.zeros_like(x)
    for o in range(kn):
        shifted = F.pad(x, (0, 0, o, 0))[:B]
        y = y + (base[stage, o][None, :] + dk[:, o]) * shifted
    return y


class _ConvIn(torch.nn.Module):
    """A layer norm followed by the first convolution stage; keeps the kernels for the second."""

    def __init__(self, norm, kp, base, gs, lin):
        super().__init__()
        self.norm, self.kp, self.base, self.gs, self.lin = norm, kp, base, gs, lin
        self.d = None

    def forward(self, h):
        x = self.norm(h)[0]
        self.d = self.lin(x, self.kp)
        return _row_conv_torch(x, self.base, self.d, 0, self.gs)[None]


class _ConvOut(torch.nn.Module):
    """A projection followed by the second convolution stage with the kernels _ConvIn kept."""

    def __init__(self, proj, conv_in):
        super().__init__()
        self.proj, self.conv_in = proj, conv_in

    def forward(self, x):
        y = self.proj(x)[0]
        return _row_conv_torch(y, self.conv_in.base, self.conv_in.d, 1, self.conv_in.gs)[None]


class HFDrafter:
    def __init__(self, cfg: di.Config, weights: dict):
        from transformers.models.qwen3.modeling_qwen3 import Qwen3Config, Qwen3DecoderLayer, Qwen3RMSNorm

        self.cfg = cfg
        hc = Qwen3Config(hidden_size=cfg.hidden, intermediate_size=cfg.intermediate,
                         num_attention_heads=cfg.heads, num_key_value_heads=cfg.kv_heads, head_dim=cfg.head_dim,
                         rms_norm_eps=cfg.eps, num_hidden_layers=cfg.layers, attention_bias=False, hidden_act="silu",
                         vocab_size=cfg.vocab)
        hc._attn_implementation = "sdpa"
        self.layers = []
        for li, lw in enumerate(weights["layers"]):
            L = Qwen3DecoderLayer(hc, layer_idx=li).double().eval()
            with torch.no_grad():
                a = L.self_attn
                a.q_proj.weight.copy_(_w(lw["q"]))
                a.k_proj.weight.copy_(_w(lw["k"]))
                a.v_proj.weight.copy_(_w(lw["v"]))
                a.o_proj.weight.copy_(_w(lw["o"]))
                a.q_norm.weight.copy_(torch.from_numpy(lw["q_norm"]).double())
                a.k_norm.weight.copy_(torch.from_numpy(lw["k_norm"]).double())
                L.mlp.gate_proj.weight.copy_(_w(lw["gate"]))
                L.mlp.up_proj.weight.copy_(_w(lw["up"]))
                L.mlp.down_proj.weight.copy_(_w(lw["down"]))
                L.input_layernorm.weight.copy_(torch.from_numpy(lw["in_norm"]).double())
                L.post_attention_layernorm.weight.copy_(torch.from_numpy(lw["post_norm"]).double())
            if cfg.body_fmt != di.F32:
                for mod in L.modules():
                    if isinstance(mod, torch.nn.Linear):
                        mod.register_forward_pre_hook(lambda m, args: (_a8_fake(args[0]),))
            if cfg.conv_kernel:  # the row convolutions around attention and the MLP
                lin = lambda x, w: self._lin(x, w, cfg.fc_fmt)
                ci = _ConvIn(L.input_layernorm, _w(lw["attn_kp"]), torch.from_numpy(lw["attn_base"]).double(),
                             cfg.conv_group, lin)
                L.input_layernorm = ci
                L.self_attn.o_proj = _ConvOut(L.self_attn.o_proj, ci)
                cm = _ConvIn(L.post_attention_layernorm, _w(lw["mlp_kp"]), torch.from_numpy(lw["mlp_base"]).double(),
                             cfg.conv_group, lin)
                L.post_attention_layernorm = cm
                L.mlp.down_proj = _ConvOut(L.mlp.down_proj, cm)
            self.layers.append(L)
        self.hidden_norm = Qwen3RMSNorm(cfg.hidden, eps=cfg.eps).double()
        self.norm = Qwen3RMSNorm(cfg.hidden, eps=cfg.eps).double()
        with torch.no_grad():
            self.hidden_norm.weight.copy_(torch.from_numpy(weights["hidden_norm"]).double())
            self.norm.weight.copy_(torch.from_numpy(weights["norm"]).double())
        self.fc = _w(weights["fc"])
        self.head = _w(weights["head"])
        self.inv = _inv_freq(cfg.rope_theta, cfg.head_dim)

    def _lin(self, x, w, fmt):
        return F.linear(_a8_fake(x) if fmt != di.F32 else x, w)

    @torch.no_grad()
    def context_kv(self, taps: np.ndarray, first: int, rotary=None):
        """Per layer (K, V) of context rows at positions first.. as [1, kv, n, hd] float64 (a
        layer with rotary[l] == 0 keeps its keys unrotated)."""
        c = self.cfg
        t = self._lin(torch.from_numpy(taps).double(), self.fc, c.fc_fmt)
        t = self.hidden_norm(t)
        n = t.shape[0]
        cos, sin = _cos_sin(np.arange(first, first + n), self.inv)
        from transformers.models.qwen3.modeling_qwen3 import apply_rotary_pos_emb

        out = []
        for li, L in enumerate(self.layers):
            a = L.self_attn
            k = a.k_norm(a.k_proj(t[None]).view(1, n, c.kv_heads, c.head_dim)).transpose(1, 2)
            v = a.v_proj(t[None]).view(1, n, c.kv_heads, c.head_dim).transpose(1, 2)
            if rotary is None or rotary[li]:
                _, k = apply_rotary_pos_emb(k, k, cos, sin)
            out.append((k, v))
        return out

    @torch.no_grad()
    def block_logits(self, kv, anchor: int, h: np.ndarray, masks=None, rotary=None) -> np.ndarray:
        """Logits of the block rows h [B][H] anchored at ``anchor`` over the context kv (the
        rows before the anchor; each layer's own length).  masks[l] (optional, [B][n_l] bool)
        hides context keys from rows, as an additive -inf; a layer with rotary[l] == 0 takes
        no rotary position (cos 1, sin 0)."""
        from transformers.cache_utils import DynamicCache

        c = self.cfg
        cache = DynamicCache()
        for li, (k, v) in enumerate(kv):
            cache.update(k.clone(), v.clone(), li)
        B = h.shape[0]
        cos, sin = _cos_sin(np.arange(anchor, anchor + B), self.inv)
        x = torch.from_numpy(h).double()[None]
        for li, L in enumerate(self.layers):
            nctx = kv[li][0].shape[2]
            mask = torch.zeros(1, 1, B, nctx + B, dtype=torch.float64)
            if masks is not None and masks[li] is not None:
                mask[0, 0, :, :nctx][torch.from_numpy(np.asarray(masks[li], bool))] = -torch.inf
            pe = (cos, sin) if rotary is None or rotary[li] else (torch.ones_like(cos), torch.zeros_like(sin))
            x = L(x, attention_mask=mask, past_key_values=cache, use_cache=True, position_embeddings=pe)
            if isinstance(x, tuple):
                x = x[0]
        x = self.norm(x)[0]
        return self._lin(x, self.head, c.head_fmt).numpy()
