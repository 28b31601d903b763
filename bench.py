#!/usr/bin/env python3
"""Benchmark of the DFlash 2 block-drafter hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input: for the long-context
workload the append of its new context rows and then the block; otherwise the block (all layers
and the head's logits for every block row of every sequence).  Inputs (weights, context, block
rows) are resident in HBM before the timed region.  `value` is the median of single steps, each
timed with HIP events after an untimed 1 GiB overwrite (L2 and the 256 MB memory-side cache then
hold none of the step's data); the same steps back to back are reported beside it.  The
8B-shaped workload is the headline; the long-context and batched workloads of the same drafter
are measured in the same run ("legs").  Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--config qwen3_8b] [--legs 1] [--cpu-baseline 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ms per DFlash draft block + achieved HBM GB/s (% of peak), 8B-shaped drafter"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
F64_MFMA_PEAK_TFS = 78.6  # MI355X dense f64 matrix, published
I8_MFMA_PEAK_OPS = 5.0e15  # MI355X dense int8 matrix, published
LEGS = ["qwen3_8b_long", "qwen3_8b_batch8"]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def workload_name(cfg) -> str:
    fmt = {0: "f32", 1: "q4_32", 2: "q8_32"}
    return (f"{cfg.key}: {cfg.layers} layers, hidden {cfg.hidden}, {cfg.heads}/{cfg.kv_heads} heads x "
            f"{cfg.head_dim}, intermediate {cfg.intermediate}, {cfg.n_taps} taps, context {cfg.ctx} rows x "
            f"{cfg.n_seqs} sequence(s), block {cfg.block}, vocab {cfg.vocab}; body {fmt[cfg.body_fmt]}, "
            f"fc {fmt[cfg.fc_fmt]}, head {fmt[cfg.head_fmt]}"
            + (f"; {cfg.append_per_block} rows appended per block" if cfg.append_per_block else ""))


def head_bytes(cfg) -> int:
    """Algorithmic bytes of one launch of the head's product: the Q8_32 (or f32) table once,
    the activations read and the logits written."""
    rows = cfg.n_seqs * cfg.block
    if cfg.head_fmt == 0:
        w = cfg.vocab * cfg.hidden * 4
        x = rows * cfg.hidden * 4
    else:
        per = 34 if cfg.head_fmt == 2 else 18
        w = cfg.vocab * (cfg.hidden // 32) * per
        x = rows * cfg.hidden + rows * (cfg.hidden // 32) * 4
    return w + x + rows * cfg.vocab * 4


def attention_kv_bytes(cfg, nctx: int) -> int:
    """Algorithmic bytes of one layer's attention chunk launch: the f32 K and V rows of every
    sequence's context read once (the block's own keys are the merge's)."""
    return cfg.n_seqs * nctx * 2 * cfg.kv_dim * 4


def attention_digit_bytes(cfg, nctx: int) -> int:
    """Bytes one layer's digit-scored attention launch reads: per context row and kv head the
    key's seven int8 digit planes (7 x head_dim), its exponent (4) and the value row (f32, or
    f16 for an f16 cache)."""
    v = cfg.head_dim * (2 if cfg.kv_f16 else 4)
    return cfg.n_seqs * nctx * cfg.kv_heads * (7 * cfg.head_dim + 4 + v)


def attention_digit_ops(cfg, nctx: int) -> int:
    """int8 operations of one layer's digit-scored launch: per q head, block row and context
    key the 28 digit pairs whose weights reach 128^-6, each a head_dim-long product."""
    return 2 * 28 * cfg.n_seqs * cfg.block * cfg.heads * nctx * cfg.head_dim


def prefill_bytes(cfg) -> int:
    """Bytes the prefill of every sequence's context must move: the FC and all layers' Wk|Wv in
    their stored formats once, the tapped rows read (f32), the K/V rows written (f32)."""
    def mbytes(rows, cols, fmt):
        return rows * cols * 4 if fmt == 0 else rows * (cols // 32) * (18 if fmt == 1 else 34)
    rows = cfg.n_seqs * cfg.ctx
    return (mbytes(cfg.hidden, cfg.tap_width, cfg.fc_fmt) + cfg.layers * mbytes(2 * cfg.kv_dim, cfg.hidden, cfg.body_fmt)
            + rows * cfg.tap_width * 4 + rows * cfg.layers * 2 * cfg.kv_dim * 4)


def attention_flops(cfg, nctx: int) -> int:
    """Flops of one layer's attention of every sequence's block: per q head and block row, the
    scores against nctx context keys + the block's own keys and the weighted sum of as many
    values (2 flops per multiply-add each)."""
    return 4 * cfg.n_seqs * cfg.block * cfg.heads * (nctx + cfg.block) * cfg.head_dim


def int8_macs(cfg) -> int:
    """Useful int8 multiply-adds of one step's quantized products (weights x activation rows):
    every body matrix and the head for the block rows, plus FC and K|V of the appended rows."""
    rows = cfg.n_seqs * cfg.block
    H, qd, kvd, I = cfg.hidden, cfg.heads * cfg.head_dim, cfg.kv_heads * cfg.head_dim, cfg.intermediate
    body = cfg.layers * ((qd + 2 * kvd) * H + H * qd + 2 * I * H + H * I)
    macs = rows * (body + cfg.vocab * H)
    if cfg.append_per_block:
        n = cfg.append_per_block * cfg.n_seqs
        macs += n * (H * cfg.n_taps * H + cfg.layers * 2 * kvd * H)
    return macs


def profile_value(name: str, key: str, sources):
    """A figure from a committed rocprofv3 summary profiles/<name>.md, or None when the file is
    missing or any kernel source it was taken on has changed since (its sha256 lines)."""
    import hashlib
    import re

    path = os.path.join(ROOT, "profiles", f"{name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    for src in sources:
        m = re.search(rf"source_sha256 {re.escape(src)}:\s*([0-9a-f]{{64}})", text)
        p = os.path.join(ROOT, "block_draft_model_dflash_amd", "csrc", src)
        if not m or not os.path.exists(p) or hashlib.sha256(open(p, "rb").read()).hexdigest() != m.group(1):
            return None
    m = re.search(rf"{re.escape(key)}:\s*([0-9.eE+-]+)", text)
    return float(m.group(1)) if m else None


KERNEL_SOURCES = ["gemm.hip", "act.hip", "attention.hip", "api.hip", "common.h", "lanes.h", "head.h"]


def cpu_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, os.cpu_count()


def cpu_baseline(cfg, weights, blocks: int):
    """The oracle as it stands on this host's cores: prefill of the context, then blocks."""
    import dflash_inputs as di
    import oracle

    m = oracle.Model(cfg, weights, max_ctx=cfg.ctx + 64, max_seqs=1)
    t = time.perf_counter()
    for p0 in range(0, cfg.ctx, 1024):
        n = min(1024, cfg.ctx - p0)
        m.append(0, p0, di.make_taps(cfg, 0, p0, n))
    prefill_s = time.perf_counter() - t
    log(f"oracle prefill {cfg.ctx} rows: {prefill_s:.1f} s")
    t = time.perf_counter()
    for i in range(blocks):
        m.block_forward([0], [cfg.ctx], di.make_block_input(cfg, 0, i)[None])
    block_ms = (time.perf_counter() - t) * 1e3 / blocks
    log(f"oracle block: {block_ms:.0f} ms ({blocks} blocks)")
    m.close()
    model, nproc = cpu_info()
    return {"value": round(block_ms, 2), "unit": "ms/block", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"one sequence of the same drafter: {cfg.ctx}-row context prefilled "
                      f"({prefill_s:.1f} s, {cfg.ctx / prefill_s:.0f} rows/s, not in value), then {blocks} "
                      f"blocks of {cfg.block} rows timed",
            "cpu_model": model, "nproc": nproc,
            "threads_note": "OpenMP threads = the host's CPU share for one GPU (OMP_NUM_THREADS, else the "
                            "cores this process may run on), not every core the host reports",
            "prefill_rows_per_s": round(cfg.ctx / prefill_s, 1)}


class Leg:
    """One workload on the GPU: the drafter, its prefilled context, its per-step inputs."""

    def __init__(self, cfg, weights, K, W):
        import numpy as np
        import torch

        import dflash_inputs as di
        from block_draft_model_dflash_amd import Drafter

        self.cfg, self.K, self.W, self.torch = cfg, K, W, torch
        self.max_ctx = cfg.ctx + (K + W) * cfg.append_per_block + 64
        self.gm = Drafter(cfg, weights, max_ctx=self.max_ctx, max_seqs=cfg.n_seqs)
        log(f"{cfg.key}: created, workspace {self.gm.nbytes / 1e9:.2f} GB")
        self.prefill_ms = self.prefill(self.gm)
        log(f"{cfg.key}: GPU prefill {cfg.n_seqs} x {cfg.ctx} rows: {self.prefill_ms:.1f} ms")
        self.seqs = list(range(cfg.n_seqs))
        self.hs = torch.from_numpy(np.stack([np.stack([di.make_block_input(cfg, s, i) for s in self.seqs])
                                             for i in range(K + W)])).cuda()
        self.app = None
        if cfg.append_per_block:
            self.app = torch.from_numpy(np.stack([di.make_taps(cfg, 0, cfg.ctx + i * cfg.append_per_block,
                                                               cfg.append_per_block) for i in range(K + W)])).cuda()
        self.logits = torch.empty((cfg.n_seqs, cfg.block, cfg.vocab), dtype=torch.float32, device="cuda")
        self.grown = 0

    def prefill(self, d):
        import dflash_inputs as di

        torch, cfg = self.torch, self.cfg
        # untimed: one 128-row append through the same kernels, then the sequence emptied again,
        # so the timed calls do not include loading the kernels' code on their first launch
        warm = torch.from_numpy(di.make_taps(cfg, 0, 0, min(128, cfg.ctx))).cuda()
        d.append(0, 0, warm)
        d.reset(0)
        torch.cuda.synchronize()
        del warm
        total = 0.0
        for s in range(cfg.n_seqs):
            for p0 in range(0, cfg.ctx, 4096):
                n = min(4096, cfg.ctx - p0)
                taps = torch.from_numpy(di.make_taps(cfg, s, p0, n)).cuda()
                torch.cuda.synchronize()
                t = time.perf_counter()
                d.append(s, p0, taps)
                torch.cuda.synchronize()
                total += (time.perf_counter() - t) * 1e3
                del taps
        return total

    def step(self, i, d=None):
        """Step i: (long context) append the next rows, then the block of every sequence."""
        d = d or self.gm
        cfg = self.cfg
        if self.app is not None:
            p = cfg.ctx + self.grown * cfg.append_per_block
            d.append(0, p, self.app[self.grown])
            self.grown += 1
            anchors = [p + cfg.append_per_block]
        else:
            anchors = [cfg.ctx] * cfg.n_seqs
        d.block_forward(self.seqs, anchors, self.hs[i], out=self.logits)

    def rewind(self, d=None):
        """The long-context workload grows by append_per_block rows a step: back to the prefill."""
        d = d or self.gm
        if self.app is not None:
            d.truncate(0, self.cfg.ctx)
            self.grown = 0
            assert d.span(0) == (0, self.cfg.ctx)

    def ctx_rows(self, i):
        cfg = self.cfg
        return cfg.ctx + (i + 1) * cfg.append_per_block if cfg.append_per_block else cfg.ctx

    def warm(self):
        """K steps back to back (after W untimed ones), wall clock around them."""
        torch = self.torch
        self.rewind()
        for i in range(self.W):
            self.step(i)
        torch.cuda.synchronize()
        self.rewind()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(self.K):
            self.step(self.W + i)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / self.K
        if self.app is not None:
            assert self.gm.span(0) == (0, self.cfg.ctx + self.K * self.cfg.append_per_block)
        return ms

    def cold(self):
        """Each of K steps on its own after an untimed overwrite of 1 GiB, HIP events on the
        step's stream: the median and spread."""
        import numpy as np

        torch = self.torch
        self.rewind()
        scrub = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(self.K)]
        for i in range(self.K):
            scrub.fill_(float(i))
            ev[i][0].record()
            self.step(self.W + i)
            ev[i][1].record()
        torch.cuda.synchronize()
        t_ms = np.array([a.elapsed_time(b) for a, b in ev])
        del scrub
        return {"median": round(float(np.median(t_ms)), 5), "p10": round(float(np.percentile(t_ms, 10)), 5),
                "p90": round(float(np.percentile(t_ms, 90)), 5), "steps": self.K}

    def kernel_events(self):
        """K steps with HIP event pairs (on the library's stream) around the head's product and
        every layer's attention chunk kernel: their summed milliseconds and launch counts."""
        import block_draft_model_dflash_amd as D

        ctx = self.gm.ctx
        self.rewind()
        D.dflash_time_stage(ctx, -1)
        D.dflash_time_stage(ctx, D.DFLASH_STAGE_HEAD)
        D.dflash_time_stage(ctx, D.DFLASH_STAGE_ATTN_CHUNKS)
        for i in range(self.K):
            self.step(self.W + i)
        head = D.dflash_read_timing(ctx, D.DFLASH_STAGE_HEAD)
        attn = D.dflash_read_timing(ctx, D.DFLASH_STAGE_ATTN_CHUNKS)
        D.dflash_time_stage(ctx, -1)
        return head, attn

    def event_pair_ms(self, n=50):
        """Median of n empty event pairs on the step's stream: what a pair adds to the kernel it
        brackets (the dispatch of the kernel and the two markers), beside a trace's durations."""
        import numpy as np

        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in ev:
            a.record()
            b.record()
        torch.cuda.synchronize()
        return round(float(np.median([a.elapsed_time(b) for a, b in ev])), 5)

    def stages(self):
        import block_draft_model_dflash_amd as D

        names = {D.DFLASH_STAGE_QKV: "qkv", D.DFLASH_STAGE_ATTENTION: "attention",
                 D.DFLASH_STAGE_ATTN_CHUNKS: "attention_chunks", D.DFLASH_STAGE_O: "o",
                 D.DFLASH_STAGE_GATE_UP: "gate_up", D.DFLASH_STAGE_DOWN: "down", D.DFLASH_STAGE_HEAD: "head",
                 D.DFLASH_STAGE_BLOCK: "block", D.DFLASH_STAGE_APPEND: "append"}
        out = {}
        for st, name in names.items():
            if st == D.DFLASH_STAGE_APPEND and self.app is None:
                continue
            self.rewind()
            D.dflash_time_stage(self.gm.ctx, st)
            for i in range(self.K):
                self.step(self.W + i)
            tot, n = D.dflash_read_timing(self.gm.ctx, st)
            D.dflash_time_stage(self.gm.ctx, -1)
            out[name] = round(tot / self.K, 5)  # ms per step, summed over the stage's launches
        return out

    def figures(self, warm_ms, cold):
        """The leg's throughput figures at the cold median (the headline statistic)."""
        import dflash_inputs as di

        cfg = self.cfg
        ms = cold["median"]
        ab = di.algorithmic_bytes(cfg, ctx_rows=self.ctx_rows(self.K // 2))
        gbs = ab["total"] / (ms * 1e-3) / 1e9
        rows = cfg.n_seqs * cfg.block
        return {
            "workload": workload_name(cfg),
            "ms_per_block": ms,
            "ms_per_block_p10_p90": [cold["p10"], cold["p90"]],
            "warm_ms_per_step": round(warm_ms, 5),
            "blocks_per_s": round(1e3 / ms * cfg.n_seqs, 2),
            "rows_per_s": round(1e3 / ms * rows, 1),
            "algorithmic_bytes_per_step": ab["total"],
            "achieved_GBps_step": round(gbs, 1),
            "frac_of_hbm_peak_step": round(gbs / HBM_PEAK_GBS, 4),
            "int8_mfma_util_step": round(int8_macs(cfg) * 2 / (ms * 1e-3) / I8_MFMA_PEAK_OPS, 5),
            "gpu_prefill_rows_per_s": round(cfg.n_seqs * cfg.ctx / (self.prefill_ms * 1e-3), 1),
            # the prefill's algorithmic bytes: FC and every layer's Wk|Wv once, the taps read, the
            # K/V rows written; it runs 128-row products, bound by their arithmetic, not by HBM
            "gpu_prefill_GBps": round(prefill_bytes(cfg) / (self.prefill_ms * 1e-3) / 1e9, 1),
        }

    def kernel_lines(self, head, attn):
        """The head's product (HBM) and the attention chunk kernel per launch, from the event
        pairs: for f64 scores its f32 K/V bytes with the f64 matrix rate beside; for digit scores
        the key digits and values it reads with the int8 and f64 matrix rates beside."""
        import block_draft_model_dflash_amd as D

        cfg, K = self.cfg, self.K
        pair = self.event_pair_ms()
        (head_ms, head_n), (attn_ms, attn_n) = head, attn
        hb = head_bytes(cfg)
        head_avg = head_ms / max(head_n, 1)
        head_gbs = hb / (head_avg * 1e-3) / 1e9
        head_line = {"bound": "hbm", "achieved": round(head_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head_gbs / HBM_PEAK_GBS, 4),
                     "traffic": profile_value(f"head_gemm_{cfg.key}_pmc", "traffic_bytes_per_launch", ["gemm.hip"]),
                     "kernel": "k_gemm_q (head logits, Q8_32 x A8_32)", "bytes_per_launch": hb,
                     "avg_launch_ms": round(head_avg, 5), "empty_event_pair_ms": pair, "launches": head_n,
                     "ms_per_step": round(head_ms / K, 5)}
        ctxs = [self.ctx_rows(i) for i in range(K)]
        digits = self.gm.last_scores() == D.DFLASH_SCORES_DIGITS
        n = max(attn_n, 1)
        attn_avg = attn_ms / n
        if digits:  # the kernel reads key digits and values; int8 scores, f64 value products
            kv = sum(attention_digit_bytes(cfg, c) for c in ctxs) * cfg.layers
            ops = sum(attention_digit_ops(cfg, c) for c in ctxs) * cfg.layers
            pv = sum(2 * cfg.n_seqs * cfg.block * cfg.heads * c * cfg.head_dim for c in ctxs) * cfg.layers
            i8_tops = ops / n / (attn_avg * 1e-3) / 1e12
            pv_tf = pv / n / (attn_avg * 1e-3) / 1e12
            name = "k_attn_gqa_dig (context keys: int8 digit-split scores, online softmax, f64 values)"
            extra = {"i8_mfma": {"achieved_TOPs": round(i8_tops, 1), "peak_TOPs": I8_MFMA_PEAK_OPS / 1e12,
                                 "frac": round(i8_tops * 1e12 / I8_MFMA_PEAK_OPS, 4), "ops_per_launch": round(ops / n)},
                     "f64_mfma": {"achieved_TFLOPs": round(pv_tf, 2), "peak_TFLOPs": F64_MFMA_PEAK_TFS,
                                  "frac": round(pv_tf / F64_MFMA_PEAK_TFS, 4), "flops_per_launch": round(pv / n)}}
        else:
            kv = sum(attention_kv_bytes(cfg, c) for c in ctxs) * cfg.layers
            flops = sum(attention_flops(cfg, c) for c in ctxs) * cfg.layers
            attn_tf = flops / n / (attn_avg * 1e-3) / 1e12
            name = "k_attn_partial (context keys: f64 scores, online softmax, f64 values)"
            extra = {"f64_mfma": {"achieved_TFLOPs": round(attn_tf, 2), "peak_TFLOPs": F64_MFMA_PEAK_TFS,
                                  "frac": round(attn_tf / F64_MFMA_PEAK_TFS, 4), "flops_per_launch": round(flops / n)}}
        attn_gbs = kv / n / (attn_avg * 1e-3) / 1e9
        attn_line = {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": profile_value(f"attn_chunks_{cfg.key}_pmc", "traffic_bytes_per_launch",
                                              ["attention.hip"]),
                     "kernel": name, "bytes_per_launch": round(kv / n), "avg_launch_ms": round(attn_avg, 5),
                     "empty_event_pair_ms": pair, "launches": attn_n, "ms_per_step": round(attn_ms / K, 5),
                     **extra}
        return (attn_line, head_line) if attn_ms > head_ms else (head_line, attn_line)

    def close(self):
        self.gm.close()
        del self.gm, self.hs, self.app, self.logits


def selection_ms(leg):
    """The candidate selection the pages run after the block (not part of the step): top 16 of
    the draft rows' logits and the greedy re-scoring with a rank-128 selector."""
    import numpy as np
    import torch

    import block_draft_model_dflash_amd as D

    cfg = leg.cfg
    rank, top, nrow = 128, 16, cfg.block - 1
    rng = np.random.default_rng(5)
    hp = torch.from_numpy(rng.standard_normal((nrow, rank)).astype(np.float32)).cuda()
    books = torch.from_numpy((rng.standard_normal((2, cfg.vocab, rank)) * 0.1).astype(np.float16).view(np.int16)).cuda()
    chosen = torch.empty(nrow, dtype=torch.int32, device="cuda")
    plain = torch.empty_like(chosen)
    scr = torch.empty(D.dflash_select_scratch_bytes(nrow, cfg.vocab, top), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    logits = leg.logits

    def sel():
        D.dflash_select(logits.data_ptr() + cfg.vocab * 4, nrow, cfg.vocab, cfg.vocab, hp.data_ptr(), rank,
                        books[0].data_ptr(), books[1].data_ptr(), cfg.vocab, top, 0, chosen.data_ptr(),
                        plain.data_ptr(), scr.data_ptr(), stream)
    for _ in range(3):
        sel()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(leg.K):
        sel()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / leg.K


def variants(leg, weights):
    """The block with the drafter's optional parts (untimed for `value`): an f16 K/V cache; for a
    single-sequence workload also the head over its first 65536 rows, the block cut to 8 rows, a
    1024-position window on layers 0, 2, 4, row convolutions of 16 columns a group and 4 offsets."""
    import torch

    import dflash_inputs as di
    from block_draft_model_dflash_amd import Drafter

    cfg, K, W = leg.cfg, leg.K, leg.W
    out = {}

    def timed(fn):
        for i in range(W):
            fn(i)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(K):
            fn(W + i)
        torch.cuda.synchronize()
        return round((time.perf_counter() - t) * 1e3 / K, 5)

    d16 = Drafter(cfg.replace(kv_f16=True), weights, max_ctx=leg.max_ctx, max_seqs=cfg.n_seqs)
    leg.prefill(d16)

    leg.rewind(d16)
    out["kv_cache_f16"] = timed(lambda i: leg.step(i, d16))
    leg.rewind(d16)
    d16.close()
    del d16
    if cfg.n_seqs != 1 or leg.app is not None:
        return out
    seqs, hs, gm = leg.seqs, leg.hs, leg.gm
    if cfg.vocab > 65536:
        short = torch.empty((1, cfg.block, 65536), dtype=torch.float32, device="cuda")
        out["head_shortlist_65536"] = timed(lambda i: gm.block_forward(seqs, [cfg.ctx], hs[i], out=short, head_rows=65536))
    if cfg.block > 8:  # the device block's cut: the anchor and the next seven rows
        hs8 = hs[:, :, :8].contiguous()
        out8 = torch.empty((1, 8, cfg.vocab), dtype=torch.float32, device="cuda")
        out["block_cut_8_rows"] = timed(lambda i: gm.block_forward(seqs, [cfg.ctx], hs8[i], out=out8))
    gm.reset(0)
    gm.set_layer_options([1024 if li % 2 == 0 else 0 for li in range(cfg.layers)], None)
    leg.prefill(gm)
    out["windows_1024_even_layers"] = timed(lambda i: gm.block_forward(seqs, [cfg.ctx], hs[i], out=leg.logits))
    ccfg = cfg.replace(conv_group=16, conv_kernel=4)
    cm = Drafter(ccfg, di.add_conv_weights(ccfg, weights), max_ctx=cfg.ctx + 64, max_seqs=1)
    leg.prefill(cm)
    out["row_conv_group16_kernel4"] = timed(lambda i: cm.block_forward(seqs, [cfg.ctx], hs[i], out=leg.logits))
    cm.close()
    return out


def main() -> int:
    import dflash_inputs as di

    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="qwen3_8b", choices=di.CONFIG_ORDER)
    ap.add_argument("--legs", type=int, default=1,
                    help="also measure the long-context and batched workloads of the same drafter")
    ap.add_argument("--cpu-baseline", type=int, default=1)
    ap.add_argument("--cpu-blocks", type=int, default=16, help="oracle blocks timed for cpu_baseline")
    ap.add_argument("--stages", type=int, default=1, help="also time each stage in its own untimed pass")
    ap.add_argument("--selection", type=int, default=1,
                    help="also time the candidate selection of one block's draft rows (top 16, rank 128)")
    ap.add_argument("--variants", type=int, default=1,
                    help="also time the block with the drafter's optional parts: an f16 cache, a head "
                         "shortlist, sliding windows, row convolutions")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed region, run one plain copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only; sharding the path over several GPUs is designed but "
              "not built, so no figure at several GPUs is produced", file=sys.stderr)
        return 2

    import torch

    cfg = di.CONFIGS[args.config]
    K, W = args.steps, args.warmup
    torch.cuda.set_device(0)
    t = time.perf_counter()
    weights = di.make_weights(cfg)
    log(f"weights of {cfg.key}: {time.perf_counter() - t:.1f} s")

    leg = Leg(cfg, weights, K, W)
    warm_ms = leg.warm()
    cold = leg.cold()
    head, attn = leg.kernel_events()
    log(f"{cfg.key}: cold {cold}, warm {warm_ms:.4f} ms/step")
    fig = leg.figures(warm_ms, cold)
    dominant, other = leg.kernel_lines(head, attn)
    stages = leg.stages() if args.stages else {}
    if stages:
        log("stages ms/step:", stages)
    sel = selection_ms(leg) if args.selection else None
    var = variants(leg, weights) if args.variants else {}
    if var:
        log("variants ms/block:", var)
    if args.copy_probe_mib:
        # a plain streaming kernel of known size (read n bytes, write n bytes): the reference
        # against which the HBM byte counters of the other kernels are scaled
        n = args.copy_probe_mib << 18  # f32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    leg.close()
    torch.cuda.empty_cache()

    legs = {}
    if args.legs and cfg.key == "qwen3_8b":
        for key in LEGS:
            lc = di.CONFIGS[key]
            lg = Leg(lc, weights, K, W)
            lw = lg.warm()
            lcold = lg.cold()
            lhead, lattn = lg.kernel_events()
            d, o = lg.kernel_lines(lhead, lattn)
            legs[key] = dict(lg.figures(lw, lcold), roofline=d, roofline_next=o,
                             stages_ms_per_step=lg.stages() if args.stages else {})
            log(f"{key}: cold {lcold}, warm {lw:.4f} ms/step")
            lg.close()
            del lg
            torch.cuda.empty_cache()

    ms = cold["median"]
    out = {
        "metric": METRIC,
        "value": ms,
        "unit": "ms/block",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8 (int8 MFMA on 4/8-bit weights) + f64 (attention, rescale) + f32",
        "data": "synthetic",
        "config": {"workload": fig["workload"], "sequences": cfg.n_seqs, "block_rows": cfg.block,
                   "context_rows": cfg.ctx, "append_rows_per_step": cfg.append_per_block},
        "value_statistic": "median of single steps, each after an untimed 1 GiB overwrite (HIP events)",
    }
    out.update({k: v for k, v in fig.items() if k not in ("workload", "ms_per_block")})
    out["measured_hbm_bytes_per_step"] = profile_value(f"step_{cfg.key}_pmc", "hbm_bytes_per_step", KERNEL_SOURCES)
    out["roofline"] = dominant
    out["roofline_next"] = other
    out["stages_ms_per_step"] = stages
    out["selection_ms_per_block"] = None if sel is None else round(sel, 5)
    out["variants_ms_per_block"] = var
    out["legs"] = legs
    for key in legs:
        legs[key]["measured_hbm_bytes_per_step"] = profile_value(f"step_{key}_pmc", "hbm_bytes_per_step",
                                                                 KERNEL_SOURCES)
    if args.cpu_baseline:
        base = di.CONFIGS["qwen3_8b"]
        same = (base.weight_seed or base.seed) == (cfg.weight_seed or cfg.seed)
        cb = cpu_baseline(base, weights if same else di.make_weights(base), args.cpu_blocks)
        if cfg.key != "qwen3_8b":
            cb["sample"] = "the same drafter at a 4096-row context (the 8B-shaped workload): " + cb["sample"]
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
