#!/usr/bin/env python3
"""Benchmark of the DFlash 2 block-drafter hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input: for the long-context
workload the append of its new context rows and then the block; otherwise the block (all layers
and the head's logits for every block row of every sequence).  Inputs (weights, context, block
rows) are resident in HBM before the timed region.  Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--config qwen3_8b] [--cpu-baseline 0|1]
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


def measured_traffic(kernel: str, workload: str, source: str):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter summary
    profiles/<kernel>_<workload>_pmc.md (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known
    size), or None when there is none or the kernel's source has changed since it was taken."""
    import hashlib
    import re

    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.md")
    src = os.path.join(ROOT, "block_draft_model_dflash_amd", "csrc", source)
    if not os.path.exists(path) or not os.path.exists(src):
        return None
    text = open(path).read()
    sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not sha or not val:
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != sha.group(1):
        return None
    return int(val.group(1))


def cpu_baseline(cfg, weights, blocks: int = 2):
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
    log(f"oracle block: {block_ms:.0f} ms")
    m.close()
    return {"value": block_ms, "unit": "ms/block", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"one sequence of the same drafter: {cfg.ctx}-row context prefilled "
                      f"({prefill_s:.1f} s, {cfg.ctx / prefill_s:.0f} rows/s, not in value), then {blocks} "
                      f"blocks of {cfg.block} rows timed",
            "prefill_rows_per_s": cfg.ctx / prefill_s}


def main() -> int:
    import dflash_inputs as di

    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="qwen3_8b", choices=di.CONFIG_ORDER)
    ap.add_argument("--cpu-baseline", type=int, default=1)
    ap.add_argument("--stages", type=int, default=1, help="also time each stage in its own untimed pass")
    ap.add_argument("--selection", type=int, default=1,
                    help="also time the candidate selection of one block's draft rows (top 16, rank 128)")
    ap.add_argument("--flush", type=int, default=1,
                    help="also time single steps after overwriting 1 GiB (cold caches), median and spread")
    ap.add_argument("--variants", type=int, default=1,
                    help="also time the block with the drafter's optional parts: a head shortlist, sliding "
                         "windows, row convolutions (single-sequence workloads)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed region, run one plain copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only; sharding the path over several GPUs is designed but "
              "not built, so no figure at several GPUs is produced", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import block_draft_model_dflash_amd as D
    from block_draft_model_dflash_amd import Drafter

    cfg = di.CONFIGS[args.config]
    K, W = args.steps, args.warmup
    torch.cuda.set_device(0)
    t = time.perf_counter()
    weights = di.make_weights(cfg)
    log(f"weights of {cfg.key}: {time.perf_counter() - t:.1f} s")
    max_ctx = cfg.ctx + (K + W) * cfg.append_per_block + 64
    gm = Drafter(cfg, weights, max_ctx=max_ctx, max_seqs=cfg.n_seqs)
    log(f"created, workspace {gm.nbytes / 1e9:.2f} GB")

    # prefill (reported, outside the step)
    prefill_ms = 0.0
    for s in range(cfg.n_seqs):
        for p0 in range(0, cfg.ctx, 4096):
            n = min(4096, cfg.ctx - p0)
            taps = torch.from_numpy(di.make_taps(cfg, s, p0, n)).cuda()
            torch.cuda.synchronize()
            t = time.perf_counter()
            gm.append(s, p0, taps)
            torch.cuda.synchronize()
            prefill_ms += (time.perf_counter() - t) * 1e3
            del taps
    log(f"GPU prefill {cfg.n_seqs} x {cfg.ctx} rows: {prefill_ms:.1f} ms")

    seqs = list(range(cfg.n_seqs))
    hs = torch.from_numpy(np.stack([np.stack([di.make_block_input(cfg, s, i) for s in seqs])
                                    for i in range(K + W)])).cuda()
    app = None
    if cfg.append_per_block:
        app = torch.from_numpy(np.stack([di.make_taps(cfg, 0, cfg.ctx + i * cfg.append_per_block,
                                                      cfg.append_per_block) for i in range(max(K, W))])).cuda()
    logits = torch.empty((cfg.n_seqs, cfg.block, cfg.vocab), dtype=torch.float32, device="cuda")

    # the long-context workload grows the context by append_per_block rows per step; rewind()
    # truncates it back to the prefill, and the next step appends right after it again
    grown = [0]

    def step(i, d=None):
        d = d or gm
        if app is not None:
            p = cfg.ctx + grown[0] * cfg.append_per_block
            d.append(0, p, app[grown[0]])
            grown[0] += 1
            anchors = [p + cfg.append_per_block]
        else:
            anchors = [cfg.ctx] * cfg.n_seqs
        d.block_forward(seqs, anchors, hs[i], out=logits)

    def rewind(d=None):
        d = d or gm
        if app is not None:
            d.truncate(0, cfg.ctx)
            grown[0] = 0
            assert d.span(0) == (0, cfg.ctx)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    rewind()

    # timed region: K steps, nothing else on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(W + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if app is not None:  # every step extended the same context
        assert gm.span(0) == (0, cfg.ctx + K * cfg.append_per_block), gm.span(0)
    ms = (t1 - t0) * 1e3 / K

    # the same K steps again with HIP events (on the library's stream) around the head's product
    # and around every layer's attention chunk kernel, the two largest kernels of the step; the
    # event pairs cost a few microseconds per step, so this repetition is not the one in `value`
    rewind()
    D.dflash_time_stage(gm.ctx, -1)
    D.dflash_time_stage(gm.ctx, D.DFLASH_STAGE_HEAD)
    D.dflash_time_stage(gm.ctx, D.DFLASH_STAGE_ATTN_CHUNKS)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(K):
        step(W + i)
    torch.cuda.synchronize()
    ms_events = (time.perf_counter() - t2) * 1e3 / K
    head_ms, head_n = D.dflash_read_timing(gm.ctx, D.DFLASH_STAGE_HEAD)
    attn_ms, attn_n = D.dflash_read_timing(gm.ctx, D.DFLASH_STAGE_ATTN_CHUNKS)
    D.dflash_time_stage(gm.ctx, -1)
    log(f"{ms:.4f} ms/step ({ms_events:.4f} with events); head {head_ms / max(head_n, 1):.4f} ms x {head_n}; "
        f"attention chunks {attn_ms / max(attn_n, 1):.4f} ms x {attn_n}")

    stages = {}
    if args.stages:
        names = {D.DFLASH_STAGE_QKV: "qkv", D.DFLASH_STAGE_ATTENTION: "attention",
                 D.DFLASH_STAGE_ATTN_CHUNKS: "attention_chunks", D.DFLASH_STAGE_O: "o",
                 D.DFLASH_STAGE_GATE_UP: "gate_up", D.DFLASH_STAGE_DOWN: "down", D.DFLASH_STAGE_HEAD: "head",
                 D.DFLASH_STAGE_BLOCK: "block", D.DFLASH_STAGE_APPEND: "append"}
        for st, name in names.items():
            if st == D.DFLASH_STAGE_APPEND and app is None:
                continue
            rewind()
            D.dflash_time_stage(gm.ctx, st)
            for i in range(K):
                step(W + i)
            tot, n = D.dflash_read_timing(gm.ctx, st)
            D.dflash_time_stage(gm.ctx, -1)
            stages[name] = round(tot / K, 5)  # ms per step, summed over the stage's launches
        log("stages ms/step:", stages)

    # each step on its own after an untimed overwrite of 1 GiB (L2 and the 256 MB MALL then hold
    # none of the step's data), timed with events on the step's stream: the median and spread of
    # single cold steps, beside `value` (K steps back to back)
    flushed = None
    if args.flush:
        rewind()
        scrub = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for i in range(K):
            scrub.fill_(float(i))
            ev[i][0].record()
            step(W + i)
            ev[i][1].record()
        torch.cuda.synchronize()
        t_ms = np.sort([a.elapsed_time(b) for a, b in ev])
        flushed = {"median": round(float(np.median(t_ms)), 5), "p10": round(float(np.percentile(t_ms, 10)), 5),
                   "p90": round(float(np.percentile(t_ms, 90)), 5), "steps": K}
        del scrub
        log("cold steps (after a 1 GiB overwrite):", flushed)

    # the candidate selection the pages run after the block (not part of the step): top 16 of the
    # draft rows' logits and the greedy re-scoring with a rank-128 selector, timed on its own
    sel_ms = None
    if args.selection:
        rank, top, nrow = 128, 16, cfg.block - 1
        rng = np.random.default_rng(5)
        hp = torch.from_numpy(rng.standard_normal((nrow, rank)).astype(np.float32)).cuda()
        books = torch.from_numpy((rng.standard_normal((2, cfg.vocab, rank)) * 0.1).astype(np.float16).view(np.int16)).cuda()
        chosen = torch.empty(nrow, dtype=torch.int32, device="cuda")
        plain = torch.empty_like(chosen)
        scr = torch.empty(D.dflash_select_scratch_bytes(nrow, cfg.vocab, top), dtype=torch.uint8, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream

        def sel():
            D.dflash_select(logits.data_ptr() + cfg.vocab * 4, nrow, cfg.vocab, cfg.vocab, hp.data_ptr(), rank,
                            books[0].data_ptr(), books[1].data_ptr(), cfg.vocab, top, 0, chosen.data_ptr(),
                            plain.data_ptr(), scr.data_ptr(), stream)
        for _ in range(3):
            sel()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(K):
            sel()
        e1.record()
        torch.cuda.synchronize()
        sel_ms = e0.elapsed_time(e1) / K

    # the same step with an f16 K/V cache (half the cache's bytes; a drafter with the same
    # weights), every workload
    variants = {}
    if args.variants:
        d16 = Drafter(cfg.replace(kv_f16=True), weights, max_ctx=max_ctx, max_seqs=cfg.n_seqs)
        for sq in range(cfg.n_seqs):
            for p0 in range(0, cfg.ctx, 4096):
                d16.append(sq, p0, torch.from_numpy(di.make_taps(cfg, sq, p0, min(4096, cfg.ctx - p0))).cuda())
        rewind(d16)  # the step counter starts over (the context is already the prefill)
        for i in range(W):
            step(i, d16)
        rewind(d16)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(K):
            step(W + i, d16)
        torch.cuda.synchronize()
        variants["kv_cache_f16"] = round((time.perf_counter() - t) * 1e3 / K, 5)
        d16.close()
        del d16

    # the block with the optional parts of the drafter the workloads do not declare (untimed for
    # `value`): the head over its first 65536 rows; the block cut to 8 rows; a 1024-position
    # window on layers 0, 2, 4;
    # row convolutions of 16 columns a group and 4 offsets (a drafter with the same weights plus
    # the convolutions')
    if args.variants and cfg.n_seqs == 1 and app is None:
        def timed(fn):
            for i in range(W):
                fn(i)
            torch.cuda.synchronize()
            t = time.perf_counter()
            for i in range(K):
                fn(W + i)
            torch.cuda.synchronize()
            return round((time.perf_counter() - t) * 1e3 / K, 5)

        def prefill(d):
            for p0 in range(0, cfg.ctx, 4096):
                d.append(0, p0, torch.from_numpy(di.make_taps(cfg, 0, p0, min(4096, cfg.ctx - p0))).cuda())
            torch.cuda.synchronize()

        if cfg.vocab > 65536:
            short = torch.empty((1, cfg.block, 65536), dtype=torch.float32, device="cuda")
            variants["head_shortlist_65536"] = timed(
                lambda i: gm.block_forward(seqs, [cfg.ctx], hs[i], out=short, head_rows=65536))
        if cfg.block > 8:  # the device block's cut: the anchor and the next seven rows
            hs8 = hs[:, :, :8].contiguous()
            out8 = torch.empty((1, 8, cfg.vocab), dtype=torch.float32, device="cuda")
            variants["block_cut_8_rows"] = timed(lambda i: gm.block_forward(seqs, [cfg.ctx], hs8[i], out=out8))
        gm.reset(0)
        gm.set_layer_options([1024 if li % 2 == 0 else 0 for li in range(cfg.layers)], None)
        prefill(gm)
        variants["windows_1024_even_layers"] = timed(lambda i: gm.block_forward(seqs, [cfg.ctx], hs[i], out=logits))
        ccfg = cfg.replace(conv_group=16, conv_kernel=4)
        cm = Drafter(ccfg, di.add_conv_weights(ccfg, weights), max_ctx=cfg.ctx + 64, max_seqs=1)
        prefill(cm)
        variants["row_conv_group16_kernel4"] = timed(lambda i: cm.block_forward(seqs, [cfg.ctx], hs[i], out=logits))
        cm.close()
        log("variants ms/block:", variants)

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

    ab = di.algorithmic_bytes(cfg, ctx_rows=cfg.ctx)
    block_gbs = ab["total"] / (ms * 1e-3) / 1e9
    rows = cfg.n_seqs * cfg.block
    # the head: algorithmic bytes per launch / its average launch time (HBM roofline)
    hb = head_bytes(cfg)
    head_avg = head_ms / max(head_n, 1)
    head_gbs = hb / (head_avg * 1e-3) / 1e9
    head_line = {"bound": "hbm", "achieved": round(head_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(head_gbs / HBM_PEAK_GBS, 4),
                 "traffic": measured_traffic("head_gemm", cfg.key, "gemm.hip"),
                 "kernel": "k_gemm_q (head logits, Q8_32 x A8_32)", "bytes_per_launch": hb,
                 "avg_launch_ms": round(head_avg, 5), "launches": head_n, "ms_per_step": round(head_ms / K, 5)}
    # attention chunks: f64 MFMA flops per launch / its average launch time (f64 matrix roofline)
    ctx_rows = [cfg.ctx + (i + 1) * cfg.append_per_block for i in range(K)] if app is not None else [cfg.ctx] * K
    flops = sum(attention_flops(cfg, n) for n in ctx_rows) * cfg.layers
    attn_avg = attn_ms / max(attn_n, 1)
    attn_tf = flops / max(attn_n, 1) / (attn_avg * 1e-3) / 1e12
    attn_line = {"bound": "mfma", "achieved": round(attn_tf, 2), "peak": F64_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                 "frac": round(attn_tf / F64_MFMA_PEAK_TFS, 4),
                 "traffic": measured_traffic("attn_chunks", cfg.key, "attention.hip"),
                 "kernel": "k_attn_partial (f64 MFMA scores, softmax and values)",
                 "flops_per_launch": round(flops / max(attn_n, 1)), "avg_launch_ms": round(attn_avg, 5),
                 "launches": attn_n, "ms_per_step": round(attn_ms / K, 5)}
    # the dominant kernel of the step is the one with the larger share of the step's time
    dominant, other = (attn_line, head_line) if attn_ms > head_ms else (head_line, attn_line)
    out = {
        "metric": METRIC,
        "value": round(ms, 5),
        "unit": "ms/block",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8 (int8 MFMA on 4/8-bit weights) + f64 (attention, rescale) + f32",
        "data": "synthetic",
        "config": {"workload": workload_name(cfg), "sequences": cfg.n_seqs, "block_rows": cfg.block,
                   "context_rows": cfg.ctx, "append_rows_per_step": cfg.append_per_block},
        "blocks_per_s": round(1e3 / ms * cfg.n_seqs, 2),
        "rows_per_s": round(1e3 / ms * rows, 1),
        "algorithmic_bytes_per_step": ab["total"],
        "achieved_GBps_step": round(block_gbs, 1),
        "frac_of_hbm_peak_step": round(block_gbs / HBM_PEAK_GBS, 4),
        "gpu_prefill_rows_per_s": round(cfg.n_seqs * cfg.ctx / (prefill_ms * 1e-3), 1),
        # the prefill's algorithmic bytes: FC and every layer's Wk|Wv once, the taps read, the K/V
        # rows written; it runs 128-row products, so it is bound by their arithmetic, not by HBM
        "gpu_prefill_GBps": round(prefill_bytes(cfg) / (prefill_ms * 1e-3) / 1e9, 1),
        "int8_mfma_util_step": round(int8_macs(cfg) * 2 / (ms * 1e-3) / I8_MFMA_PEAK_OPS, 5),
        "roofline": dominant,
        "roofline_next": other,
        "ms_per_step_with_kernel_events": round(ms_events, 5),
        "cold_ms_per_step": flushed,
        "stages_ms_per_step": stages,
        "selection_ms_per_block": None if sel_ms is None else round(sel_ms, 5),
        "variants_ms_per_block": variants,
    }
    if args.cpu_baseline and cfg.n_seqs == 1 and cfg.ctx <= 8192:
        out["cpu_baseline"] = cpu_baseline(cfg, weights)
    elif args.cpu_baseline:
        base = di.CONFIGS["qwen3_8b"]
        same = (base.weight_seed or base.seed) == (cfg.weight_seed or cfg.seed)
        cb = cpu_baseline(base, weights if same else di.make_weights(base))
        cb["sample"] = "the same drafter at a 4096-row context (the 8B-shaped workload): " + cb["sample"]
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)
    gm.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
