"""The pins bite: plant plausible mistakes in a copy of the oracle's source (a dropped term, a
wrong sign, index or operand), build each copy, and require some pin to fail on every one.
Everything here runs on the CPU.  Each broken copy runs in a child process of its own: a
planted indexing mistake can write past the oracle's buffers, and that must not corrupt the
process that runs the other tests (a child that crashes has failed loudly: caught)."""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

import dflash_inputs as di
import oracle
import test_oracle_conv as TC
import test_oracle_f16 as TF
import test_oracle_queue as TQ
import test_oracle_model as TM
import test_oracle_select as TS
import test_oracle_units as TU
import test_oracle_windows as TW

# (what the mistake is, text in dflash_oracle.c, its replacement)
MUTANTS = [
    ("mean of squares over n-1", "ms /= (double)n;", "ms /= (double)(n - 1);"),
    ("eps dropped", "sqrtf((float)ms + eps)", "sqrtf((float)ms)"),
    ("norm weight dropped", "y[i] = t * w[i];", "y[i] = t;"),
    ("rotation sign", "x[i] = (float)(a * c - b * s);", "x[i] = (float)(a * c + b * s);"),
    ("position off by one", "float p = (float)pos;", "float p = (float)(pos + 1);"),
    ("interleaved pairs", "double a = x[i], b = x[i + half];", "double a = x[2 * i], b = x[2 * i + 1];"),
    ("act scale over 128", "d[g] = amax / 127.0f;", "d[g] = amax / 128.0f;"),
    ("truncating quantizer", "float r = nearbyintf(t);", "float r = truncf(t);"),
    ("one scale per row", "dw[g] = og_f16_to_f64(w.scales[(size_t)r * groups + g]);",
     "dw[g] = og_f16_to_f64(w.scales[(size_t)r * groups]);"),
    ("nibble order swapped", "int nib = (k & 1) ? (b >> 4) : (b & 15);", "int nib = (k & 1) ? (b & 15) : (b >> 4);"),
    ("unsigned nibbles", "return nib >= 8 ? nib - 16 : nib;", "return nib;"),
    ("attention scale dropped", "s[j] = dot * (double)scale;", "s[j] = dot;"),
    ("wrong kv head for the context", "(((size_t)l * g->max_ctx + (size_t)(lo - s->first + c)) * kvh + gi) * hd;",
     "(((size_t)l * g->max_ctx + (size_t)(lo - s->first + c)) * kvh + (kvh - 1 - gi)) * hd;"),
    ("causal block rows", "vvs[gi] + (size_t)c0 * hd, nk - (int)c0, hd, scale,",
     "vvs[gi] + (size_t)c0 * hd, nctx - (int)c0 + r + 1, hd, scale,"),
    ("context past the anchor read", "int64_t hi = anchor < s->first + s->len ? anchor : s->first + s->len;",
     "int64_t hi = s->first + s->len;"),
    ("a row's window counted from the anchor row", "int64_t from = anchor + r + 1 - w;", "int64_t from = anchor + 1 - w;"),
    ("window one position long", "int64_t from = anchor + r + 1 - w;", "int64_t from = anchor + r - w;"),
    ("dropped rows still read", "base = s->first + s->dropped[l];", "base = s->first;"),
    ("truncate keeps the dropped count", "if (s->dropped[l] > keep) s->dropped[l] = keep;", "(void)keep;"),
    ("the drop keeps twice the window", "s->dropped[l] += held - w;", "s->dropped[l] += held - 2 * w;"),
    ("a no-rope layer's context rotated", "if (m->rotary[l]) og_rope_head(tmp, hd, p, m->inv_freq);",
     "og_rope_head(tmp, hd, p, m->inv_freq);"),
    ("a no-rope layer's queries rotated", "og_rmsnorm_row(qh, L->q_norm, hd, eps, tmp);\n        if (m->rotary[l]) og_rope_head",
     "og_rmsnorm_row(qh, L->q_norm, hd, eps, tmp);\n        if (1) og_rope_head"),
    ("a convolution one offset short", "for (int o = 0; o < kn && o <= r; o++) {", "for (int o = 0; o < kn - 1 && o <= r; o++) {"),
    ("a convolution skips the block's first row", "for (int o = 0; o < kn && o <= r; o++) {",
     "for (int o = 0; o < kn && o < r; o++) {"),
    ("the dynamic kernel of another group", "+ (size_t)so * groups + i / gs];", "+ (size_t)so * groups + i % groups];"),
    ("the second stage takes the first stage's kernels", "const int so = stage * kn + o;", "const int so = o;"),
    ("dynamic kernels dropped", "const double k = (double)base[(size_t)so * hidden + i] + (double)d[",
     "const double k = (double)base[(size_t)so * hidden + i] + 0.0 * (double)d["),
    ("the MLP's kernels projected with the attention's matrix", "mm(g->conv_fmt, L->mlp_kp, pr, H, x, B, dm);",
     "mm(g->conv_fmt, L->attn_kp, pr, H, x, B, dm);"),
    ("a cut block reads the rows of the whole block", "block_one(m, seqs[i], anchors[i], block_rows, h + per * i, x + per * i);",
     "block_one(m, seqs[i], anchors[i], block_rows, h + (size_t)m->g.block * m->g.hidden * i, x + per * i);"),
    ("f16 rounding truncates", "return copysign(nearbyint(a / step) * step, x);", "return copysign(trunc(a / step) * step, x);"),
    ("f16 steps one bit too coarse", "ldexp(1.0, e - 11 > -24 ? e - 11 : -24)", "ldexp(1.0, e - 10 > -24 ? e - 10 : -24)"),
    ("f16 subnormal steps too fine", "ldexp(1.0, e - 11 > -24 ? e - 11 : -24)", "ldexp(1.0, e - 11 > -26 ? e - 11 : -26)"),
    ("the f16 cache keeps keys in f32", "s->k[off + d] = (float)og_round_f16(s->k[off + d]);", "(void)0;"),
    ("waiting rows settled without rounding to chunks", "int64_t over = (s->npend - g->pending_rows + 63) / 64 * 64;",
     "int64_t over = s->npend - g->pending_rows;"),
    ("a truncation keeps the waiting rows", "if (s->npend > wait) s->npend = wait;", "(void)wait;"),
    ("the span leaves out the waiting rows", "m->seqs[seq].len + m->seqs[seq].npend; /* Drafter::next_position */",
     "m->seqs[seq].len; /* Drafter::next_position */"),
    ("the block reads before settling", "  for (int i = 0; i < n_seqs; i++) og_ctx_settle(m, seqs[i]); /* a block reads settled rows */\n  const og_geometry* g = &m->g;",
     "  const og_geometry* g = &m->g;"),
    ("the shortlist takes the whole head", "mm(g->head_fmt, m->w.head, head_rows, g->hidden,",
     "mm(g->head_fmt, m->w.head, head_rows > 16 ? head_rows - 16 : head_rows, g->hidden,"),
    ("silu sign", "a[i] = (float)(gv / (1.0 + exp(-gv)) * (double)u[i]);", "a[i] = (float)(gv / (1.0 + exp(gv)) * (double)u[i]);"),
    ("gate and up swapped", "og_silu_mul(gt, up, B * I, a);", "og_silu_mul(up, gt, B * I, a);"),
    ("attention residual dropped", "h[i] = h[i] + o[i];\n    for (int r = 0; r < B; r++) og_rmsnorm_row(h + (size_t)r * H, L->post_norm",
     "h[i] = o[i];\n    for (int r = 0; r < B; r++) og_rmsnorm_row(h + (size_t)r * H, L->post_norm"),
    ("post-norm weight is the in-norm's", "og_rmsnorm_row(h + (size_t)r * H, L->post_norm, H, eps,",
     "og_rmsnorm_row(h + (size_t)r * H, L->in_norm, H, eps,"),
    ("k-norm on the context is the q-norm", "og_rmsnorm_row(kh, L->k_norm, hd, (float)g->eps, tmp);",
     "og_rmsnorm_row(kh, L->q_norm, hd, (float)g->eps, tmp);"),
    ("context rotated at its index, not its position", "og_rope_head(tmp, hd, p, m->inv_freq);",
     "og_rope_head(tmp, hd, (int64_t)row, m->inv_freq);"),
    ("hidden norm skipped", "og_rmsnorm_row(t + (size_t)i * H, m->w.hidden_norm, H, (float)g->eps, tn + (size_t)i * H);",
     "memcpy(tn + (size_t)i * H, t + (size_t)i * H, sizeof(float) * H);"),
    ("a gap keeps the old first", "    truncate_to(m, s, 0);\n    s->first = pos;", "    truncate_to(m, s, 0);\n    s->first = s->first;"),
    ("softmax max not subtracted consistently", "s[j] = exp(s[j] - top);", "s[j] = exp(s[j] - top) * (j == 0 ? 2.0 : 1.0);"),
    ("top-k keeps the later of equal values", "while (at < len && vals[at] >= v) at++;",
     "while (at < len && vals[at] > v) at++;"),
    ("the chain restarts at the anchor", "    prev = tok;\n    chosen[j] = tok;", "    prev = anchor;\n    chosen[j] = tok;"),
    ("the last largest score wins", "if (sc > best) {", "if (sc >= best) {"),
    ("predecessor read from the successor book", "pc[r] = f16f(pred[(size_t)prev * rank + r])",
     "pc[r] = f16f(succ[(size_t)prev * rank + r])"),
]

CHECKS = [
    (TS.test_top_k_pages_worked_example, ()),
    (TS.test_top_k_is_the_head_of_the_value_then_index_order, ()),
    (TS.test_select_reduces_to_top_1, ()),
    (TS.test_select_chooses_among_the_candidates_and_follows_the_chain, ()),
    (TS.test_select_brute_force_small, ()),
    (TU.test_rmsnorm_against_torch, (4096,)),
    (TU.test_rope_against_transformers_rotate_half, (4095,)),
    (TU.test_rope_invariants, ()),
    (TU.test_quant_act_nearest_code_brute_force, ()),
    (TU.test_quant_act_zero_group_and_ties, ()),
    (TU.test_canonical_formats_by_hand, ()),
    (TU.test_quantized_matmul_against_dense, (di.Q4_32,)),
    (TU.test_quantized_matmul_against_dense, (di.Q8_32,)),
    (TU.test_attention_against_torch_sdpa, ()),
    (TU.test_attention_special_cases, ()),
    (TU.test_silu_against_torch, ()),
    (TM.test_forward_matches_transformers_qwen3_layers, (TM.SHARP,)),
    (TM.test_forward_matches_transformers_qwen3_layers, (TM.QTINY,)),
    (TM.test_anchor_row_vs_draft_rows_non_causal, ()),
    (TM.test_context_past_the_anchor_is_not_read, ()),
    (TM.test_append_chunking_truncate_and_reset, ()),
    (TW.test_windows_and_no_rope_match_transformers, ()),
    (TW.test_window_drop_bookkeeping, ()),
    (TW.test_no_rope_everywhere_is_position_free, ()),
    (TW.test_shortlist_head_is_a_prefix, ()),
    (TW.test_block_cut_to_its_first_rows_matches_transformers, ()),
    (TQ.test_queue_counts_by_hand, ()),
    (TQ.test_deferral_leaves_the_cache_and_the_block_unchanged, ()),
    (TQ.test_window_drops_follow_the_settles, ()),
    (TF.test_round_f16_against_numpy, ()),
    (TF.test_f16_cache_holds_the_rounded_rows, ()),
    (TF.test_f16_cache_block_matches_transformers, ()),
    (TC.test_row_conv_against_torch_conv1d, ()),
    (TC.test_row_conv_reach, ()),
    (TC.test_identity_convolutions_give_the_plain_layer, ()),
    (TC.test_convolutions_match_transformers, ()),
]


def _caught(fn, args) -> bool:
    try:
        fn(*args)
    except (AssertionError, ValueError):
        return True
    return False


_CHILD = """
import sys
sys.path[:0] = {paths!r}
import oracle
oracle.use_library({so!r})
import test_oracle_mutants as M
for fn, args in M.CHECKS:
    if M._caught(fn, args):
        print("caught by", fn.__name__, flush=True)
        sys.exit(0)
sys.exit(1)
"""


def _run_mutant(src: str, what: str, old: str, new: str, work: str) -> str:
    i = [m[0] for m in MUTANTS].index(what)
    path = os.path.join(work, f"mutant{i}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = oracle.build(src=path, out=os.path.join(work, f"libmutant{i}.so"), opt="-O1")
    here = os.path.dirname(os.path.abspath(__file__))
    paths = [here, os.path.dirname(here)]
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", _CHILD.format(paths=paths, so=so)], capture_output=True, text=True,
                       env=env, timeout=600)
    if r.returncode == 0:
        return "caught"
    if r.returncode < 0:
        return f"crashed (signal {-r.returncode})"
    return "not caught:\n" + r.stdout[-2000:] + r.stderr[-2000:]


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    src = open(oracle.SRC).read()
    for what, old, _ in MUTANTS:
        assert src.count(old) == 1, f"mutation site for '{what}' not unique in the oracle source"
    work = str(tmp_path_factory.mktemp("mutants"))
    workers = max(1, min(8, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(workers) as ex:
        futs = {what: ex.submit(_run_mutant, src, what, old, new, work) for what, old, new in MUTANTS}
        return {what: f.result() for what, f in futs.items()}


@pytest.mark.parametrize("what", [m[0] for m in MUTANTS])
def test_every_planted_mistake_fails_a_pin(what, mutant_results):
    res = mutant_results[what]
    assert res == "caught" or res.startswith("crashed"), f"no pin caught: {what}: {res}"
