"""The algorithmic bytes the bench divides by its times (the roofline's numerator), against the
per-part sizes of the 8B-shaped workloads worked out by hand from their geometry: a Q4_32 group
of 32 weights is 16 bytes of codes and a 2-byte f16 scale (18), a Q8_32 group 32 + 2 (34); the
context's K/V rows are read in f32; the logits are written in f32.  Also bench.py's refusal of
more than one GPU.  CPU only."""
import pytest

import dflash_inputs as di

MB = 1e6


def test_eight_b_block_bytes():
    """hidden 4096, q 32 x 128, kv 8 x 128, intermediate 12288, 5 layers, vocab 151936, Q4 body,
    Q8 head, 4096 context rows, 16 rows:
      Wq|Wk|Wv 6144 x 128 groups x 18 = 14.16 MB, Wo 4096 x 128 x 18 = 9.44 MB,
      gate|up 24576 x 128 x 18 = 56.62 MB, down 4096 x 384 x 18 = 28.31 MB: 108.53 MB a layer;
      head 151936 x 128 x 34 = 661.23 MB; K/V 4096 x 5 x 2 x 1024 x 4 = 167.77 MB;
      logits 16 x 151936 x 4 = 9.72 MB."""
    ab = di.algorithmic_bytes(di.CONFIGS["qwen3_8b"])
    assert ab["body"] == 5 * (14_155_776 + 9_437_184 + 56_623_104 + 28_311_552)
    assert ab["head"] == 661_225_472
    assert ab["kv"] == 167_772_160
    assert ab["logits"] == 9_723_904
    assert ab["total"] / MB == pytest.approx(1381.36, abs=0.01)


def test_long_context_step_bytes():
    """The same drafter reading 32768 context rows, plus the append of 16 rows: FC 4096 x 640
    groups x 34 = 89.13 MB, every layer's Wk|Wv 5 x 2048 x 128 x 18 = 23.59 MB, the taps 16 x
    20480 x 4 = 1.31 MB, the K/V rows written 16 x 5 x 2 x 1024 x 4 = 0.66 MB."""
    ab = di.algorithmic_bytes(di.CONFIGS["qwen3_8b_long"], ctx_rows=32768)
    assert ab["kv"] == 1_342_177_280
    assert ab["append_fc"] == 89_128_960
    assert ab["append_kv_w"] == 23_592_960
    assert ab["append_taps"] == 1_310_720
    assert ab["append_kv_write"] == 655_360
    assert ab["total"] / MB == pytest.approx(2670.45, abs=0.01)
    # the bench's first step reads the 16 rows it just appended as well
    assert di.algorithmic_bytes(di.CONFIGS["qwen3_8b_long"], ctx_rows=32784)["kv"] == 32784 * 5 * 2 * 1024 * 4


def test_batched_forward_bytes():
    """Eight sequences of 8192 rows, 16 rows each: the weights once (1203.86 MB), K/V 8 x 8192 x
    5 x 2 x 1024 x 4 = 2684.35 MB, logits 128 x 151936 x 4 = 77.79 MB."""
    ab = di.algorithmic_bytes(di.CONFIGS["qwen3_8b_batch8"])
    assert ab["body"] + ab["head"] == 542_638_080 + 661_225_472
    assert ab["kv"] == 2_684_354_560
    assert ab["logits"] == 77_791_232
    assert ab["total"] / MB == pytest.approx(3966.01, abs=0.01)


def test_bench_refuses_more_than_one_gpu():
    """One GPU is measured: `--gpus 2` exits with status 2 and says why, before touching a GPU."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
    assert not r.stdout.strip().startswith("{")  # no bench line
