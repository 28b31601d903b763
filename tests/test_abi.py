"""The C-ABI library builds for gfx950, loads on a CPU-only host and exports every entry point
include/dflash.h declares; host-side argument checks (no GPU call is made here)."""
import ctypes as C
import os
import re

import pytest

import block_draft_model_dflash_amd as D
import dflash_inputs as di
from block_draft_model_dflash_amd.drafter import geometry

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "dflash.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert _declared() == sorted(D.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = D.lib()
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing


def test_library_is_built_for_gfx950():
    data = open(D.LIB_PATH, "rb").read()
    assert b"gfx950" in data


@pytest.mark.parametrize("key", di.CONFIG_ORDER)
def test_workspace_sizes_of_the_workloads(key):
    c = di.CONFIGS[key]
    g = geometry(c, c.ctx + 64, c.n_seqs)
    n = D.dflash_workspace_bytes(g)
    # at least the packed weights and the f32 K/V cache
    ab = di.algorithmic_bytes(c)
    cache = 2 * c.layers * c.n_seqs * (c.ctx + 64) * c.kv_dim * 4
    assert n >= ab["body"] + ab["head"] + cache


@pytest.mark.parametrize("change,code", [
    ({"head_dim": 96}, D.DFLASH_ENOTSUP),
    ({"heads": 6, "kv_heads": 4}, D.DFLASH_EINVAL),
    ({"block": 1}, D.DFLASH_EINVAL),
    ({"block": 17}, D.DFLASH_ENOTSUP),
    ({"hidden": 4000}, D.DFLASH_ENOTSUP),
    ({"layers": 0}, D.DFLASH_EINVAL),
    ({"body_fmt": 7}, D.DFLASH_EINVAL),
    ({"conv_kernel": -1}, D.DFLASH_EINVAL),
    ({"conv_kernel": 4, "conv_group": 24}, D.DFLASH_EINVAL),  # 24 does not divide 2048
    ({"conv_kernel": 4, "conv_group": 16, "g.conv_fmt": D.DFLASH_F32}, D.DFLASH_ENOTSUP),  # f32 beside a q4 body
    ({"conv_kernel": 1, "conv_group": 512}, D.DFLASH_ENOTSUP),  # 8 kernel rows: not a whole n-tile
])
def test_geometry_checks(change, code):
    c = di.CONFIGS["small_q"].replace(**{k: v for k, v in change.items() if not k.startswith("g.")})
    g = geometry(c, 600, 1)
    for k, v in change.items():  # fields of the C geometry alone
        if k.startswith("g."):
            setattr(g, k[2:], v)
    with pytest.raises(D.DFlashError) as e:
        D.dflash_workspace_bytes(g)
    assert e.value.code == code
    assert "geometry" in D.dflash_last_error(None)


def test_convolution_workspace():
    c = di.CONFIGS["qwen3_8b"]
    plain = D.dflash_workspace_bytes(geometry(c, c.ctx + 64, 1))
    conv = D.dflash_workspace_bytes(geometry(c.replace(conv_group=16, conv_kernel=4), c.ctx + 64, 1))
    # two Q8_32 kernel projections of 2048 x 4096 per layer, at least
    assert conv - plain >= c.layers * 2 * (2048 // 16) * (4096 // 128) * 2176


def test_too_many_rows_refused():
    c = di.CONFIGS["qwen3_8b"]
    with pytest.raises(D.DFlashError) as e:
        D.dflash_workspace_bytes(geometry(c, 100, 9))  # 9 sequences x 16 rows > 128
    assert e.value.code == D.DFLASH_ENOTSUP


@pytest.mark.parametrize("f16", [0, 1])
def test_cache_rows_within_32_bit_offsets(f16):
    """Attention addresses a (sequence, kv head)'s cache rows with 32-bit byte offsets: a
    max_ctx whose rows reach 2^31 bytes is refused, one row less is accepted.  Where the scores
    come from digits (head_dim 128, four q heads per kv head) the keys' digit rows (7 x 128 bytes
    a row) count too."""
    c = di.CONFIGS["small_q"].replace(kv_f16=bool(f16))
    row_bytes = c.head_dim * (2 if f16 else 4)
    if c.head_dim == 128 and c.heads == 4 * c.kv_heads:
        row_bytes = max(row_bytes, 7 * 128)
    limit = -(-(1 << 31) // row_bytes)  # the first max_ctx whose rows reach 2^31 bytes
    g = geometry(c, limit - 1, 1)
    assert D.dflash_workspace_bytes(g) > 0
    with pytest.raises(D.DFlashError) as e:
        D.dflash_workspace_bytes(geometry(c, limit, 1))
    assert e.value.code == D.DFLASH_ENOTSUP


def test_null_arguments_refused_before_any_gpu_work():
    L = D.lib()
    g = geometry(di.CONFIGS["tiny_f32"], 128, 1)
    out = C.c_void_p()
    assert L.dflash_create(C.byref(g), None, None, 0, None, C.byref(out)) == D.DFLASH_EINVAL
    assert L.dflash_ctx_append(None, 0, 0, None, 0) == D.DFLASH_EINVAL
    assert L.dflash_block_forward(None, 1, None, None, None, None) == D.DFLASH_EINVAL
    assert L.dflash_quant_act(None, 1, 32, None, None, None) == D.DFLASH_EINVAL
    n = C.c_size_t()
    assert L.dflash_packed_bytes(D.DFLASH_Q4_32, 16, 100, C.byref(n)) == D.DFLASH_EINVAL
    assert L.dflash_packed_bytes(D.DFLASH_Q4_32, 32, 256, C.byref(n)) == 0 and n.value == 2 * 2 * 1152
    assert L.dflash_packed_bytes(D.DFLASH_Q8_32, 16, 128, C.byref(n)) == 0 and n.value == 2176
    assert L.dflash_gemm_scratch_bytes(64, 256, 129, 0, C.byref(n)) == D.DFLASH_EINVAL


def test_selection_arguments_refused_before_any_gpu_work():
    L = D.lib()
    n = C.c_size_t()
    assert L.dflash_top_k_scratch_bytes(2, 100, 0, C.byref(n)) == D.DFLASH_EINVAL
    assert L.dflash_top_k_scratch_bytes(2, 100, 65, C.byref(n)) == D.DFLASH_EINVAL
    assert L.dflash_top_k_scratch_bytes(2, 10, 11, C.byref(n)) == D.DFLASH_EINVAL
    assert L.dflash_top_k_scratch_bytes(2, 151936, 16, C.byref(n)) == D.DFLASH_OK and n.value > 0
    # the chunks' lists of a row (ceil(width / 4096) * k entries) must fit one merge of 4096
    assert L.dflash_top_k_scratch_bytes(2, 262144, 64, C.byref(n)) == D.DFLASH_OK
    assert L.dflash_top_k_scratch_bytes(2, 262145, 64, C.byref(n)) == D.DFLASH_EINVAL
    assert L.dflash_select_scratch_bytes(2, 262145, 64, C.byref(n)) == D.DFLASH_EINVAL
    assert L.dflash_top_k(None, 2, 100, 100, 4, None, None, None, None) == D.DFLASH_EINVAL
    # the allocation-free top-k refuses sizes past its fixed array before touching the GPU
    fake = 256  # never dereferenced
    assert L.dflash_top_k_noalloc(fake, 128, 151936, 151936, 64, fake, fake, None) == D.DFLASH_EINVAL
    assert "131072" in D.dflash_last_error(None)
    assert L.dflash_top_k_noalloc(None, 2, 100, 100, 4, fake, fake, None) == D.DFLASH_EINVAL
    assert L.dflash_select_scratch_bytes(15, 151936, 16, C.byref(n)) == D.DFLASH_OK
    # width beyond the codebooks' vocabulary, anchor outside it, rank 0: refused
    fake = 256  # never dereferenced: the checks come first
    assert L.dflash_select(fake, 1, 200, 200, fake, 8, fake, fake, 100, 4, 0, fake, fake, fake, None) == D.DFLASH_EINVAL
    assert L.dflash_select(fake, 1, 100, 100, fake, 8, fake, fake, 100, 4, 100, fake, fake, fake, None) == D.DFLASH_EINVAL
    assert L.dflash_select(fake, 1, 100, 100, fake, 0, fake, fake, 100, 4, 0, fake, fake, fake, None) == D.DFLASH_EINVAL
