"""dflash_top_k_noalloc (the top-k with its chunk lists in the library's fixed device array)
against dflash_top_k (caller scratch) through the C ABI: equal indices and values on two calls in
a row, the second smaller than the first, and a size past the array refused."""
import numpy as np
import pytest

import block_draft_model_dflash_amd as D

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _both(x, rows, width, ld, k):
    stream = torch.cuda.current_stream().cuda_stream
    vals = torch.empty((rows, k), dtype=torch.float32, device="cuda")
    idx = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    vals_r, idx_r = torch.empty_like(vals), torch.empty_like(idx)
    D.dflash_top_k_noalloc(x.data_ptr(), rows, width, ld, k, vals.data_ptr(), idx.data_ptr(), stream)
    scr = torch.empty(D.dflash_top_k_scratch_bytes(rows, width, k), dtype=torch.uint8, device="cuda")
    D.dflash_top_k(x.data_ptr(), rows, width, ld, k, vals_r.data_ptr(), idx_r.data_ptr(), scr.data_ptr(), stream)
    torch.cuda.synchronize()
    return vals.cpu().numpy(), idx.cpu().numpy(), vals_r.cpu().numpy(), idx_r.cpu().numpy()


def test_noalloc_top_k_matches_the_scratch_entry_point_on_two_calls():
    rng = np.random.default_rng(77)
    # a large call (38 chunks of a 151936-wide row, many rows, ties planted), then a smaller one:
    # the second must not see the first's leftovers in the shared array
    for rows, width, ld, k in [(120, 151936, 151936 + 16, 24), (3, 5000, 5000, 7)]:
        xh = rng.standard_normal((rows, ld)).astype(np.float32)
        xh[:, 100:140] = xh[:, 99:100]  # runs of equal values: the earlier index ranks first
        x = torch.from_numpy(xh).cuda()
        v, i, vr, ir = _both(x, rows, width, ld, k)
        np.testing.assert_array_equal(i, ir)
        np.testing.assert_array_equal(v, vr)
        # and the top-k itself: the largest values of each row, largest first
        want = -np.sort(-xh[:, :width], axis=1)[:, :k]
        np.testing.assert_array_equal(v, want)


def test_noalloc_top_k_refuses_sizes_past_its_array():
    x = torch.zeros((128, 151936), dtype=torch.float32, device="cuda")
    out = torch.empty((128, 64), dtype=torch.float32, device="cuda")
    idx = torch.empty((128, 64), dtype=torch.int32, device="cuda")
    with pytest.raises(D.DFlashError) as e:  # 128 * 38 * 64 entries > 131072
        D.dflash_top_k_noalloc(x.data_ptr(), 128, 151936, 151936, 64, out.data_ptr(), idx.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    assert e.value.code == D.DFLASH_EINVAL
    assert "131072" in D.dflash_last_error(None)
