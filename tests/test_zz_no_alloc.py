"""The allocation-free permutation (moe_permute_noalloc) against moe_permute, through the C ABI.

Two calls in a row on the library's shared device scratch, the second with a smaller input,
each compared with moe_permute (its own workspace) on the same input: indices, split_sizes,
offsets, probabilities and the permuted rows (bf16 and MXFP8 bytes) bit for bit, and the
bad-expert-id flag.
"""
import numpy as np
import pytest
import torch

from gpu_util import cfg_small, gpu, log, need_gpu
from moe_inputs import get_config, make_inputs

KEYS = ("split_sizes", "offsets", "row_id_map", "src_index", "prob_perm", "x_perm", "x_perm_scales")


def _same(a, b):
    # rows past offsets[E] exist only when a bad expert id dropped a pair; nothing writes them
    n = int(a["offsets"][-1].item())
    assert int(b["offsets"][-1].item()) == n
    for key in KEYS:
        if a[key] is None:
            assert b[key] is None, key
            continue
        x, y = a[key], b[key]
        if key in ("src_index", "prob_perm", "x_perm", "x_perm_scales"):
            x, y = x[:n], y[:n]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), key


@gpu
@pytest.mark.parametrize("perm_dtype", ["bf16", "mxfp8"])
def test_noalloc_permute_matches_workspace_permute(perm_dtype):
    m = need_gpu()
    big = get_config(5).with_(T=4096, H=256, I=256)            # 64 experts, top-8, Zipf routing
    small = cfg_small(T=300, H=128, I=128, E=8, k=2)
    for cfg in (big, small):
        log(f"noalloc permute {perm_dtype} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k}")
        d = make_inputs(cfg).to("cuda")
        ref = m.moe_permute(d.x, d.topk_idx, d.topk_prob, cfg.E, perm_dtype)
        got = m.moe_permute_noalloc(d.x, d.topk_idx, d.topk_prob, cfg.E, perm_dtype)
        torch.cuda.synchronize()
        _same(ref, got)
        assert m.moe_read_device_error(got["error_flag"]) == 0
        assert int(got["split_sizes"].sum().item()) == cfg.T * cfg.k


@gpu
def test_noalloc_permute_flag_and_index_only():
    m = need_gpu()
    log("noalloc permute: bad id, then a smaller clean call without rows")
    idx = torch.tensor([[0, 1], [2, 7], [1, 3], [3, 0]], dtype=torch.int32, device="cuda")   # 7 >= E = 4
    prob = torch.full((4, 2), 0.5, device="cuda")
    got = m.moe_permute_noalloc(None, idx, prob, 4)
    ref = m.moe_permute(None, idx, prob, 4)
    assert m.moe_read_device_error(got["error_flag"]) == 1
    _same(ref, got)
    got2 = m.moe_permute_noalloc(None, idx[:3].clamp(max=3), prob[:3], 4)
    ref2 = m.moe_permute(None, idx[:3].clamp(max=3), prob[:3], 4)
    assert m.moe_read_device_error(got2["error_flag"]) == 0
    _same(ref2, got2)
    np.testing.assert_array_equal(got2["split_sizes"].cpu().numpy(), [1, 2, 1, 2])


@gpu
def test_noalloc_permute_rejects_oversized_problem():
    m = need_gpu()
    log("noalloc permute: beyond the scratch")
    T, E, k = 130753, 256, 2
    idx = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    with pytest.raises(m.MoeError) as ei:
        m.moe_permute_noalloc(None, idx, None, E)
    assert ei.value.status == 2
