"""GPU parity: permutation and MXFP8 quantization must be bit-exact against the oracle."""
import numpy as np
import pytest
import torch

from gpu_util import cfg_small, gpu, inputs_with_counts, log, need_gpu
from moe_inputs import get_config, make_inputs
from moe_inputs.generate import routing_with_counts
from oracle import numerics as nm
from oracle.permute import permute as oracle_permute

ROUTINGS = [
    ("cfg1", get_config(1), None),
    ("zipf-zero-expert", get_config(3).with_(T=3000, H=256, I=256), None),
    ("finegrained-e64-k8", get_config(5).with_(T=1500, H=128, I=128), None),
    ("zeros-first-middle-last", cfg_small(T=300, H=128, I=128, E=8, k=2), [0, 235, 1, 31, 0, 33, 300, 0]),
    ("edge-sizes", cfg_small(T=600, H=64, I=128, E=7, k=2), [255, 257, 1, 31, 33, 600, 23]),
    ("one-expert", cfg_small(T=257, H=64, I=128, E=1, k=1), None),
    ("all-to-one", cfg_small(T=513, H=64, I=128, E=4, k=1), [0, 0, 513, 0]),
    ("tiny-T1", cfg_small(T=1, H=64, I=128, E=4, k=2), None),
    # H not a multiple of 512 (a partial last chunk), with whole 128-column scale words, and with not
    ("h384", cfg_small(T=200, H=384, I=128, E=4, k=2), None),
    ("h160", cfg_small(T=200, H=160, I=128, E=4, k=2), None),
    # the count scan's slicing: 1024 / E slices per expert over the 64-token blocks, with a
    # slice length that is not a whole number of 8-block batches (24 experts, 469 blocks: 12
    # per slice), 64 blocks per slice (256 experts), and more slices than blocks with E * S
    # short of 1024 (3 experts: 341 slices, 79 blocks)
    ("scan-e24-469-blocks", cfg_small(T=30000, H=64, I=128, E=24, k=6), None),
    ("scan-e256-256-blocks", cfg_small(T=16384, H=64, I=128, E=256, k=8), None),
    ("scan-e3-79-blocks", cfg_small(T=5000, H=64, I=128, E=3, k=2), None),
]


def _inputs(cfg, counts):
    if counts is None:
        return make_inputs(cfg, weights=False)
    idx, pr = routing_with_counts(counts, cfg.T, cfg.k, 5)
    return make_inputs(cfg, topk_idx=idx, topk_prob=pr, weights=False)


@gpu
@pytest.mark.parametrize("name,cfg,counts", ROUTINGS, ids=[r[0] for r in ROUTINGS])
@pytest.mark.parametrize("perm_dtype", ["bf16", "mxfp8"])
def test_permute_bit_exact(name, cfg, counts, perm_dtype):
    m = need_gpu()
    log(f"permute {name} {perm_dtype} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k}")
    inp = _inputs(cfg, counts)
    d = inp.to("cuda")
    res = m.moe_permute(d.x, d.topk_idx, d.topk_prob, cfg.E, perm_dtype)
    torch.cuda.synchronize()
    ref = oracle_permute(inp.topk_idx.numpy(), cfg.E)
    np.testing.assert_array_equal(res["split_sizes"].cpu().numpy(), ref.split_sizes)
    np.testing.assert_array_equal(res["offsets"].cpu().numpy(), ref.offsets)
    np.testing.assert_array_equal(res["row_id_map"].cpu().numpy(), ref.row_id_map)
    np.testing.assert_array_equal(res["src_index"].cpu().numpy(), ref.src_index)
    np.testing.assert_array_equal(res["prob_perm"].cpu().numpy(),
                                  inp.topk_prob.numpy().reshape(-1)[ref.src_index])
    assert m.moe_read_device_error(res["workspace"]) == 0
    x64 = inp.x.to(torch.float64).numpy()
    tok = ref.token_of_row
    if perm_dtype == "bf16":
        got = res["x_perm"].cpu().view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(got, nm.bf16_bits(nm.round_bf16(x64)[tok]))
    else:
        c, s = nm.quantize_mxfp8(x64, axis=1)
        np.testing.assert_array_equal(res["x_perm"].cpu().numpy(), c[tok])
        np.testing.assert_array_equal(res["x_perm_scales"].cpu().numpy(), s[tok])


@gpu
def test_permute_out_of_range_id_sets_flag():
    m = need_gpu()
    log("permute out-of-range id")
    idx = torch.tensor([[0, 1], [2, 7], [1, 3]], dtype=torch.int32, device="cuda")   # 7 >= E = 4
    prob = torch.full((3, 2), 0.5, device="cuda")
    res = m.moe_permute(None, idx, prob, 4, "bf16")
    flag = m.moe_read_device_error(res["workspace"])
    assert flag == 1
    rmap = res["row_id_map"].cpu().numpy()
    assert rmap[3] == -1
    assert res["split_sizes"].cpu().numpy().tolist() == [1, 2, 1, 1]
    valid = np.delete(np.arange(6), 3)
    assert sorted(rmap[valid].tolist()) == list(range(5))
    # a clean call afterwards clears the flag
    res2 = m.moe_permute(None, idx.clamp(max=3), prob, 4, "bf16")
    assert m.moe_read_device_error(res2["workspace"]) == 0


def _quant_inputs():
    g = np.random.default_rng(42)
    a = g.standard_normal((300, 256)) * 10.0 ** g.integers(-8, 8, (300, 1))
    a[7] = 0.0
    a[11, :64] = 1e-41          # f32 subnormals
    a[12] = 448.0 * 2.0 ** g.integers(-5, 5, 256)
    return a


@gpu
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
# rows x cols / 8 lane groups: a multiple of 16 (scale bytes stored as words), or not (the last
# partial 16-lane group stores bytes)
@pytest.mark.parametrize("shape", [(300, 256), (7, 96), (1, 32)])
def test_mxfp8_quantize_rowwise_bit_exact(dtype, shape):
    m = need_gpu()
    log(f"mxfp8_quantize axis0 {dtype} {shape}")
    a = torch.from_numpy(_quant_inputs()[:shape[0], :shape[1]].copy()).to(dtype)
    q, s = m.mxfp8_quantize(a.cuda(), axis=0)
    rc, rs = nm.quantize_mxfp8(a.to(torch.float64).numpy(), axis=1)
    np.testing.assert_array_equal(q.cpu().numpy(), rc)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)


@gpu
def test_mxfp8_quantize_exhaustive_bf16():
    """Every finite positive bf16 value as a block amax (the other 31 elements
    fixed fractions of it), both signs."""
    m = need_gpu()
    log("mxfp8_quantize exhaustive bf16 amax")
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    b = nm.bf16_from_bits(bits)
    fr = np.linspace(-1, 1, 31)
    blk = np.concatenate([b[:, None], nm.round_bf16(b[:, None] * fr[None, :])], axis=1)
    blk = np.concatenate([blk, -blk])
    t = torch.from_numpy(blk).to(torch.bfloat16)
    q, s = m.mxfp8_quantize(t.cuda(), axis=0)
    rc, rs = nm.quantize_mxfp8(blk, axis=1)
    np.testing.assert_array_equal(q.cpu().numpy(), rc)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)


@gpu
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
# the last case spans several 128-row workgroup tiles of the padded token axis
@pytest.mark.parametrize("sizes", [[0, 5, 32, 33, 0, 70], [257], [1, 0, 0, 64, 31], [130, 0, 400, 7, 129, 1]])
def test_mxfp8_quantize_colwise_segments_bit_exact(sizes, dtype):
    m = need_gpu()
    log(f"mxfp8_quantize axis1 segments {sizes} {dtype}")
    g = np.random.default_rng(len(sizes))
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    x = torch.from_numpy(g.standard_normal((int(off[-1]), 96))).to(torch.bfloat16)
    if dtype == "f32":
        x = x.to(torch.float32) * (1 + torch.from_numpy(g.uniform(0, 1e-3, tuple(x.shape))).to(torch.float32))
    q, s = m.mxfp8_quantize(x.cuda(), axis=1, group_offsets=torch.from_numpy(off).cuda())
    rc, rs = nm.quantize_mxfp8_segments_t(x.to(torch.float64).numpy(), off)
    rp = rc.shape[1]
    np.testing.assert_array_equal(q.cpu().numpy()[:, :rp], rc)
    np.testing.assert_array_equal(s.cpu().numpy()[:, :rp // 32], rs)
    # the columns past the last segment are padding: codes 0, scale bytes 0 (the binding allocates
    # the outputs uninitialised, so these bytes come from the kernel)
    assert not q.cpu().numpy()[:, rp:].any() and not s.cpu().numpy()[:, rp // 32:].any()
