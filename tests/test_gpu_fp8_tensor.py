"""GPU parity of the per-tensor-scaled FP8 variant (one fp32 scale per operand tensor).

The standalone quantizer is compared byte for byte (codes and fp32 scales) with the oracle,
the forward normwise with the oracle's FP8 forward (the MXFP8 tolerance, 2e-2: the same E4M3
elements; what differs between the two sides is the fp32 vs fp64 arithmetic ahead of each
rounding, so a few codes may sit one step apart).
"""
import numpy as np
import pytest
import torch

from gpu_util import MXFP8_TOL, cfg_small, gpu, log, need_gpu, to_np
from moe_inputs import get_config, make_inputs
from moe_inputs.generate import routing_with_counts
from oracle import mlp
from oracle import numerics as nm


def _bf16(g, shape, lo, hi):
    v = g.standard_normal(shape) * np.exp2(g.integers(lo, hi, shape))
    return torch.from_numpy(v).to(torch.bfloat16)


QUANT_CASES = [
    # name, rows per segment, cols
    ("one-tensor", [300], 64),
    ("segments", [0, 1, 31, 33, 256, 0, 700, 5], 128),
    ("many", [17] * 64 + [0] * 3 + [1000], 32),
]


@gpu
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("name,sizes,cols", QUANT_CASES, ids=[c[0] for c in QUANT_CASES])
def test_fp8_tensor_quantize_bit_exact(name, sizes, cols, dtype):
    m = need_gpu()
    log(f"fp8_tensor_quantize {name} {dtype} rows={sum(sizes)} cols={cols}")
    g = np.random.default_rng(31)
    rows = sum(sizes)
    x = _bf16(g, (rows, cols), -10, 6)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    if len(sizes) > 3:
        # an all-zero segment (scale 1), one of values whose scale overflows fp32 (clamped to
        # the largest float), and one with a signed zero and subnormal products
        z0, z1 = int(off[3]), int(off[4])
        x[z0:z1] = 0.0
        t0, t1 = int(off[4]), int(off[5])
        x[t0:t1] = _bf16(g, (t1 - t0, cols), -140, -133)
        x[int(off[6])] = -0.0
    if dtype == "f32":
        x = x.to(torch.float32) * (1 + torch.from_numpy(g.uniform(0, 1e-3, (rows, cols))).to(torch.float32))
    offs = None if len(sizes) == 1 else torch.from_numpy(off).cuda()
    q, s = m.fp8_tensor_quantize(x.cuda(), offs)
    torch.cuda.synchronize()
    rc, rs = nm.quantize_fp8_segments(x.to(torch.float64).numpy(), off)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rc)


FWD_CASES = [
    ("ragged", cfg_small(T=700, H=256, I=384, E=4, k=2), None),
    ("zeros-first-middle-last", cfg_small(T=400, H=128, I=256, E=8, k=2), [0, 400, 1, 31, 0, 33, 335, 0]),
    ("one-expert", cfg_small(T=300, H=128, I=128, E=1, k=1), None),
    ("f32-io", get_config(1), None),
    ("finegrained-e64-k8", get_config(5).with_(T=512, H=256, I=256, precision="bf16"), None),
    # K = 384: three MX stages with 12-byte unit-scale rows
    ("row-scales", cfg_small(T=300, H=384, I=256, E=4, k=2), None),
]


def _inputs(cfg, counts):
    if counts is None:
        return make_inputs(cfg)
    idx, pr = routing_with_counts(counts, cfg.T, cfg.k, 5)
    return make_inputs(cfg, topk_idx=idx, topk_prob=pr)


@gpu
@pytest.mark.parametrize("name,cfg,counts", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_fp8_matches_oracle(name, cfg, counts):
    m = need_gpu()
    log(f"fwd fp8 {name} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}")
    inp = _inputs(cfg, counts)
    d = inp.to("cuda")
    out, ctx = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "fp8")
    torch.cuda.synchronize()
    ref = mlp.forward(inp.x, inp.topk_idx.numpy(), inp.topk_prob, inp.w1, inp.w2, "fp8", cfg.x_dtype)
    got = to_np(out)
    assert np.all(np.isfinite(got))
    err = mlp.normwise_rel_err(got, ref.out)
    log(f"  normwise err {err:.3e} (tol {MXFP8_TOL})")
    assert err < MXFP8_TOL
    np.testing.assert_array_equal(ctx["perm"]["split_sizes"].cpu().numpy(), ref.perm.split_sizes)


@gpu
def test_forward_fp8_split_last_round():
    """The down projection's last-round tiles split along K (fp32 partials summed by the fixup
    pass) carry the per-tensor dequantization too; experts 3 and 7 against the oracle."""
    m = need_gpu()
    counts = [600, 700, 768, 514, 640, 520, 700, 600]
    cfg = cfg_small(T=sum(counts) // 2, H=3072, I=4096, E=8, k=2)
    log(f"fwd fp8 split-tail T={cfg.T} H={cfg.H} I={cfg.I}")
    inp = _inputs(cfg, counts)
    d = inp.to("cuda")
    out, _ = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "fp8")
    torch.cuda.synchronize()
    idx = inp.topk_idx.numpy()
    experts = (3, 7)
    rows = np.all(np.isin(idx, experts), axis=1)
    assert rows.sum() >= 16
    ref = mlp.forward(inp.x, idx, inp.topk_prob, inp.w1, inp.w2, "fp8", cfg.x_dtype, experts=experts)
    err = mlp.normwise_rel_err(to_np(out)[rows], ref.out[rows])
    log(f"  {rows.sum()} tokens, normwise err {err:.3e}")
    assert err < MXFP8_TOL


@gpu
def test_forward_fp8_deterministic_and_rejections():
    m = need_gpu()
    log("fwd fp8 determinism and error paths")
    cfg = cfg_small(T=600, H=256, I=256, E=8, k=2)
    d = make_inputs(cfg).to("cuda")
    a, _ = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "fp8")
    b, _ = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "fp8")
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    with pytest.raises(m.MoeError) as ei:      # forward only: no saved activations
        m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "fp8", save_for_backward=True)
    assert ei.value.status == 2
    counts = np.bincount(make_inputs(cfg).topk_idx.numpy().ravel(), minlength=cfg.E).tolist()
    with pytest.raises(m.MoeError) as ei:      # no per-expert-loop variant
        m.moe_grouped_mlp_fwd_loop(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, counts, "fp8")
    assert ei.value.status == 2
    bad = cfg_small(T=64, H=192, I=128, E=2, k=1)   # H % 128 != 0
    e = make_inputs(bad).to("cuda")
    with pytest.raises(m.MoeError) as ei:
        m.moe_grouped_mlp_fwd(e.x, e.topk_idx, e.topk_prob, e.w1, e.w2, "fp8")
    assert ei.value.status == 2


@gpu
def test_forward_fp8_cached_weights_equal_per_call_quantization():
    """Weights quantized once (quantize_weights(..., "fp8")) give bit-identical outputs to the
    per-call quantization; the cached codes and scales are the oracle's."""
    m = need_gpu()
    cfg = cfg_small(T=600, H=256, I=384, E=8, k=2)
    log("fwd fp8 cached weights")
    inp = make_inputs(cfg)
    d = inp.to("cuda")
    wq = m.quantize_weights(d.w1, d.w2, "fp8")
    a, _ = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "fp8")
    b, _ = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "fp8", w_quant=wq)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    c1, s1 = nm.quantize_fp8_tensor(inp.w1[5].to(torch.float64).numpy())
    np.testing.assert_array_equal(wq[0][5].cpu().numpy(), c1)
    assert wq[1][5].item() == float(s1)
    c2, s2 = nm.quantize_fp8_tensor(inp.w2[2].to(torch.float64).numpy())
    np.testing.assert_array_equal(wq[2][2].cpu().numpy(), c2)
    assert wq[3][2].item() == float(s2)


@gpu
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fp8_tensor_quantize_hand_derived_cases(dtype):
    """The hand-derived tensors of tests/golden/fp8_tensor_cases.txt through the GPU quantizer
    (each padded with zeros to a multiple of 8 columns, which changes neither amax nor codes)."""
    from test_oracle_fp8_tensor import _golden
    from fractions import Fraction
    m = need_gpu()
    log(f"fp8_tensor_quantize hand-derived cases {dtype}")
    for name, s, vals, codes in _golden():
        n = (len(vals) + 7) // 8 * 8
        x = torch.zeros((1, n), dtype=torch.float64)
        x[0, :len(vals)] = torch.tensor(vals, dtype=torch.float64)
        x = x.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
        q, sc = m.fp8_tensor_quantize(x.cuda())
        torch.cuda.synchronize()
        assert Fraction(sc.item()) == s, name
        assert q.cpu().numpy()[0, :len(vals)].tolist() == codes, name
