"""GPU parity: grouped MLP forward against the fp64 oracle (normwise relative error).

BF16: 5e-3; MXFP8: 2e-2 (the tolerances fixed for this layer).  The cases span
several 256-row tiles with ragged tails, zero-token experts in the first, middle
and last positions, the edge sizes 1, 31, 33, 255, 257, one expert, every token
on one expert, and the fine-grained 64-expert top-8 shape.
"""
import numpy as np
import pytest
import torch

from gpu_util import BF16_TOL, MXFP8_TOL, cfg_small, gpu, log, need_gpu, to_np
from moe_inputs import get_config, make_inputs
from moe_inputs.generate import routing_with_counts
from oracle import mlp
from oracle import numerics as nm

CASES = [
    # name, cfg, counts (None = the cfg's own routing)
    ("cfg1-tiny-f32io", get_config(1), None),
    ("ragged-bf16", cfg_small(T=700, H=256, I=384, E=4, k=2), None),
    ("zeros-first-middle-last", cfg_small(T=400, H=128, I=256, E=8, k=2), [0, 400, 1, 31, 0, 33, 335, 0]),
    ("edge-sizes", cfg_small(T=600, H=128, I=128, E=7, k=2), [255, 257, 1, 31, 33, 600, 23]),
    ("one-expert", cfg_small(T=300, H=128, I=128, E=1, k=1), None),
    ("all-to-one", cfg_small(T=520, H=128, I=256, E=4, k=1), [0, 0, 520, 0]),
    ("finegrained-e64-k8", get_config(5).with_(T=512, H=256, I=256, precision="bf16"), None),
    ("zipf-zero-expert", get_config(3).with_(T=1024, H=256, I=384, precision="bf16"), None),
    # K of a single 128-byte stage in both GEMMs (BF16: the K loop without the two-ahead loads)
    ("one-stage-k", cfg_small(T=300, H=64, I=64, E=4, k=2), None),
    # FC1 with a single-stage K, FC2 with two stages
    ("mixed-depth", cfg_small(T=300, H=64, I=128, E=4, k=2), None),
    # MXFP8 FC1 with K = 384: three stages but 12-byte scale rows (scale words read per lane)
    ("mx-row-scales", cfg_small(T=300, H=384, I=256, E=4, k=2), None),
    # several rounds of tiles in every GEMM under skewed routing with an empty expert: the weight
    # gradients' largest-expert-first, snake-dealt rounds (4 and 2 rounds), FC1 in 2 rounds, and
    # token segments starting at every 128-row offset modulo 512 (the MXFP8 scale-group shift)
    ("multiround-skew", cfg_small(T=1024, H=1024, I=2048, E=16, k=2),
     [600, 0, 300, 250, 200, 150, 120, 100, 80, 70, 60, 50, 30, 20, 10, 8]),
    # one token routed to every expert (k = E): every expert holds a single row
    ("one-token-all-experts", cfg_small(T=1, H=128, I=128, E=8, k=8), None),
    # the largest expert count with few tokens: 256 experts of a few rows each, 25 of them empty
    ("e256-sparse", cfg_small(T=64, H=128, I=256, E=256, k=8), None),
]


def _inputs(cfg, counts):
    if counts is None:
        return make_inputs(cfg)
    idx, pr = routing_with_counts(counts, cfg.T, cfg.k, 5)
    return make_inputs(cfg, topk_idx=idx, topk_prob=pr)


def _run(m, inp, compute):
    d = inp.to("cuda")
    out, ctx = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, compute)
    torch.cuda.synchronize()
    return out, ctx


@gpu
@pytest.mark.parametrize("name,cfg,counts", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("compute", ["bf16", "mxfp8"])
def test_forward_matches_oracle(name, cfg, counts, compute):
    m = need_gpu()
    if compute == "mxfp8" and (cfg.H % 128 or cfg.I % 128):
        pytest.skip("MXFP8 path needs H, I multiples of 128")
    log(f"fwd {name} {compute} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}")
    inp = _inputs(cfg, counts)
    out, ctx = _run(m, inp, compute)
    ref = mlp.forward(inp.x, inp.topk_idx.numpy(), inp.topk_prob, inp.w1, inp.w2, compute, cfg.x_dtype)
    got = to_np(out)
    assert np.all(np.isfinite(got))
    err = mlp.normwise_rel_err(got, ref.out)
    tol = BF16_TOL if compute == "bf16" else MXFP8_TOL
    log(f"  normwise err {err:.3e} (tol {tol})")
    assert err < tol
    np.testing.assert_array_equal(ctx["perm"]["split_sizes"].cpu().numpy(), ref.perm.split_sizes)


# experts whose last 256-row tile holds 0, 44, 64, 65, 128, 129, 192 and 1 rows
TAIL_COUNTS = [256, 300, 64, 65, 128, 129, 192, 513]


@gpu
@pytest.mark.parametrize("compute", ["bf16", "mxfp8"])
def test_forward_ragged_tails_per_expert(compute):
    """Each expert's tokens (top-1, so an output row belongs to one expert) match the oracle on
    their own, so a wrong ragged tile cannot hide inside the layer-wide error."""
    m = need_gpu()
    cfg = cfg_small(T=sum(TAIL_COUNTS), H=256, I=384 if compute == "bf16" else 256, E=8, k=1)
    log(f"fwd ragged tails {compute} counts={TAIL_COUNTS}")
    inp = _inputs(cfg, TAIL_COUNTS)
    out, _ = _run(m, inp, compute)
    idx = inp.topk_idx.numpy()
    ref = mlp.forward(inp.x, idx, inp.topk_prob, inp.w1, inp.w2, compute, cfg.x_dtype)
    got = to_np(out)
    tol = BF16_TOL if compute == "bf16" else MXFP8_TOL
    for e in range(cfg.E):
        rows = np.nonzero(idx[:, 0] == e)[0]
        assert len(rows) == TAIL_COUNTS[e]
        err = mlp.normwise_rel_err(got[rows], ref.out[rows])
        log(f"  expert {e} ({len(rows)} rows) err {err:.3e}")
        assert err < tol


@gpu
@pytest.mark.parametrize("compute", ["bf16", "mxfp8"])
def test_forward_split_last_round(compute):
    """Down-projection tiles of the last, partly filled round are split along K and summed by
    the fixup pass: 24 M-blocks x 12 N-tiles = 288 tiles over 256 workgroups, the 32 tiles of
    that round all belong to the last expert.  The oracle runs experts 3 and 7 (tokens routed
    to both are compared) -- every expert's arithmetic is the same."""
    m = need_gpu()
    counts = [600, 700, 768, 514, 640, 520, 700, 600]     # 3 M-blocks of 256 rows each
    cfg = cfg_small(T=sum(counts) // 2, H=3072, I=4096, E=8, k=2)
    log(f"fwd split-tail {compute} T={cfg.T} H={cfg.H} I={cfg.I}")
    inp = _inputs(cfg, counts)
    out, ctx = _run(m, inp, compute)
    idx = inp.topk_idx.numpy()
    experts = (3, 7)
    rows = np.all(np.isin(idx, experts), axis=1)
    assert rows.sum() >= 16
    ref = mlp.forward(inp.x, idx, inp.topk_prob, inp.w1, inp.w2, compute, cfg.x_dtype, experts=experts)
    err = mlp.normwise_rel_err(to_np(out)[rows], ref.out[rows])
    tol = BF16_TOL if compute == "bf16" else MXFP8_TOL
    log(f"  {rows.sum()} tokens, normwise err {err:.3e} (tol {tol})")
    assert err < tol


@gpu
@pytest.mark.parametrize("compute", ["bf16", "mxfp8"])
def test_forward_split_last_round_short_k(compute):
    """Short K with a nearly empty last round (the 64-expert layer's FC2 shape): K = I = 1408 is
    11 MXFP8 stages (its E8M0 rows are not whole 16-byte groups, the four-lane scale loads) or
    22 BF16 ones, and 130 M-blocks x 2 N-tiles = 260 tiles leave 4 for the last round, which
    runs unsplit (K is too short for parts of kMinSplitUnits stages).  Experts 3 and 7 (the
    last tiles are expert 7's; the routing pairs them) are compared."""
    m = need_gpu()
    counts = [4096] * 6 + [4100, 4100]                    # 16 x 6 + 17 x 2 = 130 M-blocks
    cfg = cfg_small(T=sum(counts) // 2, H=512, I=1408, E=8, k=2)
    log(f"fwd short-K split-tail {compute} T={cfg.T} H={cfg.H} I={cfg.I}")
    inp = _inputs(cfg, counts)
    out, ctx = _run(m, inp, compute)
    idx = inp.topk_idx.numpy()
    experts = (3, 7)
    rows = np.all(np.isin(idx, experts), axis=1)
    assert rows.sum() >= 1024
    ref = mlp.forward(inp.x, idx, inp.topk_prob, inp.w1, inp.w2, compute, cfg.x_dtype, experts=experts)
    err = mlp.normwise_rel_err(to_np(out)[rows], ref.out[rows])
    tol = BF16_TOL if compute == "bf16" else MXFP8_TOL
    log(f"  {rows.sum()} tokens, normwise err {err:.3e} (tol {tol})")
    assert err < tol


def _fused_h_check(m, inp):
    """Forward with the FC1 epilogue's debug outputs: the E4M3 codes and E8M0 scales its fused
    quantizer wrote must be the oracle quantizer's bytes for the kernel's own fp32 h (one
    result exists for a given input).  Returns (the kernel's fp32 h, its codes)."""
    d = inp.to("cuda")
    out, ctx = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "mxfp8", debug_h=True)
    plain, _ = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "mxfp8")
    torch.cuda.synchronize()
    # FC2 read the caller's code buffers: the output is the production call's, bit for bit
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                       plain.view(torch.int16) if plain.dtype == torch.bfloat16 else plain.view(torch.int32))
    dbg = ctx["debug"]
    h32 = dbg["h_f32"].cpu().numpy().astype(np.float64)
    codes = dbg["h_codes"].cpu().numpy()
    scales = dbg["h_scales"].cpu().numpy()
    rc, rs = nm.quantize_mxfp8(h32, axis=1)
    np.testing.assert_array_equal(scales, rs)
    np.testing.assert_array_equal(codes, rc)
    return h32, codes


@gpu
@pytest.mark.parametrize("name,cfg,counts", CASES, ids=[c[0] for c in CASES])
def test_fused_h_quantizer_bytes(name, cfg, counts):
    """The fused MXFP8 quantizer of h in the FC1 epilogue, byte for byte against the oracle's
    quantizer applied to the epilogue's own fp32 h."""
    m = need_gpu()
    if cfg.H % 128 or cfg.I % 128:
        pytest.skip("MXFP8 path needs H, I multiples of 128")
    log(f"fused h quantizer {name} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}")
    inp = _inputs(cfg, counts)
    h32, codes = _fused_h_check(m, inp)
    ref = mlp.forward(inp.x, inp.topk_idx.numpy(), inp.topk_prob, inp.w1, inp.w2, "mxfp8", cfg.x_dtype)
    # the kernel's fp32 h against the oracle's fp64 h (same operands; fp32 vs fp64 arithmetic).
    # Codes of the oracle's fp64 h are only counted, not compared: the last bits of h differ, so
    # a value at a rounding tie may land on either side.
    err = mlp.normwise_rel_err(h32, ref.h)
    oc, _ = nm.quantize_mxfp8(ref.h, axis=1)
    flips = int(np.count_nonzero(oc != codes))
    log(f"  bytes equal; h fp32 vs fp64 err {err:.2e}; codes differing from Q(fp64 h): {flips} of {codes.size}")
    # fp32 accumulation and the hardware exp / reciprocal against fp64: ~1e-5 relative here; a wrong
    # side output would be off by O(1)
    assert err < 1e-3


@gpu
def test_forward_cached_mxfp8_weights_equal_per_call_quantization():
    """Weights quantized once (quantize_weights) give bit-identical outputs to the per-call
    quantization, in the grouped and the per-expert-loop forward."""
    m = need_gpu()
    cfg = cfg_small(T=600, H=256, I=256, E=8, k=2)
    log("fwd cached MXFP8 weights")
    inp = make_inputs(cfg)
    d = inp.to("cuda")
    wq = m.quantize_weights(d.w1, d.w2)
    a, _ = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "mxfp8")
    b, _ = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "mxfp8", w_quant=wq)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # the oracle's weight bytes are the cached ones, for every expert and both projections
    for e in range(cfg.E):
        c1, s1 = nm.quantize_mxfp8(inp.w1[e].to(torch.float64).numpy(), axis=1)
        c2, s2 = nm.quantize_mxfp8(inp.w2[e].to(torch.float64).numpy(), axis=1)
        np.testing.assert_array_equal(wq[0][e].cpu().numpy(), c1)
        np.testing.assert_array_equal(wq[1][e].cpu().numpy(), s1)
        np.testing.assert_array_equal(wq[2][e].cpu().numpy(), c2)
        np.testing.assert_array_equal(wq[3][e].cpu().numpy(), s2)


@gpu
def test_weight_quantizer_tables():
    """mxfp8_quantize_weights (the kernels the forward and backward run per call on their weight
    tables): row-wise and transposed column-wise bytes of every matrix against the oracle, and
    matrices whose skip entry is 0 left untouched."""
    m = need_gpu()
    log("weight quantizer tables")
    g = np.random.default_rng(31)
    E, rows, cols = 5, 352, 192
    w = torch.from_numpy(g.standard_normal((E, rows, cols)).astype(np.float32) * 0.02).to(torch.bfloat16)
    w[2, 5:37] = 0.0          # all-zero blocks along both axes
    w[3] *= 1e-30             # subnormal-range values (bf16 keeps the fp32 exponent range)
    dw = w.to("cuda")
    skip = torch.tensor([1, 0, 3, 1, 0], dtype=torch.int32, device="cuda")
    q0, s0 = m.mxfp8_quantize_weights(dw, axis=0)
    q1, s1 = m.mxfp8_quantize_weights(dw, axis=1)
    q2, s2 = m.mxfp8_quantize_weights([dw[e] for e in range(E)], axis=1, skip=skip)
    torch.cuda.synchronize()
    for e in range(E):
        we = w[e].to(torch.float64).numpy()
        rc, rs = nm.quantize_mxfp8(we, axis=1)
        np.testing.assert_array_equal(q0[e].cpu().numpy(), rc)
        np.testing.assert_array_equal(s0[e].cpu().numpy(), rs)
        cc, cs = nm.quantize_mxfp8(we, axis=0)             # blocks along rows, [rows, cols/..]
        np.testing.assert_array_equal(q1[e].cpu().numpy(), cc.T)
        np.testing.assert_array_equal(s1[e].cpu().numpy(), cs.T)
        if skip[e].item() == 0:
            assert int(q2[e].count_nonzero()) == 0 and int(s2[e].count_nonzero()) == 0
        else:
            np.testing.assert_array_equal(q2[e].cpu().numpy(), cc.T)
            np.testing.assert_array_equal(s2[e].cpu().numpy(), cs.T)


@gpu
def test_forward_deterministic():
    m = need_gpu()
    log("fwd determinism")
    cfg = cfg_small(T=700, H=256, I=384, E=4, k=2)
    inp = make_inputs(cfg)
    for compute in ("bf16", "mxfp8"):
        if compute == "mxfp8":
            cfg2 = cfg.with_(I=256)
            inp = make_inputs(cfg2)
        a, _ = _run(m, inp, compute)
        b, _ = _run(m, inp, compute)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@gpu
def test_forward_rejects_bad_shapes():
    m = need_gpu()
    log("fwd error paths")
    cfg = cfg_small(T=64, H=96, I=128, E=2, k=1)   # H % 64 != 0
    inp = make_inputs(cfg).to("cuda")
    with pytest.raises(m.MoeError) as ei:
        m.moe_grouped_mlp_fwd(inp.x, inp.topk_idx, inp.topk_prob, inp.w1, inp.w2, "bf16")
    assert ei.value.status == 2
