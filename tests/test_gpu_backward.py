"""GPU parity: grouped MLP backward (dX, dprob, dW1, dW2) against the fp64 oracle.

Normwise relative error per tensor: 5e-3 (BF16), 2e-2 (MXFP8).  Experts with no
tokens must get dW exactly zero.
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
    ("cfg1-tiny-f32io", get_config(1), None),
    ("ragged-bf16", cfg_small(T=700, H=256, I=384, E=4, k=2), None),
    ("zeros-first-middle-last", cfg_small(T=400, H=128, I=256, E=8, k=2), [0, 400, 1, 31, 0, 33, 335, 0]),
    ("edge-sizes", cfg_small(T=600, H=128, I=128, E=7, k=2), [255, 257, 1, 31, 33, 600, 23]),
    ("one-expert", cfg_small(T=300, H=128, I=128, E=1, k=1), None),
    # 8 FC1-dgrad tiles with a long K: the last (only) round is split into K parts (4 for BF16,
    # 2 for MXFP8) that a fixup kernel sums
    ("split-k-dgrad", cfg_small(T=600, H=256, I=2048, E=4, k=2), None),
    ("finegrained-e64-k8", get_config(5).with_(T=512, H=256, I=256, precision="bf16"), None),
    ("zipf-zero-expert", get_config(3).with_(T=1024, H=256, I=384, precision="bf16"), None),
    # MXFP8 dgrads in the deep pipeline (K % 512 == 0): FC2 dgrad K = H = 512 (one scale group),
    # FC1 dgrad K = 2I = 1536 (three groups), an empty expert first
    ("deep-mx-dgrad", cfg_small(T=700, H=512, I=768, E=4, k=2), [0, 500, 699, 201]),
    # FC1 dgrad K = 4608 (36 stages) split in 2 parts: the second part starts at stage 18, inside
    # a scale group
    ("deep-mx-split-odd", cfg_small(T=640, H=1024, I=2304, E=3, k=2), None),
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
        return make_inputs(cfg, with_dy=True)
    idx, pr = routing_with_counts(counts, cfg.T, cfg.k, 5)
    return make_inputs(cfg, topk_idx=idx, topk_prob=pr, with_dy=True)


@gpu
@pytest.mark.parametrize("name,cfg,counts", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("compute", ["bf16", "mxfp8"])
def test_backward_matches_oracle(name, cfg, counts, compute):
    m = need_gpu()
    if compute == "mxfp8" and (cfg.H % 128 or cfg.I % 128):
        pytest.skip("MXFP8 path needs H, I multiples of 128")
    log(f"bwd {name} {compute} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}")
    inp = _inputs(cfg, counts)
    d = inp.to("cuda")
    out, ctx = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, compute, save_for_backward=True)
    dx, dprob, dw1, dw2 = m.moe_grouped_mlp_bwd(d.dy, ctx, d.w1, d.w2)
    torch.cuda.synchronize()
    fw = mlp.forward(inp.x, inp.topk_idx.numpy(), inp.topk_prob, inp.w1, inp.w2, compute, cfg.x_dtype)
    bw = mlp.backward(fw, inp.x, inp.dy, inp.w1, inp.w2)
    tol = BF16_TOL if compute == "bf16" else MXFP8_TOL
    errs = {
        "out": mlp.normwise_rel_err(to_np(out), fw.out),
        "dx": mlp.normwise_rel_err(to_np(dx), bw.dx),
        "dprob": mlp.normwise_rel_err(to_np(dprob), bw.dprob),
        "dw1": mlp.normwise_rel_err(to_np(dw1), bw.dw1),
        "dw2": mlp.normwise_rel_err(to_np(dw2), bw.dw2),
    }
    log("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k_, v in errs.items():
        assert v < tol, (k_, v)
    split = ctx["perm"]["split_sizes"].cpu().numpy()
    for e in np.nonzero(split == 0)[0]:
        assert torch.count_nonzero(dw1[e]).item() == 0 and torch.count_nonzero(dw2[e]).item() == 0


@gpu
def test_backward_deterministic():
    m = need_gpu()
    log("bwd determinism")
    cfg = cfg_small(T=700, H=256, I=256, E=4, k=2)
    d = make_inputs(cfg, with_dy=True).to("cuda")
    res = []
    for _ in range(2):
        out, ctx = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "bf16", save_for_backward=True)
        res.append(m.moe_grouped_mlp_bwd(d.dy, ctx, d.w1, d.w2))
    for a, b in zip(*res):
        assert torch.equal(a, b)


@gpu
def test_backward_cached_transposed_weights():
    """MXFP8 backward with the dgrad weights quantized once (quantize_weights(..., transposed=True))
    gives the same bits as the per-call quantization, which skips experts without tokens."""
    m = need_gpu()
    log("bwd cached transposed MXFP8 weights")
    cfg = cfg_small(T=400, H=128, I=256, E=8, k=2)
    inp = _inputs(cfg, [0, 400, 1, 31, 0, 33, 335, 0])
    d = inp.to("cuda")
    out, ctx = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "mxfp8", save_for_backward=True)
    a = m.moe_grouped_mlp_bwd(d.dy, ctx, d.w1, d.w2)
    wt = m.quantize_weights(d.w1, d.w2, "mxfp8", transposed=True)
    b = m.moe_grouped_mlp_bwd(d.dy, ctx, d.w1, d.w2, w_quant_t=wt)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@gpu
def test_forward_flag_survives_backward():
    """A forward's bad-expert-id flag lives in its own tensor: a backward that reuses the shared
    workspace afterwards does not change what it reads."""
    m = need_gpu()
    log("fwd flag after bwd")
    cfg = cfg_small(T=64, H=128, I=128, E=4, k=2)
    inp = make_inputs(cfg, with_dy=True)
    d = inp.to("cuda")
    bad = d.topk_idx.clone()
    bad[5, 1] = 9
    _, ctx_bad = m.moe_grouped_mlp_fwd(d.x, bad, d.topk_prob, d.w1, d.w2, "bf16")
    _, ctx = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "bf16", save_for_backward=True)
    m.moe_grouped_mlp_bwd(d.dy, ctx, d.w1, d.w2)
    assert m.moe_read_device_error(ctx_bad["error_flag"]) == 1
    assert m.moe_read_device_error(ctx["error_flag"]) == 0


def _check_fused_dgu(dbg, offsets, I, log_name):
    """The FC2 dgrad epilogue's MXFP8 dGU against the oracle's quantizer applied to the kernel's own
    bf16 dGU: row-wise along 2I, and along each expert's tokens in the 128-padded transposed layout
    (the 32-padded oracle layout, each segment moved to its 128-aligned start, zeros up to it), with
    the scale bytes past the last segment zero."""
    dgu = dbg["dgu_bf16"].cpu().to(torch.float64).numpy()
    rc, rs = nm.quantize_mxfp8(dgu, axis=1)
    np.testing.assert_array_equal(dbg["dgu_codes"].cpu().numpy(), rc)
    np.testing.assert_array_equal(dbg["dgu_scales"].cpu().numpy(), rs)
    tc, ts = nm.quantize_mxfp8_segments_t(dgu, offsets)
    gq, gs = dbg["dgu_t_codes"].cpu().numpy(), dbg["dgu_t_scales"].cpu().numpy()
    p32 = p128 = 0
    for e in range(len(offsets) - 1):
        me = int(offsets[e + 1] - offsets[e])
        n32, n128 = (me + 31) // 32 * 32, (me + 127) // 128 * 128
        np.testing.assert_array_equal(gq[:, p128:p128 + n32], tc[:, p32:p32 + n32], err_msg=f"codes e={e}")
        np.testing.assert_array_equal(gs[:, p128 // 32:(p128 + n32) // 32], ts[:, p32 // 32:(p32 + n32) // 32],
                                      err_msg=f"scales e={e}")
        assert not gq[:, p128 + n32:p128 + n128].any() and not gs[:, (p128 + n32) // 32:(p128 + n128) // 32].any()
        p32 += n32
        p128 += n128
    assert not gs[:, p128 // 32:].any()
    log(f"  {log_name}: fused dGU quantizer bytes equal (rows {dgu.shape[0]}, 2I {2 * I}, segment end {p128})")


@gpu
@pytest.mark.parametrize("name,cfg,counts", [c for c in CASES if c[1].H % 128 == 0 and c[1].I % 128 == 0],
                         ids=[c[0] for c in CASES if c[1].H % 128 == 0 and c[1].I % 128 == 0])
def test_fused_dgu_quantizer_bytes(name, cfg, counts):
    """MXFP8: the dGU bytes the FC2 dgrad epilogue writes for both FC1 GEMMs are bit-exact against
    the oracle's OCP quantizer of the epilogue's own bf16 dGU; that bf16 dGU is within the MXFP8
    tolerance of the oracle's."""
    m = need_gpu()
    log(f"fused dGU quantizer {name} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}")
    inp = _inputs(cfg, counts)
    d = inp.to("cuda")
    out, ctx = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "mxfp8", save_for_backward=True)
    dbg = {}
    m.moe_grouped_mlp_bwd(d.dy, ctx, d.w1, d.w2, debug=dbg)
    torch.cuda.synchronize()
    offsets = ctx["perm"]["offsets"].cpu().numpy()
    _check_fused_dgu(dbg, offsets, cfg.I, name)
    fw = mlp.forward(inp.x, inp.topk_idx.numpy(), inp.topk_prob, inp.w1, inp.w2, "mxfp8", cfg.x_dtype)
    bw = mlp.backward(fw, inp.x, inp.dy, inp.w1, inp.w2)
    err = mlp.normwise_rel_err(dbg["dgu_bf16"].cpu().to(torch.float64).numpy(), bw.dgu)
    log(f"  dgu vs oracle {err:.2e}")
    assert err < MXFP8_TOL


@gpu
@pytest.mark.parametrize("name,cfg,counts", [CASES[2], CASES[7]], ids=[CASES[2][0], CASES[7][0]])
def test_forward_quantizes_weights_for_backward(name, cfg, counts):
    """MXFP8 training: the forward's one read of the bf16 weights for both orientations gives the
    same forward output, bit for bit, and the same transposed bytes as mxfp8_quantize_weights (axis
    1) for every expert with tokens; the backward that takes them equals the one that quantizes per
    call, bit for bit."""
    m = need_gpu()
    log(f"forward quantizes W^T for the backward: {name}")
    inp = _inputs(cfg, counts)
    d = inp.to("cuda")
    out1, ctx1 = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "mxfp8", save_for_backward=True)
    out0, ctx0 = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "mxfp8", save_for_backward=True,
                                       quantize_for_backward=False)
    assert ctx1["w_quant_t"] is not None and ctx0["w_quant_t"] is None
    g1 = m.moe_grouped_mlp_bwd(d.dy, ctx1, d.w1, d.w2)
    g0 = m.moe_grouped_mlp_bwd(d.dy, ctx0, d.w1, d.w2)
    ref = m.quantize_weights(d.w1, d.w2, "mxfp8", transposed=True)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out0.view(torch.int16))
    split = ctx1["perm"]["split_sizes"].cpu().numpy()
    for t_fwd, t_ref in zip(ctx1["w_quant_t"], ref):
        for e in np.nonzero(split > 0)[0]:
            assert torch.equal(t_fwd[e], t_ref[e]), e
    for a_, b_ in zip(g1, g0):
        assert torch.equal(a_, b_)
