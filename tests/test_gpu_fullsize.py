"""GPU parity at the benchmark's full sizes, through the same entry points bench.py times.

The oracle runs on a subset of experts (the same per-expert arithmetic), and every
output that depends only on that subset is compared:
  * forward: out[t] for tokens whose k experts are all in the subset;
  * backward: dX[t] and dprob[t, :] for such tokens, and dW1_e, dW2_e of the subset
    experts in full;
  * bit-exact at full size: the permutation (all indices, split_sizes), the MXFP8 bytes
    of every permuted row of X, and the MXFP8 bytes of one expert's weights.
"""
import numpy as np
import pytest
import torch

from gpu_util import BF16_TOL, MXFP8_TOL, gpu, log, need_gpu, to_np
from moe_inputs import get_config, make_inputs
from oracle import mlp
from oracle import numerics as nm
from oracle.permute import permute as oracle_permute

slow = pytest.mark.slow


def _covered(idx, experts):
    return np.all(np.isin(idx, list(experts)), axis=1)


@gpu
@slow
@pytest.mark.timeout(900)
# The last expert's down-projection tiles fill the GEMM's last, partly occupied round, where
# they are split along K and finished by the fixup pass: each subset includes that expert.
# The per-tensor FP8 case runs the MXFP8 workload's inputs with one scale per operand tensor.
@pytest.mark.parametrize("ci,experts,prec", [(2, (0, 7), None), (3, (4, 5, 6, 7), None), (3, (4, 5, 6, 7), "fp8")],
                         ids=["mixtral-bf16", "mixtral-mxfp8-zipf", "mixtral-fp8-tensor-zipf"])
def test_fullsize_forward(ci, experts, prec):
    m = need_gpu()
    cfg = get_config(ci)
    if prec is not None:
        cfg = cfg.with_(precision=prec)
    log(f"full-size fwd {cfg.name}: generating inputs")
    inp = make_inputs(cfg)
    d = inp.to("cuda")
    out, ctx = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, cfg.precision)
    torch.cuda.synchronize()
    idx = inp.topk_idx.numpy()
    ref_perm = oracle_permute(idx, cfg.E)
    for key in ("split_sizes", "offsets", "row_id_map", "src_index"):
        np.testing.assert_array_equal(ctx["perm"][key].cpu().numpy(), getattr(ref_perm, key))
    if cfg.zero_expert is not None:
        assert ref_perm.split_sizes[cfg.zero_expert] == 0
    log(f"  oracle on experts {experts}")
    fw = mlp.forward(inp.x, idx, inp.topk_prob, inp.w1, inp.w2, cfg.precision, cfg.x_dtype, experts=experts)
    rows = _covered(idx, experts)
    assert rows.sum() >= 16, rows.sum()
    err = mlp.normwise_rel_err(to_np(out)[rows], fw.out[rows])
    tol = BF16_TOL if cfg.precision == "bf16" else MXFP8_TOL
    log(f"  {cfg.precision}: {rows.sum()} tokens compared, normwise err {err:.3e} (tol {tol})")
    assert err < tol


@gpu
@slow
@pytest.mark.timeout(900)
def test_fullsize_finegrained_forward_sampled_tokens():
    m = need_gpu()
    cfg = get_config(5)
    log(f"full-size fwd {cfg.name}: generating inputs")
    inp = make_inputs(cfg)
    d = inp.to("cuda")
    out, ctx = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, cfg.precision)
    torch.cuda.synchronize()
    idx = inp.topk_idx.numpy()
    np.testing.assert_array_equal(ctx["perm"]["split_sizes"].cpu().numpy(), np.bincount(idx.ravel(), minlength=cfg.E))
    tokens = [0, 1, 2, cfg.T // 2, cfg.T - 1]
    log(f"  oracle on tokens {tokens}")
    ref = mlp.forward_tokens(inp.x, idx, inp.topk_prob, inp.w1, inp.w2, tokens, cfg.precision, cfg.x_dtype)
    err = mlp.normwise_rel_err(to_np(out)[tokens], ref)
    log(f"  normwise err {err:.3e} (tol {MXFP8_TOL})")
    assert err < MXFP8_TOL


@gpu
@slow
@pytest.mark.timeout(900)
def test_fullsize_mxfp8_bytes():
    """Permuted X rows and one expert's weights quantized by the kernels the MXFP8 layer runs."""
    m = need_gpu()
    cfg = get_config(3)
    log("full-size MXFP8 bytes: generating inputs")
    inp = make_inputs(cfg)
    d = inp.to("cuda")
    res = m.moe_permute(d.x, d.topk_idx, d.topk_prob, cfg.E, "mxfp8")
    torch.cuda.synchronize()
    ref = oracle_permute(inp.topk_idx.numpy(), cfg.E)
    c, s = nm.quantize_mxfp8(inp.x.to(torch.float64).numpy(), axis=1)
    tok = ref.token_of_row
    np.testing.assert_array_equal(res["x_perm"].cpu().numpy(), c[tok])
    np.testing.assert_array_equal(res["x_perm_scales"].cpu().numpy(), s[tok])
    e = 6
    log(f"  weights of expert {e}")
    q1, s1 = m.mxfp8_quantize(d.w1[e], axis=0)
    rc, rs = nm.quantize_mxfp8(inp.w1[e].to(torch.float64).numpy(), axis=1)
    np.testing.assert_array_equal(q1.cpu().numpy(), rc)
    np.testing.assert_array_equal(s1.cpu().numpy(), rs)


@gpu
@slow
@pytest.mark.timeout(900)
def test_fullsize_fp8_tensor_bytes():
    """The per-tensor FP8 quantizer over the bf16 permuted rows of the MXFP8 workload, one
    tensor per expert segment (the empty expert included): codes and scales byte for byte."""
    m = need_gpu()
    cfg = get_config(3)
    log("full-size per-tensor FP8 bytes: generating inputs")
    inp = make_inputs(cfg)
    d = inp.to("cuda")
    res = m.moe_permute(d.x, d.topk_idx, d.topk_prob, cfg.E, "bf16")
    q, s = m.fp8_tensor_quantize(res["x_perm"], res["offsets"])
    torch.cuda.synchronize()
    ref = oracle_permute(inp.topk_idx.numpy(), cfg.E)
    xp = inp.x.to(torch.float64).numpy()[ref.token_of_row]
    rc, rs = nm.quantize_fp8_segments(xp, ref.offsets)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rc)


@gpu
@slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("compute", ["bf16", "mxfp8"])
def test_fullsize_backward(compute):
    """The Mixtral backward at full size (T=8192, H=4096, I=14336, E=8, top-2), in both precisions
    the benchmark times; the oracle computes experts 0 and 1 (every MXFP8 block lies inside one
    expert's segment, so this subset is exact for the oracle too)."""
    m = need_gpu()
    cfg = get_config(4)
    experts = (0, 1)
    log(f"full-size bwd {cfg.name} {compute}: generating inputs")
    inp = make_inputs(cfg)
    d = inp.to("cuda")
    out, ctx = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, compute, save_for_backward=True)
    dx, dprob, dw1, dw2 = m.moe_grouped_mlp_bwd(d.dy, ctx, d.w1, d.w2)
    torch.cuda.synchronize()
    idx = inp.topk_idx.numpy()
    log(f"  oracle on experts {experts}")
    fw = mlp.forward(inp.x, idx, inp.topk_prob, inp.w1, inp.w2, compute, cfg.x_dtype, experts=experts)
    bw = mlp.backward(fw, inp.x, inp.dy, inp.w1, inp.w2, experts=experts)
    rows = _covered(idx, experts)
    errs = {
        "dx": mlp.normwise_rel_err(to_np(dx)[rows], bw.dx[rows]),
        "dprob": mlp.normwise_rel_err(to_np(dprob)[rows], bw.dprob[rows]),
    }
    for e in experts:
        errs[f"dw1[{e}]"] = mlp.normwise_rel_err(to_np(dw1[e]), bw.dw1[e])
        errs[f"dw2[{e}]"] = mlp.normwise_rel_err(to_np(dw2[e]), bw.dw2[e])
    log(f"  {rows.sum()} tokens; " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    tol = BF16_TOL if compute == "bf16" else MXFP8_TOL
    for k, v in errs.items():
        assert v < tol, (k, v)
