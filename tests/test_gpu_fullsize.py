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


def _finegrained_sample(idx, E, T, total=512, seed=0):
    """Tokens whose outputs are compared for the 64-expert layer: for every expert, the tokens of
    the first row of its segment, of the first row of its last 256-row tile and of its last row
    (rows in a segment ascend with the token index), topped up with random tokens to `total`."""
    ref = oracle_permute(idx, E)
    toks = set()
    for e in range(E):
        lo, hi = int(ref.offsets[e]), int(ref.offsets[e + 1])
        if hi == lo:
            continue
        last_tile = lo + (hi - lo - 1) // 256 * 256
        for r in (lo, last_tile, hi - 1):
            toks.add(int(ref.token_of_row[r]))
    g = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(T), np.array(sorted(toks)))
    toks.update(int(t) for t in g.choice(rest, size=max(0, total - len(toks)), replace=False))
    return sorted(toks)


@gpu
@slow
@pytest.mark.timeout(900)
def test_fullsize_finegrained_forward_sampled_tokens():
    """The 64-expert top-8 MXFP8 layer at full size: at least 512 tokens, covering the first and
    last row of every expert and the first row of its last tile, against the oracle token by
    token (every rounding step of that layer acts within one row, so a token's output needs
    only its own row)."""
    m = need_gpu()
    cfg = get_config(5)
    log(f"full-size fwd {cfg.name}: generating inputs")
    inp = make_inputs(cfg)
    d = inp.to("cuda")
    out, ctx = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, cfg.precision)
    torch.cuda.synchronize()
    idx = inp.topk_idx.numpy()
    np.testing.assert_array_equal(ctx["perm"]["split_sizes"].cpu().numpy(), np.bincount(idx.ravel(), minlength=cfg.E))
    tokens = _finegrained_sample(idx, cfg.E, cfg.T)
    assert len(tokens) >= 512
    covered = np.unique(idx[tokens])
    assert len(covered) == int((np.bincount(idx.ravel(), minlength=cfg.E) > 0).sum())
    log(f"  oracle on {len(tokens)} tokens covering {len(covered)} experts")
    ref = mlp.forward_tokens(inp.x, idx, inp.topk_prob, inp.w1, inp.w2, tokens, cfg.precision, cfg.x_dtype)
    got = to_np(out)[tokens]
    err = mlp.normwise_rel_err(got, ref)
    worst = max(mlp.normwise_rel_err(got[i], ref[i]) for i in range(len(tokens)))
    log(f"  normwise err {err:.3e}, worst single token {worst:.3e} (tol {MXFP8_TOL})")
    assert err < MXFP8_TOL


@gpu
@slow
@pytest.mark.timeout(900)
def test_fullsize_mxfp8_bytes():
    """Every permuted X row of the MXFP8 workload, byte for byte (the permutation's fused row
    quantizer)."""
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


def _oracle_rows(w, axis, chunk=2048):
    """The oracle's MXFP8 of a bf16 matrix (axis 1: blocks along each row; axis 0: along each
    column), a band of rows (axis 1) or columns (axis 0) at a time to bound host memory."""
    w64 = w.to(torch.float64).numpy() if hasattr(w, "numpy") else w
    if axis == 1:
        parts = [nm.quantize_mxfp8(w64[r:r + chunk], axis=1) for r in range(0, w64.shape[0], chunk)]
        return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])
    parts = [nm.quantize_mxfp8(w64[:, c:c + chunk], axis=0) for c in range(0, w64.shape[1], chunk)]
    return np.concatenate([p[0] for p in parts], axis=1), np.concatenate([p[1] for p in parts], axis=1)


@gpu
@slow
@pytest.mark.timeout(900)
def test_fullsize_weight_quantizer_bytes():
    """The weight quantizer the MXFP8 layer runs on every call (mxfp8_quantize_weights, which the
    forward's per-call path and quantize_weights share): every expert's W1 and W2 at the Mixtral
    shape row-wise, as the forward GEMMs read them; and the backward's transposed, column-wise
    W1^T / W2^T of two experts."""
    m = need_gpu()
    cfg = get_config(3)
    log("full-size weight quantizer bytes: generating inputs")
    inp = make_inputs(cfg)
    d = inp.to("cuda")
    w1q, w1s, w2q, w2s = m.quantize_weights(d.w1, d.w2, "mxfp8")
    torch.cuda.synchronize()
    for e in range(cfg.E):
        log(f"  expert {e}: W1 [{2 * cfg.I}, {cfg.H}] and W2 [{cfg.H}, {cfg.I}] row-wise")
        for got_q, got_s, w in ((w1q[e], w1s[e], inp.w1[e]), (w2q[e], w2s[e], inp.w2[e])):
            rc, rs = _oracle_rows(w, axis=1)
            np.testing.assert_array_equal(got_s.cpu().numpy(), rs)
            np.testing.assert_array_equal(got_q.cpu().numpy(), rc)
    del w1q, w1s, w2q, w2s
    t1q, t1s, t2q, t2s = m.quantize_weights(d.w1, d.w2, "mxfp8", transposed=True)
    torch.cuda.synchronize()
    for e in (0, 5):
        log(f"  expert {e}: W1^T and W2^T column-wise (backward operands)")
        for got_q, got_s, w in ((t1q[e], t1s[e], inp.w1[e]), (t2q[e], t2s[e], inp.w2[e])):
            rc, rs = _oracle_rows(w, axis=0)
            np.testing.assert_array_equal(got_s.cpu().numpy(), rs.T)
            np.testing.assert_array_equal(got_q.cpu().numpy(), rc.T)


@gpu
@slow
@pytest.mark.timeout(900)
def test_fullsize_fused_h_quantizer_bytes():
    """The FC1 epilogue's fused MXFP8 quantizer of h at the full Mixtral MXFP8 workload (T=8192,
    Zipf routing), byte for byte against the oracle's quantizer on the kernel's fp32 h, for the
    rows of expert 6 (and the row count of every expert's h)."""
    m = need_gpu()
    cfg = get_config(3)
    log("full-size fused h quantizer: generating inputs")
    inp = make_inputs(cfg)
    d = inp.to("cuda")
    out, ctx = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "mxfp8", debug_h=True)
    torch.cuda.synchronize()
    off = ctx["perm"]["offsets"].cpu().numpy()
    e = 6
    lo, hi = int(off[e]), int(off[e + 1])
    dbg = ctx["debug"]
    h32 = dbg["h_f32"][lo:hi].cpu().numpy().astype(np.float64)
    rc, rs = nm.quantize_mxfp8(h32, axis=1)
    log(f"  expert {e}: {hi - lo} rows x {cfg.I}")
    np.testing.assert_array_equal(dbg["h_scales"][lo:hi].cpu().numpy(), rs)
    np.testing.assert_array_equal(dbg["h_codes"][lo:hi].cpu().numpy(), rc)
    # the kernel's h against the oracle's for the same expert
    fw = mlp.forward(inp.x, inp.topk_idx.numpy(), inp.topk_prob, inp.w1, inp.w2, "mxfp8", cfg.x_dtype,
                     experts=(e,))
    err = mlp.normwise_rel_err(h32, fw.h[lo:hi])
    flips = int(np.count_nonzero(nm.quantize_mxfp8(fw.h[lo:hi], axis=1)[0] != rc))
    log(f"  h fp32 vs fp64 err {err:.2e}; codes differing from Q(fp64 h): {flips} of {rc.size}")
    # fp32 accumulation and the hardware exp / reciprocal against fp64: ~1e-5 relative here; a wrong
    # side output would be off by O(1)
    assert err < 1e-3


@gpu
@slow
@pytest.mark.timeout(900)
def test_fullsize_fused_dgu_quantizer_bytes():
    """The FC2 dgrad epilogue's fused MXFP8 quantizer of dGU at the full Mixtral backward (T=8192,
    H=4096, I=14336, E=8 top-2), byte for byte against the oracle's quantizer on the kernel's bf16
    dGU, for the rows of the first and the last expert: row-wise along 2I, and along the tokens of
    each of the two segments in the 128-padded transposed layout."""
    m = need_gpu()
    cfg = get_config(4)
    log("full-size fused dGU quantizer: generating inputs")
    inp = make_inputs(cfg)
    d = inp.to("cuda")
    out, ctx = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, "mxfp8", save_for_backward=True)
    dbg = {}
    m.moe_grouped_mlp_bwd(d.dy, ctx, d.w1, d.w2, debug=dbg)
    torch.cuda.synchronize()
    off = ctx["perm"]["offsets"].cpu().numpy().astype(np.int64)
    pad = np.concatenate([[0], np.cumsum((np.diff(off) + 127) // 128 * 128)])
    for e in (0, cfg.E - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        g = dbg["dgu_bf16"][lo:hi].cpu().to(torch.float64).numpy()
        rc, rs = nm.quantize_mxfp8(g, axis=1)
        np.testing.assert_array_equal(dbg["dgu_codes"][lo:hi].cpu().numpy(), rc)
        np.testing.assert_array_equal(dbg["dgu_scales"][lo:hi].cpu().numpy(), rs)
        tc, ts = nm.quantize_mxfp8_segments_t(g, np.array([0, hi - lo]))
        n32 = tc.shape[1]
        p0 = int(pad[e])
        np.testing.assert_array_equal(dbg["dgu_t_codes"][:, p0:p0 + n32].cpu().numpy(), tc)
        np.testing.assert_array_equal(dbg["dgu_t_scales"][:, p0 // 32:(p0 + n32) // 32].cpu().numpy(), ts)
        log(f"  expert {e}: {hi - lo} rows x {2 * cfg.I}, both layouts equal")


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
