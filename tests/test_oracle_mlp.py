"""Pins for the oracle's grouped MLP forward/backward (CPU only).

The oracle is compared with code that shares none of its structure:
  * a pure-Python scalar loop over tokens, slots and matrix entries (tiny shapes);
  * textbook dense special cases built from torch.nn.functional in fp64
    (one expert with p = 1 is a dense SwiGLU FFN; top-k = E with p = 1/E is a
    dense SwiGLU FFN over the concatenated experts scaled by 1/E);
  * central finite differences of the oracle's own forward (rounding off);
  * torch.autograd in fp64 on a gather formulation of the layer;
  * the identity dprob[t, j] = <dY_t, z_row> / p_row.
The rounding steps themselves are pinned in test_oracle_numerics.py.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from moe_inputs import get_config, make_inputs
from moe_inputs.generate import routing_with_counts
from oracle import mlp
from oracle import numerics as nm


def tiny(T=6, H=32, I=32, E=3, k=2, seed=11, x_dtype="bf16"):
    cfg = get_config(1).with_(T=T, H=H, I=I, E=E, k=k, x_dtype=x_dtype, seed=seed)
    return make_inputs(cfg, with_dy=True)


def scalar_forward(x, idx, prob, w1, w2, precision, io):
    """Per-token, per-slot, per-entry loops written straight from the definition."""
    T, H = x.shape
    k = idx.shape[1]
    I = w2.shape[2]

    def rnd_act(row):
        if precision == "exact":
            return list(row)
        if precision == "bf16":
            return list(nm.round_bf16(np.array(row)))
        return list(nm.fake_quant_mxfp8(np.array([row]), axis=1)[0])

    def rnd_w(mat):  # rows along K
        return mat if precision != "mxfp8" else nm.fake_quant_mxfp8(mat, axis=1)

    def rnd_io(v):
        if precision == "exact":
            return v
        return float(np.float32(v)) if io == "f32" else float(nm.round_bf16(v))

    out = np.zeros((T, H))
    for t in range(T):
        xr = rnd_act([float(v) for v in x[t]])
        acc = [0.0] * H
        for j in range(k):
            e = int(idx[t, j])
            p = float(prob[t, j])
            W1 = rnd_w(w1[e])
            W2 = rnd_w(w2[e])
            gate = [sum(xr[c] * W1[n, c] for c in range(H)) for n in range(I)]
            up = [sum(xr[c] * W1[I + n, c] for c in range(H)) for n in range(I)]
            hrow = [gate[n] / (1.0 + math.exp(-gate[n])) * up[n] * p for n in range(I)]
            hq = rnd_act(hrow)
            for o in range(H):
                acc[o] += rnd_io(sum(hq[n] * W2[o, n] for n in range(I)))
        out[t] = [rnd_io(v) for v in acc]
    return out


@pytest.mark.parametrize("precision,io", [("exact", "bf16"), ("bf16", "bf16"), ("bf16", "f32"),
                                          ("mxfp8", "bf16")])
def test_forward_matches_scalar_loop(precision, io):
    inp = tiny(x_dtype="f32" if io == "f32" else "bf16")
    x, w1, w2 = mlp.f64(inp.x), mlp.f64(inp.w1), mlp.f64(inp.w2)
    idx, prob = inp.topk_idx.numpy(), inp.topk_prob.numpy()
    fw = mlp.forward(inp.x, idx, inp.topk_prob, inp.w1, inp.w2, precision, io)
    ref = scalar_forward(x, idx, prob, w1, w2, precision, io)
    if precision == "exact":
        np.testing.assert_allclose(fw.out, ref, rtol=1e-12, atol=1e-15)
    else:
        # identical roundings; only fp64 summation order differs, which can flip
        # a final rounding on an exact tie -- allow at most one io ulp
        ulp = 2.0 ** -7 if io == "bf16" else 2.0 ** -23
        assert np.all(np.abs(fw.out - ref) <= ulp * np.abs(ref) + 1e-30)
        assert np.mean(fw.out == ref) > 0.97


def test_forward_tokens_matches_forward():
    for precision in ("bf16", "mxfp8"):
        inp = tiny(T=10, seed=12)
        fw = mlp.forward(inp.x, inp.topk_idx.numpy(), inp.topk_prob, inp.w1, inp.w2, precision, "bf16")
        sel = [0, 3, 9]
        got = mlp.forward_tokens(inp.x, inp.topk_idx.numpy(), inp.topk_prob, inp.w1, inp.w2, sel,
                                 precision, "bf16")
        np.testing.assert_array_equal(got, fw.out[sel])


def dense_swiglu(x, wg, wu, wd):
    """Textbook dense SwiGLU FFN: down(silu(gate(x)) * up(x)), torch fp64."""
    return F.linear(F.silu(F.linear(x, wg)) * F.linear(x, wu), wd)


def test_single_expert_is_dense_ffn():
    inp = tiny(T=9, E=1, k=1, seed=13)
    prob = np.ones((9, 1), dtype=np.float32)
    fw = mlp.forward(inp.x, inp.topk_idx.numpy(), prob, inp.w1, inp.w2, "exact", "bf16")
    x = inp.x.double()
    I = inp.w2.shape[2]
    ref = dense_swiglu(x, inp.w1[0, :I].double(), inp.w1[0, I:].double(), inp.w2[0].double()).numpy()
    np.testing.assert_allclose(fw.out, ref, rtol=1e-12, atol=1e-14)


def _all_experts_routing(T, E):
    idx = np.tile(np.arange(E, dtype=np.int32), (T, 1))
    prob = np.full((T, E), 1.0 / E, dtype=np.float32)
    return idx, prob


@pytest.mark.parametrize("E", [4, 8])
def test_topk_equals_E_is_scaled_dense_ffn(E):
    inp = tiny(T=8, E=E, k=E, seed=14)
    idx, prob = _all_experts_routing(8, E)
    I = inp.w2.shape[2]
    wg = torch.cat([inp.w1[e, :I] for e in range(E)]).double()
    wu = torch.cat([inp.w1[e, I:] for e in range(E)]).double()
    wd = torch.cat([inp.w2[e] for e in range(E)], dim=1).double()
    x = inp.x.double()
    # exact arithmetic
    fw = mlp.forward(inp.x, idx, prob, inp.w1, inp.w2, "exact", "bf16")
    ref = dense_swiglu(x, wg, wu, wd).numpy() / E
    np.testing.assert_allclose(fw.out, ref, rtol=1e-11, atol=1e-14)
    # MXFP8 with f32 I/O: 1/E is a power of two, so quantizing h/E only shifts
    # scales; the dense form with MXFP8 operands (h blocks of 32 along E*I
    # coincide with per-expert blocks because I % 32 == 0) must agree up to the
    # f32 rounding of each expert's output.
    fq = lambda t: torch.from_numpy(nm.fake_quant_mxfp8(t.numpy(), axis=1))
    xq = fq(x)
    h = F.silu(F.linear(xq, fq(wg))) * F.linear(xq, fq(wu))
    ref8 = F.linear(fq(h), fq(wd)).numpy() / E
    fw8 = mlp.forward(inp.x, idx, prob, inp.w1, inp.w2, "mxfp8", "f32")
    np.testing.assert_allclose(fw8.out, ref8, rtol=1e-5, atol=1e-7)


# ---------------------------------------------------------------------------- backward


def _loss(inp, x, prob, w1, w2, dy):
    fw = mlp.forward(x, inp.topk_idx.numpy(), prob, w1, w2, "exact", "bf16")
    return float(np.sum(fw.out * dy))


def test_backward_finite_differences():
    inp = tiny(T=5, H=32, I=32, E=3, k=2, seed=15)
    x, w1, w2 = mlp.f64(inp.x), mlp.f64(inp.w1), mlp.f64(inp.w2)
    prob, dy = mlp.f64(inp.topk_prob), mlp.f64(inp.dy)
    fw = mlp.forward(x, inp.topk_idx.numpy(), prob, w1, w2, "exact", "bf16")
    bw = mlp.backward(fw, x, dy, w1, w2)
    g = np.random.default_rng(0)
    eps = 1e-5
    for name, arr, grad in (("x", x, bw.dx), ("prob", prob, bw.dprob), ("w1", w1, bw.dw1), ("w2", w2, bw.dw2)):
        for _ in range(6):
            pos = tuple(int(g.integers(0, n)) for n in arr.shape)
            a0 = arr[pos]
            arr[pos] = a0 + eps
            lp = _loss(inp, x, prob, w1, w2, dy)
            arr[pos] = a0 - eps
            lm = _loss(inp, x, prob, w1, w2, dy)
            arr[pos] = a0
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)) + 1e-8, (name, pos, fd, grad[pos])


def test_backward_matches_torch_autograd():
    inp = tiny(T=7, H=32, I=64, E=4, k=2, seed=16)
    idx = inp.topk_idx.long()
    x = inp.x.double().requires_grad_()
    prob = inp.topk_prob.double().requires_grad_()
    w1 = inp.w1.double().requires_grad_()
    w2 = inp.w2.double().requires_grad_()
    dy = inp.dy.double()
    I = inp.w2.shape[2]
    W1 = w1[idx]                                   # [T,k,2I,H]
    gu = torch.einsum("tkoh,th->tko", W1, x)
    hh = F.silu(gu[..., :I]) * gu[..., I:] * prob[..., None]
    z = torch.einsum("tkhi,tki->tkh", w2[idx], hh)
    out = z.sum(1)
    (out * dy).sum().backward()
    fw = mlp.forward(inp.x, inp.topk_idx.numpy(), inp.topk_prob, inp.w1, inp.w2, "exact", "bf16")
    bw = mlp.backward(fw, inp.x, inp.dy, inp.w1, inp.w2)
    np.testing.assert_allclose(fw.out, out.detach().numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(bw.dx, x.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(bw.dprob, prob.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(bw.dw1, w1.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(bw.dw2, w2.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_dprob_identity():
    inp = tiny(T=8, seed=17)
    fw = mlp.forward(inp.x, inp.topk_idx.numpy(), inp.topk_prob, inp.w1, inp.w2, "exact", "bf16")
    bw = mlp.backward(fw, inp.x, inp.dy, inp.w1, inp.w2)
    dy = mlp.f64(inp.dy)
    T, k = inp.topk_idx.shape
    for t in range(T):
        for j in range(k):
            r = fw.perm.row_id_map[t * k + j]
            ref = float(dy[t] @ fw.z[r]) / float(inp.topk_prob[t, j])
            assert abs(bw.dprob[t, j] - ref) <= 1e-10 * max(1.0, abs(ref))


def test_zero_token_expert_gets_zero_weight_grad():
    T, k = 16, 2
    counts = [0, 16, 0, 16]
    idx, prob = routing_with_counts(counts, T, k, seed=3)
    inp = tiny(T=T, E=4, k=k, seed=18)
    for precision in ("bf16", "mxfp8"):
        fw = mlp.forward(inp.x, idx, prob, inp.w1, inp.w2, precision, "bf16")
        bw = mlp.backward(fw, inp.x, inp.dy, inp.w1, inp.w2)
        for e in (0, 2):
            assert np.all(bw.dw1[e] == 0) and np.all(bw.dw2[e] == 0)
        assert np.any(bw.dw1[1] != 0) and np.any(bw.dw2[3] != 0)


def scalar_backward(inp, precision):
    """Backward written per token and slot with explicit loops over the GEMM
    entries; MXFP8 (or bf16) rounding inserted at the points of the contract."""
    x, w1, w2 = mlp.f64(inp.x), mlp.f64(inp.w1), mlp.f64(inp.w2)
    prob, dy = mlp.f64(inp.topk_prob), mlp.f64(inp.dy)
    idx = inp.topk_idx.numpy()
    T, H = x.shape
    k = idx.shape[1]
    E, I = w1.shape[0], w2.shape[2]
    q_row = (lambda a: nm.fake_quant_mxfp8(a, axis=1)) if precision == "mxfp8" else (lambda a: a)
    rb = nm.round_bf16
    xb = rb(x)
    xop = q_row(xb) if precision == "mxfp8" else xb
    w1op = nm.fake_quant_mxfp8(w1, axis=2) if precision == "mxfp8" else w1
    w2op = nm.fake_quant_mxfp8(w2, axis=2) if precision == "mxfp8" else w2
    dx = np.zeros((T, H))
    dprob = np.zeros((T, k))
    dw1 = np.zeros_like(w1)
    dw2 = np.zeros_like(w2)
    # rows per expert, in ascending token order (needed for the token-axis blocks)
    rows = {e: [(t, j) for t in range(T) for j in range(k) if idx[t, j] == e] for e in range(E)}
    for e in range(E):
        if not rows[e]:
            continue
        M = len(rows[e])
        Xe = np.array([xop[t] for t, _ in rows[e]])
        Pe = np.array([prob[t, j] for t, j in rows[e]])
        GU = np.array([[sum(Xe[m, c] * w1op[e, n, c] for c in range(H)) for n in range(2 * I)] for m in range(M)])
        Hf = np.array([[GU[m, n] / (1 + math.exp(-GU[m, n])) * GU[m, I + n] * Pe[m] for n in range(I)]
                       for m in range(M)])
        GUs, Hs = rb(GU), rb(Hf)
        DZ = np.array([dy[t] for t, _ in rows[e]])
        DZq = q_row(DZ)
        W2k = nm.fake_quant_mxfp8(w2[e], axis=0) if precision == "mxfp8" else w2[e]   # blocks along H
        W1k = nm.fake_quant_mxfp8(w1[e], axis=0) if precision == "mxfp8" else w1[e]   # blocks along 2I
        DH = np.array([[sum(DZq[m, o] * W2k[o, n] for o in range(H)) for n in range(I)] for m in range(M)])
        DGU = np.zeros((M, 2 * I))
        for m in range(M):
            t, j = rows[e][m]
            acc = 0.0
            for n in range(I):
                g, u = GUs[m, n], GUs[m, I + n]
                s = 1 / (1 + math.exp(-g))
                acc += DH[m, n] * g * s * u
                da = DH[m, n] * Pe[m]
                DGU[m, I + n] = da * g * s
                DGU[m, n] = da * u * s * (1 + g * (1 - s))
            dprob[t, j] = np.float32(acc)
        DGU = rb(DGU)
        DGUq = q_row(DGU)
        DXP = DGUq @ W1k
        for m, (t, j) in enumerate(rows[e]):
            dx[t] += rb(DXP[m])

        def colq(a):
            if precision != "mxfp8":
                return a
            Mp = (a.shape[0] + 31) // 32 * 32
            p = np.zeros((Mp, a.shape[1]))
            p[:a.shape[0]] = a
            return nm.fake_quant_mxfp8(p, axis=0)[:a.shape[0]]

        A, B = colq(DGU), colq(np.array([xb[t] for t, _ in rows[e]]))
        dw1[e] = np.array([[sum(A[m, n] * B[m, c] for m in range(M)) for c in range(H)] for n in range(2 * I)])
        A2 = colq(DZ)
        B2 = colq(Hs if precision == "mxfp8" else rb(Hf))
        dw2[e] = np.array([[sum(A2[m, o] * B2[m, n] for m in range(M)) for n in range(I)] for o in range(H)])
    return rb(dx), dprob, dw1, dw2


@pytest.mark.parametrize("precision", ["bf16", "mxfp8"])
def test_backward_matches_scalar_loop(precision):
    inp = tiny(T=4, H=32, I=32, E=2, k=2, seed=19)
    fw = mlp.forward(inp.x, inp.topk_idx.numpy(), inp.topk_prob, inp.w1, inp.w2, precision, "bf16")
    bw = mlp.backward(fw, inp.x, inp.dy, inp.w1, inp.w2)
    dx, dprob, dw1, dw2 = scalar_backward(inp, precision)
    # sums run in a different order: allow one bf16 ulp on the rounded outputs
    assert np.all(np.abs(bw.dx - dx) <= 2 ** -7 * np.abs(dx) + 1e-30)
    np.testing.assert_allclose(bw.dprob, dprob, rtol=1e-6)
    np.testing.assert_allclose(bw.dw1, dw1, rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(bw.dw2, dw2, rtol=1e-9, atol=1e-15)


# ----------------------------------------------------------------------------- the tolerance metric

@pytest.mark.parametrize("got,ref,want", [
    # 3-4-5 triangle: the difference has norm 5, the reference norm 5 / 10 / 5
    ([0.0, 0.0], [3.0, 4.0], 1.0),
    ([9.0, 4.0], [6.0, 8.0], 0.5),
    ([3.0, 4.0], [3.0, 4.0], 0.0),
    # the denominator is the reference's norm, not the result's
    ([6.0, 8.0], [3.0, 4.0], 1.0),
    # 2-D: one Frobenius norm over all entries -- a row with a zero reference row must not give
    # inf, and the result is not the largest per-row error (5 / 10 = 0.5 in the second row)
    ([[3.0, 4.0], [0.0, 1.0]], [[3.0, 4.0], [0.0, 0.0]], 0.2),
    ([[3.0, 4.0], [6.0, 13.0]], [[3.0, 4.0], [6.0, 8.0]], 5.0 / math.sqrt(125.0)),
    # both zero gives 0, a nonzero result against a zero reference gives inf
    ([0.0, 0.0, 0.0], [0.0, 0.0, 0.0], 0.0),
    ([0.0, -2.0], [0.0, 0.0], math.inf),
])
def test_normwise_rel_err_hand_values(got, ref, want):
    """||got - ref||_F / ||ref||_F on values worked out by hand."""
    v = mlp.normwise_rel_err(np.array(got), np.array(ref))
    if math.isinf(want):
        assert math.isinf(v)
    else:
        assert v == pytest.approx(want, rel=1e-15, abs=0.0)


def test_normwise_rel_err_mixed_precision_inputs():
    # bf16 values widened to fp32 against an fp64 array: the one entry that differs is off by
    # 0.5, and the reference's squares sum to 1 + 1 + 4 = 6
    got = torch.tensor([[1.0, 1.5], [2.0, 0.0]], dtype=torch.bfloat16).float().numpy()
    ref = np.array([[1.0, 1.0], [2.0, 0.0]])
    assert mlp.normwise_rel_err(got, ref) == pytest.approx(0.5 / math.sqrt(6.0), rel=1e-15)


# ----------------------------------------------------------------------------- token-axis MXFP8 operand

@pytest.mark.parametrize("M", [1, 31, 32, 45, 96])
def test_col_operand_matches_segment_quantizer(M):
    """The wgrad operand quantized along the token axis equals the brute-force-pinned
    column-wise segment quantizer (one segment, its last block zero-padded), decoded."""
    g = np.random.default_rng(100 + M)
    a = nm.round_bf16(g.standard_normal((M, 64)) * np.exp2(g.integers(-4, 5, (1, 64))))
    got = mlp._col_operand(a, "mxfp8")
    codes, scales = nm.quantize_mxfp8_segments_t(a, [0, M])          # [64, Mpad]
    deq = nm.dequantize_mxfp8(codes, scales, axis=-1)[:, :M].T
    np.testing.assert_array_equal(got, deq)
    np.testing.assert_array_equal(got, nm.fake_quant_mxfp8_segments(a, [0, M]))
    # bf16 leaves the operand alone
    np.testing.assert_array_equal(mlp._col_operand(a, "bf16"), a)


def test_mxfp8_backward_wgrad_uses_segmented_operands():
    """dW of the MXFP8 backward equals the product of the whole layer's column-wise segmented
    operands (every expert's rows a segment of the permuted token axis)."""
    inp = tiny(T=40, H=32, I=32, E=3, k=2, seed=23)
    idx = inp.topk_idx.numpy()
    fw = mlp.forward(inp.x, idx, inp.topk_prob, inp.w1, inp.w2, "mxfp8", "bf16")
    bw = mlp.backward(fw, inp.x, inp.dy, inp.w1, inp.w2)
    off = fw.perm.offsets
    tok = fw.perm.token_of_row
    xs = nm.round_bf16(mlp.f64(inp.x)[tok])
    dz = nm.round_bf16(mlp.f64(inp.dy)[tok])
    hs = nm.round_bf16(fw.h)
    dgu_q = nm.fake_quant_mxfp8_segments(bw.dgu, off)
    x_q = nm.fake_quant_mxfp8_segments(xs, off)
    dz_q = nm.fake_quant_mxfp8_segments(dz, off)
    h_q = nm.fake_quant_mxfp8_segments(hs, off)
    for e in range(3):
        lo, hi = int(off[e]), int(off[e + 1])
        np.testing.assert_allclose(bw.dw1[e], dgu_q[lo:hi].T @ x_q[lo:hi], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(bw.dw2[e], dz_q[lo:hi].T @ h_q[lo:hi], rtol=1e-12, atol=1e-14)
