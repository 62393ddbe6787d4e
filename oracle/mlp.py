"""Grouped expert MLP, forward and backward, as a plain per-expert loop in fp64.

What is computed (page "BioNeMo Uses Grouped Kernels and MXFP8": Figure 1, a
top-k router sends each token to k experts and their outputs are combined as a
weighted sum; Grouping fragmented expert workloads, the gate-up grouped linear
has out_features = 2 * intermediate_size and no bias, each expert keeps its own
weights; Fusing precision conversion and expert computation, the expert network
is gate-up linear -> ScaledSwiGLU -> down linear, ScaledSwiGLU folds the routing
probability in; Figure 4, the MXFP8 flow quantizes before the gate-up GEMM and
the down projection is a separate grouped GEMM; page "How BioNeMo cuts
overhead", How MXFP8 reduces memory use, 16-bit master weights converted to
MXFP8 for each low-precision GEMM):

    e = topk_idx[t, j],  p = topk_prob[t, j],  x = operand(X[t])
    [g | u] = x . W1_e^T                   g = first I outputs (gate), u = last I (up)
    h = silu(g) * u * p                    silu(v) = v * sigmoid(v)
    z = operand(h) . W2_e^T
    out[t] = sum_j io(z)

Readings where the pages are silent (all listed with the design notes):
  * SwiGLU = silu(gate) * up, gate = outputs [0, I) of the gate-up projection.
  * p multiplies h before the down projection (and before h is quantized), so
    the combine is an unweighted sum of the k expert outputs.
  * Operand formats: "bf16" rounds X to bf16 and h to bf16; "mxfp8" quantizes
    X and h along H / I and W1, W2 along their K (H / I) with the OCP MXFP8
    rule; "fp8" (forward only) quantizes each GEMM operand tensor with one
    scale: every W1_e and W2_e, and each expert's rows of X_perm and of h --
    the operands of that expert's GEMM -- with h rounded to bf16 first (the
    scale needs the amax of the whole tensor, so h exists in bf16 before it is
    quantized); "exact" applies no rounding at all (the derivative checks).
  * Each grouped GEMM writes its output in the layer's I/O dtype (bf16, or f32
    for f32 I/O) -- the down projection's z before the combine, the FC1 dgrad
    output before the un-permute sum; the combine sums in high precision and
    rounds once.
  * Saved activations for the backward (gate-up output, h) are bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from . import numerics as nm
from .permute import Permutation, permute


def f64(a) -> np.ndarray:
    """Exact fp64 copy of a numpy array or a CPU torch tensor (bf16 / f32)."""
    if hasattr(a, "detach"):
        import torch
        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def silu(v):
    return v / (1.0 + np.exp(-v))


def sigmoid(v):
    return 1.0 / (1.0 + np.exp(-v))


def round_io(v, io_dtype: str, precision: str):
    if precision == "exact":
        return v
    if io_dtype == "f32":
        return v.astype(np.float32).astype(np.float64)
    return nm.round_bf16(v)


def activation_operand(x, precision: str):
    """X (or h) as the grouped GEMM sees it: rows along K."""
    if precision == "exact":
        return x
    if precision == "bf16":
        return nm.round_bf16(x)
    if precision == "mxfp8":
        return nm.fake_quant_mxfp8(x, axis=1)
    if precision == "fp8":          # x: the rows of one expert (one tensor)
        return nm.fake_quant_fp8_tensor(nm.round_bf16(x))
    raise ValueError(precision)


def weight_operand(w_e, precision: str, k_axis: int = 1):
    """A bf16 master weight as the GEMM sees it (MXFP8: blocks along the GEMM's K)."""
    if precision in ("exact", "bf16"):
        return w_e
    if precision == "fp8":
        return nm.fake_quant_fp8_tensor(w_e)
    return nm.fake_quant_mxfp8(w_e, axis=k_axis)


def expert_forward(xq, p, w1q, w2q, precision: str, io_dtype: str):
    """One expert on its rows.  xq: operand rows [M, H]; p: [M] probabilities;
    w1q [2I, H], w2q [H, I]: the expert's weights as the GEMMs consume them."""
    I = w2q.shape[1]
    gu = xq @ w1q.T                                  # [M, 2I]
    g, u = gu[:, :I], gu[:, I:]
    h = silu(g) * u * p[:, None]
    hq = activation_operand(h, precision)
    z = hq @ w2q.T                                   # [M, H]
    return gu, h, hq, round_io(z, io_dtype, precision)


@dataclass
class Forward:
    perm: Permutation
    precision: str
    io_dtype: str
    x_perm: np.ndarray        # [R, H] operand values (bf16, MXFP8-dequantized or exact)
    prob_perm: np.ndarray     # [R]
    gu: np.ndarray            # [R, 2I] fp64 gate-up output
    h: np.ndarray             # [R, I] fp64 scaled SwiGLU output (before rounding)
    h_op: np.ndarray          # [R, I] h as the down projection consumes it
    z: np.ndarray             # [R, H] down projection output in the I/O dtype
    out: np.ndarray           # [T, H]
    extra: dict = field(default_factory=dict)


def forward(x, topk_idx, topk_prob, w1, w2, precision: str = "bf16", io_dtype: str = "bf16",
            experts=None) -> Forward:
    """Whole layer.  x [T,H]; topk_idx/prob [T,k]; w1 [E,2I,H]; w2 [E,H,I].

    experts: optional subset of expert ids; only their rows are computed (the
    same arithmetic), and out[t] is NaN for tokens routed to any other expert.
    """
    xs = f64(x)
    idx = np.asarray(topk_idx)
    prob = f64(topk_prob)
    T, H = xs.shape
    k = idx.shape[1]
    E = int(w1.shape[0])
    I = int(w2.shape[2])
    perm = permute(idx, E)
    tok = perm.token_of_row
    if precision == "fp8":
        x_perm = nm.round_bf16(xs)[tok]     # quantized per expert segment below
    else:
        x_perm = activation_operand(xs, precision)[tok]
    p_perm = prob.reshape(-1)[perm.src_index]
    R = T * k
    gu = np.zeros((R, 2 * I))
    h = np.zeros((R, I))
    hq = np.zeros((R, I))
    z = np.zeros((R, H))
    off = perm.offsets
    todo = set(range(E)) if experts is None else set(int(e) for e in experts)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        if e not in todo:
            z[lo:hi] = np.nan
            continue
        if precision == "fp8":
            x_perm[lo:hi] = activation_operand(x_perm[lo:hi], precision)
        g_, h_, hq_, z_ = expert_forward(x_perm[lo:hi], p_perm[lo:hi],
                                         weight_operand(f64(w1[e]), precision),
                                         weight_operand(f64(w2[e]), precision), precision, io_dtype)
        gu[lo:hi], h[lo:hi], hq[lo:hi], z[lo:hi] = g_, h_, hq_, z_
    out = np.zeros((T, H))
    for j in range(k):
        out += z[perm.row_id_map.reshape(T, k)[:, j]]
    out = round_io(out, io_dtype, precision)
    return Forward(perm, precision, io_dtype, x_perm, p_perm, gu, h, hq, z, out)


def forward_tokens(x, topk_idx, topk_prob, w1, w2, tokens, precision="bf16", io_dtype="bf16",
                   weight_cache: Optional[dict] = None) -> np.ndarray:
    """out[t] for the listed tokens only (same arithmetic as `forward`, row by row).

    Every rounding step of the layer acts within one row of X or h, or within
    one row of a weight, so a token's output does not depend on other tokens.
    That is not so for per-tensor FP8 (the scale of an expert's rows depends on
    all of them), which `forward` computes instead.
    """
    if precision == "fp8":
        raise ValueError("per-tensor FP8 couples the rows of an expert; use forward")
    idx = np.asarray(topk_idx)
    prob = f64(topk_prob)
    cache = {} if weight_cache is None else weight_cache
    outs = []
    for t in tokens:
        xt = f64(x[t:t + 1])
        xq = activation_operand(xt, precision)
        acc = np.zeros(xt.shape[1])
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            if ("w", e) not in cache:
                cache[("w", e)] = (weight_operand(f64(w1[e]), precision),
                                   weight_operand(f64(w2[e]), precision))
            w1q, w2q = cache[("w", e)]
            _, _, _, z = expert_forward(xq, np.array([prob[t, j]]), w1q, w2q, precision, io_dtype)
            acc += z[0]
        outs.append(round_io(acc, io_dtype, precision))
    return np.stack(outs)


@dataclass
class Backward:
    dx: np.ndarray        # [T, H] in the I/O dtype
    dprob: np.ndarray     # [T, k] (float32 values)
    dw1: np.ndarray       # [E, 2I, H]
    dw2: np.ndarray       # [E, H, I]
    dgu: np.ndarray       # [R, 2I] (bf16 values unless exact)
    dx_perm: np.ndarray   # [R, H] in the I/O dtype


def _col_operand(a, precision):
    """Operand whose K is the token axis (one expert's segment): MXFP8 blocks of
    32 rows per column, the last block zero-padded."""
    if precision != "mxfp8":
        return a
    M = a.shape[0]
    Mp = (M + 31) // 32 * 32
    pad = np.zeros((Mp, a.shape[1]))
    pad[:M] = a
    return nm.fake_quant_mxfp8(pad, axis=0)[:M]


def backward(fw: Forward, x, dy, w1, w2, experts=None) -> Backward:
    """Gradients of sum(out * dy) w.r.t. X, topk_prob, W1 and W2.

        dz = dY[token of row];  dh = dz . W2_e          (FC2 dgrad)
        a = silu(g) u;  dprob = sum_i dh_i a_i;  da = dh p
        du = da silu(g);  dg = da u silu'(g),  silu'(g) = s (1 + g (1 - s)), s = sigmoid(g)
        dX_perm = dGU . W1_e;  dX[t] = sum_j dX_perm[row(t, j)]
        dW1_e = dGU^T . X_perm;  dW2_e = dz^T . h

    MXFP8 operands are quantized along each GEMM's own K: dgrad FC2 (dz along
    H, W2 along H), wgrad FC2 (dz and h along tokens), dgrad FC1 (dGU along 2I,
    W1 along 2I), wgrad FC1 (dGU and X_perm along tokens).  dGU is rounded to
    bf16 before it feeds FC1's GEMMs; saved GU and h are bf16; dY enters the
    GEMMs rounded to bf16.

    experts: optional subset (as in `forward`); gradients that depend on any
    other expert are NaN.
    """
    prec, io = fw.precision, fw.io_dtype
    if prec == "fp8":
        raise ValueError("the per-tensor FP8 variant is forward only")
    perm = fw.perm
    T, k = perm.row_id_map.size // perm.k, perm.k
    R = T * k
    E = int(w1.shape[0])
    I = int(w2.shape[2])
    H = int(w2.shape[1])
    dys = f64(dy)
    tok = perm.token_of_row
    # dz is a GEMM operand: rounded to bf16 (a no-op for bf16 I/O), like X in the forward
    dz = dys[tok] if prec == "exact" else nm.round_bf16(dys[tok])
    rnd = (lambda v: v) if prec == "exact" else nm.round_bf16
    gu_s = rnd(fw.gu)
    h_s = fw.h_op if prec != "mxfp8" else nm.round_bf16(fw.h)
    xs = f64(x)
    # saved X_perm is bf16 (under MXFP8 it is re-quantized along tokens for the dW1 GEMM)
    x_s = fw.x_perm if prec != "mxfp8" else nm.round_bf16(xs[tok])
    dgu = np.zeros((R, 2 * I))
    dx_perm = np.zeros((R, H))
    dprob_perm = np.zeros(R)
    dw1 = np.zeros((E, 2 * I, H))
    dw2 = np.zeros((E, H, I))
    off = perm.offsets
    todo = set(range(E)) if experts is None else set(int(e) for e in experts)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if e not in todo:
            dx_perm[lo:hi] = np.nan
            dprob_perm[lo:hi] = np.nan
            dw1[e] = np.nan
            dw2[e] = np.nan
            continue
        if hi == lo:
            continue
        w1e, w2e = f64(w1[e]), f64(w2[e])
        dz_e = dz[lo:hi]
        dzq = activation_operand(dz_e, prec) if prec == "mxfp8" else dz_e
        w2q = weight_operand(w2e, prec, k_axis=0)        # K = H (rows of W2)
        dh = dzq @ w2q                                   # [M, I]
        g, u = gu_s[lo:hi, :I], gu_s[lo:hi, I:]
        s = sigmoid(g)
        sl = g * s
        a = sl * u
        p = fw.prob_perm[lo:hi][:, None]
        dprob_perm[lo:hi] = np.sum(dh * a, axis=1)
        da = dh * p
        du = da * sl
        dg = da * u * (s * (1.0 + g * (1.0 - s)))
        dgu_e = rnd(np.concatenate([dg, du], axis=1))
        dgu[lo:hi] = dgu_e
        dguq = activation_operand(dgu_e, prec) if prec == "mxfp8" else dgu_e
        w1q = weight_operand(w1e, prec, k_axis=0)        # K = 2I (rows of W1)
        dx_perm[lo:hi] = round_io(dguq @ w1q, io, prec)
        dw1[e] = _col_operand(dgu_e, prec).T @ _col_operand(x_s[lo:hi], prec)
        dw2[e] = _col_operand(dz_e, prec).T @ _col_operand(h_s[lo:hi], prec)
    dx = np.zeros((T, H))
    rm = perm.row_id_map.reshape(T, k)
    for j in range(k):
        dx += dx_perm[rm[:, j]]
    dx = round_io(dx, io, prec)
    dprob = dprob_perm[perm.row_id_map].reshape(T, k)
    if prec != "exact":
        dprob = dprob.astype(np.float32).astype(np.float64)
    return Backward(dx, dprob, dw1, dw2, dgu, dx_perm)


def normwise_rel_err(got, ref) -> float:
    """||got - ref||_F / ||ref||_F in fp64 (0 when both are zero)."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(r.ravel())
    num = np.linalg.norm((g - r).ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
