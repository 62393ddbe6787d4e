"""Pins of the oracle's per-tensor FP8 quantizer (one fp32 scale s = 448 / amax per tensor).

The pages (page "BioNeMo Uses Grouped Kernels and MXFP8", Reducing memory pressure with
MXFP8; page "How BioNeMo cuts overhead", How MXFP8 reduces memory use) name FP8 beside
MXFP8 and tell them apart by the scaling granularity only.  What is checked here does not
reuse the oracle's arithmetic: the fp32 rounding of the scale and of each product is done on
exact fractions, element codes by nearest-value search over the E4M3 table, and torch's own
float8 cast serves as the library cross-check.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import numerics as nm
from test_oracle_numerics import brute_e4m3_code

FLT_MAX = float(np.finfo(np.float32).max)


def fp32_round(x: Fraction) -> float:
    """Nearest fp32 value of an exact rational (ties to even), by bisection on the bit
    patterns of positive floats (monotone in value); overflow gives inf."""
    if x == 0:
        return 0.0
    sgn = -1.0 if x < 0 else 1.0
    a = abs(x)
    lo, hi = 0, 0x7F800000                    # +0 .. +inf as uint32 patterns
    while hi - lo > 1:                        # largest pattern with value <= a
        mid = (lo + hi) // 2
        v = np.array([mid], dtype=np.uint32).view(np.float32)[0]
        if Fraction(float(v)) <= a:
            lo = mid
        else:
            hi = mid
    below = float(np.array([lo], dtype=np.uint32).view(np.float32)[0])
    if Fraction(below) == a:
        return sgn * below
    above = float(np.array([lo + 1], dtype=np.uint32).view(np.float32)[0])
    if math.isinf(above):                     # past the largest finite value: overflow
        half = Fraction(FLT_MAX) + Fraction(2) ** (127 - 24)
        return sgn * (math.inf if a >= half else FLT_MAX)
    db, da = a - Fraction(below), Fraction(above) - a
    if db < da or (db == da and lo % 2 == 0):
        return sgn * below
    return sgn * above


def ref_scale(amax: float) -> float:
    if amax == 0:
        return 1.0
    s = fp32_round(Fraction(448) / Fraction(amax))
    return FLT_MAX if math.isinf(s) else s


def bf16_values(g, n, lo_exp=-20, hi_exp=10):
    v = g.standard_normal(n) * np.exp2(g.integers(lo_exp, hi_exp, n))
    return torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()


def test_scale_is_correctly_rounded_fp32_division():
    g = np.random.default_rng(11)
    amaxes = list(np.abs(bf16_values(g, 300, -130, 120)))
    amaxes += [0.0, 1.0, 448.0, 3.0, 7.0, 2.0 ** -133, 2.0 ** -126, 3.3895313892515355e38,
               2.0 ** -100, 1.0e-38]
    for a in amaxes:
        got = float(nm.fp8_tensor_scale(a))
        assert got == ref_scale(float(a)), a


def test_scale_edge_cases():
    assert float(nm.fp8_tensor_scale(0.0)) == 1.0
    assert float(nm.fp8_tensor_scale(2.0 ** -133)) == FLT_MAX          # 448 * 2^133 overflows fp32
    assert float(nm.fp8_tensor_scale(448.0)) == 1.0
    assert float(nm.fp8_tensor_scale(7.0)) == 64.0


def test_codes_brute_force():
    g = np.random.default_rng(12)
    for trial in range(6):
        x = bf16_values(g, 200, -12 - 3 * trial, 4)
        if trial == 5:
            x[:50] = 0.0
            x[50:60] = -0.0
        codes, s = nm.quantize_fp8_tensor(x)
        assert float(s) == ref_scale(float(np.max(np.abs(x))))
        for v, c in zip(x, codes):
            q = fp32_round(Fraction(float(v)) * Fraction(float(s)))
            if q == 0.0:
                q = math.copysign(0.0, v)
            assert c == brute_e4m3_code(q), (v, s, c)


def test_codes_match_torch_float8_cast():
    g = np.random.default_rng(13)
    for scale_exp in (-30, -6, 0, 5, 40):
        x = bf16_values(g, 5000, scale_exp - 8, scale_exp + 2)
        codes, s = nm.quantize_fp8_tensor(x)
        q = torch.from_numpy(x.astype(np.float32)) * torch.tensor(float(s), dtype=torch.float32)
        ref = q.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(codes, ref)


def test_amax_element_maps_to_448():
    g = np.random.default_rng(14)
    for e in range(-60, 60, 7):
        x = bf16_values(g, 257, e - 6, e)
        codes, _ = nm.quantize_fp8_tensor(x)
        i = int(np.argmax(np.abs(x)))
        assert codes[i] == (0xFE if x[i] < 0 else 0x7E)
        assert np.all((codes & 0x7F) != 0x7F)                      # never NaN


def test_power_of_two_invariance():
    g = np.random.default_rng(15)
    x = bf16_values(g, 1000, -8, 3)
    c0, s0 = nm.quantize_fp8_tensor(x)
    for j in (-20, -3, 1, 9, 30):
        c, s = nm.quantize_fp8_tensor(np.ldexp(x, j))
        np.testing.assert_array_equal(c, c0)
        assert float(s) == math.ldexp(float(s0), -j)


def test_dequantization_error_bound():
    g = np.random.default_rng(16)
    for trial in range(4):
        x = bf16_values(g, 4000, -16, 2 + trial)
        codes, s = nm.quantize_fp8_tensor(x)
        d = nm.dequantize_fp8_tensor(codes, s)
        # half a unit in the last place of E4M3 (relative 2^-4 for normals, 2^-10 absolute for
        # subnormals, in the scaled domain), plus the fp32 rounding of the product
        bound = (np.abs(x) * 2.0 ** -4 + 2.0 ** -10 / float(s)) * (1 + 2.0 ** -20)
        assert np.all(np.abs(d - x) <= bound)


def test_segments_each_on_their_own():
    g = np.random.default_rng(17)
    x = bf16_values(g, 40 * 8, -6, 3).reshape(40, 8)
    x[12:15] = 0.0                                     # an all-zero segment
    off = [0, 5, 5, 12, 15, 33, 40]                    # an empty segment second
    codes, scales = nm.quantize_fp8_segments(x, off)
    assert scales[1] == 1.0 and scales[3] == 1.0
    for gi in range(len(off) - 1):
        lo, hi = off[gi], off[gi + 1]
        if hi == lo:
            continue
        c, s = nm.quantize_fp8_tensor(x[lo:hi])
        np.testing.assert_array_equal(codes[lo:hi], c)
        assert scales[gi] == s
    # a segment's scale does not see the other segments' values
    assert scales[0] == np.float32(ref_scale(float(np.max(np.abs(x[0:5])))))


def test_rejects_values_not_in_fp32():
    with pytest.raises(ValueError):
        nm.quantize_fp8_tensor(np.array([1.0 + 2.0 ** -40]))


# ---------------------------------------------------------------------------- the FP8 forward

from oracle import mlp                                        # noqa: E402
from test_oracle_mlp import tiny                              # noqa: E402
from test_oracle_numerics import TAB_C, TAB_V                 # noqa: E402

DECODE = {int(c): float(v) for c, v in zip(TAB_C, TAB_V)}


def scalar_fake_quant(vals):
    """One tensor (a flat list of floats) through per-tensor FP8 and back, element by element."""
    amax = max((abs(v) for v in vals), default=0.0)
    s = ref_scale(amax)
    out = []
    for v in vals:
        q = fp32_round(Fraction(v) * Fraction(s))
        if q == 0.0:
            q = math.copysign(0.0, v)
        out.append(DECODE[brute_e4m3_code(q)] / s)
    return out


def scalar_forward_fp8(x, idx, prob, w1, w2):
    """Loops over experts, their rows (ascending token order) and matrix entries."""
    T, H = x.shape
    k = idx.shape[1]
    E, I = w2.shape[0], w2.shape[2]
    xb = [[float(v) for v in nm.round_bf16(np.asarray(x[t], dtype=np.float64))] for t in range(T)]
    z = {}
    for e in range(E):
        rows = [(t, j) for t in range(T) for j in range(k) if int(idx[t, j]) == e]
        if not rows:
            continue
        flat = scalar_fake_quant([v for (t, j) in rows for v in xb[t]])
        xq = [flat[n * H:(n + 1) * H] for n in range(len(rows))]
        W1 = scalar_fake_quant([float(v) for v in np.asarray(w1[e], dtype=np.float64).ravel()])
        W2 = scalar_fake_quant([float(v) for v in np.asarray(w2[e], dtype=np.float64).ravel()])
        hs = []
        for n, (t, j) in enumerate(rows):
            gu = [sum(xq[n][c] * W1[i * H + c] for c in range(H)) for i in range(2 * I)]
            p = float(prob[t, j])
            h = [gu[i] / (1.0 + math.exp(-gu[i])) * gu[I + i] * p for i in range(I)]
            hs.append([float(v) for v in nm.round_bf16(np.array(h))])
        flat = scalar_fake_quant([v for row in hs for v in row])
        for n, (t, j) in enumerate(rows):
            hq = flat[n * I:(n + 1) * I]
            z[(t, j)] = [sum(hq[i] * W2[c * I + i] for i in range(I)) for c in range(H)]
    out = np.zeros((T, H))
    for t in range(T):
        acc = [0.0] * H
        for j in range(k):
            zb = nm.round_bf16(np.array(z[(t, j)]))
            acc = [a + float(b) for a, b in zip(acc, zb)]
        out[t] = nm.round_bf16(np.array(acc))
    return out


def test_fp8_forward_matches_scalar_loop():
    inp = tiny(T=7, H=32, I=32, E=3, k=2, seed=21)
    w1 = inp.w1.to(torch.float64).numpy()
    w2 = inp.w2.to(torch.float64).numpy()
    idx = inp.topk_idx.numpy()
    prob = inp.topk_prob.to(torch.float64).numpy()
    fw = mlp.forward(inp.x, idx, inp.topk_prob, inp.w1, inp.w2, "fp8", "bf16")
    ref = scalar_forward_fp8(inp.x.to(torch.float64).numpy(), idx, prob, w1, w2)
    # the two sum in different orders, so a bf16 rounding of the output may differ by one unit
    diff = np.abs(fw.out - ref)
    assert np.all(diff <= 2.0 ** -7 * np.abs(ref) + 1e-30)
    assert np.mean(diff == 0) > 0.95


def test_fp8_forward_is_exact_on_representable_operands():
    """Every operand tensor holds E4M3 values times 2^j with amax = 448 * 2^j exactly, so each
    scale is the power of two 2^-j and the quantization loses nothing: the gate-up output equals
    the BF16 path's (the same fp64 products of the same values)."""
    inp = tiny(T=16, H=32, I=32, E=4, k=2, seed=22)
    g = np.random.default_rng(23)
    finite = TAB_V[np.abs(TAB_V) <= 448]

    def build(shape, j, fix_axis_rows):
        v = g.choice(finite, size=shape) * 2.0 ** j
        if fix_axis_rows:
            v[..., 0] = 448.0 * 2.0 ** j              # every row holds the amax
        else:
            v.reshape(shape[0], -1)[:, 0] = -448.0 * 2.0 ** j   # one amax element per tensor
        return torch.from_numpy(v).to(torch.bfloat16)
    x = build(tuple(inp.x.shape), -6, True)
    w1 = build(tuple(inp.w1.shape), -12, False)
    w2 = build(tuple(inp.w2.shape), -10, False)
    idx = inp.topk_idx.numpy()
    f8 = mlp.forward(x, idx, inp.topk_prob, w1, w2, "fp8", "bf16")
    fb = mlp.forward(x, idx, inp.topk_prob, w1, w2, "bf16", "bf16")
    np.testing.assert_array_equal(f8.x_perm, fb.x_perm)
    np.testing.assert_array_equal(f8.gu, fb.gu)
    np.testing.assert_array_equal(f8.h, fb.h)


def test_fp8_forward_close_to_bf16():
    inp = tiny(T=64, H=64, I=64, E=4, k=2, seed=24)
    idx = inp.topk_idx.numpy()
    f8 = mlp.forward(inp.x, idx, inp.topk_prob, inp.w1, inp.w2, "fp8", "bf16")
    fb = mlp.forward(inp.x, idx, inp.topk_prob, inp.w1, inp.w2, "bf16", "bf16")
    fm = mlp.forward(inp.x, idx, inp.topk_prob, inp.w1, inp.w2, "mxfp8", "bf16")
    err = mlp.normwise_rel_err(f8.out, fb.out)
    err_mx = mlp.normwise_rel_err(fm.out, fb.out)
    # both keep 4 significant bits per element (E4M3), so on N(0,1)-like data their distance
    # from the BF16 path is of the same size (about 6-8 % here, four roundings deep)
    assert 0.5 * err_mx < err < 1.5 * err_mx, (err, err_mx)


def test_fp8_rejected_where_rows_are_coupled():
    inp = tiny()
    idx = inp.topk_idx.numpy()
    with pytest.raises(ValueError):
        mlp.forward_tokens(inp.x, idx, inp.topk_prob, inp.w1, inp.w2, [0], "fp8")
    fw = mlp.forward(inp.x, idx, inp.topk_prob, inp.w1, inp.w2, "fp8")
    with pytest.raises(ValueError):
        mlp.backward(fw, inp.x, inp.dy, inp.w1, inp.w2)


# ---------------------------------------------------------------------------- hand-derived cases

import os                                                      # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_tensor_cases.txt")


def _golden():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line.startswith("tensor "):
            continue
        parts = [p.strip() for p in line.split("|")]
        name = parts[0].split()[1]
        s = Fraction(parts[1].split("=")[1])
        vals, codes = [], []
        for tok in parts[2].split():
            v, c = tok.split("=")
            vals.append(float(v))
            codes.append(int(c, 16))
        out.append((name, s, vals, codes))
    return out


@pytest.mark.parametrize("name,s,vals,codes", _golden(), ids=[g[0] for g in _golden()])
def test_golden_fp8_tensor_cases(name, s, vals, codes):
    c, got_s = nm.quantize_fp8_tensor(np.array(vals))
    assert Fraction(float(got_s)) == s
    np.testing.assert_array_equal(c, np.array(codes, dtype=np.uint8))
