"""Pins for the oracle's rounding and MXFP8 quantizer (CPU only).

Each check compares oracle.numerics with something other than itself: a
brute-force nearest-value search over the 254 finite E4M3FN codes, hand-worked
blocks (tests/golden/mxfp8_blocks.txt), torch's CPU float8 / bfloat16 casts,
closed forms and invariants (round trip, power-of-two scaling).
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import numerics as nm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp8_blocks.txt")

# ---------------------------------------------------------------------------- brute-force E4M3


def _e4m3_table():
    """All finite E4M3FN values from their bit fields (written independently of the oracle)."""
    codes, vals = [], []
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue  # NaN
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 7
        v = (m / 8.0) * 2.0 ** (1 - 7) if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        codes.append(c)
        vals.append(s * v)
    return np.array(codes), np.array(vals)


TAB_C, TAB_V = _e4m3_table()


def brute_e4m3_code(q: float) -> int:
    """Nearest finite E4M3FN value; ties -> even mantissa; |q| > 448 -> +-448; zero keeps sign."""
    if abs(q) > 448.0:
        return 0x7E | (0x80 if q < 0 else 0)
    d = np.abs(TAB_V - q)
    best = d.min()
    cand = [int(c) for c, dd in zip(TAB_C, d) if dd == best]
    # +0 and -0 are the same value: keep only the zero with the sign of q
    zsign = 0x80 if math.copysign(1.0, q) < 0 else 0x00
    cand = [c for c in cand if (c & 0x7F) != 0 or c == zsign]
    if len(cand) > 1:
        cand = [c for c in cand if (c & 1) == 0]
    assert len(cand) == 1, (q, cand)
    return cand[0]


def brute_floor_log2(a: float) -> int:
    e = 0
    while 2.0 ** e > a:
        e -= 1
    while 2.0 ** (e + 1) <= a:
        e += 1
    return e


def brute_block(v):
    v = [float(x) for x in v]
    amax = max(abs(x) for x in v)
    s = -127 if amax == 0 else max(-127, min(127, brute_floor_log2(amax) - 8))
    return s + 127, [brute_e4m3_code(x / 2.0 ** s) for x in v]


# ---------------------------------------------------------------------------- bf16


def test_round_bf16_matches_torch_cast():
    g = np.random.default_rng(1)
    x = np.concatenate([
        g.standard_normal(20000).astype(np.float32),
        (g.standard_normal(20000) * 1e-38).astype(np.float32),     # bf16 subnormals
        (g.standard_normal(20000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32),
    ])
    # exact float32 halfway cases
    hw = (g.integers(0, 2 ** 16, 5000).astype(np.uint32) << 16) | 0x8000
    x = np.concatenate([x, hw.view(np.float32)[np.isfinite(hw.view(np.float32))]])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = nm.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_round_bf16_no_double_rounding_from_fp64():
    # 1 + 2^-8 + 2^-40: nearest bf16 is 1 + 2^-7; rounding through float32 first would give 1.0
    assert nm.round_bf16(1.0 + 2 ** -8 + 2 ** -40) == 1.0 + 2 ** -7
    assert nm.round_bf16(1.0 + 2 ** -8) == 1.0           # exact tie -> even
    assert nm.round_bf16(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6
    assert nm.round_bf16(-(1.0 + 2 ** -8 + 2 ** -40)) == -(1.0 + 2 ** -7)


def test_bf16_bits_roundtrip():
    b = np.arange(0, 2 ** 16, dtype=np.uint16)
    v = nm.bf16_from_bits(b)
    fin = np.isfinite(v)
    np.testing.assert_array_equal(nm.bf16_bits(v[fin]), b[fin])


# ---------------------------------------------------------------------------- E4M3


def test_decode_matches_table_and_torch():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    np.testing.assert_array_equal(nm.decode_e4m3(codes), TAB_V)
    t = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(nm.decode_e4m3(codes), t)
    assert np.isnan(nm.decode_e4m3(np.array([0x7F, 0xFF]))).all()
    np.testing.assert_array_equal(nm.encode_e4m3(TAB_V), codes)


def test_round_e4m3_brute_force():
    g = np.random.default_rng(2)
    pos = np.sort(TAB_V[TAB_V > 0])
    mids = (pos[:-1] + pos[1:]) / 2
    q = np.concatenate([
        TAB_V, mids, -mids, mids * (1 + 1e-12), mids * (1 - 1e-12),
        g.uniform(-520, 520, 3000), g.standard_normal(3000) * 0.01, g.standard_normal(2000) * 1e-3,
        [0.0, -0.0, 2 ** -10, -2 ** -10, 3 * 2 ** -11, 448.0, 463.99, 464.0, 464.01, 500.0, -464.0, 1e6],
    ])
    got = nm.encode_e4m3(nm.round_e4m3(q))
    ref = np.array([brute_e4m3_code(float(v)) for v in q], dtype=np.uint8)
    np.testing.assert_array_equal(got, ref)


def test_round_e4m3_matches_torch_cast_within_range():
    g = np.random.default_rng(3)
    q = np.concatenate([g.uniform(-448, 448, 20000), g.standard_normal(20000) * 0.05]).astype(np.float32)
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = nm.encode_e4m3(nm.round_e4m3(q.astype(np.float64)))
    np.testing.assert_array_equal(got, ref)


# ---------------------------------------------------------------------------- E8M0 / blocks


def test_shared_exponent_brute_force_and_torch_decode():
    g = np.random.default_rng(4)
    a = np.concatenate([2.0 ** np.arange(-140, 128), 2.0 ** np.arange(-120, 120) * (1 - 2 ** -20),
                        np.abs(g.standard_normal(500)) * 10.0 ** g.integers(-30, 30, 500), [0.0]])
    s = nm.mx_shared_exponent(a)
    ref = np.array([-127 if v == 0 else max(-127, min(127, brute_floor_log2(v) - 8)) for v in a])
    np.testing.assert_array_equal(s, ref)
    byte = (s + 127).astype(np.uint8)
    t = torch.from_numpy(byte).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    np.testing.assert_array_equal(nm.decode_e8m0(byte), t)


def _golden_blocks():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line.startswith("block "):
            continue
        parts = [p.strip() for p in line.split("|")]
        name = parts[0].split()[1]
        sbyte = int(parts[1], 16)
        fill_v, fill_c = parts[3].split()[1].split("=")
        vals = [float(fill_v)] * 32
        codes = [int(fill_c, 16)] * 32
        for tok in parts[2].split():
            i, rest = tok.split(":")
            v, c = rest.split("=")
            vals[int(i)] = float(v)
            codes[int(i)] = int(c, 16)
        out.append((name, sbyte, np.array(vals), np.array(codes, dtype=np.uint8)))
    return out


@pytest.mark.parametrize("name,sbyte,vals,codes", _golden_blocks(), ids=lambda x: x if isinstance(x, str) else "")
def test_golden_blocks(name, sbyte, vals, codes):
    c, s = nm.quantize_mxfp8(vals[None, :])
    assert int(s[0, 0]) == sbyte, name
    np.testing.assert_array_equal(c[0], codes)
    bs, bc = brute_block(vals)
    assert bs == sbyte and list(bc) == list(codes)


def test_quantize_blocks_brute_force_random():
    g = np.random.default_rng(5)
    x = g.standard_normal((40, 96)) * 10.0 ** g.integers(-6, 6, (40, 1))
    x[3] = 0.0
    x[5, :32] = -x[5, :32]
    x = nm.round_bf16(x)
    c, s = nm.quantize_mxfp8(x)
    for r in range(x.shape[0]):
        for b in range(3):
            bs, bc = brute_block(x[r, 32 * b:32 * b + 32])
            assert s[r, b] == bs
            assert list(c[r, 32 * b:32 * b + 32]) == bc


def test_exhaustive_bf16_as_block_amax():
    """Every finite positive bf16 value b as the amax of a block; the other 31
    elements are b times fixed fractions (rounded to bf16)."""
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    b = nm.bf16_from_bits(bits)
    fr = np.linspace(-1, 1, 31)
    blk = nm.round_bf16(b[:, None] * fr[None, :])
    blk = np.concatenate([b[:, None], blk], axis=1)
    c, s = nm.quantize_mxfp8(blk)
    # scale: closed form from the bf16 exponent field
    ef = (bits.astype(np.int64) >> 7) & 0xFF
    sub = ef == 0
    exp = np.where(sub, -127, np.clip(ef - 127 - 8, -127, 127))
    np.testing.assert_array_equal(s[:, 0].astype(np.int64) - 127, exp)
    # elements: brute force over the 254 codes, vectorised
    q = blk / np.ldexp(1.0, s[:, 0].astype(np.int64) - 127)[:, None]
    ref = _vector_brute(q.ravel()).reshape(q.shape)
    np.testing.assert_array_equal(c, ref)


def _vector_brute(q):
    pos_v = TAB_V[TAB_C < 0x80]
    pos_c = TAB_C[TAB_C < 0x80]
    a = np.minimum(np.abs(q), 448.0)
    out = np.empty(q.size, dtype=np.uint8)
    for lo in range(0, q.size, 1 << 16):
        aa = a[lo:lo + (1 << 16)]
        d = np.abs(aa[:, None] - pos_v[None, :])
        best = d.min(axis=1, keepdims=True)
        tie = d == best
        # prefer even code among the nearest
        even = tie & ((pos_c[None, :] & 1) == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), tie.argmax(axis=1))
        out[lo:lo + aa.size] = pos_c[pick]
    neg = np.signbit(q)
    return (out | np.where(neg, 0x80, 0)).astype(np.uint8)


def test_round_trip_of_representable_blocks():
    g = np.random.default_rng(6)
    n = 500
    sexp = g.integers(-120, 120, n)
    codes = g.choice(TAB_C, size=(n, 32))
    # force a max element with magnitude in [256, 448] so the rule re-derives s
    big = TAB_C[(np.abs(TAB_V) >= 256) & (np.abs(TAB_V) <= 448)]
    codes[:, 7] = g.choice(big, size=n)
    vals = nm.decode_e4m3(codes) * np.ldexp(1.0, sexp)[:, None]
    c, s = nm.quantize_mxfp8(vals)
    np.testing.assert_array_equal(s[:, 0].astype(np.int64), sexp + 127)
    # +0 / -0 codes both decode to zero; compare values and sign
    np.testing.assert_array_equal(nm.decode_e4m3(c), nm.decode_e4m3(codes))
    np.testing.assert_array_equal(nm.dequantize_mxfp8(c, s), vals)
    # values are bf16-exact too: the bf16 round trip is the identity
    np.testing.assert_array_equal(nm.round_bf16(vals), vals)


def test_power_of_two_scaling():
    g = np.random.default_rng(7)
    x = nm.round_bf16(g.standard_normal((64, 64)))
    c0, s0 = nm.quantize_mxfp8(x)
    for j in (-20, -3, 1, 5, 40):
        c, s = nm.quantize_mxfp8(x * 2.0 ** j)
        np.testing.assert_array_equal(c, c0)
        np.testing.assert_array_equal(s.astype(int), s0.astype(int) + j)


def test_axis0_equals_transpose():
    g = np.random.default_rng(8)
    x = g.standard_normal((64, 40))
    c, s = nm.quantize_mxfp8(x, axis=0)
    ct, st = nm.quantize_mxfp8(x.T, axis=1)
    np.testing.assert_array_equal(c, ct.T)
    np.testing.assert_array_equal(s, st.T)


def test_segments_restart_and_pad():
    g = np.random.default_rng(9)
    sizes = [0, 5, 32, 33, 0, 70]
    off = np.concatenate([[0], np.cumsum(sizes)])
    x = g.standard_normal((off[-1], 64))
    codes, scales = nm.quantize_mxfp8_segments_t(x, off)
    pad = nm.padded_segments(off)
    assert list(np.diff(pad)) == [0, 32, 32, 64, 0, 96]
    for gi in range(len(sizes)):
        lo, hi = off[gi], off[gi + 1]
        seg = np.zeros((pad[gi + 1] - pad[gi], 64))
        seg[:hi - lo] = x[lo:hi]
        for col in range(64):
            for b in range(seg.shape[0] // 32):
                bs, bc = brute_block(seg[32 * b:32 * b + 32, col])
                assert scales[col, pad[gi] // 32 + b] == bs
                assert list(codes[col, pad[gi] + 32 * b:pad[gi] + 32 * b + 32]) == bc
    fq = nm.fake_quant_mxfp8_segments(x, off)
    assert fq.shape == x.shape
    assert np.max(np.abs(fq - x) / (np.abs(x) + 1e-3)) < 0.2
