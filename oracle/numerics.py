"""Rounding and block-scaled formats, written from their definitions (fp64).

Formats (page "BioNeMo Uses Grouped Kernels and MXFP8", Reducing memory
pressure with MXFP8, Figure 3; page "How BioNeMo cuts overhead", How MXFP8
reduces memory use):
  * BF16: 1 sign, 8 exponent, 7 mantissa bits.
  * MXFP8: E4M3 elements plus one shared E8M0 scale per 32 consecutive values.
  * FP8 (same sections): 8-bit values whose scaling is coarser than MXFP8's
    per-32-value blocks -- read as one scale per tensor (below).
The pages do not spell out the scale rule or the rounding; the readings taken
for MXFP8 are the OCP Microscaling (MX) v1.0 ones:
  * shared exponent s = floor(log2(amax)) - 8, where 8 is the exponent of the
    largest normal E4M3 value (448 = 1.75 * 2^8); s is clamped to [-127, 127],
    so an all-zero block gets s = -127 (E8M0 byte 0x00); E8M0 byte = s + 127;
  * element = v / 2^s rounded to E4M3FN (OCP variant: bias 7, no infinities,
    max 448, subnormals n * 2^-9) with round-to-nearest, ties to even, and
    saturated to +-448; the sign of a value that rounds to zero is kept.
For per-tensor FP8 the readings are current scaling of each tensor as a whole:
  * s = 448 / amax as an fp32 division (correctly rounded), amax = max |v|
    over the tensor; amax == 0 gives s = 1, and an s that overflows fp32 is
    clamped to the largest finite fp32 value;
  * element = E4M3FN(fp32(v * s)): the product rounded once to fp32, then to
    E4M3FN as above (nearest, ties to even, saturated to +-448, zero keeps its
    sign); the value the code stands for is decode(code) / s.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest normal E4M3 value
E4M3_EMIN = -6         # exponent of the smallest normal E4M3 value
E4M3_MBITS = 3
MX_BLOCK = 32


# ----------------------------------------------------------------------------- bf16

def round_bf16(x) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even); fp64 in, fp64 out, no double rounding.

    bf16 has 8 significant bits; for a normal value with exponent e the
    spacing is 2^(e-7).  Subnormal bf16 values share the spacing 2^-133.
    Overflow goes to +-inf as in IEEE round-to-nearest.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                       # a = m * 2^e, m in [0.5, 1)
    exp_unb = np.maximum(e - 1, -126)        # floor(log2 a), subnormals share -126
    ulp = np.ldexp(1.0, exp_unb - 7)
    r = np.rint(a / ulp) * ulp               # np.rint: round half to even
    r = np.where(r > 3.3895313892515355e38, np.inf, r)  # above the largest bf16 value
    r = np.where(a == 0, 0.0, r)
    return np.copysign(r, x)


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of values that are exactly representable in bf16."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(b) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16)).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- E4M3 / E8M0

def round_e4m3(q) -> np.ndarray:
    """Round fp64 values to the nearest E4M3FN value (ties to even), saturating at +-448.

    Normal E4M3 values with exponent e in [-6, 8] are spaced 2^(e-3); the
    subnormals share the spacing 2^-9 of the lowest binade.  A value that
    rounds up to the next power of two simply lands on that binade's first
    value, which is representable.
    """
    q = np.asarray(q, dtype=np.float64)
    a = np.abs(q)
    _, e = np.frexp(a)
    exp_unb = np.maximum(e - 1, E4M3_EMIN)
    ulp = np.ldexp(1.0, exp_unb - E4M3_MBITS)
    r = np.rint(a / ulp) * ulp
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, q)


def encode_e4m3(v) -> np.ndarray:
    """Code byte of values that are exactly representable in E4M3FN (|v| <= 448)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = np.signbit(v).astype(np.uint8)
    _, e = np.frexp(a)
    normal = a >= 2.0 ** E4M3_EMIN
    ex = np.where(normal, e - 1 + 7, 0)
    mant = np.where(normal,
                    (a / np.ldexp(1.0, e - 1) - 1.0) * 8.0,
                    a / 2.0 ** -9)
    mant_i = mant.astype(np.int64)
    if np.any(mant_i != mant) or np.any(a > E4M3_MAX):
        raise ValueError("value not representable in E4M3FN")
    return ((sign.astype(np.int64) << 7) | (ex.astype(np.int64) << 3) | mant_i).astype(np.uint8)


def decode_e4m3(code) -> np.ndarray:
    """fp64 value of E4M3FN code bytes (0x7F / 0xFF are NaN)."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(ex == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, ex - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def decode_e8m0(byte) -> np.ndarray:
    """2^(byte - 127); 0xFF is NaN."""
    b = np.asarray(byte, dtype=np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


def mx_shared_exponent(amax) -> np.ndarray:
    """s = floor(log2(amax)) - 8, clamped to [-127, 127]; amax == 0 gives -127."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)                    # amax = m * 2^e, m in [0.5, 1)
    s = (e - 1) - E4M3_EMAX
    s = np.where(amax == 0, -127, s)
    return np.clip(s, -127, 127).astype(np.int64)


# ----------------------------------------------------------------------------- MXFP8 blocks

def quantize_mxfp8(x, axis: int = -1):
    """OCP MXFP8 along `axis` in blocks of 32 consecutive values.

    Returns (codes uint8 with x's shape, scales uint8 with that axis divided by
    32).  The axis length must be a multiple of 32.
    """
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    n = x.shape[-1]
    if n % MX_BLOCK:
        raise ValueError("axis length must be a multiple of 32")
    blk = x.reshape(*x.shape[:-1], n // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blk), axis=-1)
    s = mx_shared_exponent(amax)
    q = blk / np.ldexp(1.0, s)[..., None]    # exact: division by a power of two
    codes = encode_e4m3(round_e4m3(q)).reshape(x.shape)
    scales = (s + 127).astype(np.uint8)
    return np.moveaxis(codes, -1, axis), np.moveaxis(scales, -1, axis)


def dequantize_mxfp8(codes, scales, axis: int = -1) -> np.ndarray:
    c = np.moveaxis(np.asarray(codes), axis, -1)
    s = np.moveaxis(np.asarray(scales), axis, -1)
    v = decode_e4m3(c).reshape(*c.shape[:-1], c.shape[-1] // MX_BLOCK, MX_BLOCK)
    v = v * decode_e8m0(s)[..., None]
    return np.moveaxis(v.reshape(c.shape), -1, axis)


def fake_quant_mxfp8(x, axis: int = -1) -> np.ndarray:
    """dequantize(quantize(x)) along `axis`."""
    c, s = quantize_mxfp8(x, axis)
    return dequantize_mxfp8(c, s, axis)


def padded_segments(offsets):
    """Per-segment starts in a token axis where every segment is padded to a multiple of 32."""
    offsets = np.asarray(offsets, dtype=np.int64)
    sizes = np.diff(offsets)
    pad = (sizes + MX_BLOCK - 1) // MX_BLOCK * MX_BLOCK
    return np.concatenate([[0], np.cumsum(pad)]).astype(np.int64)


def quantize_mxfp8_segments_t(x, offsets):
    """Column-wise MXFP8 of x [R, C] along the row axis, restarted per segment.

    Segment g holds rows [offsets[g], offsets[g+1]); it is zero-padded at its
    end to a multiple of 32 rows, quantized in blocks of 32 rows per column,
    and written transposed: codes [C, Rpad] (segment g in columns
    [pad[g], pad[g+1])), scales [C, Rpad/32].  Padding codes are 0x00.
    """
    x = np.asarray(x, dtype=np.float64)
    R, C = x.shape
    pad = padded_segments(offsets)
    Rp = int(pad[-1])
    xt = np.zeros((C, Rp), dtype=np.float64)
    for g in range(len(offsets) - 1):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        xt[:, pad[g]:pad[g] + (hi - lo)] = x[lo:hi].T
    return quantize_mxfp8(xt, axis=-1)


def fake_quant_mxfp8_segments(x, offsets) -> np.ndarray:
    """dequantize(quantize) of the column-wise segmented MXFP8, returned as [R, C]."""
    x = np.asarray(x, dtype=np.float64)
    R, C = x.shape
    codes, scales = quantize_mxfp8_segments_t(x, offsets)
    deq = dequantize_mxfp8(codes, scales, axis=-1)        # [C, Rp]
    pad = padded_segments(offsets)
    out = np.empty_like(x)
    for g in range(len(offsets) - 1):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        out[lo:hi] = deq[:, pad[g]:pad[g] + (hi - lo)].T
    return out


# ----------------------------------------------------------------------------- per-tensor FP8

FLT_MAX = float(np.finfo(np.float32).max)


def fp8_tensor_scale(amax) -> np.float32:
    """s = 448 / amax in fp32; 1 for amax == 0; clamped to the largest finite fp32 value."""
    a = np.float32(amax)
    if a == 0:
        return np.float32(1.0)
    with np.errstate(over="ignore"):
        s = np.float32(E4M3_MAX) / a                 # one IEEE fp32 division
    return np.float32(FLT_MAX) if np.isinf(s) else np.float32(s)


def quantize_fp8_tensor(x):
    """Per-tensor-scaled E4M3 of x (values exactly representable in fp32, e.g. bf16).

    Returns (codes uint8 with x's shape, s as np.float32).
    """
    x64 = np.asarray(x, dtype=np.float64)
    x32 = x64.astype(np.float32)
    if not np.array_equal(x32.astype(np.float64), x64, equal_nan=True):
        raise ValueError("per-tensor FP8 input must be exactly representable in fp32")
    amax = float(np.max(np.abs(x64))) if x64.size else 0.0
    s = fp8_tensor_scale(amax)
    q = (x32 * s).astype(np.float64)                 # fp32 product, then E4M3
    return encode_e4m3(round_e4m3(q)), s


def dequantize_fp8_tensor(codes, s) -> np.ndarray:
    return decode_e4m3(codes) / np.float64(s)


def fake_quant_fp8_tensor(x) -> np.ndarray:
    """dequantize(quantize(x)) with one scale for all of x."""
    c, s = quantize_fp8_tensor(x)
    return dequantize_fp8_tensor(c, s)


def quantize_fp8_segments(x, offsets):
    """Per-tensor FP8 of each row segment [offsets[g], offsets[g+1]) of x [R, C] on its own.

    Returns (codes [R, C] uint8, scales [G] float32); an empty segment gets s = 1.
    """
    x = np.asarray(x, dtype=np.float64)
    off = np.asarray(offsets, dtype=np.int64)
    codes = np.zeros(x.shape, dtype=np.uint8)
    scales = np.ones(len(off) - 1, dtype=np.float32)
    for g in range(len(off) - 1):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi > lo:
            codes[lo:hi], scales[g] = quantize_fp8_tensor(x[lo:hi])
    return codes, scales
