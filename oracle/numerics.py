"""Storage-precision rounding used by the oracle.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The oracle computes in fp64 but sees every weight and input as the value stored on the device
(bf16), and it rounds the logits to bf16 before the sampler statistics, because the sampler reads
the logits the decoder returns (diffusers DiffusionGemmaPipeline docs, class description: the
model returns logits of shape [batch, canvas_length, vocab_size], and the scheduler works on them).

bf16 keeps 8 significant bits (1 implicit + 7 stored) and the binary32 exponent range.  Rounding
is to nearest, ties to even; values beyond the largest finite bf16 after rounding become inf.
"""
import numpy as np

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(x):
    """Nearest bf16 value of each float64 input (round to nearest, ties to even), as float64."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    ax = np.abs(xf)
    m, e = np.frexp(ax)                       # ax = m * 2**e, m in [0.5, 1)
    # normal range: 8 significant bits -> quantum 2**(e-8); below 2**-126 the quantum is 2**-133
    q_exp = np.where(e - 8 < -133, -133, e - 8)
    q = np.ldexp(1.0, q_exp)
    r = np.rint(ax / q) * q                   # np.rint rounds half to even; ax/q is exact
    r = np.where(r > _BF16_MAX, np.inf, r)
    out[:] = np.copysign(r, xf)
    out[~finite] = x[~finite]
    return out


def bf16_bits(x):
    """bf16 bit patterns (uint16) of the nearest bf16 values of float64 inputs."""
    r = round_bf16(x).astype(np.float32)      # exact: every bf16 value is a binary32 value
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f64(bits):
    """Exact value of bf16 bit patterns, as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ---- OCP FP8 E4M3 ("e4m3fn") ------------------------------------------------------------------
# 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no infinities; the all-ones magnitude
# code 0x7F is NaN, so the largest finite value is 1.75 * 2**8 = 448; normals from 2**-6,
# subnormals m * 2**-9 (m = 1..7).  Used for the expert and LM-head weights and their inputs in
# the fp8 configuration.  The pages only say FP8 (the model card quotes its speed on H100 in
# FP8); the reading taken: per-row scale = amax / 448, round to nearest even, saturate at +-448,
# fp32 accumulation, output = accumulator * input scale * weight scale.

E4M3_MAX = 448.0


def round_e4m3(x):
    """Nearest e4m3 value of each float64 input (ties to even); magnitudes beyond 448 saturate
    to 448; NaN stays NaN.  Returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    xf = np.where(nan | ~np.isfinite(x), np.where(nan, 0.0, np.sign(x) * 1e300), x)
    ax = np.abs(xf)
    _, e = np.frexp(ax)                       # ax in [2**(e-1), 2**e)
    # 4 significant bits in the normal range -> quantum 2**(e-4); subnormal quantum 2**-9
    q_exp = np.maximum(e - 4, -9)
    q = np.ldexp(1.0, q_exp)
    r = np.rint(ax / q) * q                   # exact quotient; rint = half to even
    r = np.minimum(r, E4M3_MAX)
    out = np.copysign(r, xf)
    out[nan] = np.nan
    return out


def e4m3_code(v):
    """uint8 code of e4m3 values (outputs of round_e4m3); NaN -> 0x7F."""
    v = np.asarray(v, dtype=np.float64)
    nan = np.isnan(v)
    a = np.abs(np.where(nan, 0.0, v))
    _, e = np.frexp(a)                        # a in [2**(e-1), 2**e)
    normal = a >= 2.0 ** -6
    exp_field = np.where(normal, e - 1 + 7, 0)
    mant = np.where(normal, (a / np.ldexp(1.0, e - 1) - 1.0) * 8.0, a / 2.0 ** -9)
    code = (exp_field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = code | (np.signbit(v).astype(np.int64) << 7)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


def e4m3_value(code):
    """Exact value of e4m3 codes, as float64 (0x7F / 0xFF -> NaN)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 7
    val = np.where(ef == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, ef - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def quantize_rows_e4m3(x):
    """Per-row symmetric e4m3 quantisation along the last axis, decided in binary32:
    s = fp32(max |x|) / 448 (binary32 division; s = 1 for an all-zero row) and
    q = e4m3(fp32(x) / s) (binary32 division, then nearest-even with saturation).
    Returns (q as float64 e4m3 values, s as float64), so that x ~ q * s."""
    xf = np.asarray(x, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(xf), axis=-1)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (xf / s[..., None]).astype(np.float32)
    return round_e4m3(y.astype(np.float64)), s.astype(np.float64)
