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
