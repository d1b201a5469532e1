"""FP8 (OCP E4M3) inputs for exact attention, fp64 -- TEST INFRASTRUCTURE
ONLY (see the package docstring for who may import it).

[xinc] "4. 减少访存的几种办法" notes that matrix products may run on FP8
operands while accumulation, normalisation and the softmax keep a wider
format.  What such a forward must reach is still standard attention
([xinc] "6. 标准注意力为什么慢"), evaluated on the values the 8-bit codes
stand for: with one fp32 scale per tensor, element x of Q stands for
q_scale * e4m3(x), likewise K and V.  The oracle is that definition: decode
the codes exactly, apply the tensor scales, run standard_attention.  The
GPU side also rounds the probabilities to E4M3 before the P V product; that
rounding is not part of the definition, and the parity tests bound its
effect from the arithmetic instead of modelling it here.

E4M3 ("fn" variant of the OCP 8-bit floating point formats): 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits; no infinities; the one
all-ones exponent-and-mantissa pattern (codes 0x7F and 0xFF) is NaN, so the
largest finite magnitude is 1.75 * 2^8 = 448; exponent field 0 holds the
subnormals m/8 * 2^-6.
"""

import numpy as np

from .attention import standard_attention, standard_attention_rows


def decode_e4m3(codes):
    """E4M3 codes (uint8 array) -> fp64 values, from the field definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32))
    subnormal = np.ldexp(m / 8.0, -6)
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def fp8_values(q8, k8, v8, q_scale, k_scale, v_scale):
    """The fp64 values (q, k, v) that the codes and tensor scales stand for.
    The scales are the fp32 values the GPU receives, widened exactly."""
    return (float(np.float32(q_scale)) * decode_e4m3(q8),
            float(np.float32(k_scale)) * decode_e4m3(k8),
            float(np.float32(v_scale)) * decode_e4m3(v8))


def fp8_attention(q8, k8, v8, scale, q_scale, k_scale, v_scale):
    """Standard attention of the decoded, scaled FP8 inputs: (o, lse)."""
    q, k, v = fp8_values(q8, k8, v8, q_scale, k_scale, v_scale)
    return standard_attention(q, k, v, float(np.float32(scale)))


def fp8_attention_rows(q8, k8, v8, scale, q_scale, k_scale, v_scale, rows):
    """fp8_attention for selected (b, h, i) query rows only."""
    q, k, v = fp8_values(q8, k8, v8, q_scale, k_scale, v_scale)
    return standard_attention_rows(q, k, v, float(np.float32(scale)), rows)
