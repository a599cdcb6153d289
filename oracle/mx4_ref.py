"""MXFP4 block codec (E2M1 element codes, one E8M0 scale per 32 values).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The hgpu.org abstract of the MXFP4 MoE training recipe on Hopper keeps the
GEMMs in FP8 and stores activations and expert-parallel payloads as MXFP4,
converting FP8/FP4 directly and turning row-blocked FP4 into column blocks
with new scales.  The element format (E2M1) and the power-of-two scale byte
(E8M0) are the OCP microscaling formats "MXFP4" names; the abstract gives
no scale rule, so this codec takes the same reading as the MXFP8 codec
(``mx_ref``), with E2M1's largest value 6 = 1.5 * 2^2:

  * amax = max |v| over the block of 32;
  * scale exponent e = clamp(floor(log2 amax) - 2, -127, 127); an all-zero
    block takes e = -127; the stored byte is e + 127;
  * code = E2M1(v / 2^e): the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes
    0..7; bit 3 is the sign, bit 0 the mantissa), ties to the even code,
    saturated to +-6; the sign survives rounding to zero (-0 -> 0x8);
  * decode: E2M1 value * 2^(byte - 127);
  * storage: two codes a byte, the element of lower index in the low
    nibble (the layout is the GPU path's; this module returns one code per
    array element).

Pinned by tests/test_oracle_mx4_pins.py: every finite bfloat16 bit pattern
under a sweep of block exponents against a brute-force nearest-value
search over the E2M1 table, the scale exponent against a search for the
smallest e that keeps |v|/2^e below 8, hand-derived points
(tests/golden/e2m1_points.json), and the half-spacing error bound.
"""

import numpy as np

E2M1_MAX = 6.0
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
MX_BLOCK = 32


def e2m1_round(v):
    """Nearest E2M1 value (ties to even code), saturated to +-6; the sign of
    v is kept.  float64 in and out."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)                   # a = m * 2^ex, m in [0.5, 1)
    binade = np.maximum(ex - 1, 0)        # [0, 2) share the 0.5 spacing
    spacing = np.ldexp(1.0, binade - 1)   # one mantissa bit
    q = np.rint(a / spacing) * spacing    # rint: half to even multiple
    q = np.minimum(q, E2M1_MAX)
    return np.copysign(q, v)


def e2m1_encode(v):
    """uint8 E2M1 codes (0..15) of v, rounded as in e2m1_round."""
    v = np.asarray(v, dtype=np.float64)
    q = np.abs(e2m1_round(v))
    code = np.searchsorted(E2M1_VALUES, q).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 3)


def e2m1_decode(codes):
    c = np.asarray(codes).astype(np.int64)
    return np.where(c & 8, -1.0, 1.0) * E2M1_VALUES[c & 7]


def e8m0_exponent4(amax):
    """Block scale exponent for block maxima amax (any shape)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)
    e = np.clip((ex - 1) - 2, -127, 127)  # floor(log2 amax) - emax(E2M1)
    return np.where(amax == 0.0, -127, e).astype(np.int64)


def quantize_blocks4(v):
    """Blocks along the last axis (length <= 32).  Returns (codes uint8 of
    v's shape, scale bytes uint8 of shape[:-1])."""
    v = np.asarray(v, dtype=np.float64)
    e = e8m0_exponent4(np.max(np.abs(v), axis=-1))
    codes = e2m1_encode(v / np.ldexp(1.0, e)[..., None])
    return codes, (e + 127).astype(np.uint8)


def dequantize_blocks4(codes, scales):
    e = np.asarray(scales).astype(np.int64) - 127
    return e2m1_decode(codes) * np.ldexp(1.0, e)[..., None]


def quantize_rows4(a):
    """MXFP4 along the last axis of [R, C] (C % 32 == 0): codes [R, C] (one
    a element), scales [R, C/32]."""
    a = np.asarray(a, dtype=np.float64)
    R, C = a.shape
    if C % MX_BLOCK:
        raise ValueError("columns must be a multiple of 32")
    codes, scales = quantize_blocks4(a.reshape(R, C // MX_BLOCK, MX_BLOCK))
    return codes.reshape(R, C), scales


def dequantize_rows4(codes, scales):
    R, C = codes.shape
    return dequantize_blocks4(codes.reshape(R, C // MX_BLOCK, MX_BLOCK),
                              scales).reshape(R, C)


def quantize_segments4(a, seg_offsets):
    """MXFP4 along the rows of [R, C], blocks of 32 rows restarting at each
    segment start (the last block of a segment holds the remaining rows).
    Returns (codes [R, C], list of (row0, row1, scale bytes [C]))."""
    a = np.asarray(a, dtype=np.float64)
    codes = np.zeros(a.shape, dtype=np.uint8)
    blocks = []
    offs = [int(o) for o in seg_offsets]
    for s in range(len(offs) - 1):
        for b0 in range(offs[s], offs[s + 1], MX_BLOCK):
            b1 = min(b0 + MX_BLOCK, offs[s + 1])
            c, sc = quantize_blocks4(a[b0:b1].T)
            codes[b0:b1] = c.T
            blocks.append((b0, b1, sc))
    return codes, blocks


def dequantize_segments4(codes, blocks):
    out = np.zeros(codes.shape, dtype=np.float64)
    for b0, b1, sc in blocks:
        out[b0:b1] = dequantize_blocks4(codes[b0:b1].T, sc).T
    return out


def pack_nibbles(codes):
    """Two codes a byte along the last axis (even index in the low
    nibble)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
