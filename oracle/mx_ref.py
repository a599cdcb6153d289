"""MXFP8 block codec (E4M3 element codes, one E8M0 scale per 32 values).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Efficient MoE Training for Biological Foundation Models", Challenge 2:
MXFP8 stores 8-bit values and gives every block of 32 consecutive values its
own scaling factor.  The element format (E4M3) and the power-of-two scale
byte (E8M0) are the OCP microscaling formats the name refers to; the pages
do not spell out the scale rule, so this codec takes the plainest reading of
"MX" block scaling:

  * amax = max |v| over the block;
  * scale exponent e = clamp(floor(log2 amax) - 8, -127, 127), with 8 the
    exponent of E4M3's largest normal (448 = 1.75 * 2^8); an all-zero block
    takes e = -127; the stored byte is e + 127;
  * code = E4M3(v / 2^e), rounded to nearest, ties to even mantissa, and
    saturated to +-448 (E4M3 "FN": bias 7, no infinities, 0x7F/0xFF NaN,
    subnormal step 2^-9); the sign survives rounding to zero (-0 -> 0x80);
  * decode: E4M3 value * 2^(byte - 127).

Pinned by tests/test_oracle_pins.py: every finite bfloat16 bit pattern
against a brute-force nearest-value search over the E4M3 table, torch's
float8_e4m3fn cast wherever no saturation happens, the scale exponent
against a search for the smallest e that keeps |v|/2^e below 2^9, and the
half-spacing error bound.
"""

import numpy as np

E4M3_MAX = 448.0
MX_BLOCK = 32


def e4m3_round(v):
    """Nearest E4M3 value (ties to even mantissa), saturated to +-448.
    Input and output are float64 arrays; the sign of v is kept."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)                   # a = m * 2^ex, m in [0.5, 1)
    binade = np.maximum(ex - 1, -6)       # subnormals share the 2^-6 binade
    spacing = np.ldexp(1.0, binade - 3)   # 3 mantissa bits
    q = np.rint(a / spacing) * spacing    # rint: half to even multiple
    q = np.minimum(q, E4M3_MAX)
    return np.copysign(q, v)


def e4m3_encode(v):
    """uint8 E4M3 codes of v (rounded and saturated as in e4m3_round)."""
    v = np.asarray(v, dtype=np.float64)
    q = np.abs(e4m3_round(v))
    sign = np.signbit(v).astype(np.uint8) << 7
    _, ex = np.frexp(q)
    e_unb = ex - 1
    normal = q >= 2.0 ** -6
    # normal: (1 + m/8) * 2^E, biased exponent E + 7 in bits 6..3
    mant_n = np.where(normal, q / np.ldexp(1.0, e_unb) * 8.0 - 8.0, 0.0)
    code_n = ((e_unb + 7).astype(np.int64) << 3) + mant_n.astype(np.int64)
    # subnormal: m * 2^-9
    code_s = (q / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_n, code_s).astype(np.uint8)
    return code | sign


def e4m3_decode(codes):
    """float64 values of uint8 E4M3 codes (0x7F/0xFF decode to NaN)."""
    c = np.asarray(codes).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9,
                   (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    out = s * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e8m0_exponent(amax):
    """Block scale exponent e for block maxima amax (any shape)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)
    e = (ex - 1) - 8                      # floor(log2 amax) - emax(E4M3)
    e = np.clip(e, -127, 127)
    return np.where(amax == 0.0, -127, e).astype(np.int64)


def quantize_blocks(v):
    """Quantize blocks laid out along the last axis (length <= 32 each
    block; the caller reshapes).  Returns (codes uint8 same shape,
    scale bytes uint8 shape[:-1])."""
    v = np.asarray(v, dtype=np.float64)
    amax = np.max(np.abs(v), axis=-1)
    e = e8m0_exponent(amax)
    codes = e4m3_encode(v / np.ldexp(1.0, e)[..., None])
    return codes, (e + 127).astype(np.uint8)


def dequantize_blocks(codes, scales):
    """Inverse of quantize_blocks (exact)."""
    e = np.asarray(scales).astype(np.int64) - 127
    return e4m3_decode(codes) * np.ldexp(1.0, e)[..., None]


def quantize_rows(a):
    """MX along the last axis of a 2-D array [R, C] (C % 32 == 0): blocks of
    32 consecutive columns.  Returns codes [R, C] and scales [R, C/32]."""
    a = np.asarray(a, dtype=np.float64)
    R, C = a.shape
    if C % MX_BLOCK:
        raise ValueError("columns must be a multiple of 32")
    codes, scales = quantize_blocks(a.reshape(R, C // MX_BLOCK, MX_BLOCK))
    return codes.reshape(R, C), scales


def dequantize_rows(codes, scales):
    R, C = codes.shape
    return dequantize_blocks(codes.reshape(R, C // MX_BLOCK, MX_BLOCK),
                             scales).reshape(R, C)


def quantize_segments(a, seg_offsets):
    """MX along rows of a [R, C], blocks of 32 consecutive rows that restart
    at each segment start seg_offsets[s] (the last block of a segment holds
    the remaining rows; its amax covers those rows only).

    Returns (codes [R, C] uint8, scales list of (row0, row1, bytes[C])).
    """
    a = np.asarray(a, dtype=np.float64)
    codes = np.zeros(a.shape, dtype=np.uint8)
    blocks = []
    offs = [int(o) for o in seg_offsets]
    for s in range(len(offs) - 1):
        for b0 in range(offs[s], offs[s + 1], MX_BLOCK):
            b1 = min(b0 + MX_BLOCK, offs[s + 1])
            c, sc = quantize_blocks(a[b0:b1].T)      # blocks along rows
            codes[b0:b1] = c.T
            blocks.append((b0, b1, sc))
    return codes, blocks


def dequantize_segments(codes, blocks):
    out = np.zeros(codes.shape, dtype=np.float64)
    for b0, b1, sc in blocks:
        out[b0:b1] = dequantize_blocks(codes[b0:b1].T, sc).T
    return out
