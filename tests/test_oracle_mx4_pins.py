"""Pins of the oracle's MXFP4 codec (oracle/mx4_ref.py): every finite
bfloat16 bit pattern, under a sweep of block exponents, against a
brute-force nearest-value search over the E2M1 table built from the bit
fields; hand-worked format points; the block-scale rule against a direct
search; the half-spacing error bound; segment-restarting token-axis
blocks; and the nibble packing.  CPU only."""

import json
import os

import numpy as np
import pytest

from oracle import mx4_ref as M4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v32 = bits.view(np.float32)
    return v32[np.isfinite(v32)].astype(np.float64)


def _e2m1_table():
    """Non-negative E2M1 values, code by code from the fields (two
    exponent bits with bias 1, one mantissa bit, subnormal at exponent
    field 0)."""
    vals = []
    for code in range(8):
        e, m = code >> 1, code & 1
        vals.append(m * 0.5 if e == 0 else (1 + m / 2.0) * 2.0 ** (e - 1))
    return np.array(vals)


def _bruteforce(v):
    """(value, code) of the nearest table entry; on a tie the even code;
    beyond the table the largest."""
    tab = _e2m1_table()
    a = np.abs(v)
    d = np.abs(a[:, None] - tab[None, :])
    best = np.min(d, axis=1, keepdims=True)
    cand = d == best
    # among the closest entries prefer an even code (a tie has one of each)
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    code = np.where(even.any(axis=1), np.argmax(even, axis=1),
                    np.argmax(cand, axis=1))
    code = np.where(a > tab[-1], 7, code)
    val = np.copysign(tab[code], v)
    return val, (code | (np.signbit(v) << 3)).astype(np.uint8)


@pytest.mark.parametrize("shift", [0, -1, 2, -7, 5, 120, -130])
def test_e2m1_round_exhaustive_bf16(shift):
    v = np.ldexp(_all_finite_bf16(), shift)
    v = v[np.isfinite(v)]
    ref_val, ref_code = _bruteforce(v)
    np.testing.assert_array_equal(M4.e2m1_round(v), ref_val)
    np.testing.assert_array_equal(M4.e2m1_encode(v), ref_code)


def test_e2m1_decode_all_codes():
    tab = _e2m1_table()
    codes = np.arange(16, dtype=np.uint8)
    dec = M4.e2m1_decode(codes)
    np.testing.assert_array_equal(np.abs(dec), np.concatenate([tab, tab]))
    assert np.all(np.signbit(dec[8:]) | (dec[8:] == 0))
    # every code survives decode -> encode (the signed zero included)
    np.testing.assert_array_equal(
        M4.e2m1_encode(np.where(codes >= 8, -1.0, 1.0) * np.abs(dec)), codes)


def test_e2m1_hand_points():
    with open(os.path.join(GOLDEN, "e2m1_points.json")) as fh:
        pts = json.load(fh)["points"]
    for p in pts:
        v = float(eval(p["value"], {"__builtins__": {}}))
        got = int(M4.e2m1_encode(np.array([v]))[0])
        assert got == int(p["code"], 16), (p, hex(got))


def _search_exponent(amax):
    """Smallest e in [-127, 127] with amax / 2^e < 8 (E2M1's top binade
    ends at 8); zero gives -127."""
    if amax == 0.0:
        return -127
    e = -300
    while amax / 2.0 ** e >= 8.0:
        e += 1
    return int(np.clip(e, -127, 127))


def test_scale_exponent_against_search():
    rng = np.random.default_rng(0)
    amax = np.concatenate([
        np.abs(_all_finite_bf16())[::97],
        2.0 ** rng.integers(-140, 128, 500),
        [0.0, 2.0 ** -149, 2.0 ** -126, 6.0, 7.99, 8.0, 3.3e38]])
    got = M4.e8m0_exponent4(amax)
    ref = np.array([_search_exponent(a) for a in amax])
    np.testing.assert_array_equal(got, ref)


def test_block_quantize_error_bound_and_saturation():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((4000, 32)) * 2.0 ** rng.integers(
        -30, 30, (4000, 1))
    v[::7, 3] *= 100.0
    v = v.astype(np.float32).astype(np.float64)
    codes, scales = M4.quantize_blocks4(v)
    deq = M4.dequantize_blocks4(codes, scales)
    e = scales.astype(np.int64) - 127
    w = v / np.ldexp(1.0, e)[:, None]
    aw = np.abs(w)
    # half a step: 0.25 below 2, 2^(binade - 2) above
    binade = np.floor(np.log2(np.where(aw > 0, aw, 1.0)))
    half = np.where(aw < 2.0, 0.25, 2.0 ** (binade - 2))
    unsat = aw <= 6.0
    err = np.abs(w - deq / np.ldexp(1.0, e)[:, None])
    assert np.all(err[unsat] <= half[unsat])
    top = np.max(aw, axis=1)
    assert np.all((top >= 4.0) & (top < 8.0))
    sat = aw > 6.0
    np.testing.assert_array_equal(
        np.abs(deq[sat]), (6.0 * np.ldexp(1.0, e)[:, None]
                           * np.ones_like(v))[sat])


def test_zero_block():
    codes, scales = M4.quantize_blocks4(np.zeros((1, 32)))
    assert scales[0] == 0 and np.all(codes == 0)
    codes, scales = M4.quantize_blocks4(-np.zeros((1, 32)))
    assert scales[0] == 0 and np.all(codes == 0x8)


def test_rows_segments_and_packing():
    rng = np.random.default_rng(2)
    a = rng.standard_normal((70, 64)).astype(np.float32).astype(np.float64)
    codes, scales = M4.quantize_rows4(a)
    assert scales.shape == (70, 2) and codes.max() < 16
    np.testing.assert_array_equal(codes[:, 32:],
                                  M4.quantize_blocks4(a[:, 32:])[0])
    offs = [0, 0, 33, 33, 70]
    sc, blocks = M4.quantize_segments4(a, offs)
    assert [(b0, b1) for b0, b1, _ in blocks] == [(0, 32), (32, 33),
                                                  (33, 65), (65, 70)]
    for b0, b1, s in blocks:
        c, s_ref = M4.quantize_blocks4(a[b0:b1].T)
        np.testing.assert_array_equal(sc[b0:b1], c.T)
        np.testing.assert_array_equal(s, s_ref)
    # packing: element 2i in the low nibble of byte i
    p = M4.pack_nibbles(codes)
    assert p.shape == (70, 32)
    np.testing.assert_array_equal(p[:, 0] & 0xF, codes[:, 0])
    np.testing.assert_array_equal(p[:, 0] >> 4, codes[:, 1])
    np.testing.assert_array_equal(M4.unpack_nibbles(p), codes)
