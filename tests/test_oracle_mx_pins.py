"""Pins of the oracle's MXFP8 codec: every finite bfloat16 bit pattern
against a brute-force nearest-value search over the E4M3 table, torch's
float8_e4m3fn cast where no saturation happens, hand-worked format points,
the block-scale rule against a direct search, the half-spacing error bound
and the segment-restarting token-axis blocks.  CPU only."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import mx_ref as M

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v32 = bits.view(np.float32)
    return v32[np.isfinite(v32)].astype(np.float64)


def _e4m3_table():
    """All non-negative finite E4M3 values from the bit layout: code ->
    value, built from the field definitions one code at a time."""
    vals = []
    for code in range(0x7F):                  # 0x7F is NaN
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(m / 8.0 * 2.0 ** -6)
        else:
            vals.append((1 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals)


def _bruteforce_round(v):
    """Nearest finite E4M3 value by search: bracket |v| between the table
    neighbours lo <= |v| <= hi and keep the closer one (the even code on a
    tie); above the largest finite value only lo exists."""
    tab = _e4m3_table()
    a = np.abs(v)
    i_hi = np.searchsorted(tab, a, side="left")      # first tab >= a
    i_lo = np.clip(i_hi - 1, 0, tab.size - 1)
    exact = (i_hi < tab.size) & (tab[np.minimum(i_hi, tab.size - 1)] == a)
    out = np.empty_like(a)
    for n in range(a.size):
        if exact[n]:
            out[n] = a[n]
            continue
        if i_hi[n] >= tab.size:                      # beyond the table
            out[n] = tab[-1]
            continue
        lo, hi = i_lo[n], i_hi[n]
        dl, dh = a[n] - tab[lo], tab[hi] - a[n]
        if dl < dh:
            out[n] = tab[lo]
        elif dh < dl:
            out[n] = tab[hi]
        else:
            out[n] = tab[lo] if lo % 2 == 0 else tab[hi]
    return np.copysign(out, v)


@pytest.mark.parametrize("shift", [0, -3, 5, -9, 9, 120, -130])
def test_e4m3_round_exhaustive_bf16(shift):
    v = _all_finite_bf16() * 2.0 ** shift
    got = M.e4m3_round(v)
    ref = _bruteforce_round(v)
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(np.signbit(got), np.signbit(v))


def test_e4m3_encode_decode_roundtrip_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    vals = M.e4m3_decode(codes)
    finite = np.isfinite(vals)
    assert (~finite).sum() == 2                 # 0x7F and 0xFF
    np.testing.assert_array_equal(M.e4m3_encode(vals[finite]),
                                  codes[finite])


def test_e4m3_matches_torch_cast_without_saturation():
    v = _all_finite_bf16()
    v = v[np.abs(v) <= 448.0]
    ours = M.e4m3_encode(v)
    theirs = torch.from_numpy(v.astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, theirs)


def test_e4m3_hand_points():
    with open(os.path.join(GOLDEN, "e4m3_points.json")) as fh:
        pts = json.load(fh)["points"]
    for p in pts:
        v = float(eval(p["value"]))
        assert int(M.e4m3_encode(np.array([v]))[0]) == int(p["code"], 16), p


def _search_exponent(amax):
    """Smallest e with amax / 2^e < 2^9 (the top binade of a block lands on
    [256, 512)), clamped to [-127, 127]; zero blocks take -127."""
    if amax == 0.0:
        return -127
    e = -300
    while amax / 2.0 ** e >= 512.0:
        e += 1
    return int(np.clip(e, -127, 127))


def test_scale_exponent_against_search():
    rng = np.random.default_rng(0)
    amax = np.concatenate([
        np.abs(_all_finite_bf16())[::97],
        2.0 ** rng.integers(-140, 128, 500),
        [0.0, 2.0 ** -149, 2.0 ** -126, 448.0, 511.9, 512.0, 3.3e38]])
    got = M.e8m0_exponent(amax)
    ref = np.array([_search_exponent(a) for a in amax])
    np.testing.assert_array_equal(got, ref)


def test_block_quantize_error_bound_and_saturation():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((4000, 32)) * 2.0 ** rng.integers(
        -30, 30, (4000, 1))
    v[::7, 3] *= 100.0                         # an outlier per block
    v = v.astype(np.float32).astype(np.float64)
    codes, scales = M.quantize_blocks(v)
    deq = M.dequantize_blocks(codes, scales)
    e = scales.astype(np.int64) - 127
    w = v / np.ldexp(1.0, e)[:, None]
    aw = np.abs(w)
    unsat = (aw <= 448.0) & (aw >= 2.0 ** -6)
    binade = np.floor(np.log2(np.where(aw > 0, aw, 1.0)))
    bound = np.ldexp(1.0, e)[:, None] * 2.0 ** -4 * 2.0 ** binade
    assert np.all(np.abs(v - deq)[unsat] <= bound[unsat])
    # every block's largest element lands in the top binade [256, 512)
    top = np.max(aw, axis=1)
    assert np.all((top >= 256.0) & (top < 512.0))
    # saturated elements decode to exactly +-448 * 2^e
    sat = aw > 448.0
    np.testing.assert_array_equal(
        np.abs(deq[sat]), (448.0 * np.ldexp(1.0, e)[:, None]
                           * np.ones_like(v))[sat])


def test_zero_block():
    codes, scales = M.quantize_blocks(np.zeros((1, 32)))
    assert scales[0] == 0 and np.all(codes == 0)
    codes, scales = M.quantize_blocks(-np.zeros((1, 32)))
    assert scales[0] == 0 and np.all(codes == 0x80)


def test_rows_and_segments():
    rng = np.random.default_rng(2)
    a = rng.standard_normal((70, 64)).astype(np.float32).astype(np.float64)
    codes, scales = M.quantize_rows(a)
    assert scales.shape == (70, 2)
    np.testing.assert_array_equal(
        codes[:, 32:], M.quantize_blocks(a[:, 32:])[0])
    offs = [0, 0, 33, 33, 70]                  # empty and ragged segments
    sc, blocks = M.quantize_segments(a, offs)
    spans = [(b0, b1) for b0, b1, _ in blocks]
    assert spans == [(0, 32), (32, 33), (33, 65), (65, 70)]
    # a block's codes are those of the same rows quantized on their own
    for b0, b1, s in blocks:
        c, s_ref = M.quantize_blocks(a[b0:b1].T)
        np.testing.assert_array_equal(sc[b0:b1], c.T)
        np.testing.assert_array_equal(s, s_ref)
    deq = M.dequantize_segments(sc, blocks)
    assert np.max(np.abs(deq - a)) <= 2.0 ** -4 * np.max(np.abs(a)) * 2
