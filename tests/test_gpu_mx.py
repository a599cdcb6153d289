"""GPU parity of the MXFP8 quantizer (moe_mxfp8_quantize) against the
oracle codec: codes and scale bytes bit-exact.

Row blocks: every finite bfloat16 bit pattern appears as an element, in
blocks of similar magnitude (sorted) and of mixed magnitude (shuffled), so
every scale exponent, the subnormal range, ties and saturation are hit.
Token blocks: segments restarting the 32-row blocks, empty and ragged
segments, the 128-row padding of the transposed layout."""

import numpy as np
import pytest
import torch

from oracle import mx_ref as M

gpu = pytest.mark.gpu
if torch.cuda.is_available():
    from mixture_experts_expert_top_amd import moe


def _dev():
    return torch.device("cuda:0")


def _all_finite_bf16_bits():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = (bits.astype(np.uint32) << 16).view(np.float32)
    return bits[np.isfinite(v)]


def _to_gpu_bf16(bits16):
    return torch.from_numpy(bits16.view(np.int16).copy()).to(_dev()).view(
        torch.bfloat16)


def _as_f64(bits16):
    return (bits16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _quant_rows_gpu(bits16_2d):
    R, C = bits16_2d.shape
    src = _to_gpu_bf16(bits16_2d.reshape(-1)).reshape(R, C)
    codes = torch.empty(R, C, dtype=torch.uint8, device=_dev())
    scales = torch.empty(R, C // 32, dtype=torch.uint8, device=_dev())
    moe.moe_mxfp8_quantize(src, 0, None, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


@gpu
@pytest.mark.parametrize("arrangement", ["sorted", "shuffled", "reversed"])
def test_quantize_rows_every_bf16(arrangement):
    bits = _all_finite_bf16_bits()
    vals = _as_f64(bits)
    if arrangement == "sorted":
        order = np.argsort(np.abs(vals), kind="stable")
    elif arrangement == "shuffled":
        order = np.random.default_rng(0).permutation(bits.size)
    else:
        order = np.argsort(-np.abs(vals), kind="stable")
    bits = bits[order]
    n = bits.size // 256 * 256
    blk = bits[:n].reshape(-1, 256)                     # rows of 8 blocks
    codes, scales = _quant_rows_gpu(blk)
    ref_codes, ref_scales = M.quantize_rows(_as_f64(blk))
    np.testing.assert_array_equal(scales, ref_scales)
    np.testing.assert_array_equal(codes, ref_codes)


@gpu
def test_quantize_rows_special_blocks():
    rng = np.random.default_rng(1)
    rows = []
    rows.append(np.zeros(64))                          # zero block -> byte 0
    rows.append(-np.zeros(64))                         # -0 keeps its sign
    rows.append(np.full(64, 448.0))
    rows.append(np.full(64, 2.0 ** -133))              # bf16 subnormals
    r = rng.standard_normal(64)
    r[3] = 1e4                                         # outlier in block 0
    rows.append(r)
    rows.append(rng.standard_normal(64) * 1e-30)
    a = np.stack(rows).astype(np.float32)
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)    # truncate to bf16
    codes, scales = _quant_rows_gpu(bits)
    ref_codes, ref_scales = M.quantize_rows(_as_f64(bits))
    np.testing.assert_array_equal(scales, ref_scales)
    np.testing.assert_array_equal(codes, ref_codes)
    assert scales[0, 0] == 0 and np.all(codes[1] == 0x80)


def _expected_tokens(a64, offs, rows_pad):
    """Oracle segment blocks mapped to the transposed, 128-padded layout."""
    R, C = a64.shape
    codes_ref, blocks = M.quantize_segments(a64, offs)
    exp_codes = np.zeros((C, rows_pad), dtype=np.uint8)
    exp_scales = np.zeros((C, rows_pad // 32), dtype=np.uint8)
    pad_off = 0
    for s in range(len(offs) - 1):
        s0, s1 = offs[s], offs[s + 1]
        exp_codes[:, pad_off:pad_off + (s1 - s0)] = codes_ref[s0:s1].T
        for b0, b1, sc in blocks:
            if s0 <= b0 < s1:
                exp_scales[:, (pad_off + (b0 - s0)) // 32] = sc
        pad_off += (s1 - s0 + 127) // 128 * 128
    return exp_codes, exp_scales


@gpu
@pytest.mark.parametrize("offs", [
    [0, 300],                              # one segment (passed as NULL)
    [0, 0, 33, 33, 70, 200, 201],          # empty, ragged, single-row
    [0, 128, 256, 300, 512],               # exact multiples
])
def test_quantize_tokens_segments(offs):
    rng = np.random.default_rng(len(offs))
    R, C = offs[-1], 264
    a = (rng.standard_normal((R, C)) *
         2.0 ** rng.integers(-20, 20, (R, 1))).astype(np.float32)
    a[::17] *= 300.0
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    a64 = _as_f64(bits)
    nseg = len(offs) - 1
    rows_pad = moe.moe_mxfp8_padded_rows(R, nseg)
    src = _to_gpu_bf16(bits.reshape(-1)).reshape(R, C)
    codes = torch.full((C, rows_pad), 0x5A, dtype=torch.uint8, device=_dev())
    scales = torch.full((C, rows_pad // 32), 0x5A, dtype=torch.uint8,
                        device=_dev())
    seg = None if nseg == 1 else torch.tensor(offs, dtype=torch.int32,
                                              device=_dev())
    moe.moe_mxfp8_quantize(src, 1, seg, codes, scales, rows_pad)
    torch.cuda.synchronize()
    exp_codes, exp_scales = _expected_tokens(a64, offs, rows_pad)
    np.testing.assert_array_equal(scales.cpu().numpy(), exp_scales)
    np.testing.assert_array_equal(codes.cpu().numpy(), exp_codes)


@gpu
@pytest.mark.parametrize("R,C", [(128, 64), (256, 320), (384, 1024), (128, 576)])
def test_quantize_weight_both_layouts(R, C):
    """moe_mxfp8_quantize_weight: the row-wise codes equal the oracle's row
    blocks and the column-wise (transposed) codes its one-segment blocks
    along the rows, and both equal the two separate moe_mxfp8_quantize
    calls bit for bit."""
    rng = np.random.default_rng(R + C)
    a = (rng.standard_normal((R, C)) *
         2.0 ** rng.integers(-30, 30, (R, 1))).astype(np.float32)
    a[:, ::13] *= 500.0
    a[5] = 0.0                              # an all-zero row block
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    a64 = _as_f64(bits)
    src = _to_gpu_bf16(bits.reshape(-1)).reshape(R, C)
    u8 = dict(dtype=torch.uint8, device=_dev())
    rc, rs = torch.full((R, C), 0x5A, **u8), torch.full((R, C // 32), 0x5A, **u8)
    cc, cs = torch.full((C, R), 0x5A, **u8), torch.full((C, R // 32), 0x5A, **u8)
    moe.moe_mxfp8_quantize_weight(src, rc, rs, cc, cs)
    sep_rc, sep_rs = torch.empty_like(rc), torch.empty_like(rs)
    sep_cc, sep_cs = torch.empty_like(cc), torch.empty_like(cs)
    moe.moe_mxfp8_quantize(src, 0, None, sep_rc, sep_rs)
    moe.moe_mxfp8_quantize(src, 1, None, sep_cc, sep_cs, R)
    torch.cuda.synchronize()
    codes_ref, scales_ref = M.quantize_rows(a64)
    np.testing.assert_array_equal(rc.cpu().numpy(), codes_ref)
    np.testing.assert_array_equal(rs.cpu().numpy(), scales_ref)
    exp_codes, exp_scales = _expected_tokens(a64, [0, R], R)
    np.testing.assert_array_equal(cc.cpu().numpy(), exp_codes)
    np.testing.assert_array_equal(cs.cpu().numpy(), exp_scales)
    for got, sep in ((rc, sep_rc), (rs, sep_rs), (cc, sep_cc), (cs, sep_cs)):
        assert torch.equal(got, sep)
