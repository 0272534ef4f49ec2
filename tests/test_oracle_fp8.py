"""Pins for oracle.fp8 and the FP8-cache paths of the oracle: every E4M3
code against torch's independent float8_e4m3fn conversion, rounding of
in-range values against torch, the saturation reading by hand, FP8 decode
against the pinned bf16 decode on the same values, the scales' closed
forms, and the quantising append against a plain append of pre-quantised
rows."""

import numpy as np
import pytest
import torch

from oracle import append as ap
from oracle import attention as att
from oracle import fp8
from oracle import page_table as pt


def test_every_code_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_rounding_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(4000) * s for s in (1e-3, 0.1, 1.0, 30.0, 200.0)])
    x = x[np.abs(x) <= 448.0]
    # exact ties: midpoints between neighbouring codes
    vals = fp8.e4m3_to_f64(np.arange(0, 126, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([x, mids, -mids]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.f64_to_e4m3(x.astype(np.float64)), ref)


def test_saturation_reading():
    got = fp8.f64_to_e4m3(np.array([464.0, 479.0, 480.0, 1e6, -1e6, np.nan, -0.0]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7F, 0x80]


def test_fp8_decode_equals_bf16_decode_on_the_same_values():
    # every E4M3 value is exactly a bf16 value: widen the codes to bf16 bits
    rng = np.random.default_rng(1)
    indptr, idx, last = pt.page_table([37, 16, 5, 90], 16)
    codes = rng.integers(0, 256, size=(int(indptr[-1]), 2, 16, 2, 16), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38  # no NaN codes
    vals = fp8.e4m3_to_f64(codes).astype(np.float32)
    bf16_bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(att.bf16_to_f64(bf16_bits), fp8.e4m3_to_f64(codes))
    q = (rng.standard_normal((4, 8, 16)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    o1, l1 = att.decode(q, bf16_bits, indptr, idx, last, 2)
    o2, l2 = att.decode_fp8(q, codes, indptr, idx, last, 2)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12) and np.allclose(l1, l2, rtol=0, atol=1e-12)
    # scales: k_scale multiplies the logits like sm_scale; v_scale scales o
    o3, l3 = att.decode_fp8(q, codes, indptr, idx, last, 2, k_scale=2.0, v_scale=0.5)
    o4, l4 = att.decode(q, bf16_bits, indptr, idx, last, 2, sm_scale=2.0 / 4.0)
    assert np.allclose(o3, 0.5 * o4, atol=1e-12) and np.allclose(l3, l4, atol=1e-12)


def test_quantised_append_equals_append_of_quantised_rows():
    rng = np.random.default_rng(2)
    indptr, idx, last = pt.page_table([20, 33], 16)
    cache = rng.integers(0, 120, size=(int(indptr[-1]), 2, 16, 2, 8), dtype=np.uint8)
    k = (rng.standard_normal((3, 2, 8)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    v = (rng.standard_normal((3, 2, 8)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    b, pos = np.array([0, 1, 1]), np.array([19, 31, 32])
    out = ap.append_quantized(cache, k, v, b, pos, indptr, idx, k_scale=0.5, v_scale=2.0)
    # power-of-two scales: x / scale is exact in any precision
    kq = fp8.f64_to_e4m3(att.bf16_to_f64(k) / 0.5)
    vq = fp8.f64_to_e4m3(att.bf16_to_f64(v) / 2.0)
    assert np.array_equal(out, ap.append(cache, kq, vq, b, pos, indptr, idx))
    assert fp8.e4m3_to_f64(out[idx[1], 0, 3]).tolist() == fp8.e4m3_to_f64(kq[0]).tolist()


def test_quantised_append_rounds_the_float32_product():
    """A non-power-of-two scale where the precision of x / scale decides the
    code.  x = 91 * 2^-10 (bf16 0x3DB6) and scale 7: the exact quotient is
    13 * 2^-10 = 6.5 * 2^-9, the midpoint of the E4M3 subnormal codes 0x06
    (6 * 2^-9) and 0x07 (7 * 2^-9), which ties to the even code 0x06.  The
    library's contract rounds the float32 product x * fl32(1 / 7) instead:
    fl32(1 / 7) = 0x3E124925 lies above 1 / 7 and the product rounds to
    0x3C500001, one float32 ulp above the midpoint, so the stored code is
    0x07 (0x87 for -x).  An oracle that divided in float64 gives 0x06 here."""
    assert np.float32(1.0 / 7.0).view(np.uint32) == 0x3E124925
    assert (np.float32(91 * 2.0 ** -10) * np.float32(1.0 / 7.0)).view(np.uint32) == 0x3C500001
    indptr, idx, last = pt.page_table([2], 16)
    cache = np.zeros((1, 2, 16, 1, 2), dtype=np.uint8)
    x = np.array([[[0x3DB6, 0xBDB6]]], dtype=np.uint16)   # +-91 * 2^-10, one token
    out = ap.append_quantized(cache, x, x, np.array([0]), np.array([1]), indptr, idx,
                              k_scale=7.0, v_scale=7.0)
    assert out[0, 0, 1, 0].tolist() == [0x07, 0x87]
    assert out[0, 1, 1, 0].tolist() == [0x07, 0x87]
    # the exact quotient would tie to the even code
    assert fp8.f64_to_e4m3(np.array([13 * 2.0 ** -10])).tolist() == [0x06]
    # x = 9 * 2^-10 and scale 0.6, received as fl32(0.6) = 0x3F19999A: the
    # exact x / fl32(0.6) lies just below the midpoint 7.5 * 2^-9 of codes 0x07
    # and 0x08, but the float32 product x * fl32(1 / fl32(0.6)) rounds to the
    # midpoint itself (0x3C700000), which ties to the even code 0x08
    assert np.float32(0.6).view(np.uint32) == 0x3F19999A
    inv = np.float32(1.0 / float(np.float32(0.6)))
    assert (np.float32(9 * 2.0 ** -10) * inv).view(np.uint32) == 0x3C700000
    y = np.array([[[0x3C10]]], dtype=np.uint16)            # 9 * 2^-10
    out6 = ap.append_quantized(np.zeros((1, 2, 16, 1, 1), np.uint8), y, y, np.array([0]),
                               np.array([0]), indptr, idx, k_scale=0.6, v_scale=0.6)
    assert out6[0, :, 0, 0, 0].tolist() == [0x08, 0x08]
    assert fp8.f64_to_e4m3(np.array([9 * 2.0 ** -10 / float(np.float32(0.6))])).tolist() == [0x07]
