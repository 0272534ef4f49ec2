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
