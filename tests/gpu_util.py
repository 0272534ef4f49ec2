"""Helpers for the GPU parity tests: move seeded inputs to the device, run
the library through its binding, and compare with the oracle."""

from __future__ import annotations

import sys

import numpy as np

TOL_O = 1e-2    # max abs error on the bf16 output
TOL_LSE = 1e-3  # max abs error on lse


def say(*args):
    print("[gpu-case]", *args, file=sys.stderr, flush=True)


def bits_to_dev(bits: np.ndarray):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_to_f64(t) -> np.ndarray:
    import torch

    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def dev_bits(t) -> np.ndarray:
    """Bit patterns of a 2-byte (bf16) or 1-byte (FP8 codes) device tensor."""
    import torch

    if t.element_size() == 1:
        return t.detach().contiguous().view(torch.uint8).cpu().numpy()
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def codes_to_dev(codes: np.ndarray):
    """uint8 E4M3 codes to a float8_e4m3fn tensor on the GPU."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).cuda().view(
        torch.float8_e4m3fn)


_RUNNERS = {}


def runner(max_batch=512, max_nnz=1 << 17, max_qo_heads=64, num_slots=0):
    import paged_kv_decode_11_amd as pkd

    key = (max_batch, max_nnz, max_qo_heads, num_slots)
    if key not in _RUNNERS:
        _RUNNERS[key] = pkd.DecodePlanRun(max_batch, max_nnz, max_qo_heads, 128, num_slots)
    return _RUNNERS[key]


def decode(batch, q_dev, cache_dev, r=None, sm_scale=None, return_lse=True, **opts):
    """Plan + run; returns (o [B,Hq,D] bf16 tensor, lse tensor or None)."""
    import torch

    r = r or runner()
    idx = torch.from_numpy(batch.kv_indices.astype(np.int32)).cuda()
    r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, batch.num_qo_heads, batch.num_kv_heads,
           batch.head_dim, batch.page_size, **opts)
    res = r.run(q_dev, cache_dev, return_lse=return_lse, sm_scale=sm_scale)
    torch.cuda.synchronize()
    return res if return_lse else (res, None)


def o_tolerance(o_ref: np.ndarray) -> np.ndarray:
    """Elementwise bound on |o - o_ref| for a bf16 output: 1e-2, or, where a
    correctly rounded bf16 value can itself be further off (|o_ref| >= 4, half
    an ulp is 2**(e - 8) for |o_ref| in [2**e, 2**(e + 1))), that half ulp
    plus 1e-3 of fp32 arithmetic."""
    a = np.abs(o_ref)
    e = np.floor(np.log2(np.maximum(a, 1e-30)))
    return np.maximum(TOL_O, np.exp2(e - 8) + 1e-3)


def check_o(o_got: np.ndarray, o_ref: np.ndarray, label=""):
    """o against the oracle within o_tolerance.  Elements whose bound is
    above 1e-2 (|o_ref| >= 4, where a correctly rounded bf16 value may itself
    be further off) are reported on stderr, so a run shows when the relaxed
    part of the bound was used."""
    assert np.all(np.isfinite(o_got)), f"{label}: non-finite output"
    err = np.abs(o_got - o_ref)
    tol = o_tolerance(o_ref)
    bad = err > tol
    assert not bad.any(), (f"{label}: {int(bad.sum())} elements over tolerance; "
                           f"max |o - o_ref| = {err.max()} at |o_ref| = "
                           f"{np.abs(o_ref).ravel()[np.argmax(err)]}")
    wide = tol > TOL_O
    if wide.any():
        say(f"{label}: {int(wide.sum())} of {wide.size} outputs have |o_ref| >= 4 (bound half a "
            f"bf16 ulp + 1e-3); largest error there {float(err[wide].max()):.3g}, elsewhere "
            f"{float(err[~wide].max()) if (~wide).any() else 0.0:.3g}")
    return float(err.max())


def check_lse(lse_got: np.ndarray, lse_ref: np.ndarray, label=""):
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_got), fin), f"{label}: lse finiteness differs"
    assert np.all(lse_got[~fin] == lse_ref[~fin]), f"{label}: infinite lse differs"
    err = float(np.max(np.abs(lse_got[fin] - lse_ref[fin]))) if fin.any() else 0.0
    assert err <= TOL_LSE, f"{label}: max |lse - lse_ref| = {err}"
    return err


def assert_close(o_dev, lse_dev, o_ref, lse_ref, requests=None, label=""):
    o = dev_to_f64(o_dev)
    rows = slice(None) if requests is None else list(requests)
    err_o = check_o(o[rows], o_ref[rows], label)
    if lse_dev is not None:
        lse = lse_dev.detach().cpu().numpy().astype(np.float64)
        return err_o, check_lse(lse[rows], lse_ref[rows], label)
    return err_o, None


def compact_pages(batch, cache_dev, requests):
    """Copy the pages of `requests` from a device cache to the host; return a
    compact host cache and the remapped page table for those requests (as a
    smaller batch, in the given order)."""
    import torch

    rows, lens = [], []
    for i in requests:
        rows.append(batch.kv_indices[batch.kv_indptr[i]:batch.kv_indptr[i + 1]])
        lens.append(int(batch.kv_lens[i]))
    pages = np.unique(np.concatenate(rows))
    sel = torch.from_numpy(pages.astype(np.int64)).cuda()
    host = dev_bits(cache_dev.index_select(0, sel))
    remap = {int(p): j for j, p in enumerate(pages)}
    indptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    indices = np.array([remap[int(p)] for r in rows for p in r], dtype=np.int32)
    last = np.array([batch.kv_last_page_len[i] for i in requests], dtype=np.int32)
    return host, indptr, indices, last
