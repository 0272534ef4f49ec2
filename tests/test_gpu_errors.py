"""Failure modes at the boundary (aicassindra "Failure modes in production";
pinghaoyang, interface pitfalls): run before plan, a batch that is not the
planned one, dtype and layout mismatches, a workspace too small.  All are
refused on the host before any kernel runs."""

import numpy as np
import pytest

import workloads
from paged_kv_decode_11_amd import _lib
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _inputs():
    rng = np.random.default_rng(5)
    batch = workloads.make_batch([40, 3], 16, 16, 32, 8, 128, rng)
    q = workloads.host_query(batch, rng)
    cache = workloads.host_cache(batch, rng)
    return batch, gu.bits_to_dev(q), gu.bits_to_dev(cache)


def test_run_before_plan_is_stale():
    import paged_kv_decode_11_amd as pkd

    batch, q, cache = _inputs()
    r = pkd.DecodePlanRun(max_batch=4, max_nnz=64, max_qo_heads=32)
    with pytest.raises(pkd.PkdError) as e:
        r.run(q, cache)
    assert e.value.code == _lib.PKD_ERR_STALE_PLAN


def test_batch_mismatch_is_stale_and_plan_id_advances():
    import torch
    import paged_kv_decode_11_amd as pkd

    batch, q, cache = _inputs()
    r = pkd.DecodePlanRun(max_batch=4, max_nnz=64, max_qo_heads=32)
    assert r.plan_id == 0
    idx = torch.from_numpy(batch.kv_indices).cuda()
    r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, 32, 8, 128, 16)
    assert r.plan_id == 1
    r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, 32, 8, 128, 16)
    assert r.plan_id == 2
    with pytest.raises(pkd.PkdError) as e:
        r.run(q[:1].contiguous(), cache)
    assert e.value.code == _lib.PKD_ERR_STALE_PLAN


def test_dtype_and_layout_errors():
    import torch
    import paged_kv_decode_11_amd as pkd

    batch, q, cache = _inputs()
    r = pkd.DecodePlanRun(max_batch=4, max_nnz=64, max_qo_heads=32)
    idx = torch.from_numpy(batch.kv_indices).cuda()
    with pytest.raises(pkd.PkdError) as e:
        r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, 32, 8, 128, 16,
               q_data_type=torch.float16, kv_data_type=torch.float16)
    assert e.value.code == _lib.PKD_ERR_UNSUPPORTED
    with pytest.raises(pkd.PkdError) as e:
        r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, 32, 8, 128, 16, kv_layout="HND")
    assert e.value.code == _lib.PKD_ERR_UNSUPPORTED
    with pytest.raises(pkd.PkdError) as e:
        r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, 32, 8, 64, 16)
    assert e.value.code == _lib.PKD_ERR_UNSUPPORTED
    r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, 32, 8, 128, 16)
    with pytest.raises(pkd.PkdError) as e:
        r.run(q.to(torch.float16), cache)
    assert e.value.code == _lib.PKD_ERR_DTYPE_MISMATCH


def test_fp8_cache_errors():
    """An E4M3 cache: a page size and a kernel it is not built for, scales on
    a bf16 cache, invalid scales, and a run whose cache dtype is not the
    plan's."""
    import torch
    import paged_kv_decode_11_amd as pkd

    batch, q, cache = _inputs()
    fp8 = torch.float8_e4m3fn
    r = pkd.DecodePlanRun(max_batch=4, max_nnz=64, max_qo_heads=32)
    idx = torch.from_numpy(batch.kv_indices).cuda()
    args = (batch.kv_indptr, idx, batch.kv_last_page_len, 32, 8, 128)
    with pytest.raises(pkd.PkdError) as e:
        r.plan(*args, 128, kv_data_type=fp8)
    assert e.value.code == _lib.PKD_ERR_UNSUPPORTED
    with pytest.raises(pkd.PkdError) as e:
        r.plan(*args, 16, kv_data_type=fp8, variant="dot2")
    assert e.value.code == _lib.PKD_ERR_UNSUPPORTED
    r.plan(*args, 16)
    with pytest.raises(pkd.PkdError) as e:
        r.run(q, cache, k_scale=0.5)
    assert e.value.code == _lib.PKD_ERR_INVALID_ARG
    codes = torch.zeros(cache.shape, dtype=torch.uint8, device="cuda").view(fp8)
    with pytest.raises(pkd.PkdError) as e:
        r.run(q, codes)
    assert e.value.code == _lib.PKD_ERR_DTYPE_MISMATCH
    r.plan(*args, 16, kv_data_type=fp8)
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(pkd.PkdError) as e:
            r.run(q, codes, v_scale=bad)
        assert e.value.code == _lib.PKD_ERR_INVALID_ARG
    with pytest.raises(pkd.PkdError) as e:
        r.run(q, cache)
    assert e.value.code == _lib.PKD_ERR_DTYPE_MISMATCH
    sr = pkd.SharedPlanRun(2, 4, 64, 32, 8)
    with pytest.raises(pkd.PkdError) as e:  # shared-prefix plans need pages of 16-64 tokens
        sr.plan(np.array([0, 2]), batch.kv_indptr[:2], idx[:3].contiguous(),
                batch.kv_last_page_len[:1], 32, 8, 128, 8, kv_data_type=fp8)
    assert e.value.code == _lib.PKD_ERR_UNSUPPORTED
    k = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    i32 = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(pkd.PkdError) as e:
        pkd.append_paged_kv_cache(k, k, i32, i32, cache, idx, torch.from_numpy(
            batch.kv_indptr).cuda(), k_scale=2.0)
    assert e.value.code == _lib.PKD_ERR_INVALID_ARG


def test_bad_page_table_rejected():
    import torch
    import paged_kv_decode_11_amd as pkd

    batch, q, cache = _inputs()
    r = pkd.DecodePlanRun(max_batch=4, max_nnz=64, max_qo_heads=32)
    idx = torch.from_numpy(batch.kv_indices).cuda()
    last = batch.kv_last_page_len.copy()
    last[1] = 0  # the exact-multiple mistake: 0 instead of page_size
    with pytest.raises(pkd.PkdError) as e:
        r.plan(batch.kv_indptr, idx, last, 32, 8, 128, 16)
    assert e.value.code == _lib.PKD_ERR_INVALID_ARG
    assert r.plan_id == 0


def test_workspace_too_small():
    import torch
    import paged_kv_decode_11_amd as pkd

    rng = np.random.default_rng(6)
    batch = workloads.make_batch([4000] * 4, 16, 1100, 32, 8, 128, rng)
    # capacity for 4 requests on 8 slots = 16 items; one page per chunk needs 1000
    r = pkd.DecodePlanRun(max_batch=4, max_nnz=1100, max_qo_heads=32, num_slots=8)
    idx = torch.from_numpy(batch.kv_indices).cuda()
    with pytest.raises(pkd.PkdError) as e:
        r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, 32, 8, 128, 16, fixed_chunk_pages=1)
    assert e.value.code == _lib.PKD_ERR_WORKSPACE_TOO_SMALL
    r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, 32, 8, 128, 16)  # derived chunks fit


def test_pageable_host_workspace_rejected():
    """The plan upload reads the staging area from the GPU, so pkd_plan
    refuses host memory the device cannot map (checked on the host)."""
    import torch
    import paged_kv_decode_11_amd as pkd

    batch, q, cache = _inputs()
    r = pkd.DecodePlanRun(max_batch=4, max_nnz=64, max_qo_heads=32)
    idx = torch.from_numpy(batch.kv_indices).cuda()
    hb = r.host_workspace.numel()
    raw = torch.empty(hb + 256, dtype=torch.uint8)  # ordinary pageable memory
    off = (-raw.data_ptr()) % 256
    r._host_raw, r.host_workspace = raw, raw[off: off + hb]
    with pytest.raises(pkd.PkdError) as e:
        r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, 32, 8, 128, 16)
    assert e.value.code == _lib.PKD_ERR_INVALID_ARG
    assert r.plan_id == 0


def test_run_shape_mismatch_refused_before_launch():
    """q, cache, out or lse whose shape is not the plan's: refused by the
    binding (PlanMismatchError, status PKD_ERR_STALE_PLAN) before pkd_run,
    so nothing is read or written past a buffer."""
    import torch
    import paged_kv_decode_11_amd as pkd

    batch, q, cache = _inputs()
    r = pkd.DecodePlanRun(max_batch=4, max_nnz=64, max_qo_heads=64)
    idx = torch.from_numpy(batch.kv_indices).cuda()
    r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, 32, 8, 128, 16)
    assert r.plan_shape == dict(batch=2, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                                page_size=16, q_dtype=_lib.PKD_DTYPE_BF16,
                                kv_dtype=_lib.PKD_DTYPE_BF16, kind=_lib.PKD_PLAN_DECODE)
    sentinel = torch.full((2, 32, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    bad_cases = [
        dict(q=q[:, :16].contiguous()),                                        # fewer heads
        dict(kv=cache.view(cache.shape[0] // 2, 2, 32, 8, 128)
             if cache.shape[0] % 2 == 0 else cache[:, :, :8].contiguous()),    # other page size
        dict(kv=cache.view(cache.shape[0], 2, 16, 4, 256)),                    # other head split
        dict(out=torch.empty((2, 32, 64), dtype=torch.bfloat16, device="cuda")),
        dict(lse=torch.empty((2, 16), dtype=torch.float32, device="cuda")),
    ]
    for case in bad_cases:
        with pytest.raises(pkd.PlanMismatchError):
            r.run(case.get("q", q), case.get("kv", cache), out=case.get("out", sentinel),
                  lse=case.get("lse"))
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())  # nothing ran
    sr = pkd.SharedPlanRun(2, 4, 64, 32, 8)
    assert sr.plan_shape is None
    with pytest.raises(pkd.PkdError) as e:
        sr.run(q, cache)
    assert e.value.code == _lib.PKD_ERR_STALE_PLAN


@pytest.mark.parametrize("variant,P,kv", [("dot2", 16, "bf16"), ("mfma", 16, "bf16"),
                                          ("mfma_pv", 16, "bf16"), ("dot2", 4, "bf16"),
                                          ("mfma", 4, "bf16"), ("mfma_pv", 4, "bf16"),
                                          ("mfma", 32, "e4m3")])
@pytest.mark.parametrize("chunk", [0, 1])
def test_out_of_range_page_id_in_decode(variant, P, kv, chunk):
    """kv_indices entries outside [0, num_pages) (one past the end, far past
    it, negative) at an item's first page, in its middle and at its last
    page: every decode kernel reads page 0 in their place, sets
    PKD_DEVERR_PAGE_ID, and otherwise computes the oracle's result with page
    0 substituted."""
    import torch
    from oracle import attention as att

    rng = np.random.default_rng(70 + P + chunk)
    lens = [5 * P + 3, 3 * P, 2, 7 * P + 1]
    need = sum(-(-l // P) for l in lens)
    batch = workloads.make_batch(lens, P, need + 4, 32, 8, 128, rng)
    num_pages = batch.num_pages
    bad_idx = batch.kv_indices.copy()
    bad_idx[batch.kv_indptr[0]] = num_pages              # first page of request 0
    bad_idx[batch.kv_indptr[0] + 2] = -1                 # a middle page
    bad_idx[batch.kv_indptr[3] + 6] = num_pages + 1000   # request 3's last page
    bad_idx[batch.kv_indptr[2]] = 1 << 30                # the one-page request
    sub = np.where((bad_idx < 0) | (bad_idx >= num_pages), 0, bad_idx).astype(np.int32)
    q = workloads.host_query(batch, rng)
    gu.say("bad page id", variant, "P", P, kv, "chunk", chunk)
    r = gu.runner()
    opts = dict(fixed_chunk_pages=chunk) if chunk else {}
    if kv == "e4m3":
        codes = workloads.host_cache_e4m3(batch, rng)
        r.plan(batch.kv_indptr, torch.from_numpy(bad_idx).cuda(), batch.kv_last_page_len, 32, 8,
               128, P, kv_data_type=torch.float8_e4m3fn, **opts)
        o, lse = r.run(gu.bits_to_dev(q), gu.codes_to_dev(codes), return_lse=True,
                       k_scale=1.0 / 64, v_scale=1.0 / 32)
        o_ref, lse_ref = att.decode_fp8(q, codes, batch.kv_indptr, sub, batch.kv_last_page_len, 8,
                                        k_scale=1.0 / 64, v_scale=1.0 / 32)
    else:
        cache = workloads.host_cache(batch, rng)
        r.plan(batch.kv_indptr, torch.from_numpy(bad_idx).cuda(), batch.kv_last_page_len, 32, 8,
               128, P, variant=variant, **opts)
        o, lse = r.run(gu.bits_to_dev(q), gu.bits_to_dev(cache), return_lse=True)
        o_ref, lse_ref = att.decode(q, cache, batch.kv_indptr, sub, batch.kv_last_page_len, 8)
    torch.cuda.synchronize()
    assert r.read_device_error() == _lib.PKD_DEVERR_PAGE_ID
    assert r.read_device_error() == 0  # read clears the flag
    gu.assert_close(o, lse, o_ref, lse_ref, label=f"bad page id {variant} P{P}")


@pytest.mark.parametrize("variant", ["dot2", "mfma", "mfma_pv", "e4m3"])
@pytest.mark.parametrize("P", [1, 2])
def test_out_of_range_page_id_off_lane_zero(variant, P):
    """With pages of 1 or 2 tokens each lane reads the page ids of its own
    rows, and the rows of a wave's lane 0 skip pages 1, 3 and 5 of a tile.
    Out-of-range ids only there still raise PKD_DEVERR_PAGE_ID (the flag is
    the wave's, not lane 0's), and page 0 stands in for them."""
    import torch
    from oracle import attention as att

    rng = np.random.default_rng(90 + P)
    lens = [40, 33, 7 * P + 5, 64]
    need = sum(-(-l // P) for l in lens)
    batch = workloads.make_batch(lens, P, need + 4, 32, 8, 128, rng)
    num_pages = batch.num_pages
    bad_idx = batch.kv_indices.copy()
    ip = batch.kv_indptr
    bad_idx[ip[0] + 1] = num_pages
    bad_idx[ip[1] + 3] = -5
    bad_idx[ip[3] + 5] = num_pages + 77
    sub = np.where((bad_idx < 0) | (bad_idx >= num_pages), 0, bad_idx).astype(np.int32)
    q = workloads.host_query(batch, rng)
    gu.say("bad page id off lane 0", variant, "P", P)
    r = gu.runner()
    idx = torch.from_numpy(bad_idx).cuda()
    if variant == "e4m3":  # the FP8 kernel (per-lane rows of 2 K and 4 V loads)
        codes = workloads.host_cache_e4m3(batch, rng)
        r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, 32, 8, 128, P,
               kv_data_type=torch.float8_e4m3fn)
        o, lse = r.run(gu.bits_to_dev(q), gu.codes_to_dev(codes), return_lse=True,
                       k_scale=1.0 / 64, v_scale=1.0 / 32)
        o_ref, lse_ref = att.decode_fp8(q, codes, batch.kv_indptr, sub, batch.kv_last_page_len, 8,
                                        k_scale=1.0 / 64, v_scale=1.0 / 32)
    else:
        cache = workloads.host_cache(batch, rng)
        r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, 32, 8, 128, P, variant=variant)
        o, lse = r.run(gu.bits_to_dev(q), gu.bits_to_dev(cache), return_lse=True)
        o_ref, lse_ref = att.decode(q, cache, batch.kv_indptr, sub, batch.kv_last_page_len, 8)
    torch.cuda.synchronize()
    assert r.read_device_error() == _lib.PKD_DEVERR_PAGE_ID
    gu.assert_close(o, lse, o_ref, lse_ref, label=f"bad page id off lane 0 {variant} P{P}")
