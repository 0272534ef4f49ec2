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
    """An E4M3 cache: page sizes and kernels it is not built for, scales on a
    bf16 cache, invalid scales, and a run whose cache dtype is not the plan's."""
    import torch
    import paged_kv_decode_11_amd as pkd

    batch, q, cache = _inputs()
    fp8 = torch.float8_e4m3fn
    r = pkd.DecodePlanRun(max_batch=4, max_nnz=64, max_qo_heads=32)
    idx = torch.from_numpy(batch.kv_indices).cuda()
    args = (batch.kv_indptr, idx, batch.kv_last_page_len, 32, 8, 128)
    with pytest.raises(pkd.PkdError) as e:
        r.plan(*args, 8, kv_data_type=fp8)
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
    with pytest.raises(pkd.PkdError) as e:
        sr.plan(np.array([0, 2]), batch.kv_indptr[:2], idx[:3].contiguous(),
                batch.kv_last_page_len[:1], 32, 8, 128, 16, kv_data_type=fp8)
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
