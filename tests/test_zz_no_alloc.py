"""pkd_plan_static, the plan that needs no workspaces (its plan image and
partial states live in the library's own device array), against pkd_plan
with caller-owned workspaces, through the C ABI: on the same inputs the
runs after either plan give the same bits, and both meet the oracle's bar
(max |o - o_ref| <= 1e-2, or half a bf16 ulp above 4; |lse - lse_ref| <=
1e-3).  Two calls in a row, the second with a smaller batch; unsplit and
forced-split plans (so the partial states in the static array are used).
Also: a plan too large for the array is refused on the host, a run after
another handle's static plan is refused as stale, and a run captured in a
graph replays correctly after later static plans."""

import numpy as np
import pytest

import workloads
from oracle import attention as att
from paged_kv_decode_11_amd import _lib
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

P, HQ, HKV = 16, 32, 8


def _inputs(seed, B, max_len):
    rng = np.random.default_rng(seed)
    batch = workloads.random_batch(rng, B, max_len, P, HQ, HKV, 128)
    q = workloads.host_query(batch, rng)
    cache = workloads.host_cache(batch, rng, poison=True)
    return batch, q, cache


def _run(r, batch, q_dev, cache_dev, **opts):
    import torch

    r.plan(batch.kv_indptr, torch.from_numpy(batch.kv_indices).cuda(), batch.kv_last_page_len,
           HQ, HKV, 128, P, **opts)
    o, lse = r.run(q_dev, cache_dev, return_lse=True)
    torch.cuda.synchronize()
    assert r.read_device_error() == 0
    return o, lse


def test_static_plan_matches_workspace_plan():
    import torch
    import paged_kv_decode_11_amd as pkd

    static = pkd.StaticPlanRun()
    # room for the forced two-page chunks (about 1,900 items)
    ws = pkd.DecodePlanRun(max_batch=1024, max_nnz=1 << 14, max_qo_heads=HQ)
    for call, (B, max_len, seed) in enumerate([(40, 3000, 11), (6, 700, 12)]):
        batch, q, cache = _inputs(seed, B, max_len)
        q_dev, cache_dev = gu.bits_to_dev(q), gu.bits_to_dev(cache)
        o_ref, lse_ref = att.decode(q, cache, batch.kv_indptr, batch.kv_indices,
                                    batch.kv_last_page_len, HKV)
        for opts in ({}, {"fixed_chunk_pages": 2}):
            gu.say("no-alloc call", call, "B", B, "opts", opts)
            o_s, lse_s = _run(static, batch, q_dev, cache_dev, **opts)
            o_w, lse_w = _run(ws, batch, q_dev, cache_dev, **opts)
            assert static.planned_variant == ws.planned_variant
            assert torch.equal(o_s.view(torch.int16), o_w.view(torch.int16)), "o differs"
            assert torch.equal(lse_s.view(torch.int32), lse_w.view(torch.int32)), "lse differs"
            gu.assert_close(o_s, lse_s, o_ref, lse_ref, label=f"static call {call} {opts}")


def test_static_plan_limits_and_sharing():
    import torch
    import paged_kv_decode_11_amd as pkd

    # 2,400 one-page chunks of 64 query heads: 2,400 x 64 x 129 x 4 bytes of
    # partial states, above PKD_STATIC_FLOAT_BYTES; refused before any launch
    big = pkd.StaticPlanRun()
    lens = [600 * P] * 4
    rng = np.random.default_rng(3)
    b = workloads.make_batch(lens, P, 2400, 64, HKV, 128, rng)
    with pytest.raises(pkd.PkdError) as e:
        big.plan(b.kv_indptr, torch.from_numpy(b.kv_indices).cuda(), b.kv_last_page_len, 64, HKV,
                 128, P, fixed_chunk_pages=1)
    assert e.value.code == _lib.PKD_ERR_WORKSPACE_TOO_SMALL
    assert big.plan_id == 0

    # two handles share the array: the older plan is refused as stale
    batch, q, cache = _inputs(21, 5, 400)
    q_dev, cache_dev = gu.bits_to_dev(q), gu.bits_to_dev(cache)
    a, c = pkd.StaticPlanRun(), pkd.StaticPlanRun()
    idx = torch.from_numpy(batch.kv_indices).cuda()
    a.plan(batch.kv_indptr, idx, batch.kv_last_page_len, HQ, HKV, 128, P)
    c.plan(batch.kv_indptr, idx, batch.kv_last_page_len, HQ, HKV, 128, P)
    with pytest.raises(pkd.PkdError) as e:
        a.run(q_dev, cache_dev)
    assert e.value.code == _lib.PKD_ERR_STALE_PLAN
    o, lse = _run(a, batch, q_dev, cache_dev)  # plans again, then runs
    o_ref, lse_ref = att.decode(q, cache, batch.kv_indptr, batch.kv_indices,
                                batch.kv_last_page_len, HKV)
    gu.assert_close(o, lse, o_ref, lse_ref, label="static after re-plan")


def test_static_plan_graph_replay():
    import torch
    import paged_kv_decode_11_amd as pkd

    MAXB, pool = 16, 1200
    rng = np.random.default_rng(8)
    r = pkd.StaticPlanRun()
    full = workloads.make_batch([1] * MAXB, P, pool, HQ, HKV, 128, rng)
    cache = workloads.host_cache(full, rng, fill_pages="all")
    cd = gu.bits_to_dev(cache)
    q_buf = torch.zeros((MAXB, HQ, 128), dtype=torch.bfloat16, device="cuda")
    o_buf = torch.zeros((MAXB, HQ, 128), dtype=torch.bfloat16, device="cuda")
    lse_buf = torch.zeros((MAXB, HQ), dtype=torch.float32, device="cuda")

    def step(B, seed):
        g = np.random.default_rng(seed)
        b = workloads.make_batch(g.integers(1, 1000, size=B), P, pool, HQ, HKV, 128, g)
        return b, workloads.normal_bf16(g, (B, HQ, 128))

    b0, q0 = step(MAXB, 1)
    r.plan(b0.kv_indptr, torch.from_numpy(b0.kv_indices).cuda(), b0.kv_last_page_len, HQ, HKV,
           128, P)
    q_buf.copy_(gu.bits_to_dev(q0))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        r.run(q_buf, cd, out=o_buf, lse=lse_buf)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r.run(q_buf, cd, out=o_buf, lse=lse_buf)
    torch.cuda.synchronize()
    for B, seed, fixed in [(MAXB, 2, 0), (9, 3, 3), (MAXB, 4, 0)]:
        b, q = step(B, seed)
        gu.say("static graph step", B, seed, fixed)
        r.plan(b.kv_indptr, torch.from_numpy(b.kv_indices).cuda(), b.kv_last_page_len, HQ, HKV,
               128, P, fixed_chunk_pages=fixed)
        q_buf[:B].copy_(gu.bits_to_dev(q))
        for _ in range(2):
            o_buf.zero_()
            g.replay()
            torch.cuda.synchronize()
            o_ref, lse_ref = att.decode(q, cache, b.kv_indptr, b.kv_indices, b.kv_last_page_len,
                                        HKV)
            gu.assert_close(o_buf[:B], lse_buf[:B], o_ref, lse_ref, label=f"static replay {seed}")


@pytest.mark.parametrize("page", [16, 1])
def test_static_plan_fp8_cache(page):
    """An FP8 E4M3 cache through pkd_plan_static: the same bits as after a
    plan on caller-owned workspaces, and the oracle's bar; two calls, the
    second smaller, unsplit and forced-split."""
    import torch
    import paged_kv_decode_11_amd as pkd

    fp8 = torch.float8_e4m3fn
    static = pkd.StaticPlanRun()
    ws = pkd.DecodePlanRun(max_batch=1024, max_nnz=1 << 14, max_qo_heads=HQ)
    for call, (B, max_len, seed) in enumerate([(24, 1500, 21), (5, 400, 22)]):
        rng = np.random.default_rng(seed + page)
        batch = workloads.random_batch(rng, B, max_len, page, HQ, HKV, 128)
        q = workloads.host_query(batch, rng)
        codes = workloads.host_cache_e4m3(batch, rng, poison=True)
        q_dev, c_dev = gu.bits_to_dev(q), gu.codes_to_dev(codes)
        o_ref, lse_ref = att.decode_fp8(q, codes, batch.kv_indptr, batch.kv_indices,
                                        batch.kv_last_page_len, HKV, k_scale=1 / 64, v_scale=1 / 32)
        idx = torch.from_numpy(batch.kv_indices).cuda()
        for opts in ({}, {"fixed_chunk_pages": 2 if page >= 16 else 48}):
            gu.say("no-alloc fp8 call", call, "P", page, "B", B, "opts", opts)
            outs = []
            for r in (static, ws):
                r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, HQ, HKV, 128, page,
                       kv_data_type=fp8, **opts)
                o, lse = r.run(q_dev, c_dev, return_lse=True, k_scale=1 / 64, v_scale=1 / 32)
                torch.cuda.synchronize()
                assert r.read_device_error() == 0
                outs.append((o, lse))
            (o_s, lse_s), (o_w, lse_w) = outs
            assert torch.equal(o_s.view(torch.int16), o_w.view(torch.int16)), "o differs"
            assert torch.equal(lse_s.view(torch.int32), lse_w.view(torch.int32)), "lse differs"
            gu.assert_close(o_s, lse_s, o_ref, lse_ref, label=f"static fp8 P{page} call {call}")
