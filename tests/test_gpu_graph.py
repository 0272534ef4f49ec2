"""Graph replay: a run captured once in a HIP graph (torch.cuda.CUDAGraph)
keeps producing the oracle's result after later plans refill the same
workspaces with other batches (aicassindra "Plan and run"; pinghaoyang,
CUDA-graph sections).  Each replay is followed by eager work and a
synchronisation, and every replay is checked."""

import numpy as np
import pytest

import workloads
from oracle import attention as att
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("variant", ["auto", "dot2", "mfma_pv"])
def test_graph_replay_across_plans(variant):
    import torch
    import paged_kv_decode_11_amd as pkd

    P, Hq, Hkv, MAXB = 16, 32, 8, 24
    rng = np.random.default_rng(77)
    pool = 2000
    r = pkd.DecodePlanRun(max_batch=MAXB, max_nnz=pool, max_qo_heads=Hq)
    # one cache for all steps; q and o buffers of the maximum batch
    full = workloads.make_batch([1] * MAXB, P, pool, Hq, Hkv, 128, rng)
    cache = workloads.host_cache(full, rng, fill_pages="all")
    cd = gu.bits_to_dev(cache)
    q_buf = torch.zeros((MAXB, Hq, 128), dtype=torch.bfloat16, device="cuda")
    o_buf = torch.zeros((MAXB, Hq, 128), dtype=torch.bfloat16, device="cuda")
    lse_buf = torch.zeros((MAXB, Hq), dtype=torch.float32, device="cuda")

    def make_step(B, seed, fixed=0):
        g = np.random.default_rng(seed)
        lens = g.integers(1, 1200, size=B)
        b = workloads.make_batch(lens, P, pool, Hq, Hkv, 128, g)
        q = workloads.normal_bf16(g, (B, Hq, 128))
        return b, q, fixed

    # dummy plan at the maximum batch, then capture run on it
    b0, q0, _ = make_step(MAXB, 1)
    r.plan(b0.kv_indptr, torch.from_numpy(b0.kv_indices).cuda(), b0.kv_last_page_len, Hq, Hkv,
           128, P, variant=variant)
    q_buf.copy_(gu.bits_to_dev(q0))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        r.run(q_buf, cd, out=o_buf, lse=lse_buf)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        r.run(q_buf, cd, out=o_buf, lse=lse_buf)
    torch.cuda.synchronize()

    steps = [(MAXB, 2, 0), (17, 3, 2), (5, 4, 1), (MAXB, 5, 0)]
    for B, seed, fixed in steps:
        b, q, fixed = make_step(B, seed, fixed)
        gu.say("graph step", variant, B, seed, fixed)
        idx = torch.from_numpy(b.kv_indices).cuda()
        r.plan(b.kv_indptr, idx, b.kv_last_page_len, Hq, Hkv, 128, P, fixed_chunk_pages=fixed,
               variant=variant)
        q_buf[:B].copy_(gu.bits_to_dev(q))
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1000, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        o_ref, lse_ref = att.decode(q, cache, b.kv_indptr, b.kv_indices, b.kv_last_page_len, Hkv)
        gu.assert_close(o_buf[:B], lse_buf[:B], o_ref, lse_ref, label=f"replay-{variant}-{seed}")


def test_merge_long_and_short_entries_across_replays():
    """Merge-list entries of up to 10 states and of up to 300 (one request cut
    into 300 one-page chunks): eager, and a run captured on a plan of one
    kind replayed after a plan of the other."""
    import torch
    import paged_kv_decode_11_amd as pkd

    P, Hq, Hkv = 16, 32, 8
    pool = 1400
    rng = np.random.default_rng(91)
    r = pkd.DecodePlanRun(max_batch=1024, max_nnz=pool, max_qo_heads=Hq)
    full = workloads.make_batch([1] * 4, P, pool, Hq, Hkv, 128, rng)
    cache = workloads.host_cache(full, rng, fill_pages="all")
    cd = gu.bits_to_dev(cache)
    q = workloads.normal_bf16(rng, (4, Hq, 128))
    qd = gu.bits_to_dev(q)
    o_buf = torch.zeros((4, Hq, 128), dtype=torch.bfloat16, device="cuda")
    lse_buf = torch.zeros((4, Hq), dtype=torch.float32, device="cuda")
    # shallow: at most 10 chunks per request; deep: 300 one-page chunks
    shallow = workloads.make_batch([160, 90, 33, 7], P, pool, Hq, Hkv, 128, rng)
    deep = workloads.make_batch([300 * P, 70 * P - 3, 5, 1000], P, pool, Hq, Hkv, 128, rng)

    def plan(b, fixed):
        r.plan(b.kv_indptr, torch.from_numpy(b.kv_indices).cuda(), b.kv_last_page_len, Hq, Hkv,
               128, P, fixed_chunk_pages=fixed)

    for b, fixed in ((shallow, 1), (deep, 1)):
        gu.say("merge entries eager", int(b.kv_lens.max()), fixed)
        plan(b, fixed)
        r.run(qd, cd, out=o_buf, lse=lse_buf)
        torch.cuda.synchronize()
        o_ref, lse_ref = att.decode(q, cache, b.kv_indptr, b.kv_indices, b.kv_last_page_len, Hkv)
        gu.assert_close(o_buf, lse_buf, o_ref, lse_ref, label="merge entries eager")
    for first, then in (((shallow, 1), (deep, 1)), ((deep, 1), (shallow, 1))):
        plan(*first)
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            r.run(qd, cd, out=o_buf, lse=lse_buf, stream=s)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            r.run(qd, cd, out=o_buf, lse=lse_buf)
        torch.cuda.synchronize()
        plan(*then)
        b = then[0]
        for _ in range(2):
            o_buf.zero_()
            g.replay()
            torch.cuda.synchronize()
            o_ref, lse_ref = att.decode(q, cache, b.kv_indptr, b.kv_indices, b.kv_last_page_len,
                                        Hkv)
            gu.assert_close(o_buf, lse_buf, o_ref, lse_ref, label="merge entries replay")
        del g


@pytest.mark.parametrize("longest", [300, 64, 40])
@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (4, 1), (8, 8)])
def test_merge_mixed_entries(Hq, Hkv, longest):
    """One plan whose merge list holds entries of a few states (one round
    trip by 32 lanes) and of more: one workgroup per task while no entry has
    more than 64 states, else cut across head_dim over several workgroups;
    with 4 or 8 query heads a block of 8 tasks spans several entries, short
    and long ones together."""
    import torch
    import paged_kv_decode_11_amd as pkd

    P = 16
    pool = 1200
    rng = np.random.default_rng(57 + Hq + longest)
    lens = [longest * P, 10 * P, 3 * P + 2, 40 * P - 7, 17 * P, 16 * P, 5, 1]
    b = workloads.make_batch(lens, P, pool, Hq, Hkv, 128, rng)
    cache = workloads.host_cache(b, rng, poison=True)
    q = workloads.normal_bf16(rng, (len(lens), Hq, 128))
    r = pkd.DecodePlanRun(max_batch=1024, max_nnz=pool, max_qo_heads=Hq)
    gu.say("merge mixed entries", Hq, Hkv, longest)
    r.plan(b.kv_indptr, torch.from_numpy(b.kv_indices).cuda(), b.kv_last_page_len, Hq, Hkv, 128,
           P, fixed_chunk_pages=1)
    o, lse = r.run(gu.bits_to_dev(q), gu.bits_to_dev(cache), return_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = att.decode(q, cache, b.kv_indptr, b.kv_indices, b.kv_last_page_len, Hkv)
    gu.assert_close(o, lse, o_ref, lse_ref, label="merge mixed entries")
