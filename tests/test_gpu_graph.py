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
