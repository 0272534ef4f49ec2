"""Merge kernels on the GPU against the oracle's merge, and the composable
shared-prefix format: prefix state and suffix state computed by two plans
and merged must equal single-format attention over prefix + suffix."""

import math

import numpy as np
import pytest

import workloads
from oracle import attention as att
from oracle import merge as mg
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _states(rng, n, H, spread=3.0):
    o = workloads.normal_bf16(rng, (n, H, 128))
    lse = (rng.standard_normal((n, H)) * spread).astype(np.float32)
    return o, lse


def test_merge_state_matches_oracle():
    import torch

    rng = np.random.default_rng(1)
    n, H = 37, 32
    oa, la = _states(rng, n, H)
    ob, lb = _states(rng, n, H)
    la[0, :4] = -np.inf           # one empty side
    la[1, 0] = lb[1, 0] = -np.inf  # both empty
    gu.say("merge_state", n, H)
    import paged_kv_decode_11_amd as pkd
    o, lse = pkd.merge_state(gu.bits_to_dev(oa), torch.from_numpy(la).cuda(), gu.bits_to_dev(ob),
                             torch.from_numpy(lb).cuda())
    torch.cuda.synchronize()
    ref_o, ref_l = mg.merge_rows(att.bf16_to_f64(oa), la.astype(np.float64), att.bf16_to_f64(ob),
                                 lb.astype(np.float64))
    got_l = lse.cpu().numpy().astype(np.float64)
    assert got_l[1, 0] == -math.inf and np.all(gu.dev_to_f64(o)[1, 0] == 0)
    gu.check_lse(got_l, ref_l, "merge_state")
    gu.check_o(gu.dev_to_f64(o), ref_o, "merge_state")


def test_merge_state_in_place():
    import torch
    import paged_kv_decode_11_amd as pkd

    rng = np.random.default_rng(2)
    oa, la = _states(rng, 9, 8)
    ob, lb = _states(rng, 9, 8)
    da, dla = gu.bits_to_dev(oa), torch.from_numpy(la).cuda()
    pkd.merge_state(da, dla, gu.bits_to_dev(ob), torch.from_numpy(lb).cuda(), out=da, lse_out=dla)
    torch.cuda.synchronize()
    ref_o, ref_l = mg.merge_rows(att.bf16_to_f64(oa), la.astype(np.float64), att.bf16_to_f64(ob),
                                 lb.astype(np.float64))
    gu.check_o(gu.dev_to_f64(da), ref_o, "in-place")
    gu.check_lse(dla.cpu().numpy().astype(np.float64), ref_l, "in-place")


@pytest.mark.parametrize("k", [1, 2, 7, 64, 300])
def test_merge_states_matches_oracle(k):
    import torch
    import paged_kv_decode_11_amd as pkd

    rng = np.random.default_rng(10 + k)
    n, H = 5, 16
    o = workloads.normal_bf16(rng, (n, k, H, 128))
    lse = (rng.standard_normal((n, k, H)) * 4).astype(np.float32)
    if k > 2:
        lse[0, 1, :] = -np.inf
    gu.say("merge_states k", k)
    out, lse_out = pkd.merge_states(gu.bits_to_dev(o), torch.from_numpy(lse).cuda())
    torch.cuda.synchronize()
    of = att.bf16_to_f64(o)
    ref_o = np.zeros((n, H, 128))
    ref_l = np.zeros((n, H))
    for i in range(n):
        for h in range(H):
            ref_o[i, h], ref_l[i, h] = mg.merge_many(
                [(of[i, c, h], float(lse[i, c, h])) for c in range(k)])
    gu.check_o(gu.dev_to_f64(out), ref_o, f"merge_states k={k}")
    gu.check_lse(lse_out.cpu().numpy().astype(np.float64), ref_l, f"merge_states k={k}")


def test_split_partials_merge_like_unsplit():
    """Splitting a request into many chunks and merging their partial states
    gives the unsplit result (up to rounding)."""
    rng = np.random.default_rng(3)
    batch = workloads.make_batch([4000, 2500], 16, 500, 32, 8, 128, rng)
    q = workloads.host_query(batch, rng)
    cache = workloads.host_cache(batch, rng)
    qd, cd = gu.bits_to_dev(q), gu.bits_to_dev(cache)
    o1, l1 = gu.decode(batch, qd, cd, min_chunk_tokens=100000)  # no split
    o2, l2 = gu.decode(batch, qd, cd, fixed_chunk_pages=3)      # 84 + 53 chunks
    gu.check_o(gu.dev_to_f64(o2), gu.dev_to_f64(o1), "split-vs-unsplit")
    gu.check_lse(l2.cpu().numpy().astype(np.float64), l1.cpu().numpy().astype(np.float64),
                 "split-vs-unsplit")


def test_composable_shared_prefix_small():
    """The composable format on a small case: prefix plan (every row points at
    the shared prefix pages) and suffix plan, merged with pkd_merge_state,
    against the oracle on the single-format page table."""
    import torch
    import paged_kv_decode_11_amd as pkd

    rng = np.random.default_rng(4)
    P, n_req, prefix_pages = 16, 6, 9
    suffix = rng.integers(1, 70, size=n_req)
    pool = 200
    perm = rng.permutation(pool)
    pre = perm[:prefix_pages]
    s_indptr, s_idx, s_last = workloads.allocate_pages(suffix, P, perm[prefix_pages:])
    single_rows = [np.concatenate([pre, s_idx[s_indptr[i]:s_indptr[i + 1]]]) for i in range(n_req)]
    mk = workloads.PagedBatch
    single = mk(P, 32, 8, 128, pool, (prefix_pages * P + suffix).astype(np.int64),
                np.concatenate([[0], np.cumsum([len(r) for r in single_rows])]).astype(np.int32),
                np.concatenate(single_rows).astype(np.int32), s_last.astype(np.int32))
    prefix = mk(P, 32, 8, 128, pool, np.full(n_req, prefix_pages * P, dtype=np.int64),
                (np.arange(n_req + 1) * prefix_pages).astype(np.int32),
                np.tile(pre, n_req).astype(np.int32), np.full(n_req, P, dtype=np.int32))
    suf = mk(P, 32, 8, 128, pool, suffix.astype(np.int64), s_indptr, s_idx, s_last)
    q = workloads.host_query(single, rng)
    cache = workloads.host_cache(single, rng, poison=True)
    qd, cd = gu.bits_to_dev(q), gu.bits_to_dev(cache)
    o_p, l_p = gu.decode(prefix, qd, cd, r=gu.runner())
    o_s, l_s = gu.decode(suf, qd, cd, r=gu.runner(max_batch=64, max_nnz=4096))
    o, lse = pkd.merge_state(o_p, l_p, o_s, l_s)
    torch.cuda.synchronize()
    o_ref, lse_ref = att.decode(q, cache, single.kv_indptr, single.kv_indices,
                                single.kv_last_page_len, 8)
    gu.assert_close(o, lse, o_ref, lse_ref, label="composable-small")
