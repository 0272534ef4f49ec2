"""Parity at the full workload sizes, in the launch configuration the
benchmark times (default plan on the handle's default slot count).  The
cache is filled on the device; the pages of sampled requests are copied
back and the oracle computes those requests one by one."""

import numpy as np
import pytest

import workloads
from oracle import attention as att
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _sampled_check(name, requests, used_only=False, seed_offset=0, **opts):
    import torch

    spec, rng, b = workloads.workload(name)
    batch = b["main"]
    gu.say(name, "B", batch.batch, "T", batch.total_tokens, "nnz", batch.nnz, "pool",
           batch.num_pages, "requests", requests)
    cache = workloads.device_cache(batch, spec.seed + 100 + seed_offset, "cuda",
                                   used_only=used_only)
    q = workloads.host_query(batch, rng)
    r = gu.runner(max_batch=512, max_nnz=1 << 17)
    o, lse = gu.decode(batch, gu.bits_to_dev(q), cache, r=r, **opts)
    host, indptr, indices, last = gu.compact_pages(batch, cache, requests)
    del cache
    torch.cuda.empty_cache()
    o_ref, lse_ref = att.decode(q[list(requests)], host, indptr, indices, last,
                                batch.num_kv_heads)
    return gu.assert_close(o[list(requests)], lse[list(requests)], o_ref, lse_ref, label=name)


def test_skewed_full_size():
    # the 100k-token request (index 63, split across most slots) and three
    # 512-token requests
    _sampled_check("skewed", [63, 0, 31, 62])


def test_skewed_full_size_dot2_kernel():
    _sampled_check("skewed", [63, 5], variant="dot2")


def test_llama8b_layer_full_size():
    _, _, b = workloads.workload("llama8b_step")
    lens = b["main"].kv_lens
    _sampled_check("llama8b_step", [int(np.argmax(lens)), int(np.argmin(lens)), 17])


def test_wide_gqa_full_size_pv_kernel():
    _, _, b = workloads.workload("wide_gqa")
    lens = b["main"].kv_lens
    order = np.argsort(lens)
    _sampled_check("wide_gqa", [int(order[-1]), int(order[0]), int(order[128])], used_only=True,
                   variant="mfma_pv")


def test_llama8b_layer_full_size_pv_kernel():
    _, _, b = workloads.workload("llama8b_step")
    lens = b["main"].kv_lens
    _sampled_check("llama8b_step", [int(np.argmax(lens)), 5], variant="mfma_pv")


def test_wide_gqa_full_size():
    _, _, b = workloads.workload("wide_gqa")
    lens = b["main"].kv_lens
    order = np.argsort(lens)
    _sampled_check("wide_gqa", [int(order[-1]), int(order[0]), int(order[128])], used_only=True)


def test_token_sparse_full():
    """page_size 1, every request checked."""
    spec, rng, b = workloads.workload("token_sparse")
    batch = b["main"]
    q = workloads.host_query(batch, rng)
    cache = workloads.host_cache(batch, rng)
    gu.say("token_sparse", batch.batch, batch.total_tokens)
    o, lse = gu.decode(batch, gu.bits_to_dev(q), gu.bits_to_dev(cache))
    o_ref, lse_ref = att.decode(q, cache, batch.kv_indptr, batch.kv_indices,
                                batch.kv_last_page_len, batch.num_kv_heads)
    gu.assert_close(o, lse, o_ref, lse_ref, label="token_sparse")


def test_shared_prefix_composable_full():
    """Prefix state (32 rows over the same 512 pages) and suffix state from
    two plans, merged, against the single-format oracle on 8 requests."""
    import torch
    import paged_kv_decode_11_amd as pkd

    spec, rng, b = workloads.workload("shared_prefix")
    main, prefix, suffix = b["main"], b["prefix"], b["suffix"]
    q = workloads.host_query(main, rng)
    cache = workloads.host_cache(main, rng)
    gu.say("shared_prefix", main.batch, main.total_tokens)
    qd, cd = gu.bits_to_dev(q), gu.bits_to_dev(cache)
    o_p, l_p = gu.decode(prefix, qd, cd, r=gu.runner(max_batch=512, max_nnz=1 << 17))
    o_s, l_s = gu.decode(suffix, qd, cd, r=gu.runner(max_batch=64, max_nnz=1 << 12))
    o, lse = pkd.merge_state(o_p, l_p, o_s, l_s)
    o1, l1 = gu.decode(main, qd, cd, r=gu.runner(max_batch=512, max_nnz=1 << 17))
    torch.cuda.synchronize()
    req = [0, 3, 7, 12, 18, 24, 29, 31]
    o_ref, lse_ref = att.decode(q, cache, main.kv_indptr, main.kv_indices,
                                main.kv_last_page_len, main.num_kv_heads, requests=req)
    gu.assert_close(o, lse, o_ref, lse_ref, requests=req, label="composable")
    gu.assert_close(o1, l1, o_ref, lse_ref, requests=req, label="single-format")
