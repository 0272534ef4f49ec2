"""Appending new tokens to the paged cache on the GPU, through the C ABI,
against oracle.append: the positions helper and the cache after the append
must match bit for bit; then decode over the grown cache against the fp64
oracle (max abs error <= 1e-2 on o, <= 1e-3 on lse)."""

import numpy as np
import pytest

import workloads
from oracle import append as ap
from oracle import attention as att
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _grown_batch(rng, old, add, P, Hkv, spare=5):
    """Old and grown page tables over one pool: each request keeps its pages
    and takes fresh ones as it grows."""
    pool = sum(-(-(l + a) // P) for l, a in zip(old, add)) + spare
    perm = rng.permutation(pool)
    old_pages, new_pages, c = [], [], 0
    for l0, a in zip(old, add):
        n1 = -(-(l0 + a) // P)
        pages = perm[c:c + n1]
        c += n1
        old_pages.append(pages[:-(-l0 // P)])
        new_pages.append(pages)

    def table(lists, lens):
        indptr = np.concatenate([[0], np.cumsum([len(p) for p in lists])]).astype(np.int32)
        return (indptr, np.concatenate(lists).astype(np.int32),
                np.array([l - (-(-l // P) - 1) * P for l in lens], np.int32))

    return pool, table(old_pages, old), table(new_pages, [l + a for l, a in zip(old, add)])


def _dev_i32(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("P,Hkv", [(1, 8), (4, 2), (16, 8), (16, 1), (64, 8)])
def test_append_matches_oracle_bit_exact(P, Hkv):
    import paged_kv_decode_11_amd as pkd
    import torch

    rng = np.random.default_rng(100 * P + Hkv)
    old = rng.integers(1, 200, size=11).tolist()
    add = rng.integers(0, 50, size=11).tolist()
    add[0], add[1] = 1, 2 * P + 3  # one token; a run across page boundaries
    pool, (oi, ox, ol), (ni, nx, nl) = _grown_batch(rng, old, add, P, Hkv)
    gu.say("append", "P", P, "Hkv", Hkv, "new tokens", sum(add))
    cache = workloads.normal_bf16(rng, (pool, 2, P, Hkv, 128))
    n_new = int(sum(add))
    k_new = workloads.normal_bf16(rng, (n_new, Hkv, 128))
    v_new = workloads.normal_bf16(rng, (n_new, Hkv, 128))
    append_indptr = np.concatenate([[0], np.cumsum(add)]).astype(np.int32)

    b_ref, p_ref = ap.batch_indices_positions(append_indptr, ni, nl, P)
    b_dev, p_dev = pkd.append_positions(_dev_i32(append_indptr), _dev_i32(ni), _dev_i32(nl), P)
    assert np.array_equal(b_dev.cpu().numpy(), b_ref)
    assert np.array_equal(p_dev.cpu().numpy(), p_ref)

    cache_dev = gu.bits_to_dev(cache)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkd.append_paged_kv_cache(gu.bits_to_dev(k_new), gu.bits_to_dev(v_new), b_dev, p_dev, cache_dev,
                              _dev_i32(nx), _dev_i32(ni), device_error=err)
    torch.cuda.synchronize()
    want = ap.append(cache, k_new, v_new, b_ref, p_ref, ni, nx)
    assert np.array_equal(gu.dev_bits(cache_dev), want)
    assert int(err.item()) == 0


def test_out_of_range_tokens_are_not_written():
    import paged_kv_decode_11_amd as pkd
    import torch

    rng = np.random.default_rng(7)
    pool, _, (ni, nx, nl) = _grown_batch(rng, [20, 5], [0, 0], 16, 8)
    cache = workloads.normal_bf16(rng, (pool, 2, 16, 8, 128))
    k = workloads.normal_bf16(rng, (4, 8, 128))
    b = np.array([0, 0, 1, 5], np.int32)       # request 5 does not exist
    pos = np.array([19, 32, -1, 0], np.int32)  # 32 is past request 0's pages, -1 is negative
    cache_dev = gu.bits_to_dev(cache)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkd.append_paged_kv_cache(gu.bits_to_dev(k), gu.bits_to_dev(k), _dev_i32(b), _dev_i32(pos),
                              cache_dev, _dev_i32(nx), _dev_i32(ni), device_error=err)
    torch.cuda.synchronize()
    want = ap.append(cache, k, k, b[:1], pos[:1], ni, nx)
    assert np.array_equal(gu.dev_bits(cache_dev), want)
    assert int(err.item()) != 0


def test_append_then_decode():
    """One generated token per request appended, then the decode of the
    grown batch against the oracle on the grown cache."""
    import paged_kv_decode_11_amd as pkd
    import torch

    rng = np.random.default_rng(11)
    old = [37, 16, 5, 300, 128, 1]
    pool, _, (ni, nx, nl) = _grown_batch(rng, old, [1] * len(old), 16, 8)
    cache = workloads.normal_bf16(rng, (pool, 2, 16, 8, 128))
    k_new = workloads.normal_bf16(rng, (len(old), 8, 128))
    v_new = workloads.normal_bf16(rng, (len(old), 8, 128))
    q = workloads.normal_bf16(rng, (len(old), 32, 128))
    append_indptr = np.arange(len(old) + 1, dtype=np.int32)
    cache_dev = gu.bits_to_dev(cache)
    b_dev, p_dev = pkd.append_positions(_dev_i32(append_indptr), _dev_i32(ni), _dev_i32(nl), 16)
    pkd.append_paged_kv_cache(gu.bits_to_dev(k_new), gu.bits_to_dev(v_new), b_dev, p_dev,
                              cache_dev, _dev_i32(nx), _dev_i32(ni))
    r = gu.runner(max_batch=64, max_nnz=1 << 12)
    r.plan(ni, _dev_i32(nx), nl, 32, 8, 128, 16)
    o, lse = r.run(gu.bits_to_dev(q), cache_dev, return_lse=True)
    torch.cuda.synchronize()
    b_ref, p_ref = ap.batch_indices_positions(append_indptr, ni, nl, 16)
    grown = ap.append(cache, k_new, v_new, b_ref, p_ref, ni, nx)
    o_ref, lse_ref = att.decode(q, grown, ni, nx, nl, 8)
    gu.assert_close(o, lse, o_ref, lse_ref, label="append-then-decode")
