"""Pins for oracle.attention against things other than itself: exact bf16
widening, brute force with exactly rounded sums, torch's
scaled_dot_product_attention in float64 on a dense layout that this test
scatters into pages on its own, and closed forms."""

import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as att
from oracle import page_table as pt


def test_bf16_widening_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x3F81, 0x0001, 0x4049],
                    dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, math.inf, -math.inf, 1.0 + 2.0 ** -7, 2.0 ** -133,
            3.140625]
    got = att.bf16_to_f64(bits)
    for g, w in zip(got, want):
        assert g == w
    assert math.isnan(att.bf16_to_f64(np.array([0x7FC0], dtype=np.uint16))[0])


def _tiny_case(seed, P=4, Hq=4, Hkv=2, D=8, lens=None, poison=True):
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(1, 3 * P + 2, size=3)
    batch = workloads.make_batch(lens, P, int(sum(-(-l // P) for l in lens)) + 5, Hq, Hkv, D, rng)
    q = workloads.host_query(batch, rng)
    cache = workloads.host_cache(batch, rng, poison=poison)
    return batch, q, cache


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_vectorized_matches_bruteforce(seed):
    batch, q, cache = _tiny_case(seed)
    args = (q, cache, batch.kv_indptr, batch.kv_indices, batch.kv_last_page_len, batch.num_kv_heads)
    o1, l1 = att.decode(*args)
    o2, l2 = att.decode_bruteforce(*args)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs(l1 - l2)) < 1e-12
    assert np.all(np.isfinite(o1)) and np.all(np.isfinite(l1))  # poison never read


@pytest.mark.parametrize("P,Hq,Hkv", [(16, 32, 8), (1, 4, 4), (4, 8, 2), (8, 6, 3)])
def test_matches_torch_sdpa_on_dense_layout(P, Hq, Hkv):
    """Dense per-request K/V -> scattered into a permuted pool by this test
    -> oracle gathers back; compare with torch SDPA (float64, CPU) on the
    dense tensors, GQA expanded with repeat_interleave."""
    rng = np.random.default_rng(100 + P)
    D = 16
    lens = [1, P, P + 1, 3 * P + 2, 40]
    indptr, indices, last = pt.page_table(lens, P, page_ids=rng.permutation(400))
    cache = np.zeros((400, 2, P, Hkv, D), dtype=np.uint16)
    q = workloads.normal_bf16(rng, (len(lens), Hq, D))
    dense = []
    for i, L in enumerate(lens):
        kv = workloads.normal_bf16(rng, (2, L, Hkv, D))
        dense.append(kv)
        for t in range(L):
            page = indices[indptr[i] + t // P]
            cache[page, 0, t % P] = kv[0, t]
            cache[page, 1, t % P] = kv[1, t]
    o, lse = att.decode(q, cache, indptr, indices, last, Hkv)
    g = Hq // Hkv
    for i, L in enumerate(lens):
        qt = torch.from_numpy(att.bf16_to_f64(q[i])).view(1, Hq, 1, D)
        K = torch.from_numpy(att.bf16_to_f64(dense[i][0])).permute(1, 0, 2)  # [Hkv, L, D]
        V = torch.from_numpy(att.bf16_to_f64(dense[i][1])).permute(1, 0, 2)
        K = K.repeat_interleave(g, dim=0).unsqueeze(0).contiguous()
        V = V.repeat_interleave(g, dim=0).unsqueeze(0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qt, K, V).view(Hq, D).numpy()
        logits = (qt @ K.transpose(-1, -2)).view(Hq, L) / math.sqrt(D)
        ref_lse = torch.logsumexp(logits, dim=-1).numpy()
        assert np.max(np.abs(o[i] - ref)) < 1e-12
        assert np.max(np.abs(lse[i] - ref_lse)) < 1e-12


def _one_request_cache(K, V, P=4):
    """Lay one request's K, V ([L, 1, D] float arrays exactly representable
    in bf16) into pages 0.. of a fresh pool."""
    L = K.shape[0]
    n = -(-L // P)
    cache = np.zeros((n + 1, 2, P, 1, K.shape[-1]), dtype=np.uint16)
    kb = workloads.f32_to_bf16_bits(K.astype(np.float32))
    vb = workloads.f32_to_bf16_bits(V.astype(np.float32))
    for t in range(L):
        cache[t // P, 0, t % P] = kb[t]
        cache[t // P, 1, t % P] = vb[t]
    indptr, indices, last = pt.page_table([L], P)
    return cache, indptr, indices, last


def test_closed_form_single_token():
    rng = np.random.default_rng(3)
    D = 8
    K = rng.integers(-4, 5, size=(1, 1, D)).astype(np.float64)
    V = rng.integers(-4, 5, size=(1, 1, D)).astype(np.float64)
    qv = rng.integers(-3, 4, size=(1, 1, D)).astype(np.float64)
    cache, indptr, indices, last = _one_request_cache(K, V)
    q = workloads.f32_to_bf16_bits(qv.astype(np.float32))
    o, lse = att.decode(q, cache, indptr, indices, last, 1)
    assert np.array_equal(o[0, 0], V[0, 0])                      # o = v_0
    assert lse[0, 0] == pytest.approx(math.fsum(qv[0, 0] * K[0, 0]) / math.sqrt(D), abs=1e-14)


def test_closed_form_zero_query_and_zero_scale():
    rng = np.random.default_rng(4)
    L, D = 23, 8
    K = rng.integers(-4, 5, size=(L, 1, D)).astype(np.float64)
    V = rng.integers(-4, 5, size=(L, 1, D)).astype(np.float64)
    cache, indptr, indices, last = _one_request_cache(K, V)
    q0 = np.zeros((1, 1, D), dtype=np.uint16)
    o, lse = att.decode(q0, cache, indptr, indices, last, 1)
    assert np.max(np.abs(o[0, 0] - V[:, 0].mean(axis=0))) < 1e-14   # uniform weights
    assert lse[0, 0] == pytest.approx(math.log(L), abs=1e-14)
    q1 = workloads.normal_bf16(rng, (1, 1, D))
    o, lse = att.decode(q1, cache, indptr, indices, last, 1, sm_scale=0.0)
    assert np.max(np.abs(o[0, 0] - V[:, 0].mean(axis=0))) < 1e-14
    assert lse[0, 0] == pytest.approx(math.log(L), abs=1e-14)


def test_closed_form_identical_keys():
    rng = np.random.default_rng(5)
    L, D = 37, 8
    k_row = rng.integers(-3, 4, size=D).astype(np.float64)
    K = np.tile(k_row, (L, 1, 1))
    V = rng.integers(-4, 5, size=(L, 1, D)).astype(np.float64)
    qv = rng.integers(-3, 4, size=(1, 1, D)).astype(np.float64)
    cache, indptr, indices, last = _one_request_cache(K, V)
    q = workloads.f32_to_bf16_bits(qv.astype(np.float32))
    o, lse = att.decode(q, cache, indptr, indices, last, 1)
    s = math.fsum(qv[0, 0] * k_row) / math.sqrt(D)
    assert np.max(np.abs(o[0, 0] - V[:, 0].mean(axis=0))) < 1e-13
    assert lse[0, 0] == pytest.approx(s + math.log(L), abs=1e-13)


def test_page_order_permutation_invariance():
    """Attention is a function of the key set: listing a request's full pages
    in another order leaves (o, lse) unchanged."""
    rng = np.random.default_rng(6)
    P, Hq, Hkv, D = 4, 4, 2, 8
    batch = workloads.make_batch([4 * P], P, 10, Hq, Hkv, D, rng)
    q = workloads.host_query(batch, rng)
    cache = workloads.host_cache(batch, rng)
    o1, l1 = att.decode(q, cache, batch.kv_indptr, batch.kv_indices, batch.kv_last_page_len, Hkv)
    perm = batch.kv_indices[::-1].copy()
    o2, l2 = att.decode(q, cache, batch.kv_indptr, perm, batch.kv_last_page_len, Hkv)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


def test_gqa_group_one_is_plain_multihead():
    """g = 1: query head h reads KV head h; equal to running each head alone."""
    batch, q, cache = _tiny_case(9, Hq=3, Hkv=3)
    o, lse = att.decode(q, cache, batch.kv_indptr, batch.kv_indices, batch.kv_last_page_len, 3)
    for h in range(3):
        o1, l1 = att.decode(q[:, h:h + 1], cache[:, :, :, h:h + 1], batch.kv_indptr,
                            batch.kv_indices, batch.kv_last_page_len, 1)
        assert np.max(np.abs(o[:, h] - o1[:, 0])) < 1e-15
        assert np.max(np.abs(lse[:, h] - l1[:, 0])) < 1e-15


def test_request_state_full_range_equals_decode():
    batch, q, cache = _tiny_case(12)
    o, lse = att.decode(q, cache, batch.kv_indptr, batch.kv_indices, batch.kv_last_page_len, 2)
    for i in range(batch.batch):
        L = int(batch.kv_lens[i])
        o1, l1 = att.request_state(q, cache, batch.kv_indptr, batch.kv_indices,
                                   batch.kv_last_page_len, 2, i, 0, L)
        assert np.max(np.abs(o1 - o[i])) < 1e-15 and np.max(np.abs(l1 - lse[i])) < 1e-15
