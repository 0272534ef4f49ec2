"""Pins for oracle.merge: merging the states of disjoint key sets must give
the state of their union exactly (to float64 rounding), and the merge is
commutative, associative and has the empty state as identity."""

import math

import numpy as np
import pytest

import workloads
from oracle import attention as att
from oracle import merge as mg


def _request(seed, L=57, P=4, Hq=4, Hkv=2, D=8):
    rng = np.random.default_rng(seed)
    batch = workloads.make_batch([L], P, -(-L // P) + 3, Hq, Hkv, D, rng)
    q = workloads.host_query(batch, rng)
    cache = workloads.host_cache(batch, rng, poison=True)
    return batch, q, cache


def _state(batch, q, cache, t0, t1):
    return att.request_state(q, cache, batch.kv_indptr, batch.kv_indices,
                             batch.kv_last_page_len, batch.num_kv_heads, 0, t0, t1)


@pytest.mark.parametrize("cut", [1, 4, 20, 56])
def test_two_way_split_is_exact(cut):
    batch, q, cache = _request(1)
    L = int(batch.kv_lens[0])
    full_o, full_l = _state(batch, q, cache, 0, L)
    a_o, a_l = _state(batch, q, cache, 0, cut)
    b_o, b_l = _state(batch, q, cache, cut, L)
    for h in range(q.shape[1]):
        o, lse = mg.merge_two(a_o[h], a_l[h], b_o[h], b_l[h])
        assert np.max(np.abs(o - full_o[h])) < 1e-12
        assert abs(lse - full_l[h]) < 1e-12


def test_many_way_split_is_exact():
    batch, q, cache = _request(2, L=200)
    cuts = [0, 3, 17, 64, 65, 130, 200]
    full_o, full_l = _state(batch, q, cache, 0, 200)
    parts = [_state(batch, q, cache, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    for h in range(q.shape[1]):
        o, lse = mg.merge_many([(p[0][h], p[1][h]) for p in parts])
        assert np.max(np.abs(o - full_o[h])) < 1e-12
        assert abs(lse - full_l[h]) < 1e-12


def test_commutative_associative_identity():
    rng = np.random.default_rng(3)
    s = [(rng.standard_normal(8), float(rng.normal() * 5)) for _ in range(3)]
    ab = mg.merge_two(*s[0], *s[1])
    ba = mg.merge_two(*s[1], *s[0])
    assert np.max(np.abs(ab[0] - ba[0])) < 1e-15 and abs(ab[1] - ba[1]) < 1e-15
    left = mg.merge_two(*ab, *s[2])
    bc = mg.merge_two(*s[1], *s[2])
    right = mg.merge_two(*s[0], *bc)
    assert np.max(np.abs(left[0] - right[0])) < 1e-14 and abs(left[1] - right[1]) < 1e-14
    empty = (np.zeros(8), -math.inf)
    ident = mg.merge_two(*s[0], *empty)
    assert np.array_equal(ident[0], s[0][0]) and ident[1] == s[0][1]


def test_empty_states():
    o, lse = mg.merge_two(np.zeros(4), -math.inf, np.zeros(4), -math.inf)
    assert lse == -math.inf and np.array_equal(o, np.zeros(4))
    o, lse = att.attention_state(np.zeros(4), np.zeros((0, 4)), np.zeros((0, 4)), 0.5)
    assert lse == -math.inf and np.array_equal(o, np.zeros(4))


def test_weights_follow_lse_difference():
    """Two states whose lse differ by ln 3 combine with weights 3/4 and 1/4
    and lse = lse_b + ln 4."""
    o_a, o_b = np.ones(4), -np.ones(4)
    o, lse = mg.merge_two(o_a, 0.7 + math.log(3.0), o_b, 0.7)
    assert np.max(np.abs(o - 0.5)) < 1e-15
    assert lse == pytest.approx(0.7 + math.log(4.0), abs=1e-15)


def test_merge_rows_matches_scalar_merge():
    rng = np.random.default_rng(4)
    oa, ob = rng.standard_normal((3, 2, 5)), rng.standard_normal((3, 2, 5))
    la, lb = rng.standard_normal((3, 2)), rng.standard_normal((3, 2))
    o, lse = mg.merge_rows(oa, la, ob, lb)
    for i in range(3):
        for h in range(2):
            o1, l1 = mg.merge_two(oa[i, h], la[i, h], ob[i, h], lb[i, h])
            assert np.array_equal(o[i, h], o1) and lse[i, h] == l1
