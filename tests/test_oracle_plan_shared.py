"""Pins for the shared-prefix (composable) plan of oracle.plan_ref: a
schedule worked out by hand, the reduction to the decode plan when every
group is one request and there is one KV head, and invariants any correct
schedule must satisfy (every page of every (group, row block, KV head)
covered once and in order, consistent partial ids and merge list)."""

import numpy as np
import pytest

from oracle import page_table as pt
from oracle import plan_ref


def test_hand_worked_two_groups():
    # group 0: 3 requests over 4 full pages (64 tokens); group 1: 1 request
    # over one page holding 5 tokens.  P 16, S 4, gqa 4 (32 requests per
    # block), 2 KV heads, min_chunk_tokens 16.
    # T_eff = 64 + 5 = 69; 69 * 2 = 138; ceil(138 / 4) = 35 tokens -> 3 pages.
    # group 0: chunks of 3 and 1 pages (48 and 16 tokens), split; its
    # requests r = 0, 1, 2 get partial ids 2r + j.  group 1: one chunk.
    # Costs (alpha l_q + beta l_kv): 3 + 48 = 51, 3 + 16 = 19, 1 + 5 = 6,
    # each for heads 0 and 1.  LPT: 51 -> s0, 51 -> s1, 19 -> s2, 19 -> s3,
    # 6 -> s2 (19 = 19, lower id), 6 -> s3.
    p = plan_ref.plan_shared([0, 3, 4], [0, 4, 5], [16, 5], 16, 4, 4, 2, min_chunk_tokens=16)
    assert p["chunk_pages"] == 3 and p["t_eff"] == 69 and p["rows_per_block"] == 32
    assert p["slot_indptr"].tolist() == [0, 1, 2, 4, 6]
    assert p["items"].tolist() == [
        [0, 0, 3, 16, 0, 48, 0, 0],
        [0, 0, 3, 16, 0, 48, 0, 1],
        [0, 3, 1, 16, 1, 16, 0, 0], [1, 4, 1, 5, -1, 5, 0, 0],
        [0, 3, 1, 16, 1, 16, 0, 1], [1, 4, 1, 5, -1, 5, 0, 1]]
    assert p["merges"].tolist() == [[0, 0, 2], [1, 2, 2], [2, 4, 2]]
    assert p["groups"].tolist() == [[0, 3, 2, 0], [3, 1, 1, -1]]
    assert p["n_partials"] == 6 and p["slot_loads"].tolist() == [51, 51, 25, 25]


@pytest.mark.parametrize("seed", range(4))
def test_one_request_groups_and_one_head_reduce_to_decode_plan(seed):
    rng = np.random.default_rng(seed)
    P = [16, 1, 8, 32][seed]
    lens = rng.integers(1, 3000, size=int(rng.integers(1, 40)))
    indptr, _, last = pt.page_table(lens, P)
    B = len(lens)
    S = [1, 7, 64, 256][seed]
    opts = [dict(), dict(min_chunk_tokens=16), dict(fixed_chunk_pages=2), dict(alpha=3, beta=2)][seed]
    d = plan_ref.plan(indptr, last, P, S, **opts)
    s = plan_ref.plan_shared(np.arange(B + 1), indptr, last, P, S, 4, 1, **opts)
    assert s["chunk_pages"] == d["chunk_pages"]
    assert np.array_equal(s["slot_indptr"], d["slot_indptr"])
    assert np.array_equal(s["items"][:, :5], d["items"])
    assert not s["items"][:, 6:].any()
    assert np.array_equal(s["merges"], d["merges"])
    assert s["n_partials"] == d["n_partials"]


@pytest.mark.parametrize("seed", range(6))
def test_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    P = [16, 32, 64, 16, 16, 32][seed]
    G = int(rng.integers(1, 6))
    gqa = [1, 2, 4, 8, 4, 8][seed]
    Hkv = [8, 4, 8, 2, 1, 8][seed]
    rows = rng.integers(1, 300, size=G)
    qo = np.concatenate([[0], np.cumsum(rows)])
    lens = rng.integers(1, 20000, size=G)
    indptr, _, last = pt.page_table(lens, P)
    S = int(rng.integers(1, 300))
    p = plan_ref.plan_shared(qo, indptr, last, P, S, gqa, Hkv, min_chunk_tokens=[128, 16, 1, 512, 128, 64][seed])
    tq = 128 // gqa
    items = p["items"]
    assert items.shape[0] == p["num_items"] and p["slot_indptr"][-1] == p["num_items"]
    # every (group, block, head) covers the group's pages once, in chunk order
    for g in range(G):
        nb = -(-int(rows[g]) // tq)
        for b in range(nb):
            for h in range(Hkv):
                sel = items[(items[:, 0] == g) & (items[:, 6] == b) & (items[:, 7] == h)]
                sel = sel[np.argsort(sel[:, 1])]
                assert sel[0, 1] == indptr[g]
                assert np.array_equal(sel[1:, 1], sel[:-1, 1] + sel[:-1, 2])
                assert sel[-1, 1] + sel[-1, 2] == indptr[g + 1]
                assert sel[:, 5].sum() == lens[g]
                assert np.array_equal(sel[:, 5], (sel[:, 2] - 1) * P + sel[:, 3])
                k = sel.shape[0]
                assert p["groups"][g].tolist()[:3] == [qo[g], rows[g], k]
                if k == 1:
                    assert sel[0, 4] == -1
                else:
                    base = p["groups"][g][3]
                    assert sel[:, 4].tolist() == list(range(base, base + k))
    # partial ids: every request of a split group owns k consecutive ids;
    # together they tile [0, n_partials)
    ids = []
    for req, first, k in p["merges"].tolist():
        ids.extend(range(first, first + k))
    assert sorted(ids) == list(range(p["n_partials"]))
    assert p["merges"][:, 0].tolist() == sorted(p["merges"][:, 0].tolist())
    # LPT bound: max load <= mean load + largest item cost
    costs = []
    for it in items:
        g, b = it[0], it[6]
        lq = min(tq, rows[g] - b * tq)
        costs.append(lq + it[5])
    assert p["slot_loads"].sum() == sum(costs)
    assert p["slot_loads"].max() <= p["slot_loads"].mean() + max(costs)
