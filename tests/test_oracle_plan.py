"""Pins for oracle.plan_ref: schedules worked out by hand from the
longest-first rule, agreement of the heap and plain-scan implementations,
and invariants any correct schedule must satisfy."""

import numpy as np
import pytest

from oracle import page_table as pt
from oracle import plan_ref


def test_hand_worked_lpt_without_splits():
    # costs 5,4,3,3,3 on two slots (alpha 0, beta 1, page_size 1, no split):
    # 5 -> s0; 4 -> s1; 3 -> s1 (4<5); 3 -> s0 (5<7); 3 -> s1 (7<8).
    # Loads 8 and 10 (LPT is not optimal here: 9/9 exists).
    indptr, _, last = pt.page_table([5, 4, 3, 3, 3], 1)
    for impl in (plan_ref.plan, plan_ref.plan_naive):
        p = impl(indptr, last, 1, 2, fixed_chunk_pages=1000, alpha=0, beta=1)
        assert p["slot_indptr"].tolist() == [0, 2, 5]
        assert p["items"].tolist() == [
            [0, 0, 5, 1, -1], [3, 12, 3, 1, -1],
            [1, 5, 4, 1, -1], [2, 9, 3, 1, -1], [4, 15, 3, 1, -1]]
        assert p["slot_loads"].tolist() == [8, 10]
        assert p["n_split"] == 0 and p["n_partials"] == 0 and p["merges"].shape == (0, 3)


def test_hand_worked_split_and_writethrough():
    # P 16, S 4, lengths 100 and 20, min_chunk_tokens 16:
    # T = 120, ceil(120/4) = 30 tokens -> 2 pages per chunk.
    # request 0: 7 pages (last holds 4) -> chunks of 2,2,2,1 pages, lengths
    # 32,32,32,4, partial ids 0..3; request 1: 2 pages (20 tokens) -> one
    # chunk, written through.  Costs 33,33,33,5 and 21; LPT gives the three
    # 33s to slots 0-2, the 21 to slot 3, then the 5 to slot 3 (load 21).
    indptr, _, last = pt.page_table([100, 20], 16)
    for impl in (plan_ref.plan, plan_ref.plan_naive):
        p = impl(indptr, last, 16, 4, min_chunk_tokens=16)
        assert p["chunk_pages"] == 2
        assert p["slot_indptr"].tolist() == [0, 1, 2, 3, 5]
        assert p["items"].tolist() == [
            [0, 0, 2, 16, 0], [0, 2, 2, 16, 1], [0, 4, 2, 16, 2],
            [1, 7, 2, 4, -1], [0, 6, 1, 4, 3]]
        assert p["merges"].tolist() == [[0, 0, 4]]
        assert p["n_partials"] == 4 and p["n_split"] == 1 and p["num_items"] == 5


def test_hand_worked_all_partials():
    # The same schedule as above with every request's states as partials:
    # request 1's one chunk now gets partial id 4 (after request 0's four)
    # and a merge-list entry of its own; slots and order do not change.
    indptr, _, last = pt.page_table([100, 20], 16)
    for impl in (plan_ref.plan, plan_ref.plan_naive):
        p = impl(indptr, last, 16, 4, min_chunk_tokens=16, all_partials=True)
        assert p["slot_indptr"].tolist() == [0, 1, 2, 3, 5]
        assert p["items"].tolist() == [
            [0, 0, 2, 16, 0], [0, 2, 2, 16, 1], [0, 4, 2, 16, 2],
            [1, 7, 2, 4, 4], [0, 6, 1, 4, 3]]
        assert p["merges"].tolist() == [[0, 0, 4], [1, 4, 1]]
        assert p["n_partials"] == 5 and p["n_split"] == 2
    # the worked example, none of it split: ids 0, 1, 2, one per request
    indptr, _, last = pt.page_table([37, 16, 5], 16)
    p = plan_ref.plan(indptr, last, 16, 512, all_partials=True)
    assert p["items"].tolist() == [[0, 0, 3, 5, 0], [1, 3, 1, 16, 1], [2, 4, 1, 5, 2]]
    assert p["merges"].tolist() == [[0, 0, 1], [1, 1, 1], [2, 2, 1]]


def test_worked_example_batch_is_not_split():
    # [37,16,5] at P 16 on 512 slots: cp = max(ceil(128/16), ceil(ceil(58/512)/16)) = 8
    indptr, _, last = pt.page_table([37, 16, 5], 16)
    p = plan_ref.plan(indptr, last, 16, 512)
    assert p["chunk_pages"] == 8
    assert p["items"].tolist() == [[0, 0, 3, 5, -1], [1, 3, 1, 16, -1], [2, 4, 1, 5, -1]]
    assert p["slot_indptr"][:4].tolist() == [0, 1, 2, 3] and p["slot_indptr"][-1] == 3


def _check_invariants(p, indptr, last, P, S, fixed):
    lens = pt.kv_lengths(indptr, last, P)
    T = int(lens.sum())
    items = p["items"]
    cp = p["chunk_pages"]
    assert p["slot_indptr"][0] == 0 and p["slot_indptr"][-1] == items.shape[0]
    assert np.all(np.diff(p["slot_indptr"]) >= 0)
    # coverage: each request's chunks tile its page range in order
    by_req = {}
    for r, pb, npg, ll, out in items.tolist():
        by_req.setdefault(r, []).append((pb, npg, ll, out))
    total = 0
    for i in range(len(last)):
        ch = sorted(by_req[i])
        pos = int(indptr[i])
        outs = []
        for j, (pb, npg, ll, out) in enumerate(ch):
            assert pb == pos and 1 <= npg <= cp
            pos += npg
            final = j == len(ch) - 1
            assert ll == (int(last[i]) if final else P)
            total += (npg - 1) * P + ll
            outs.append(out)
        assert pos == int(indptr[i + 1])
        if len(ch) == 1:
            assert outs == [-1]
        else:
            assert outs == list(range(outs[0], outs[0] + len(ch)))
    assert total == T
    # merge map: split requests ascending with contiguous partial ids
    m = p["merges"]
    assert m.shape[0] == p["n_split"]
    if m.shape[0]:
        assert np.all(np.diff(m[:, 0]) > 0)
        assert m[0, 1] == 0 and np.all(m[1:, 1] == (m[:-1, 1] + m[:-1, 2]))
        assert int(m[:, 2].sum()) == p["n_partials"]
    # list-scheduling bound and the item-count bound
    costs = 1 + ((items[:, 2].astype(np.int64) - 1) * P + items[:, 3])
    assert p["slot_loads"].max() <= costs.sum() / S + costs.max()
    if not fixed:
        assert items.shape[0] <= S + 2 * len(last)
    # each slot's list is longest-first
    for s in range(S):
        c = costs[p["slot_indptr"][s]:p["slot_indptr"][s + 1]]
        assert np.all(np.diff(c) <= 0)


@pytest.mark.parametrize("seed", range(12))
def test_heap_and_scan_agree_and_invariants_hold(seed):
    rng = np.random.default_rng(seed)
    P = [1, 16, 16, 4][seed % 4]
    S = [1, 3, 7, 64, 512][seed % 5]
    B = int(rng.integers(1, 40))
    lens = rng.integers(1, 3000, size=B)
    if seed % 3 == 0:
        lens[0] = 50_000
    indptr, _, last = pt.page_table(lens, P)
    fixed = [0, 0, 1, 3][seed % 4]
    mct = [128, 16, 256][seed % 3]
    a = plan_ref.plan(indptr, last, P, S, fixed_chunk_pages=fixed, min_chunk_tokens=mct)
    b = plan_ref.plan_naive(indptr, last, P, S, fixed_chunk_pages=fixed, min_chunk_tokens=mct)
    for k in ("slot_indptr", "items", "merges", "slot_loads"):
        assert np.array_equal(a[k], b[k]), k
    _check_invariants(a, indptr, last, P, S, fixed)


def test_workload_item_counts():
    import workloads

    for name, S in (("llama8b_step", 512), ("skewed", 512), ("wide_gqa", 512)):
        _, _, batches = workloads.workload(name)
        bt = batches["main"]
        p = plan_ref.plan(bt.kv_indptr, bt.kv_last_page_len, bt.page_size, S)
        assert p["num_items"] <= S + 2 * bt.batch
        _check_invariants(p, bt.kv_indptr, bt.kv_last_page_len, bt.page_size, S, 0)
