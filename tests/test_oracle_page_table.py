"""Pins for oracle.page_table: the pages' worked example, the length
identity, and hand-counted page boundaries."""

import json
import os

import numpy as np
import pytest

from oracle import page_table as pt

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_table_worked_example.json")


def test_worked_example_matches_pages():
    g = json.load(open(GOLDEN))
    indptr, indices, last = pt.page_table(g["kv_lens"], g["page_size"])
    assert indptr.tolist() == g["kv_indptr"]
    assert indices.tolist() == g["kv_indices"]
    assert last.tolist() == g["kv_last_page_len"]
    assert indptr.dtype == np.int32 and indices.dtype == np.int32 and last.dtype == np.int32


# (length, pages, fill of last page), counted by hand
HAND = {
    16: [(1, 1, 1), (15, 1, 15), (16, 1, 16), (17, 2, 1), (32, 2, 16), (33, 3, 1),
         (100, 7, 4), (100_000, 6250, 16)],
    1: [(1, 1, 1), (2, 2, 1), (7, 7, 1)],
    4: [(3, 1, 3), (4, 1, 4), (5, 2, 1), (8, 2, 4)],
}


@pytest.mark.parametrize("page_size", sorted(HAND))
def test_page_boundaries_by_hand(page_size):
    for length, pages, fill in HAND[page_size]:
        indptr, indices, last = pt.page_table([length], page_size)
        assert int(indptr[1]) == pages, (length, page_size)
        assert int(last[0]) == fill, (length, page_size)
        assert indices.tolist() == list(range(pages))


def test_exact_multiple_never_writes_zero():
    # a length that is an exact multiple of P keeps a full last page (the
    # failure mode the aicassindra page warns about is writing 0 here)
    for P in (1, 2, 16, 64):
        for m in (1, 2, 5):
            _, _, last = pt.page_table([m * P], P)
            assert int(last[0]) == P


def test_length_identity_random():
    rng = np.random.default_rng(11)
    for P in (1, 3, 16, 32):
        lens = rng.integers(1, 500, size=40)
        perm = rng.permutation(30_000)
        indptr, indices, last = pt.page_table(lens, P, page_ids=perm)
        n = np.diff(indptr.astype(np.int64))
        # every request's pages hold its tokens and no page is wasted
        assert np.all((n - 1) * P < lens) and np.all(lens <= n * P)
        assert np.all((last >= 1) & (last <= P))
        assert np.array_equal(pt.kv_lengths(indptr, last, P), lens)
        assert indices.tolist() == perm[: indptr[-1]].tolist()
        pt.check(indptr, last, P)


def test_check_rejects_bad_tables():
    with pytest.raises(ValueError):
        pt.check([0, 2], [0], 16)          # last_page_len 0
    with pytest.raises(ValueError):
        pt.check([0, 2], [17], 16)         # last_page_len > P
    with pytest.raises(ValueError):
        pt.check([1, 2], [3], 16)          # indptr[0] != 0
    with pytest.raises(ValueError):
        pt.check([0, 2, 2], [3, 3], 16)    # a request with no page
    with pytest.raises(ValueError):
        pt.page_table([0], 16)


def test_workload_allocator_agrees_with_oracle():
    """The input generator's page allocator and the oracle's page table are
    written separately; they must agree."""
    import workloads

    rng = np.random.default_rng(5)
    for P in (1, 16):
        lens = rng.integers(1, 300, size=25)
        perm = rng.permutation(20_000)
        a = workloads.allocate_pages(lens, P, perm)
        b = pt.page_table(lens, P, page_ids=perm)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
