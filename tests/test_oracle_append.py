"""Pins for oracle.append: the worked example's lengths grown by one token
(one request crossing into a fresh page), the identity "append, then gather
through the grown page table = the old tokens followed by the new rows" on
random batches with multi-token appends, untouched slots, and positions
outside a request's pages."""

import numpy as np

from oracle import append as ap
from oracle import attention as att
from oracle import page_table as pt


def _grow(old_lens, add, P, rng, pool):
    """Old and new page tables sharing page ids: every request keeps its old
    pages and gets fresh ones from the pool as it grows."""
    perm = rng.permutation(pool)
    old_pages, new_pages, cursor = [], [], 0
    for l0, a in zip(old_lens, add):
        n0 = -(-l0 // P)
        n1 = -(-(l0 + a) // P)
        pages = perm[cursor:cursor + n1]
        cursor += n1
        old_pages.append(pages[:n0])
        new_pages.append(pages)
    def table(page_lists, lens):
        indptr = np.concatenate([[0], np.cumsum([len(p) for p in page_lists])]).astype(np.int32)
        idx = np.concatenate(page_lists).astype(np.int32)
        last = np.array([l - (-(-l // P) - 1) * P for l in lens], np.int32)
        return indptr, idx, last
    return table(old_pages, old_lens), table(new_pages, [l + a for l, a in zip(old_lens, add)])


def test_worked_example_one_token_each():
    # [37, 16, 5] at P 16 grows to [38, 17, 6]: request 1 was an exact
    # multiple and needs a fresh page (its new token at position 16 goes to
    # slot 0 of that page); the others write slot 5 of their third page and
    # slot 5 of their only page.
    indptr, idx, last = pt.page_table([38, 17, 6], 16)
    assert indptr.tolist() == [0, 3, 5, 6] and last.tolist() == [6, 1, 6]
    b, pos = ap.batch_indices_positions([0, 1, 2, 3], indptr, last, 16)
    assert b.tolist() == [0, 1, 2] and pos.tolist() == [37, 16, 5]
    cache = np.zeros((6, 2, 16, 1, 2), np.uint16)
    k = np.array([[[1, 2]], [[3, 4]], [[5, 6]]], np.uint16)
    v = k + 100
    out = ap.append(cache, k, v, b, pos, indptr, idx)
    assert out[2, 0, 5].tolist() == [[1, 2]] and out[2, 1, 5].tolist() == [[101, 102]]
    assert out[4, 0, 0].tolist() == [[3, 4]] and out[4, 1, 0].tolist() == [[103, 104]]
    assert out[5, 0, 5].tolist() == [[5, 6]]
    assert np.count_nonzero(out) == 3 * 2 * 2


def test_append_then_gather_is_concatenation():
    rng = np.random.default_rng(3)
    for P in (1, 4, 16, 64):
        old = rng.integers(1, 300, size=9).tolist()
        add = rng.integers(0, 70, size=9).tolist()
        pool = sum(-(-(l + a) // P) for l, a in zip(old, add)) + 5
        (oi, ox, ol), (ni, nx, nl) = _grow(old, add, P, rng, pool)
        cache = rng.integers(0, 65535, size=(pool, 2, P, 2, 8), dtype=np.uint16)
        n_new = int(sum(add))
        k = rng.integers(0, 65535, size=(n_new, 2, 8), dtype=np.uint16)
        v = rng.integers(0, 65535, size=(n_new, 2, 8), dtype=np.uint16)
        append_indptr = np.concatenate([[0], np.cumsum(add)])
        b, pos = ap.batch_indices_positions(append_indptr, ni, nl, P)
        out = ap.append(cache, k, v, b, pos, ni, nx)
        for i in range(len(old)):
            k_old, v_old = att.gather_request(cache, oi, ox, ol, i)
            k_all, v_all = att.gather_request(out, ni, nx, nl, i)
            s, e = append_indptr[i], append_indptr[i + 1]
            assert np.array_equal(k_all, np.concatenate([k_old, k[s:e]]))
            assert np.array_equal(v_all, np.concatenate([v_old, v[s:e]]))
        # nothing else changed: exactly the new tokens' rows differ
        written = set()
        for t in range(n_new):
            page = nx[ni[b[t]] + pos[t] // P]
            written.add((int(page), int(pos[t] % P)))
        for page in range(pool):
            for slot in range(P):
                if (page, slot) not in written:
                    assert np.array_equal(out[page, :, slot], cache[page, :, slot])


def test_positions_outside_the_pages_are_skipped():
    indptr, idx, last = pt.page_table([20], 16)
    cache = np.zeros((3, 2, 16, 1, 1), np.uint16)
    k = np.ones((3, 1, 1), np.uint16)
    out = ap.append(cache, k, k, np.array([0, 0, 0]), np.array([19, 32, -1]), indptr, idx)
    assert np.count_nonzero(out) == 2 and out[1, 0, 3, 0, 0] == 1
