"""Split-KV work schedule (oracle).

The shape of the algorithm is the pinghaoyang page's, section
"先切长 KV，再做最长任务优先分配" (split long KV first, then longest-first
assignment):

* the chunk bound is the total work divided by the fixed CTA count,
  L_kv = sum_i ceil(l_q(i) / T_q) l_kv(i) / N_CTA; with one query row per
  request (decode) that is T / S for T = sum of KV lengths and S slots;
* KV ranges longer than the bound are cut along the sequence into chunks;
* a work item costs C = alpha l_q + beta l_kv;
* items are sorted by cost, longest first, and each goes to the slot with the
  least accumulated cost (LPT);
* partial states are combined through a fixed reduction map, in a fixed
  order, with no atomics (same section, the Stream-K paragraph).

Requests that are not split write their output directly ("writethrough",
pinghaoyang section "Split-KV 解决的是并行度，不是减少计算量"; aicassindra
"Load balancing with split-KV": short sequences are not split).

Readings where the pages leave a step open (also in the design notes):
* chunks are whole pages;
* cp = fixed_chunk_pages when given, else
  max(ceil(min_chunk_tokens / P), ceil(ceil(T / S) / P)), min_chunk_tokens = 128;
* alpha = beta = 1 with l_q = 1, so cost = 1 + chunk length;
* ties: items are ordered by (-cost, request, chunk); an item goes to the
  least-loaded slot, the lowest slot id among equals;
* split request i gets partial ids base_i .. base_i + k_i - 1, with base_i
  the number of chunks of the split requests before it;
* with ``all_partials`` every request counts as split (a request of one
  chunk gets one partial id and a merge-list entry), so that its state can be
  merged with states from another plan; the merge list then names every
  request in order.

The least-loaded-slot choice is written twice, as a binary heap (``plan``)
and as a plain scan over the slots (``plan_naive``), and the tests require
the two to agree; both share the chunking, the item order (``_prepare``) and
the output assembly, which are pinned on their own by hand-worked schedules
and by invariants (every page once, in order; lengths summing to T).
"""

from __future__ import annotations

import heapq

import numpy as np

DEFAULT_MIN_CHUNK_TOKENS = 128


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def chunk_pages(total_tokens: int, page_size: int, num_slots: int,
                fixed_chunk_pages: int = 0,
                min_chunk_tokens: int = DEFAULT_MIN_CHUNK_TOKENS) -> int:
    if fixed_chunk_pages > 0:
        return int(fixed_chunk_pages)
    bound = _ceil_div(int(total_tokens), int(num_slots))
    return max(1, _ceil_div(int(min_chunk_tokens), page_size), _ceil_div(bound, page_size))


def work_items(kv_indptr, kv_last_page_len, page_size: int, cp: int, alpha: int, beta: int,
               all_partials: bool = False):
    """Chunks of every request, in request/chunk order, and the split map.

    Each item is a dict with request, chunk, page_begin, num_pages, last_len,
    length, out (partial id, -1 for writethrough) and cost."""
    indptr = [int(x) for x in kv_indptr]
    last = [int(x) for x in kv_last_page_len]
    items, merges = [], []
    next_partial = 0
    for i in range(len(last)):
        n = indptr[i + 1] - indptr[i]
        k = _ceil_div(n, cp)
        split = k > 1 or all_partials
        base = next_partial
        if split:
            merges.append((i, base, k))
            next_partial += k
        for j in range(k):
            pages = min(cp, n - j * cp)
            last_len = last[i] if j == k - 1 else page_size
            length = (pages - 1) * page_size + last_len
            items.append(dict(request=i, chunk=j, page_begin=indptr[i] + j * cp,
                              num_pages=pages, last_len=last_len, length=length,
                              out=base + j if split else -1,
                              cost=alpha + beta * length))
    return items, merges, next_partial


def _assemble(assignments, num_slots, items_in_order, merges, n_partials, header):
    per_slot = [[] for _ in range(num_slots)]
    for slot, item in assignments:
        per_slot[slot].append(item)
    slot_indptr = np.zeros(num_slots + 1, dtype=np.int32)
    rows = []
    for s in range(num_slots):
        slot_indptr[s + 1] = slot_indptr[s] + len(per_slot[s])
        for it in per_slot[s]:
            rows.append((it["request"], it["page_begin"], it["num_pages"], it["last_len"],
                         it["out"]))
    items_arr = np.array(rows, dtype=np.int32).reshape(-1, 5)
    merge_arr = np.array(merges, dtype=np.int32).reshape(-1, 3)
    loads = np.zeros(num_slots, dtype=np.int64)
    for slot, it in assignments:
        loads[slot] += it["cost"]
    return dict(header, slot_indptr=slot_indptr, items=items_arr, merges=merge_arr,
                num_items=len(items_in_order), n_partials=n_partials, n_split=len(merges),
                slot_loads=loads)


def _prepare(kv_indptr, kv_last_page_len, page_size, num_slots, fixed_chunk_pages,
             min_chunk_tokens, alpha, beta, all_partials=False):
    indptr = np.asarray(kv_indptr, dtype=np.int64)
    last = np.asarray(kv_last_page_len, dtype=np.int64)
    n = indptr[1:] - indptr[:-1]
    lengths = page_size * (n - 1) + last
    total = int(lengths.sum())
    cp = chunk_pages(total, page_size, num_slots, fixed_chunk_pages, min_chunk_tokens)
    items, merges, n_partials = work_items(indptr, last, page_size, cp, alpha, beta, all_partials)
    order = sorted(items, key=lambda it: (-it["cost"], it["request"], it["chunk"]))
    header = dict(batch=int(last.shape[0]), page_size=int(page_size), num_slots=int(num_slots),
                  chunk_pages=cp, total_tokens=total, alpha=alpha, beta=beta)
    return items, order, merges, n_partials, header


def plan(kv_indptr, kv_last_page_len, page_size: int, num_slots: int,
         fixed_chunk_pages: int = 0, min_chunk_tokens: int = DEFAULT_MIN_CHUNK_TOKENS,
         alpha: int = 1, beta: int = 1, all_partials: bool = False):
    """The schedule, with a binary heap keyed (load, slot)."""
    items, order, merges, n_partials, header = _prepare(
        kv_indptr, kv_last_page_len, page_size, num_slots, fixed_chunk_pages,
        min_chunk_tokens, alpha, beta, all_partials)
    heap = [(0, s) for s in range(num_slots)]
    assignments = []
    for it in order:
        load, slot = heapq.heappop(heap)
        assignments.append((slot, it))
        heapq.heappush(heap, (load + it["cost"], slot))
    return _assemble(assignments, num_slots, items, merges, n_partials, header)


def plan_naive(kv_indptr, kv_last_page_len, page_size: int, num_slots: int,
               fixed_chunk_pages: int = 0, min_chunk_tokens: int = DEFAULT_MIN_CHUNK_TOKENS,
               alpha: int = 1, beta: int = 1, all_partials: bool = False):
    """The same schedule with a linear scan for the least-loaded slot."""
    items, order, merges, n_partials, header = _prepare(
        kv_indptr, kv_last_page_len, page_size, num_slots, fixed_chunk_pages,
        min_chunk_tokens, alpha, beta, all_partials)
    loads = [0] * num_slots
    assignments = []
    for it in order:
        best = 0
        for s in range(1, num_slots):
            if loads[s] < loads[best]:
                best = s
        assignments.append((best, it))
        loads[best] += it["cost"]
    return _assemble(assignments, num_slots, items, merges, n_partials, header)


# ---------------------------------------------------------------------------
# Shared-prefix (composable) plans: a block row of several requests
# ---------------------------------------------------------------------------
#
# The pinghaoyang page, section "Composable Format：共享前缀与独有后缀分开算"
# (composable format: shared prefix and unique suffixes computed apart), puts
# a prefix that several requests share in one block row of the KV matrix, so
# that one workgroup reads each prefix page once for all of those requests;
# the suffixes stay one-request rows.  Here a *group* is such a block row: a
# contiguous range of request rows (qo_indptr) that all attend to the same
# pages (the group's row of kv_indptr / kv_indices / kv_last_page_len).
#
# The work of a group is cut the same way as decode work, with the chunk
# bound of the same section counting query tiles:
# L_kv = sum_g ceil(R_g / T_q) l_g / N_CTA, where R_g requests of group g are
# tiled T_q = 128 / gqa requests at a time (128 query rows per workgroup:
# gqa query heads per request).  Readings:
# * one workgroup computes one KV head of one (group, row block, chunk), so
#   N_CTA per KV head is S / Hkv and L_kv = T_eff Hkv / S with
#   T_eff = sum_g ceil(R_g / T_q) l_g;
# * cp = fixed_chunk_pages when given, else
#   max(ceil(min_chunk_tokens / P), ceil(ceil(T_eff Hkv / S) / P));
# * an item costs alpha l_q + beta l_kv, with l_q the requests in its block;
# * ties: (-cost, group, block, chunk, head), then the least-loaded slot,
#   lowest slot id among equals;
# * a split group g (k_g > 1 chunks) gives each of its requests r (0-based
#   within the group) the partial ids base_g + r k_g + j, j = 0..k_g-1, with
#   base_g the partial count of the split groups before it; the merge list
#   has one entry (request, base_g + r k_g, k_g) per request of every split
#   group, in request order;
# * with ``all_partials`` every group counts as split, as in ``plan``.

SHARED_ROWS_PER_WORKGROUP = 128


def plan_shared(qo_indptr, kv_indptr, kv_last_page_len, page_size: int, num_slots: int,
                gqa: int, num_kv_heads: int, fixed_chunk_pages: int = 0,
                min_chunk_tokens: int = DEFAULT_MIN_CHUNK_TOKENS, alpha: int = 1,
                beta: int = 1, all_partials: bool = False):
    """Schedule of a shared-prefix plan (heap LPT, as ``plan``)."""
    qo = [int(x) for x in qo_indptr]
    indptr = [int(x) for x in kv_indptr]
    last = [int(x) for x in kv_last_page_len]
    G = len(last)
    tq = SHARED_ROWS_PER_WORKGROUP // gqa
    rows = [qo[g + 1] - qo[g] for g in range(G)]
    npages = [indptr[g + 1] - indptr[g] for g in range(G)]
    lengths = [page_size * (npages[g] - 1) + last[g] for g in range(G)]
    blocks = [_ceil_div(rows[g], tq) for g in range(G)]
    t_eff = sum(blocks[g] * lengths[g] for g in range(G))
    cp = chunk_pages(t_eff * num_kv_heads, page_size, num_slots, fixed_chunk_pages,
                     min_chunk_tokens)
    items, merges, groups = [], [], []
    next_partial = 0
    for g in range(G):
        k = _ceil_div(npages[g], cp)
        split = k > 1 or all_partials
        base = next_partial if split else -1
        if split:
            for r in range(rows[g]):
                merges.append((qo[g] + r, next_partial + r * k, k))
            next_partial += rows[g] * k
        groups.append((qo[g], rows[g], k, base))
        for b in range(blocks[g]):
            lq = min(tq, rows[g] - b * tq)
            for j in range(k):
                pages = min(cp, npages[g] - j * cp)
                last_len = last[g] if j == k - 1 else page_size
                length = (pages - 1) * page_size + last_len
                for h in range(num_kv_heads):
                    items.append(dict(group=g, block=b, chunk=j, head=h,
                                      page_begin=indptr[g] + j * cp, num_pages=pages,
                                      last_len=last_len, length=length,
                                      out=base + j if split else -1,
                                      cost=alpha * lq + beta * length))
    order = sorted(items, key=lambda it: (-it["cost"], it["group"], it["block"], it["chunk"],
                                          it["head"]))
    heap = [(0, s) for s in range(num_slots)]
    per_slot = [[] for _ in range(num_slots)]
    loads = np.zeros(num_slots, dtype=np.int64)
    for it in order:
        load, slot = heapq.heappop(heap)
        per_slot[slot].append(it)
        loads[slot] += it["cost"]
        heapq.heappush(heap, (load + it["cost"], slot))
    slot_indptr = np.zeros(num_slots + 1, dtype=np.int32)
    out_rows = []
    for s in range(num_slots):
        slot_indptr[s + 1] = slot_indptr[s] + len(per_slot[s])
        for it in per_slot[s]:
            out_rows.append((it["group"], it["page_begin"], it["num_pages"], it["last_len"],
                             it["out"], it["length"], it["block"], it["head"]))
    return dict(num_groups=G, batch=qo[-1], page_size=int(page_size), num_slots=int(num_slots),
                chunk_pages=cp, total_tokens=int(sum(lengths)), t_eff=int(t_eff),
                rows_per_block=tq, slot_indptr=slot_indptr,
                items=np.array(out_rows, dtype=np.int32).reshape(-1, 8),
                merges=np.array(merges, dtype=np.int32).reshape(-1, 3),
                groups=np.array(groups, dtype=np.int32).reshape(-1, 4),
                num_items=len(items), n_partials=next_partial, n_split=len(merges),
                slot_loads=loads)
