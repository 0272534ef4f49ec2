"""Plain, slow CPU reference for paged GQA decode -- TEST INFRASTRUCTURE ONLY.

What it computes, in float64 with numpy:

* ``page_table``  -- the CSR page table for a list of KV lengths and the
  length identity l = P (n - 1) + r, 1 <= r <= P;
* ``attention``   -- softmax(q K^T / sqrt(d)) V and its log-sum-exp for each
  request and query head, gathering K and V through the page table;
* ``merge``       -- the exact combination of attention states over
  disjoint key sets;
* ``plan_ref``    -- the split-KV work schedule (chunking, longest-first
  assignment to a fixed number of workgroups, reduction map) that the
  library's host planner must reproduce bit for bit, for decode plans and
  shared-prefix (composable) plans;
* ``append``      -- writing new tokens' K and V rows into their page slots,
  and the request / position of every new token;
* ``fp8``         -- FP8 E4M3 cache values and the scale contract (decode
  over an FP8 cache is ``attention.decode_fp8``, quantising appends
  ``append.append_quantized``).

Sources: the three FlashInfer pages (aicassindra "FlashInfer, in depth";
pyshine "FlashInfer" source tour; pinghaoyang "FlashInfer 完全拆解").  Each
function cites the passage it follows.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never calls it, and it
shares no code with the library: the two meet only on the seeded inputs from
``workloads``.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against the pages' worked example, closed forms, a library routine (torch's
scaled_dot_product_attention in float64) or brute force.  No function is
"parity unpinned".
"""

from . import append, attention, fp8, merge, page_table, plan_ref  # noqa: F401
