"""Seeded synthetic inputs for paged GQA decode.

This package is shared by the tests, the benchmark and the oracle-side checks.
It draws request lengths, places pages in a pool and fills q/K/V with N(0, 1)
values rounded to bf16.  It holds none of the attention or scheduling
arithmetic: those live, independently, in the oracle and in the HIP library.
"""

from .synth import (  # noqa: F401
    PagedBatch,
    WorkloadSpec,
    WORKLOADS,
    allocate_pages,
    device_cache,
    device_cache_e4m3,
    device_query,
    e4m3_codes,
    edge_lengths,
    f32_to_bf16_bits,
    host_cache,
    host_cache_e4m3,
    host_query,
    make_batch,
    normal_bf16,
    random_batch,
    workload,
)
