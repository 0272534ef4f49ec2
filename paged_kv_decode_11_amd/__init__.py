"""Paged GQA decode attention for AMD MI355X (gfx950).

A thin Python binding over libpkd.so (C ABI in include/pkd.h): a host
scheduler that plans split-KV work once per decode step, a HIP decode kernel
that runs once per layer over a CSR-paged bf16 KV cache, a kernel that
merges split attention states, and a shared-prefix kernel that reads a
prefix several requests share once for all of them.  There is no CPU
fallback: if the library is not built, importing the binding's entry points
raises.
"""

from ._lib import PkdError, header_functions, load  # noqa: F401
from .api import (  # noqa: F401
    DecodePlanRun,
    PlanMismatchError,
    SharedPlanRun,
    StaticPlanRun,
    append_paged_kv_cache,
    append_positions,
    check_append_args,
    check_run_args,
    float_workspace_bytes,
    host_workspace_bytes,
    int_workspace_bytes,
    merge_state,
    merge_states,
    plan_host,
    plan_shared_host,
    read_pages,
    read_stream,
    run_composable,
)
