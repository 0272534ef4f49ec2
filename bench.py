#!/usr/bin/env python3
"""Paged GQA decode benchmark on one MI355X.

A step is one pass of the whole hot path over one batch: pkd_plan (host
scheduler + upload) once, then pkd_run once per layer (decode kernel + merge
kernel).  Default workload: the Llama-3-8B-like decode step (32 layers,
Hq 32 / Hkv 8 / D 128, bf16, page_size 16, batch 64 with KV lengths uniform
in [3000, 5000], pages scattered through a 32,768-page pool per layer).

Prints one JSON line for the main workload; by default the skewed batch (63
requests of 512 tokens and one of 100,000) is timed after it the same way
and reported under `targets` beside the main one, each with its fraction of
the HBM peak and the target fraction for that batch.  `value` is the
achieved KV-stream rate in GB/s
(KV bytes the step must read, 4096 B per token per layer, over the measured
step time; 2048 B with --kv-dtype e4m3).  By default a step is the plan
call followed by one replay of a
HIP graph that holds the step's runs; --no-graph launches the runs one by
one, and the eager timing is reported beside the graph one in any case.
`roofline` gives the decode kernel's own rate from HIP events
around each launch; `cpu_baseline` times the fp64 oracle on a sample of
layer 0's requests.  Inputs are synthetic and seeded.
"""

from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
# per-chunk weight (in tokens) of the shared-prefix workload's suffix plan
SUFFIX_ALPHA = 32
ROTATE_BYTES = 2 << 30  # single-layer workloads rotate caches to >= 2 GiB
METRIC = "paged GQA decode: achieved KV GB/s (% of HBM peak) and µs/layer-step"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_step",
                    choices=["llama8b_step", "skewed", "wide_gqa", "token_sparse", "tiny",
                             "shared_prefix", "shared_prefix_b16", "shared_prefix_b64",
                             "append"])
    ap.add_argument("--slots", type=int, default=0, help="persistent workgroups (0 = default)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle time budget for cpu_baseline (0 disables)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--variant", default="auto", choices=["auto", "dot2", "mfma", "mfma_pv"],
                    help="decode kernel (auto = the library's default for the shape)")
    ap.add_argument("--kv-dtype", default="bf16", choices=["bf16", "e4m3"],
                    help="KV cache element type (e4m3: FP8 codes with per-tensor scales)")
    ap.add_argument("--prefix-chunk-tokens", type=int, default=0,
                    help="shared_prefix: smallest chunk of the prefix plan in tokens (0 = the "
                         "library's default)")
    ap.add_argument("--prefix-slots", type=int, default=-1,
                    help="shared_prefix: workgroups of the shared-prefix kernel (0 = the "
                         "library's default, -1 = one per 512-token prefix item, between half "
                         "and three quarters of the compute units)")
    ap.add_argument("--suffix-slots", type=int, default=-1,
                    help="shared_prefix: workgroups of the suffix decode kernel (0 = the "
                         "library's default, -1 = the compute units the prefix plan leaves, so "
                         "the two kernels run side by side)")
    ap.add_argument("--targets", default="skewed",
                    help="comma-separated decode workloads also timed after the main one (graph "
                         "mode, no oracle), reported under `targets` ('none' skips)")
    ap.add_argument("--placement", default="scattered", choices=["scattered", "contiguous"],
                    help="page placement: the workload's random scatter, or the same lengths on "
                         "pages 0, 1, 2, ... in request order (a control for the page gather)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of this many MiB (5 times), "
                         "to calibrate HBM byte counters against a known size")
    return ap.parse_args()


# the source files a decode kernel is built from, by kernel
KERNEL_FILES = {
    "decode_mfma_kernel": ("decode_mfma.hip", "device_common.h", "plan_layout.h"),
    "decode_kernel": ("decode.hip", "device_common.h", "plan_layout.h"),
    "decode_fp8_kernel": ("decode_fp8.hip", "decode_fp8.h", "device_common.h", "plan_layout.h"),
    "decode_pv_kernel": ("decode_pv.hip", "decode_pv.h", "device_common.h", "plan_layout.h"),
    "prefix_mfma_kernel": ("prefix_mfma.hip", "prefix_mfma.h", "device_common.h",
                           "plan_layout.h"),
    "composable_kernel": ("composable.hip", "prefix_mfma.h", "decode_pv.h", "device_common.h",
                          "plan_layout.h"),
    "composable_fp8_kernel": ("composable.hip", "prefix_mfma.h", "decode_fp8.h",
                              "device_common.h", "plan_layout.h"),
}


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_FILES[kernel]:
        with open(os.path.join(ROOT, "paged_kv_decode_11_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str, kv_dtype: str):
    """HBM bytes per decode launch from committed rocprofv3 counter runs,
    if they were taken on the current kernel source."""
    tag = "" if kv_dtype == "bf16" else f"_{kv_dtype}"
    path = os.path.join(ROOT, "profiles", f"decode_{workload}{tag}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel") != kernel or rec.get("kernel_source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(batch, q_bits, cache_dev, o_dev, lse_dev, budget_s: float, fp8_scales=None):
    """Time the oracle on layer 0's requests, in order, until the budget is
    spent; also report its agreement with the GPU output on those rows.
    fp8_scales = (k_scale, v_scale) for an E4M3 cache."""
    import numpy as np
    import torch

    from oracle import attention as att

    try:
        import threadpoolctl

        blas = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas = 1
    done, tokens, elapsed, passes = [], 0, 0.0, 0
    o_gpu = o_dev.float().cpu().numpy()
    lse_gpu = lse_dev.cpu().numpy()
    err_o = err_l = 0.0
    host_pages = {}
    # requests in order; when the layer is done inside the budget, it is
    # decoded again (same inputs), so the timed sample is 10-30 s of work
    while elapsed < budget_s:
        passes += 1
        for i in range(batch.batch):
            rows = batch.kv_indices[batch.kv_indptr[i]:batch.kv_indptr[i + 1]]
            n = rows.shape[0]
            indptr = np.array([0, n], dtype=np.int32)
            idx = np.arange(n, dtype=np.int32)
            last = batch.kv_last_page_len[i:i + 1]
            if i not in host_pages:
                sel = torch.from_numpy(rows.astype(np.int64)).to(cache_dev.device)
                if fp8_scales is None:
                    host_pages[i] = cache_dev.index_select(0, sel).view(
                        torch.int16).cpu().numpy().view(np.uint16)
                else:
                    host_pages[i] = cache_dev.view(torch.uint8).index_select(0, sel).cpu().numpy()
            host = host_pages[i]
            t0 = time.perf_counter()
            if fp8_scales is None:
                o_ref, lse_ref = att.decode(q_bits[i:i + 1], host, indptr, idx, last,
                                            batch.num_kv_heads)
            else:
                o_ref, lse_ref = att.decode_fp8(q_bits[i:i + 1], host, indptr, idx, last,
                                                batch.num_kv_heads, k_scale=fp8_scales[0],
                                                v_scale=fp8_scales[1])
            elapsed += time.perf_counter() - t0
            if passes == 1:
                err_o = max(err_o, float(np.max(np.abs(o_gpu[i] - o_ref[0]))))
                err_l = max(err_l, float(np.max(np.abs(lse_gpu[i] - lse_ref[0]))))
                done.append(i)
            tokens += int(batch.kv_lens[i])
            if elapsed >= budget_s:
                break
    kv_bytes = tokens * batch.kv_bytes_per_token() // (1 if fp8_scales is None else 2)
    gbs = kv_bytes / elapsed / 1e9
    us_layer = elapsed * 1e6 * batch.total_tokens / tokens
    return {
        "value": round(gbs, 6), "unit": "GB/s", "cores": int(blas),
        "kind": "oracle",
        "sample": f"layer 0, requests 0..{done[-1]} ({len(done)} of {batch.batch}), "
                  f"{passes} pass(es), {tokens} KV tokens decoded, numpy fp64, {elapsed:.1f} s",
        "us_per_layer_step": round(us_layer, 1),
        "affinity_cpus": len(os.sched_getaffinity(0)),
    }, {"max_abs_err_o": err_o, "max_abs_err_lse": err_l, "requests_checked": len(done)}


def read_ceilings(caches, batch, reps: int = 6) -> dict:
    """Context for the decode kernel's rate: what this GPU reads with the
    library's read-only kernels (no compute) over the same caches, rotated
    like the decode runs.  `stream_gbs`: each cache (first 4 GiB at most) read
    front to back.  `page_gather_gbs`: the pages the batch uses, whole, in a
    seeded random order.  Each the best of 256 and 512 workgroups (larger
    grids read slower)."""
    import numpy as np
    import torch

    import paged_kv_decode_11_amd as pkd

    def timed(fn, nbytes):
        for i in range(2):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9

    flat = [c.view(-1).view(torch.uint8) for c in caches]
    span = min(flat[0].numel(), 4 << 30) // 16 * 16
    sink = torch.empty(512 * 512, dtype=torch.int32, device=caches[0].device)
    stream = max(timed(lambda i: pkd.read_stream(flat[i % len(flat)][:span], grid=g, sink=sink),
                       span) for g in (256, 512))
    page_bytes = flat[0].numel() // batch.num_pages
    pages = np.unique(batch.kv_indices)
    ids = np.random.Generator(np.random.PCG64(12345)).permutation(pages).astype(np.int32)
    ids_dev = torch.from_numpy(ids).to(caches[0].device)
    gather = max(timed(lambda i: pkd.read_pages(flat[i % len(flat)], batch.num_pages, page_bytes,
                                                ids_dev, grid=g, sink=sink), ids.size * page_bytes)
                 for g in (256, 512))
    return {"stream_gbs": round(stream, 1), "page_gather_gbs": round(gather, 1),
            "page_bytes": int(page_bytes), "pages": int(ids.size),
            "kernels": "read_stream_kernel, read_pages_kernel (read_ceiling.hip)"}


def calibrate_copy(mib: int) -> None:
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give
    the scale between counter units and bytes moved."""
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 5
    print(json.dumps({"calibrate_copy_bytes_read": n, "calibrate_copy_bytes_written": n,
                      "copies": 5, "gbs_read_plus_write": round(2 * n / dt / 1e9, 1)}), flush=True)


def time_graph(fn, steps: int, warmup: int, before=None) -> float:
    """ms per replay of a graph holding fn(); `before` runs on the host ahead
    of each replay (a plan)."""
    import torch

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    for _ in range(warmup):
        if before:
            before()
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        if before:
            before()
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del g
    return ms


def plan_chunk_pages(r) -> int:
    """Chunk size (pages) of the handle's current plan, read back from its
    int workspace header."""
    import torch

    import paged_kv_decode_11_amd as pkd

    hdr = r.int_workspace[4 * pkd._lib.HEADER_BASE: 4 * (pkd._lib.HEADER_BASE + 32)].cpu()
    return int(hdr.view(torch.int32)[pkd._lib.H["CHUNK_PAGES"]])


def bench_shared_prefix(args):
    """32 requests over one 8192-token prefix plus their own suffixes, one
    layer, caches rotated over R copies.  Composable: the prefix state of all
    requests from one shared-prefix plan (the prefix read once per KV head),
    the suffix states from a decode plan, merged row by row.  Single format:
    one decode plan over each request's prefix + suffix pages.  `value` is
    the KV bytes the composable step streams (prefix once, suffixes) over its
    time.  With --kv-dtype e4m3 every format runs over E4M3 codes with
    per-tensor scales."""
    import numpy as np
    import torch

    import paged_kv_decode_11_amd as pkd
    import workloads

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    spec, rng, b = workloads.workload(args.workload)
    main, prefix, suffix = b["main"], b["prefix"], b["suffix"]
    fp8 = args.kv_dtype == "e4m3"
    kv_tok = main.kv_bytes_per_token() // (2 if fp8 else 1)
    kv = dict(kv_data_type=torch.float8_e4m3fn) if fp8 else {}
    scales = dict(k_scale=1.0 / 64, v_scale=1.0 / 64) if fp8 else {}
    n_prefix_pages = int(prefix.kv_indptr[1])
    prefix_tokens = int(prefix.kv_lens[0])
    unique_bytes = (prefix_tokens + suffix.total_tokens) * kv_tok
    single_bytes = main.total_tokens * kv_tok
    R = 8  # cache copies: R x unique bytes well above the last-level cache
    log(f"shared_prefix: B={main.batch} prefix={prefix_tokens} suffix tokens={suffix.total_tokens} "
        f"unique {unique_bytes / 1e6:.1f} MB, single-format {single_bytes / 1e6:.1f} MB, R={R}")
    base = (workloads.device_cache_e4m3(main, spec.seed * 1000, dev) if fp8 else
            workloads.device_cache(main, spec.seed * 1000, dev, used_only=True))
    caches = [base] + [base.clone() for _ in range(R - 1)]
    qs = [workloads.device_query(main, spec.seed * 7919 + j, dev) for j in range(R)]
    H = main.num_qo_heads

    # single format
    r1 = pkd.DecodePlanRun(max_batch=main.batch, max_nnz=main.nnz, max_qo_heads=H, device=0)
    idx_main = torch.from_numpy(main.kv_indices.astype(np.int32)).to(dev)
    outs1 = [torch.empty_like(qs[0]) for _ in range(R)]
    lses1 = [torch.empty((main.batch, H), dtype=torch.float32, device=dev) for _ in range(R)]

    def plan1():
        r1.plan(main.kv_indptr, idx_main, main.kv_last_page_len, H, main.num_kv_heads, 128, 16,
                **kv)

    def run1():
        for j in range(R):
            r1.run(qs[j], caches[j], out=outs1[j], lse=lses1[j], **scales)

    # composable: one shared-prefix plan (all 32 requests over the prefix
    # pages) and one decode plan (each request's own suffix), both writing
    # every chunk's state as a partial; pkd_run_composable runs the prefix
    # kernel, the suffix decode and one merge
    # The compute units split between the two plans so that both attention
    # kernels run in one launch side by side: the prefix plan gets one slot
    # per item of 512 prefix tokens (row blocks of 128 query rows x KV heads
    # x chunks), at least half of the units and at most three quarters; the
    # suffix plan the rest.  (Measured: 128 + 128 best for 16 and 32
    # requests, 192 + 64 for 64 requests, over a 256-CU part.)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    g = H // main.num_kv_heads
    row_blocks = -(-main.batch * g // 128)
    pre_items = row_blocks * main.num_kv_heads * -(-prefix_tokens // 512)
    pre_slots = min(max(pre_items, cus // 2), cus - cus // 4)
    rp = pkd.SharedPlanRun(4, main.batch, n_prefix_pages, H, main.num_kv_heads,
                           num_slots=pre_slots if args.prefix_slots < 0 else args.prefix_slots,
                           device=0)
    rs = pkd.DecodePlanRun(max_batch=suffix.batch, max_nnz=suffix.nnz, max_qo_heads=H,
                           num_slots=(cus - pre_slots if args.suffix_slots < 0
                                      else args.suffix_slots),
                           device=0)
    qo = np.array([0, main.batch], np.int32)
    kv_indptr = np.array([0, n_prefix_pages], np.int32)
    idx_pre = torch.from_numpy(prefix.kv_indices[:n_prefix_pages].astype(np.int32)).to(dev)
    idx_suf = torch.from_numpy(suffix.kv_indices.astype(np.int32)).to(dev)
    outs2 = [torch.empty_like(qs[0]) for _ in range(R)]
    lses2 = [torch.empty((main.batch, H), dtype=torch.float32, device=dev) for _ in range(R)]

    pre_opts = {"min_chunk_tokens": args.prefix_chunk_tokens} if args.prefix_chunk_tokens else {}

    def plan2():
        rp.plan(qo, kv_indptr, idx_pre, prefix.kv_last_page_len[:1], H, main.num_kv_heads, 128, 16,
                all_partials=True, **pre_opts, **kv)
        # alpha = 32: each chunk weighs 32 tokens on top of its own in the
        # slot assignment, so that no slot gets three of the short suffix
        # chunks (the launch's last workgroup) while most get one
        rs.plan(suffix.kv_indptr, idx_suf, suffix.kv_last_page_len, H, main.num_kv_heads, 128, 16,
                all_partials=True, alpha=SUFFIX_ALPHA, **kv)

    def run2():
        for j in range(R):
            pkd.run_composable(rp, rs, qs[j], caches[j], out=outs2[j], lse=lses2[j], **scales)

    # the same states through separate calls (prefix run with its merge,
    # suffix run with its merge, merge_state): five launches per layer
    rp5 = pkd.SharedPlanRun(4, main.batch, n_prefix_pages, H, main.num_kv_heads, device=0)
    rs5 = pkd.DecodePlanRun(max_batch=suffix.batch, max_nnz=suffix.nnz, max_qo_heads=H, device=0)
    op = [torch.empty_like(qs[0]) for _ in range(R)]
    lp = [torch.empty((main.batch, H), dtype=torch.float32, device=dev) for _ in range(R)]
    os_ = [torch.empty_like(qs[0]) for _ in range(R)]
    ls = [torch.empty((main.batch, H), dtype=torch.float32, device=dev) for _ in range(R)]
    outs5 = [torch.empty_like(qs[0]) for _ in range(R)]
    lses5 = [torch.empty((main.batch, H), dtype=torch.float32, device=dev) for _ in range(R)]

    def plan5():
        rp5.plan(qo, kv_indptr, idx_pre, prefix.kv_last_page_len[:1], H, main.num_kv_heads, 128,
                 16, **pre_opts, **kv)
        rs5.plan(suffix.kv_indptr, idx_suf, suffix.kv_last_page_len, H, main.num_kv_heads, 128, 16,
                 alpha=SUFFIX_ALPHA, **kv)

    def run5():
        for j in range(R):
            rp5.run(qs[j], caches[j], out=op[j], lse=lp[j], **scales)
            rs5.run(qs[j], caches[j], out=os_[j], lse=ls[j], **scales)
            pkd.merge_state(op[j], lp[j], os_[j], ls[j], out=outs5[j], lse_out=lses5[j])

    plan1()
    plan2()
    plan5()
    run1()
    run2()
    run5()
    torch.cuda.synchronize()
    # the formats agree (each is checked against the oracle by the tests)
    diff = max(float((outs1[j].float() - outs2[j].float()).abs().max()) for j in range(R))
    dlse = max(float((lses1[j] - lses2[j]).abs().max()) for j in range(R))
    diff5 = max(float((outs5[j].float() - outs2[j].float()).abs().max()) for j in range(R))
    log(f"formats agree: max |o1 - o2| {diff:.3g}, max |lse1 - lse2| {dlse:.3g}, "
        f"five-launch vs one-call {diff5:.3g}")

    # per-launch times of the composable layer (eager, HIP events recorded by
    # the library): prefix handle = prefix kernel; suffix handle = suffix
    # decode, then the merge
    rp.profile_enable(True)
    rs.profile_enable(True)
    for _ in range(args.steps):
        plan2()
        run2()
    torch.cuda.synchronize()
    attn_ms, merge_ms, runs = rp.profile_read()
    rs.profile_read()
    rp.profile_enable(False)
    rs.profile_enable(False)
    # pkd_run_composable runs both attention kernels in one launch when the
    # two handles' slots fit the compute units side by side and the suffix
    # plan runs the matrix-core P.V kernel
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    one_launch = rp.num_slots + rs.num_slots <= cus and (fp8 or rs.planned_variant == "mfma_pv")
    attn_us = attn_ms * 1e3 / runs
    prefix_merge_us = merge_ms * 1e3 / runs
    breakdown = {"attention_kernels": round(attn_us, 2), "merge": round(prefix_merge_us, 2),
                 "one_launch": one_launch, "prefix_slots": rp.num_slots,
                 "suffix_slots": rs.num_slots}
    log(f"composable launches (us): {breakdown}")

    ms1 = time_graph(run1, args.steps, args.warmup, plan1)
    ms2 = time_graph(run2, args.steps, args.warmup, plan2)
    ms5 = time_graph(run5, args.steps, args.warmup, plan5)
    us1, us2, us5 = ms1 * 1e3 / R, ms2 * 1e3 / R, ms5 * 1e3 / R
    value = unique_bytes * R / (ms2 / 1e3) / 1e9
    # the attention launch(es) read the prefix once per KV head and every
    # suffix once: the unique K/V bytes
    achieved = unique_bytes / (attn_us / 1e6) / 1e9
    roof_kernel = (("composable_fp8_kernel" if fp8 else "composable_kernel") if one_launch
                   else "prefix_mfma_kernel + decode kernel")
    log(f"single format {us1:.1f} us/layer, composable {us2:.1f} us/layer (five launches "
        f"{us5:.1f}; attention {attn_us:.1f} us, merge {prefix_merge_us:.1f} us)")
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms2, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3 kv (bf16/f16 mfma, f32 accumulate)" if fp8 else "bf16",
        "data": ("synthetic (seeded N(0,1) bf16 q, uniformly drawn E4M3 K/V codes with scales "
                 "1/64, seeded lengths and page placement)" if fp8 else
                 "synthetic (seeded N(0,1) bf16 q/K/V, seeded lengths and page placement)"),
        "config": {"workload": args.workload, "batch": main.batch, "layers": R,
                   "prefix_tokens": prefix_tokens, "suffix_tokens": suffix.total_tokens,
                   "num_qo_heads": H, "num_kv_heads": main.num_kv_heads, "head_dim": 128,
                   "page_size": 16, "slots": rp.num_slots, "kv_dtype": args.kv_dtype,
                   "parallelism": "single GPU"},
        "us_per_layer_step": round(us2, 2),
        "frac_of_hbm_peak": round(value / PEAK_HBM_GBS, 4),
        "composable_us_per_layer": round(us2, 2),
        "composable_five_launch_us_per_layer": round(us5, 2),
        "single_format_us_per_layer": round(us1, 2),
        "speedup_over_single_format": round(us1 / us2, 2),
        "unique_kv_bytes_per_layer": unique_bytes,
        "single_format_kv_bytes_per_layer": single_bytes,
        "single_format_kv_gbs": round(single_bytes * R / (ms1 / 1e3) / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": (measured_traffic(args.workload, roof_kernel, args.kv_dtype)
                                 if one_launch else None),
                     "kernel": roof_kernel, "avg_launch_us": round(attn_us, 2),
                     "algorithmic_bytes_per_launch": unique_bytes,
                     "merge_avg_launch_us": round(prefix_merge_us, 2)},
        "composable_launch_us": breakdown,
        "formats_max_abs_diff_five_launch": diff5,
        "prefix_chunk_pages": plan_chunk_pages(rp),
        "formats_max_abs_diff": {"o": diff, "lse": dlse},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bench_append(args):
    """The append kernel on the Llama-3-8B-like batch's page table: every
    token of the batch written at once (a prefill-sized append, about 1 GB
    of K/V), and one new token per request (a decode step's append).  `value`
    is the bytes the prefill-sized append moves (new rows read, cache slots
    written) over its time."""
    import numpy as np
    import torch

    import paged_kv_decode_11_amd as pkd
    import workloads

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    spec, rng, b = workloads.workload("llama8b_step")
    batch = b["main"]
    Hkv, P = batch.num_kv_heads, batch.page_size
    row = Hkv * 128 * 2
    cache = torch.zeros(batch.cache_shape(), dtype=torch.bfloat16, device=dev)
    indptr = torch.from_numpy(batch.kv_indptr.astype(np.int32)).to(dev)
    indices = torch.from_numpy(batch.kv_indices.astype(np.int32)).to(dev)
    last = torch.from_numpy(batch.kv_last_page_len.astype(np.int32)).to(dev)
    lens = batch.kv_lens.astype(np.int64)

    def setup(add):
        a_ind = torch.from_numpy(np.concatenate([[0], np.cumsum(add)]).astype(np.int32)).to(dev)
        bi, pos = pkd.append_positions(a_ind, indptr, last, P)
        n = int(np.sum(add))
        k = workloads.device_query(batch, 11, dev).new_empty((n, Hkv, 128)).normal_()
        v = torch.empty_like(k).normal_()
        return bi, pos, k, v, n

    def timed(bi, pos, k, v, steps):
        run = lambda: pkd.append_paged_kv_cache(k, v, bi, pos, cache, indices, indptr)
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            run()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    bi, pos, k, v, n_full = setup(lens)
    ms_full = timed(bi, pos, k, v, args.steps)
    moved = 2 * (2 * n_full * row)  # K and V rows, read once and written once
    value = moved / (ms_full / 1e3) / 1e9
    del k, v
    bi1, pos1, k1, v1, n1 = setup(np.ones_like(lens))
    ms_one = timed(bi1, pos1, k1, v1, max(args.steps, 20))
    log(f"append: {n_full} tokens in {ms_full * 1e3:.1f} us ({value:.0f} GB/s); "
        f"one token per request ({n1}): {ms_one * 1e3:.2f} us")
    line = {
        "metric": "paged KV append: achieved GB/s (new rows read + cache slots written)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_full, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 rows, the Llama-3-8B-like batch's page table)",
        "config": {"workload": "append", "tokens": n_full, "batch": batch.batch,
                   "num_kv_heads": Hkv, "head_dim": 128, "page_size": P,
                   "parallelism": "single GPU"},
        "decode_step_append_us": round(ms_one * 1e3, 2),
        "roofline": {"bound": "hbm", "achieved": round(value, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(value / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "append_kv_kernel", "avg_launch_us": round(ms_full * 1e3, 2),
                     "algorithmic_bytes_per_launch": moved},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


# the fraction of the HBM peak each of these workloads is held to
TARGET_FRAC = {"llama8b_step": 0.70, "skewed": 0.60}


def bench_decode(args, workload_name: str, cpu_seconds: float, ceilings: bool = True,
                 placement: str = "scattered") -> dict:
    """One decode workload: plan per step, runs per layer (graph-replayed by
    default); returns its JSON line as a dict.  Every tensor it allocates is
    freed on return."""
    import numpy as np
    import torch

    import paged_kv_decode_11_amd as pkd
    import workloads

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    spec, rng, b = workloads.workload(workload_name)
    batch = b["main"]
    if placement == "contiguous":
        # the same lengths on pages 0, 1, 2, ... in request order
        batch = workloads.make_batch(batch.kv_lens, batch.page_size, batch.num_pages,
                                     batch.num_qo_heads, batch.num_kv_heads, batch.head_dim,
                                     None, scatter=False)
    fp8 = args.kv_dtype == "e4m3"
    if fp8 and args.variant == "dot2":
        raise SystemExit("an e4m3 cache runs on its own matrix-core kernel")
    kv_tok = batch.kv_bytes_per_token() // (2 if fp8 else 1)
    kernel = None  # set from the library's plan below
    layer_bytes = batch.total_tokens * kv_tok
    if spec.num_layers > 1:
        n_layers, distinct = spec.num_layers, 2
    else:
        n_layers = min(16, max(1, math.ceil(ROTATE_BYTES / layer_bytes)))
        if workload_name == "wide_gqa":
            n_layers = 1  # its ~3.4 GB per layer already dwarfs the last-level cache
        distinct = 1
    log(f"workload {workload_name}: B={batch.batch} T={batch.total_tokens} nnz={batch.nnz} "
        f"pool={batch.num_pages} runs/step={n_layers}")

    # caches: `distinct` freshly drawn, the rest device copies (distinct addresses)
    used_only = workload_name == "wide_gqa"
    if fp8:
        fresh = [workloads.device_cache_e4m3(batch, spec.seed * 1000 + j, dev)
                 for j in range(distinct)]
    else:
        fresh = [workloads.device_cache(batch, spec.seed * 1000 + j, dev, used_only=used_only)
                 for j in range(distinct)]
    caches = []
    for layer in range(n_layers):
        if layer == 0:
            caches.append(fresh[0])
        elif distinct == 2 and layer == n_layers - 1:
            caches.append(fresh[1])
        else:
            caches.append(fresh[0 if (distinct == 1 or layer < n_layers // 2) else 1].clone())
    log("caches ready", torch.cuda.memory_allocated() / 2**30, "GiB")
    q_bits = workloads.host_query(batch, rng)
    qs = [torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).to(dev)]
    for layer in range(1, n_layers):
        qs.append(workloads.device_query(batch, spec.seed * 7919 + layer, dev))
    outs = [torch.empty_like(qs[0]) for _ in range(n_layers)]
    lses = [torch.empty((batch.batch, batch.num_qo_heads), dtype=torch.float32, device=dev)
            for _ in range(n_layers)]

    r = pkd.DecodePlanRun(max_batch=batch.batch, max_nnz=batch.nnz,
                          max_qo_heads=batch.num_qo_heads, num_slots=args.slots, device=0)
    idx = torch.from_numpy(batch.kv_indices.astype(np.int32)).to(dev)

    kv_type = torch.float8_e4m3fn if fp8 else torch.bfloat16
    # per-tensor scales that bring the uniformly drawn codes (up to 448) to
    # unit-range keys and values
    scales = dict(k_scale=1.0 / 64, v_scale=1.0 / 64) if fp8 else {}

    def plan():
        r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, batch.num_qo_heads,
               batch.num_kv_heads, batch.head_dim, batch.page_size, variant=args.variant,
               kv_data_type=kv_type)

    def run(layer):
        r.run(qs[layer], caches[layer], out=outs[layer], lse=lses[layer], **scales)

    def step():
        plan()
        for layer in range(n_layers):
            run(layer)

    plan()
    kernel = ("decode_fp8_kernel" if fp8 else
              {"mfma": "decode_mfma_kernel", "mfma_pv": "decode_pv_kernel",
               "dot2": "decode_kernel"}[r.planned_variant])
    log(f"decode kernel: {kernel}")
    # plan host cost, on its own
    torch.cuda.synchronize()
    plan_us = []
    for _ in range(20):
        t0 = time.perf_counter()
        plan()
        plan_us.append((time.perf_counter() - t0) * 1e6)
        torch.cuda.synchronize()
    plan_us.sort()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")

    r.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    decode_ms, merge_ms, runs = r.profile_read()
    r.profile_enable(False)
    eager_ms = (t1 - t0) * 1e3 / args.steps
    step_bytes = layer_bytes * n_layers
    eager = {"ms_per_step": round(eager_ms, 4),
             "us_per_layer_step": round(eager_ms * 1e3 / n_layers, 2),
             "kv_gbs": round(step_bytes / (eager_ms / 1e3) / 1e9, 1)}
    decode_us = decode_ms * 1e3 / runs
    merge_us = merge_ms * 1e3 / runs
    achieved = layer_bytes / (decode_us / 1e6) / 1e9
    log(f"eager: {eager_ms:.3f} ms/step, {eager['kv_gbs']} GB/s; decode {decode_us:.1f} us, "
        f"merge {merge_us:.1f} us per run")

    graph = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for layer in range(n_layers):
                run(layer)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            plan()
            g.replay()
        torch.cuda.synchronize()
        tg0 = time.perf_counter()
        for _ in range(args.steps):
            plan()
            g.replay()
        torch.cuda.synchronize()
        tg1 = time.perf_counter()
        g_ms = (tg1 - tg0) * 1e3 / args.steps
        # per-step spread: events around each plan + replay, steps back to
        # back (each sample runs from the previous step's end to this one's)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for e0, e1 in evs:
            e0.record()
            plan()
            g.replay()
            e1.record()
        torch.cuda.synchronize()
        per = sorted(e0.elapsed_time(e1) * 1e3 / n_layers for e0, e1 in evs)
        pct = lambda f: round(per[min(len(per) - 1, int(f * len(per)))], 2)
        graph = {"ms_per_step": round(g_ms, 4), "us_per_layer_step": round(g_ms * 1e3 / n_layers, 2),
                 "kv_gbs": round(step_bytes / (g_ms / 1e3) / 1e9, 1),
                 "us_per_layer_step_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)]}
        log(f"graph: {g_ms:.3f} ms/step, {graph['kv_gbs']} GB/s, per-step spread "
            f"{graph['us_per_layer_step_p10_p50_p90']} us/layer")
        del g

    # the headline is the graph-replayed step when graphs are on (the serving
    # mode the plan/run split exists for), else the eager step
    ms_per_step = graph["ms_per_step"] if graph else eager_ms
    value = step_bytes / (ms_per_step / 1e3) / 1e9
    # one more eager step so outputs are fresh for the parity spot check
    step()
    torch.cuda.synchronize()
    cpu = None
    spot = None
    if cpu_seconds > 0:
        log("cpu baseline (oracle) ...")
        cpu, spot = cpu_baseline(batch, q_bits, caches[0], outs[0], lses[0], cpu_seconds,
                                 (scales["k_scale"], scales["v_scale"]) if fp8 else None)

    ceiling = None
    if ceilings:
        ceiling = read_ceilings(caches, batch)
        ceiling["decode_kernel_frac_of_page_gather"] = round(
            achieved / ceiling["page_gather_gbs"], 4)
        log(f"read ceilings: {ceiling}")

    traffic = measured_traffic(workload_name, kernel, args.kv_dtype) \
        if placement == "scattered" else None
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 kv (bf16/f16 mfma, f32 accumulate)" if fp8 else "bf16",
        "data": ("synthetic (seeded N(0,1) bf16 q, uniformly drawn E4M3 K/V codes with "
                 "scales 1/64, seeded lengths and page placement)" if fp8 else
                 "synthetic (seeded N(0,1) bf16 q/K/V, seeded lengths and page placement)"),
        "config": {
            "workload": workload_name, "batch": batch.batch, "layers": n_layers,
            "num_qo_heads": batch.num_qo_heads, "num_kv_heads": batch.num_kv_heads,
            "head_dim": batch.head_dim, "page_size": batch.page_size,
            "kv_tokens_per_layer": batch.total_tokens, "pages_per_layer": batch.nnz,
            "pool_pages": batch.num_pages, "slots": r.num_slots, "kv_dtype": args.kv_dtype,
            "decode_kernel": kernel, "page_placement": placement,
            "parallelism": "single GPU",
        },
        "us_per_layer_step": round(ms_per_step * 1e3 / n_layers, 2),
        "frac_of_hbm_peak": round(value / PEAK_HBM_GBS, 4),
        "plan_host_us_median": round(plan_us[len(plan_us) // 2], 1),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "kernel": kernel,
            "avg_launch_us": round(decode_us, 2),
            "algorithmic_bytes_per_launch": layer_bytes,
            "merge_avg_launch_us": round(merge_us, 2),
        },
        "mode": "graph" if graph else "eager",
        "graph": graph,
        "eager": eager,
        "read_ceiling": ceiling,
        "cpu_baseline": cpu,
        "parity_spot_check": spot,
    }
    return line




def target_summary(line: dict) -> dict:
    """The fields of a secondary workload's line that the headline carries."""
    w = line["config"]["workload"]
    frac = line["frac_of_hbm_peak"]
    out = {"us_per_layer_step": line["us_per_layer_step"], "kv_gbs": line["value"],
           "steps": line["steps"], "warmup": line["warmup"],
           "frac_of_hbm_peak": frac, "target_frac": TARGET_FRAC.get(w),
           "meets_target": None if w not in TARGET_FRAC else bool(frac >= TARGET_FRAC[w]),
           "layers": line["config"]["layers"], "mode": line["mode"],
           "decode_kernel": line["config"]["decode_kernel"],
           "kv_tokens_per_layer": line["config"]["kv_tokens_per_layer"],
           "plan_host_us_median": line["plan_host_us_median"], "roofline": line["roofline"]}
    if line.get("graph"):
        out["us_per_layer_step_p10_p50_p90"] = line["graph"]["us_per_layer_step_p10_p50_p90"]
    return out


def main():
    args = parse()
    # No cyclic garbage collection while timing (as timeit does): a pass over
    # torch's and numpy's objects in the middle of a timed loop stalls the host
    # for milliseconds, and with it the GPU of a plan-per-step loop.  Objects
    # are still freed by reference counting; workloads collect in between.
    gc.disable()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; multi-GPU sharding is a design "
                                   "note only (see the design document)", "n_gpus": args.gpus}))
        sys.exit(2)
    if args.workload.startswith("shared_prefix"):
        bench_shared_prefix(args)
        return
    if args.workload == "append":
        bench_append(args)
        return
    w = args.workload
    extra = [t for t in args.targets.split(",") if t and t != "none" and t != w]
    # The secondary workloads run first, and their memory goes back to the
    # driver (a few GB, cleared in well under the pause below) before the
    # headline allocates: a workload timed while another one's freed caches
    # sat in torch's pool ran its graph step 2-4 us per layer slower, and
    # handing the headline's 64 GiB back to the driver instead would let its
    # clearing of that memory share HBM with the next timing.
    # A single-layer step is short (the skewed batch: about 0.37 ms for its
    # four rotated layers), so time at least 250 steps after at least 10
    # warm-up steps: about 0.1 s, past the start-up transient of the loop.
    sub_args = argparse.Namespace(**vars(args))
    sub_args.steps, sub_args.warmup = max(args.steps, 250), max(args.warmup, 10)
    subs = {}
    for t in extra:
        log(f"secondary workload {t}")
        subs[t] = target_summary(bench_decode(sub_args, t, 0.0, ceilings=False,
                                              placement=args.placement))
        log(f"{t}: {subs[t]['us_per_layer_step']} us/layer-step, "
            f"{subs[t]['frac_of_hbm_peak']} of HBM peak")
        gc.collect()
    if extra:
        import torch

        torch.cuda.empty_cache()
        time.sleep(3.0)
    line = bench_decode(args, w, args.cpu_seconds, placement=args.placement)
    if w in TARGET_FRAC:
        line["target_frac"] = TARGET_FRAC[w]
        line["meets_target"] = bool(line["frac_of_hbm_peak"] >= TARGET_FRAC[w])
    if extra:
        line["targets"] = {w: target_summary(line), **subs}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
