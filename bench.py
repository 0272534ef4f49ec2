#!/usr/bin/env python3
"""Paged GQA decode benchmark on one MI355X.

A step is one pass of the whole hot path over one batch: pkd_plan (host
scheduler + upload) once, then pkd_run once per layer (decode kernel + merge
kernel).  Default workload: the Llama-3-8B-like decode step (32 layers,
Hq 32 / Hkv 8 / D 128, bf16, page_size 16, batch 64 with KV lengths uniform
in [3000, 5000], pages scattered through a 32,768-page pool per layer).

Prints one JSON line.  `value` is the achieved KV-stream rate in GB/s
(KV bytes the step must read, 4096 B per token per layer, over the measured
step time).  By default a step is the plan call followed by one replay of a
HIP graph that holds the step's runs; --no-graph launches the runs one by
one, and the eager timing is reported beside the graph one in any case.
`roofline` gives the decode kernel's own rate from HIP events
around each launch; `cpu_baseline` times the fp64 oracle on a sample of
layer 0's requests.  Inputs are synthetic and seeded.
"""

from __future__ import annotations

import argparse
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
ROTATE_BYTES = 2 << 30  # single-layer workloads rotate caches to >= 2 GiB
METRIC = "paged GQA decode: achieved KV GB/s (% of HBM peak) and µs/layer-step"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_step",
                    choices=["llama8b_step", "skewed", "wide_gqa", "token_sparse", "tiny"])
    ap.add_argument("--slots", type=int, default=0, help="persistent workgroups (0 = default)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle time budget for cpu_baseline (0 disables)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--variant", default="auto", choices=["auto", "dot2", "mfma"],
                    help="decode kernel (auto = the matrix-core kernel)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of this many MiB (5 times), "
                         "to calibrate HBM byte counters against a known size")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("decode.hip", "decode_mfma.hip", "merge.hip", "kernels.h", "device_common.h"):
        with open(os.path.join(ROOT, "paged_kv_decode_11_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, launches_bytes: float):
    """HBM bytes per decode launch from committed rocprofv3 counter runs,
    if they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(batch, q_bits, cache_dev, o_dev, lse_dev, budget_s: float):
    """Time the oracle on layer 0's requests, in order, until the budget is
    spent; also report its agreement with the GPU output on those rows."""
    import numpy as np
    import torch

    from oracle import attention as att

    try:
        import threadpoolctl

        blas = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas = 1
    done, tokens, elapsed = [], 0, 0.0
    o_gpu = o_dev.float().cpu().numpy()
    lse_gpu = lse_dev.cpu().numpy()
    err_o = err_l = 0.0
    for i in range(batch.batch):
        rows = batch.kv_indices[batch.kv_indptr[i]:batch.kv_indptr[i + 1]]
        sel = torch.from_numpy(rows.astype(np.int64)).to(cache_dev.device)
        host = cache_dev.index_select(0, sel).view(torch.int16).cpu().numpy().view(np.uint16)
        n = rows.shape[0]
        indptr = np.array([0, n], dtype=np.int32)
        idx = np.arange(n, dtype=np.int32)
        last = batch.kv_last_page_len[i:i + 1]
        t0 = time.perf_counter()
        o_ref, lse_ref = att.decode(q_bits[i:i + 1], host, indptr, idx, last, batch.num_kv_heads)
        elapsed += time.perf_counter() - t0
        err_o = max(err_o, float(np.max(np.abs(o_gpu[i] - o_ref[0]))))
        err_l = max(err_l, float(np.max(np.abs(lse_gpu[i] - lse_ref[0]))))
        done.append(i)
        tokens += int(batch.kv_lens[i])
        if elapsed >= budget_s:
            break
    kv_bytes = tokens * batch.kv_bytes_per_token()
    gbs = kv_bytes / elapsed / 1e9
    us_layer = elapsed * 1e6 * batch.total_tokens / tokens
    return {
        "value": round(gbs, 6), "unit": "GB/s", "cores": int(blas),
        "kind": "oracle",
        "sample": f"layer 0, requests 0..{done[-1]} ({len(done)} of {batch.batch}, {tokens} KV tokens), "
                  f"numpy fp64, {elapsed:.1f} s",
        "us_per_layer_step": round(us_layer, 1),
        "affinity_cpus": len(os.sched_getaffinity(0)),
    }, {"max_abs_err_o": err_o, "max_abs_err_lse": err_l, "requests_checked": len(done)}


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


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; multi-GPU sharding is a design "
                                   "note only (see the design document)", "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    import paged_kv_decode_11_amd as pkd
    import workloads

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    spec, rng, b = workloads.workload(args.workload)
    batch = b["main"]
    kv_tok = batch.kv_bytes_per_token()
    layer_bytes = batch.total_tokens * kv_tok
    if spec.num_layers > 1:
        n_layers, distinct = spec.num_layers, 2
    else:
        n_layers = min(16, max(1, math.ceil(ROTATE_BYTES / layer_bytes)))
        if args.workload == "wide_gqa":
            n_layers = 1  # its ~3.4 GB per layer already dwarfs the last-level cache
        distinct = 1
    log(f"workload {args.workload}: B={batch.batch} T={batch.total_tokens} nnz={batch.nnz} "
        f"pool={batch.num_pages} runs/step={n_layers}")

    # caches: `distinct` freshly drawn, the rest device copies (distinct addresses)
    used_only = args.workload == "wide_gqa"
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

    def plan():
        r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, batch.num_qo_heads,
               batch.num_kv_heads, batch.head_dim, batch.page_size, variant=args.variant)

    def step():
        plan()
        for layer in range(n_layers):
            r.run(qs[layer], caches[layer], out=outs[layer], lse=lses[layer])

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
                r.run(qs[layer], caches[layer], out=outs[layer], lse=lses[layer])
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
        graph = {"ms_per_step": round(g_ms, 4), "us_per_layer_step": round(g_ms * 1e3 / n_layers, 2),
                 "kv_gbs": round(step_bytes / (g_ms / 1e3) / 1e9, 1)}
        log(f"graph: {g_ms:.3f} ms/step, {graph['kv_gbs']} GB/s")
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
    if args.cpu_seconds > 0:
        log("cpu baseline (oracle) ...")
        cpu, spot = cpu_baseline(batch, q_bits, caches[0], outs[0], lses[0], args.cpu_seconds)

    traffic = measured_traffic(args.workload, layer_bytes)
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
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/K/V, seeded lengths and page placement)",
        "config": {
            "workload": args.workload, "batch": batch.batch, "layers": n_layers,
            "num_qo_heads": batch.num_qo_heads, "num_kv_heads": batch.num_kv_heads,
            "head_dim": batch.head_dim, "page_size": batch.page_size,
            "kv_tokens_per_layer": batch.total_tokens, "pages_per_layer": batch.nnz,
            "pool_pages": batch.num_pages, "slots": r.num_slots,
            "decode_kernel": "mfma" if args.variant in ("auto", "mfma") else "dot2",
            "parallelism": "single GPU",
        },
        "us_per_layer_step": round(ms_per_step * 1e3 / n_layers, 2),
        "frac_of_hbm_peak": round(value / PEAK_HBM_GBS, 4),
        "plan_host_us_median": round(plan_us[len(plan_us) // 2], 1),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "kernel": "decode_mfma_kernel" if args.variant in ("auto", "mfma") else "decode_kernel",
            "avg_launch_us": round(decode_us, 2),
            "algorithmic_bytes_per_launch": layer_bytes,
            "merge_avg_launch_us": round(merge_us, 2),
        },
        "mode": "graph" if graph else "eager",
        "graph": graph,
        "eager": eager,
        "cpu_baseline": cpu,
        "parity_spot_check": spot,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
