"""Host-side parts of bench.py that need no GPU: the one-GPU refusal and the
bookkeeping that ties committed traffic records to kernel sources."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_kernel_source_lists_name_existing_files():
    import bench

    csrc = os.path.join(ROOT, "paged_kv_decode_11_amd", "csrc")
    for kernel, files in bench.KERNEL_FILES.items():
        for f in files:
            assert os.path.exists(os.path.join(csrc, f)), (kernel, f)
        assert len(bench.kernel_source_hash(kernel)) == 16


def test_traffic_records_are_well_formed():
    """Every committed record names a kernel bench.py knows and carries the
    fields the roofline line reads (whether its hash is current is checked
    by bench.py itself, which reports traffic as null otherwise)."""
    import glob

    import bench

    recs = glob.glob(os.path.join(ROOT, "profiles", "decode_*_traffic.json"))
    assert recs
    for path in recs:
        with open(path) as f:
            rec = json.load(f)
        assert rec["kernel"] in bench.KERNEL_FILES, path
        for key in ("bytes_per_launch", "algorithmic_bytes_per_launch", "kernel_source_hash",
                    "fetch_scale", "write_scale", "dispatches"):
            assert key in rec, (path, key)
        assert 0.5 < rec["traffic_over_algorithmic"] < 2.0, path
