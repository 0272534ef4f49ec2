"""The C-ABI library without a GPU: it loads, exports every function
include/pkd.h declares, sizes workspaces, validates page tables, and its
host scheduler (pkd_plan_host) reproduces oracle.plan_ref bit for bit."""

import ctypes
import re

import numpy as np
import pytest

import workloads
from oracle import page_table as pt
from oracle import plan_ref
import paged_kv_decode_11_amd as pkd
from paged_kv_decode_11_amd import _lib


def test_library_exports_every_declared_function():
    lib = pkd.load()
    declared = pkd.header_functions()
    assert "pkd_plan" in declared and "pkd_run" in declared and "pkd_merge_states" in declared
    for name in declared:
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding lacks {name}"


def test_header_constants_match_binding():
    text = open(_lib.HEADER_PATH).read()
    assert "#define PKD_HEADER_BASE 32" in text
    body = text[text.index("PKD_H_MAGIC = 0"):text.index("PKD_H_COUNT")]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = [t.split("=")[0].strip() for t in body.split(",")]
    names = [n[len("PKD_H_"):] for n in names if n.startswith("PKD_H_")]
    assert names == _lib.H_FIELDS


def test_workspace_sizes():
    L = pkd.load()
    S = 512
    ib = L.pkd_int_workspace_bytes(64, 16000, S)
    fb = L.pkd_float_workspace_bytes(64, S, 32, 128)
    hb = L.pkd_host_workspace_bytes(64, S)
    assert ib >= 4 * (64 + S + 1 + 8 * (S + 128) + 16000)
    assert fb == (S + 128) * 32 * 129 * 4
    assert hb >= 2 * 4 * (64 + S + 1 + 8 * (S + 128))
    assert L.pkd_int_workspace_bytes(0, 10, S) == 0
    assert L.pkd_float_workspace_bytes(1, 0, 32, 128) == 0
    assert L.pkd_host_workspace_bytes(-1, S) == 0


def _compare(p_lib, p_ref):
    assert p_lib["chunk_pages"] == p_ref["chunk_pages"]
    assert p_lib["num_items"] == p_ref["num_items"]
    assert p_lib["n_partials"] == p_ref["n_partials"]
    assert p_lib["n_split"] == p_ref["n_split"]
    assert np.array_equal(p_lib["slot_indptr"], p_ref["slot_indptr"])
    assert np.array_equal(p_lib["items"], p_ref["items"])
    assert np.array_equal(p_lib["merges"], p_ref["merges"])


def _lengths_ok(p, P):
    it = p["items"].astype(np.int64)
    assert np.array_equal(p["item_lengths"], (it[:, 2] - 1) * P + it[:, 3])
    assert not p["item_pad"].any()
    _first_items_ok(p)


def _first_items_ok(p):
    """The fixed offsets the kernels compute from the slot count (slots, the
    first-item table and the merge list), the items right after the merge
    list, and the first-item table: slot s's first item again, zeros for an empty slot."""
    h, img = p["header"], p["image"]
    S = h["SLOTS"]
    assert h["OFF_SLOTS"] == 64
    assert h["OFF_FIRST"] == -(-(64 + S + 1) // 8) * 8
    assert h["OFF_MERGE"] == h["OFF_FIRST"] + 8 * S
    assert h["OFF_ITEMS"] == -(-(h["OFF_MERGE"] + 4 * h["SPLIT"]) // 8) * 8
    items8 = img[h["OFF_ITEMS"]: h["OFF_ITEMS"] + 8 * h["ITEMS"]].reshape(-1, 8)
    ind = p["slot_indptr"]
    for s in range(S):
        want = items8[ind[s]] if ind[s] < ind[s + 1] else np.zeros(8, np.int32)
        assert np.array_equal(p["first_items"][s], want), s


@pytest.mark.parametrize("S", [1, 3, 7, 512])
@pytest.mark.parametrize("seed", range(6))
def test_plan_host_matches_oracle_bit_exact(S, seed):
    rng = np.random.default_rng(1000 * S + seed)
    P = [16, 1, 4, 16, 32, 8][seed]
    B = int(rng.integers(1, 70))
    lens = rng.integers(1, 5000 if P > 1 else 800, size=B)
    if seed % 2:
        lens[rng.integers(B)] = 60_000 if P > 1 else 9_000
    indptr, _, last = pt.page_table(lens, P)
    opts = [dict(), dict(min_chunk_tokens=16), dict(fixed_chunk_pages=3), dict(alpha=5, beta=2),
            dict(min_chunk_tokens=512), dict(fixed_chunk_pages=1)][seed]
    if S in (3, 512):
        opts["all_partials"] = True
    ref_opts = {k: v for k, v in opts.items()}
    if S == 1 and opts.get("fixed_chunk_pages") == 1 and int(indptr[-1]) > 20000:
        pytest.skip("oversized for a one-slot scan")
    p_lib = pkd.plan_host(indptr, last, 32, 8, 128, P, S, **opts)
    p_ref = plan_ref.plan(indptr, last, P, S, **ref_opts)
    _compare(p_lib, p_ref)
    _lengths_ok(p_lib, P)
    h = p_lib["header"]
    assert h["MAGIC"] == 0x31444B50 and h["VERSION"] == 3 and h["BATCH"] == B
    assert h["FLAGS"] == (_lib.PKD_PLAN_ALL_PARTIALS if opts.get("all_partials") else 0)
    if opts.get("all_partials"):
        assert p_lib["n_split"] == B and p_lib["merges"][:, 0].tolist() == list(range(B))
    assert h["SLOTS"] == S and h["PAGE_SIZE"] == P and h["NNZ"] == int(indptr[-1])
    assert h["TOTAL_TOKENS_LO"] + (h["TOTAL_TOKENS_HI"] << 32) == int(lens.sum())


@pytest.mark.parametrize("name", ["tiny", "llama8b_step", "skewed", "shared_prefix",
                                  "token_sparse", "wide_gqa", "shared_prefix_b16",
                                  "shared_prefix_b64"])
def test_plan_host_matches_oracle_on_workloads(name):
    spec, _, batches = workloads.workload(name)
    for key, bt in batches.items():
        for S in (256, 512, 768):
            p_lib = pkd.plan_host(bt.kv_indptr, bt.kv_last_page_len, spec.num_qo_heads,
                                  spec.num_kv_heads, spec.head_dim, bt.page_size, S)
            p_ref = plan_ref.plan(bt.kv_indptr, bt.kv_last_page_len, bt.page_size, S)
            _compare(p_lib, p_ref)
            _lengths_ok(p_lib, bt.page_size)


def _plan_rc(indptr, last, Hq=32, Hkv=8, P=16, S=8):
    L = pkd.load()
    indptr = np.ascontiguousarray(indptr, dtype=np.int32)
    last = np.ascontiguousarray(last, dtype=np.int32)
    out = np.zeros(4096, dtype=np.int32)
    n = ctypes.c_int64()
    return L.pkd_plan_host(indptr.ctypes.data, last.ctypes.data, last.shape[0], Hq, Hkv, 128, P, S,
                           None, out.ctypes.data, out.nbytes, ctypes.byref(n))


def test_validation_error_codes():
    assert _plan_rc([0, 3, 4], [5, 16]) == _lib.PKD_OK
    assert _plan_rc([1, 3, 4], [5, 16]) == _lib.PKD_ERR_INVALID_ARG        # indptr[0] != 0
    assert _plan_rc([0, 3, 3], [5, 16]) == _lib.PKD_ERR_INVALID_ARG        # empty request
    assert _plan_rc([0, 3, 4], [0, 16]) == _lib.PKD_ERR_INVALID_ARG        # last_page_len 0
    assert _plan_rc([0, 3, 4], [5, 17]) == _lib.PKD_ERR_INVALID_ARG        # last_page_len > P
    assert _plan_rc([0, 3, 4], [5, 16], Hq=30, Hkv=8) == _lib.PKD_ERR_INVALID_ARG
    assert _plan_rc([0], np.zeros(0)) == _lib.PKD_ERR_INVALID_ARG           # empty batch
    assert _plan_rc([0, 3, 4], [5, 16], S=0) == _lib.PKD_ERR_INVALID_ARG
    msg = pkd.load().pkd_last_error().decode()
    assert "num_slots" in msg


def test_plan_host_buffer_too_small():
    L = pkd.load()
    indptr = np.array([0, 3, 4], dtype=np.int32)
    last = np.array([5, 16], dtype=np.int32)
    out = np.zeros(16, dtype=np.int32)
    n = ctypes.c_int64()
    rc = L.pkd_plan_host(indptr.ctypes.data, last.ctypes.data, 2, 32, 8, 128, 16, 4, None,
                         out.ctypes.data, out.nbytes, ctypes.byref(n))
    assert rc == _lib.PKD_ERR_WORKSPACE_TOO_SMALL


def test_item_bound_holds_for_derived_chunks():
    rng = np.random.default_rng(3)
    for _ in range(30):
        S = int(rng.integers(1, 600))
        B = int(rng.integers(1, 300))
        P = int(rng.choice([1, 16]))
        lens = rng.integers(1, 20000 if P > 1 else 3000, size=B)
        indptr, _, last = pt.page_table(lens, P)
        p = pkd.plan_host(indptr, last, 32, 8, 128, P, S)
        assert p["num_items"] <= S + 2 * B
        assert p["n_partials"] <= p["num_items"]


@pytest.mark.parametrize("seed", range(8))
def test_plan_shared_host_matches_oracle_bit_exact(seed):
    rng = np.random.default_rng(500 + seed)
    P = [16, 32, 64, 16, 16, 32, 64, 16][seed]
    Hq, Hkv = [(32, 8), (32, 4), (64, 8), (8, 8), (16, 2), (32, 32), (64, 8), (32, 8)][seed]
    G = int(rng.integers(1, 7))
    rows = rng.integers(1, 200, size=G)
    qo = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    lens = rng.integers(1, 12000, size=G)
    indptr, _, last = pt.page_table(lens, P)
    S = [256, 7, 1, 512, 33, 256, 64, 100][seed]
    opts = [dict(), dict(min_chunk_tokens=16), dict(fixed_chunk_pages=3), dict(alpha=5, beta=2),
            dict(min_chunk_tokens=1024), dict(), dict(fixed_chunk_pages=1), dict()][seed]
    if seed in (3, 4, 7):
        opts["all_partials"] = True
    lib = pkd.plan_shared_host(qo, indptr, last, Hq, Hkv, 128, P, S, **opts)
    ref = plan_ref.plan_shared(qo, indptr, last, P, S, Hq // Hkv, Hkv, **opts)
    assert lib["chunk_pages"] == ref["chunk_pages"]
    assert lib["num_items"] == ref["num_items"] and lib["n_partials"] == ref["n_partials"]
    assert np.array_equal(lib["slot_indptr"], ref["slot_indptr"])
    assert np.array_equal(lib["items"], ref["items"])
    assert np.array_equal(lib["merges"], ref["merges"])
    assert np.array_equal(lib["groups"], ref["groups"])
    h = lib["header"]
    assert h["KIND"] == 1 and h["BATCH"] == int(qo[-1]) and h["NUM_GROUPS"] == G
    if opts.get("all_partials"):
        assert lib["n_split"] == int(qo[-1])
        assert lib["merges"][:, 0].tolist() == list(range(int(qo[-1])))
    assert h["ROWS_PER_BLOCK"] == 128 // (Hq // Hkv)
    _first_items_ok(dict(lib, first_items=lib["first_items"]))


def test_plan_shared_host_rejects_bad_groups():
    indptr, _, last = pt.page_table([100], 16)
    with pytest.raises(pkd.PkdError) as e:  # gqa 3 does not divide the 128-row block
        pkd.plan_shared_host([0, 2], indptr, last, 24, 8, 128, 16, 16)
    assert e.value.code == _lib.PKD_ERR_UNSUPPORTED
    with pytest.raises(pkd.PkdError) as e:
        pkd.plan_shared_host([0, 0], indptr, last, 32, 8, 128, 16, 16)
    assert e.value.code == _lib.PKD_ERR_INVALID_ARG


def test_read_ceiling_argument_checks():
    """The read-ceiling entry points reject bad sizes, alignment, grids and
    null pointers before any launch (the pointers here are never touched)."""
    L = _lib.load()
    inv = _lib.PKD_ERR_INVALID_ARG
    buf, sink, ids = 0x10000, 0x20000, 0x30000
    assert L.pkd_read_sink_words(3) == 3 * 512 and L.pkd_read_sink_words(0) == 0
    assert L.pkd_read_stream(buf, 24, sink, 1, None) == inv          # not a multiple of 16
    assert L.pkd_read_stream(buf, 0, sink, 1, None) == inv
    assert L.pkd_read_stream(buf + 8, 4096, sink, 1, None) == inv    # misaligned
    assert L.pkd_read_stream(buf, 4096, sink, 0, None) == inv        # grid
    assert L.pkd_read_stream(buf, 4096, sink, (1 << 20) + 1, None) == inv
    assert L.pkd_read_stream(None, 4096, sink, 1, None) == inv
    assert L.pkd_read_stream(buf, 4096, None, 1, None) == inv
    assert L.pkd_read_pages(buf, 4, 1000, ids, 4, sink, 1, None) == inv   # not a power of two
    assert L.pkd_read_pages(buf, 4, 8, ids, 4, sink, 1, None) == inv      # below 16
    assert L.pkd_read_pages(buf, 0, 1024, ids, 4, sink, 1, None) == inv   # no pages
    assert L.pkd_read_pages(buf, 4, 1024, ids, 0, sink, 1, None) == inv   # no ids
    assert L.pkd_read_pages(buf, 4, 1024, None, 4, sink, 1, None) == inv
    assert L.pkd_read_pages(buf, 4, 1024, ids, 4, sink, 0, None) == inv
