"""Shared-prefix (composable) plans on the GPU, through the C ABI: every
request's attention state over its group's pages, from the shared-prefix
kernel (each K/V tile read once per row block of the group), against the fp64
oracle run on the same table expanded to one page list per request.  Bar:
max abs error <= 1e-2 on the bf16 output and <= 1e-3 on lse."""

import numpy as np
import pytest

import workloads
from oracle import attention as att
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

_SHARED = {}


def shared_runner(max_groups=8, max_batch=512, max_nnz=1 << 15, Hq=32, Hkv=8, num_slots=0):
    import paged_kv_decode_11_amd as pkd

    key = (max_groups, max_batch, max_nnz, Hq, Hkv, num_slots)
    if key not in _SHARED:
        _SHARED[key] = pkd.SharedPlanRun(max_groups, max_batch, max_nnz, Hq, Hkv, 128, num_slots)
    return _SHARED[key]


def _groups(seed, rows, lens, P, Hq, Hkv, spare=7, poison=True):
    """Seeded groups: group g has rows[g] requests over lens[g] tokens."""
    rng = np.random.default_rng(seed)
    gb = workloads.make_batch(lens, P, int(sum(-(-l // P) for l in lens)) + spare, Hq, Hkv, 128,
                              rng)
    qo = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    B = int(qo[-1])
    q = workloads.normal_bf16(rng, (B, Hq, 128))
    cache = workloads.host_cache(gb, rng, poison=poison)
    return gb, qo, q, cache


def _expanded(gb, qo):
    """The per-request page table: request r of group g gets group g's pages."""
    G = len(qo) - 1
    indptr, indices, last = [0], [], []
    for g in range(G):
        pages = gb.kv_indices[gb.kv_indptr[g]:gb.kv_indptr[g + 1]]
        for _ in range(qo[g + 1] - qo[g]):
            indices.extend(pages.tolist())
            indptr.append(len(indices))
            last.append(int(gb.kv_last_page_len[g]))
    return (np.array(indptr, np.int32), np.array(indices, np.int32), np.array(last, np.int32))


def _run_shared(gb, qo, q_dev, cache_dev, r=None, sm_scale=None, **opts):
    import torch

    r = r or shared_runner(Hq=gb.num_qo_heads, Hkv=gb.num_kv_heads)
    idx = torch.from_numpy(gb.kv_indices.astype(np.int32)).cuda()
    r.plan(qo, gb.kv_indptr, idx, gb.kv_last_page_len, gb.num_qo_heads, gb.num_kv_heads, 128,
           gb.page_size, **opts)
    o, lse = r.run(q_dev, cache_dev, return_lse=True, sm_scale=sm_scale)
    torch.cuda.synchronize()
    return o, lse


def _check(seed, rows, lens, P, Hq, Hkv, label, sm_scale=None, **opts):
    gb, qo, q, cache = _groups(seed, rows, lens, P, Hq, Hkv)
    gu.say(label, "groups", len(rows), "rows", list(rows), "lens", list(lens), "P", P, "Hq", Hq,
           "Hkv", Hkv, opts)
    o, lse = _run_shared(gb, qo, gu.bits_to_dev(q), gu.bits_to_dev(cache), sm_scale=sm_scale,
                         **opts)
    indptr, indices, last = _expanded(gb, qo)
    o_ref, lse_ref = att.decode(q, cache, indptr, indices, last, Hkv, sm_scale=sm_scale)
    return gu.assert_close(o, lse, o_ref, lse_ref, label=label)


@pytest.mark.parametrize("P", [16, 32, 64])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_one_group_page_sizes_and_gqa(P, G):
    Hkv = 8 if G <= 4 else 4
    tq = 128 // G
    # a full row block, a partial one, and a tail tile of 9 tokens
    _check(10 * P + G, [tq + 3], [5 * P + 9], P, Hkv * G, Hkv, f"P{P}-G{G}")
    _check(11 * P + G, [tq + 3], [5 * P + 9], P, Hkv * G, Hkv, f"P{P}-G{G}-split",
           fixed_chunk_pages=1)


@pytest.mark.parametrize("rows", [1, 5, 31, 32, 33, 100])
def test_row_counts(rows):
    _check(40 + rows, [rows], [700], 16, 32, 8, f"rows{rows}")
    _check(41 + rows, [rows], [700], 16, 32, 8, f"rows{rows}-mct16", min_chunk_tokens=16)


def test_several_groups_mixed():
    _check(70, [3, 1, 40, 17], [1, 2000, 333, 16], 16, 32, 8, "groups")
    _check(71, [3, 1, 40, 17], [1, 2000, 333, 16], 16, 32, 8, "groups-split", fixed_chunk_pages=2)
    _check(72, [3, 1, 40, 17], [1, 2000, 333, 16], 16, 32, 8, "groups-scale", sm_scale=0.2,
           min_chunk_tokens=16)


def test_kv_head_counts():
    _check(80, [9, 4], [500, 77], 16, 8, 8, "Hkv8-G1")
    _check(81, [9, 4], [500, 77], 16, 16, 16, "Hkv16-G1")
    _check(82, [9, 4], [500, 77], 16, 8, 2, "Hkv2-G4", min_chunk_tokens=16)


def test_deterministic():
    import torch

    gb, qo, q, cache = _groups(90, [40, 7], [3000, 900], 16, 32, 8)
    qd, cd = gu.bits_to_dev(q), gu.bits_to_dev(cache)
    o1, l1 = _run_shared(gb, qo, qd, cd, min_chunk_tokens=16)
    o2, l2 = _run_shared(gb, qo, qd, cd, min_chunk_tokens=16)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_unbuilt_page_size_rejected():
    import torch
    import paged_kv_decode_11_amd as pkd
    from paged_kv_decode_11_amd import _lib

    gb, qo, q, cache = _groups(91, [4], [100], 8, 32, 8)
    r = shared_runner()
    idx = torch.from_numpy(gb.kv_indices.astype(np.int32)).cuda()
    with pytest.raises(pkd.PkdError) as e:
        r.plan(qo, gb.kv_indptr, idx, gb.kv_last_page_len, 32, 8, 128, 8)
    assert e.value.code == _lib.PKD_ERR_UNSUPPORTED


def test_shared_prefix_workload_composable_full():
    """The shared-prefix workload at full size: the prefix state of all 32
    requests from one shared-prefix plan (the 512 prefix pages read once per
    KV head), the suffix states from a decode plan, merged, against the
    single-format oracle on 8 requests."""
    import torch
    import paged_kv_decode_11_amd as pkd

    spec, rng, b = workloads.workload("shared_prefix")
    main, prefix, suffix = b["main"], b["prefix"], b["suffix"]
    q = workloads.host_query(main, rng)
    cache = workloads.host_cache(main, rng)
    gu.say("shared_prefix composable (shared kernel)", main.batch, main.total_tokens)
    qd, cd = gu.bits_to_dev(q), gu.bits_to_dev(cache)
    # the prefix as one group of all 32 requests
    n_pages = int(prefix.kv_indptr[1])
    qo = np.array([0, main.batch], np.int32)
    kv_indptr = np.array([0, n_pages], np.int32)
    pages = torch.from_numpy(prefix.kv_indices[:n_pages].astype(np.int32)).cuda()
    r = shared_runner(max_groups=4, max_batch=64, max_nnz=1 << 12)
    r.plan(qo, kv_indptr, pages, prefix.kv_last_page_len[:1], 32, 8, 128, 16)
    o_p, l_p = r.run(qd, cd, return_lse=True)
    o_s, l_s = gu.decode(suffix, qd, cd, r=gu.runner(max_batch=64, max_nnz=1 << 12))
    o, lse = pkd.merge_state(o_p, l_p, o_s, l_s)
    torch.cuda.synchronize()
    req = [0, 3, 7, 12, 18, 24, 29, 31]
    o_ref, lse_ref = att.decode(q, cache, main.kv_indptr, main.kv_indices, main.kv_last_page_len,
                                main.num_kv_heads, requests=req)
    gu.assert_close(o, lse, o_ref, lse_ref, requests=req, label="composable-shared-kernel")


# ---------------------------------------------------------------------------
# the composable format in one call: pkd_run_composable
# ---------------------------------------------------------------------------

def _composable_inputs(seed, rows, prefix_lens, suffix_lens, P, Hq, Hkv, fp8=False):
    """Groups over prefixes and every request's own suffix, in one pool: the
    group table, the suffix table and the cache (E4M3 codes when fp8)."""
    rng = np.random.default_rng(seed)
    lens = list(prefix_lens) + list(suffix_lens)
    need = int(sum(-(-l // P) for l in lens))
    allb = workloads.make_batch(lens, P, need + 5, Hq, Hkv, 128, rng)
    G = len(prefix_lens)
    gi = allb.kv_indptr
    gb = workloads.PagedBatch(P, Hq, Hkv, 128, allb.num_pages,
                              np.asarray(prefix_lens, np.int64), gi[:G + 1].copy(),
                              allb.kv_indices[:gi[G]].copy(), allb.kv_last_page_len[:G].copy())
    sb = workloads.PagedBatch(P, Hq, Hkv, 128, allb.num_pages,
                              np.asarray(suffix_lens, np.int64), (gi[G:] - gi[G]).astype(np.int32),
                              allb.kv_indices[gi[G]:].copy(), allb.kv_last_page_len[G:].copy())
    qo = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    q = workloads.normal_bf16(rng, (int(qo[-1]), Hq, 128))
    cache = (workloads.host_cache_e4m3(allb, rng, poison=True) if fp8
             else workloads.host_cache(allb, rng, poison=True))
    return gb, sb, qo, q, cache


def _composable_ref(gb, sb, qo, q, cache, Hkv, sm_scale=None):
    from oracle import merge as om

    indptr, indices, last = _expanded(gb, qo)
    o_p, l_p = att.decode(q, cache, indptr, indices, last, Hkv, sm_scale=sm_scale)
    o_s, l_s = att.decode(q, cache, sb.kv_indptr, sb.kv_indices, sb.kv_last_page_len, Hkv,
                          sm_scale=sm_scale)
    return om.merge_rows(o_p, l_p, o_s, l_s)


def _plan_both(rp, rs, gb, sb, qo, P, Hq, Hkv, popts=None, sopts=None, fp8=False):
    import torch

    kv = dict(kv_data_type=torch.float8_e4m3fn) if fp8 else {}
    rp.plan(qo, gb.kv_indptr, torch.from_numpy(gb.kv_indices.astype(np.int32)).cuda(),
            gb.kv_last_page_len, Hq, Hkv, 128, P, all_partials=True, **kv, **(popts or {}))
    rs.plan(sb.kv_indptr, torch.from_numpy(sb.kv_indices.astype(np.int32)).cuda(),
            sb.kv_last_page_len, Hq, Hkv, 128, P, all_partials=True, **kv, **(sopts or {}))


@pytest.mark.parametrize("side_by_side", [False, True])
@pytest.mark.parametrize("case", range(7))
def test_run_composable(case, side_by_side):
    """Prefix groups and per-request suffixes in one call against the
    oracle's merge of the two exact states; unsplit and split on either side,
    one-token suffixes, several groups, group sizes 1-8; with the default
    slot counts (three launches) and with half of the compute units per
    handle (both attention kernels in one launch, KV head counts 2 and 8
    among the cases)."""
    import torch
    import paged_kv_decode_11_amd as pkd

    P, Hq, Hkv, rows, plens, popts, sopts = [
        (16, 32, 8, [32], [8 * 16 + 5], {}, {}),
        (16, 32, 8, [5, 40, 1], [300, 2000, 17], {"fixed_chunk_pages": 2}, {"fixed_chunk_pages": 1}),
        (32, 64, 8, [20], [1000], {"min_chunk_tokens": 32}, {}),
        (64, 8, 8, [9, 3], [700, 64], {}, {"fixed_chunk_pages": 3}),
        (16, 16, 2, [33], [5000], {}, {"min_chunk_tokens": 16}),
        (16, 32, 8, [2, 2, 2, 2], [16, 32, 48, 1], {"fixed_chunk_pages": 1}, {}),
        # the suffix plan weighing each chunk 32 tokens more (as the benchmark does)
        (16, 32, 8, [32], [4096], {}, {"alpha": 32}),
    ][case]
    B = int(sum(rows))
    rng = np.random.default_rng(600 + case)
    slens = rng.integers(1, 900, size=B).tolist()
    slens[0] = 1
    gb, sb, qo, q, cache = _composable_inputs(610 + case, rows, plens, slens, P, Hq, Hkv)
    gu.say("composable", case, "side by side", side_by_side, "rows", rows, "prefix", plens, "P", P,
           "Hq", Hq, "Hkv", Hkv)
    # workspaces with room for the forced one- and two-page chunks
    slots = _half_cus() if side_by_side else 0
    rp = pkd.SharedPlanRun(64, 256, 1 << 14, Hq, Hkv, num_slots=slots)
    rs = pkd.DecodePlanRun(max_batch=1024, max_nnz=1 << 14, max_qo_heads=Hq, num_slots=slots)
    _plan_both(rp, rs, gb, sb, qo, P, Hq, Hkv, popts, sopts)
    o, lse = pkd.run_composable(rp, rs, gu.bits_to_dev(q), gu.bits_to_dev(cache), return_lse=True)
    torch.cuda.synchronize()
    assert rp.read_device_error() == 0 and rs.read_device_error() == 0
    o_ref, lse_ref = _composable_ref(gb, sb, qo, q, cache, Hkv)
    gu.assert_close(o, lse, o_ref, lse_ref, label=f"composable-{case}")


def test_run_composable_refusals():
    import torch
    import paged_kv_decode_11_amd as pkd
    from paged_kv_decode_11_amd import _lib

    gb, sb, qo, q, cache = _composable_inputs(620, [4], [100], [5, 6, 7, 8], 16, 32, 8)
    qd, cd = gu.bits_to_dev(q), gu.bits_to_dev(cache)
    rp = pkd.SharedPlanRun(2, 16, 1 << 10, 32, 8)
    rs = pkd.DecodePlanRun(max_batch=16, max_nnz=1 << 10, max_qo_heads=32)
    idx_g = torch.from_numpy(gb.kv_indices.astype(np.int32)).cuda()
    idx_s = torch.from_numpy(sb.kv_indices.astype(np.int32)).cuda()
    # plans without all_partials
    rp.plan(qo, gb.kv_indptr, idx_g, gb.kv_last_page_len, 32, 8, 128, 16)
    rs.plan(sb.kv_indptr, idx_s, sb.kv_last_page_len, 32, 8, 128, 16)
    with pytest.raises(pkd.PkdError) as e:
        pkd.run_composable(rp, rs, qd, cd)
    assert e.value.code == _lib.PKD_ERR_INVALID_ARG
    _plan_both(rp, rs, gb, sb, qo, 16, 32, 8)
    with pytest.raises(pkd.PkdError) as e:   # handles swapped
        pkd.run_composable(rs, rp, qd, cd)
    assert e.value.code == _lib.PKD_ERR_INVALID_ARG
    # a suffix plan for another batch
    rs.plan(sb.kv_indptr[:3], idx_s, sb.kv_last_page_len[:2], 32, 8, 128, 16, all_partials=True)
    with pytest.raises(pkd.PkdError) as e:
        pkd.run_composable(rp, rs, qd, cd)
    assert e.value.code == _lib.PKD_ERR_STALE_PLAN
    # scales on a bf16 cache; a plan pair whose cache dtypes differ
    _plan_both(rp, rs, gb, sb, qo, 16, 32, 8)
    with pytest.raises(pkd.PkdError) as e:
        pkd.run_composable(rp, rs, qd, cd, k_scale=0.5)
    assert e.value.code == _lib.PKD_ERR_INVALID_ARG
    rs.plan(sb.kv_indptr, idx_s, sb.kv_last_page_len, 32, 8, 128, 16, all_partials=True,
            kv_data_type=torch.float8_e4m3fn)
    with pytest.raises(pkd.PkdError) as e:
        pkd.run_composable(rp, rs, qd, cd)
    assert e.value.code == _lib.PKD_ERR_DTYPE_MISMATCH


def _half_cus():
    import torch

    return torch.cuda.get_device_properties(0).multi_processor_count // 2


@pytest.mark.parametrize("side_by_side", [False, True])
def test_run_composable_graph_replay(side_by_side):
    """A composable run captured once replays correctly after both handles
    are planned again for other lengths: with the default slot counts (the
    three kernels one after the other) and with half of the compute units
    for each handle (both attention kernels in one launch, then the
    merge)."""
    import torch
    import paged_kv_decode_11_amd as pkd

    P, Hq, Hkv, rows = 16, 32, 8, [6, 10]
    B = sum(rows)
    slots = _half_cus() if side_by_side else 0
    rp = pkd.SharedPlanRun(4, 64, 1 << 12, Hq, Hkv, num_slots=slots)
    rs = pkd.DecodePlanRun(max_batch=512, max_nnz=1 << 12, max_qo_heads=Hq, num_slots=slots)
    steps = []
    for seed in range(3):
        rng = np.random.default_rng(700 + seed)
        plens = rng.integers(1, 1500, size=2).tolist()
        slens = rng.integers(1, 600, size=B).tolist()
        steps.append(_composable_inputs(710 + seed, rows, plens, slens, P, Hq, Hkv))
    pool = max(s[0].num_pages for s in steps)
    # one device cache large enough for every step's pool
    cd = torch.zeros((pool, 2, P, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    q_buf = torch.zeros((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    o_buf = torch.zeros((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    lse_buf = torch.zeros((B, Hq), dtype=torch.float32, device="cuda")
    gb, sb, qo, q, cache = steps[0]
    _plan_both(rp, rs, gb, sb, qo, P, Hq, Hkv)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pkd.run_composable(rp, rs, q_buf, cd, out=o_buf, lse=lse_buf, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pkd.run_composable(rp, rs, q_buf, cd, out=o_buf, lse=lse_buf)
    torch.cuda.synchronize()
    for n, (gb, sb, qo, q, cache) in enumerate(steps[1:] + steps[:1]):
        gu.say("composable graph step", n)
        _plan_both(rp, rs, gb, sb, qo, P, Hq, Hkv, sopts={"fixed_chunk_pages": n + 1})
        cd[:cache.shape[0]].copy_(gu.bits_to_dev(cache))
        q_buf.copy_(gu.bits_to_dev(q))
        for _ in range(2):
            o_buf.zero_()
            g.replay()
            torch.cuda.synchronize()
            o_ref, lse_ref = _composable_ref(gb, sb, qo, q, cache, Hkv)
            gu.assert_close(o_buf, lse_buf, o_ref, lse_ref, label=f"composable replay {n}")


@pytest.mark.parametrize("name", ["shared_prefix", "shared_prefix_b16", "shared_prefix_b64"])
def test_shared_prefix_workload_run_composable_full(name):
    """A shared-prefix workload at full size through pkd_run_composable,
    against the single-format oracle on 8 requests (the last among them)."""
    import torch
    import paged_kv_decode_11_amd as pkd

    spec, rng, b = workloads.workload(name)
    main, prefix, suffix = b["main"], b["prefix"], b["suffix"]
    q = workloads.host_query(main, rng)
    cache = workloads.host_cache(main, rng)
    gu.say("shared_prefix run_composable", main.batch, main.total_tokens)
    qd, cd = gu.bits_to_dev(q), gu.bits_to_dev(cache)
    n_pages = int(prefix.kv_indptr[1])
    rp = pkd.SharedPlanRun(4, 64, 1 << 12, 32, 8)
    rs = pkd.DecodePlanRun(max_batch=64, max_nnz=1 << 12, max_qo_heads=32)
    rp.plan(np.array([0, main.batch], np.int32), np.array([0, n_pages], np.int32),
            torch.from_numpy(prefix.kv_indices[:n_pages].astype(np.int32)).cuda(),
            prefix.kv_last_page_len[:1], 32, 8, 128, 16, all_partials=True)
    rs.plan(suffix.kv_indptr, torch.from_numpy(suffix.kv_indices.astype(np.int32)).cuda(),
            suffix.kv_last_page_len, 32, 8, 128, 16, all_partials=True)
    o, lse = pkd.run_composable(rp, rs, qd, cd, return_lse=True)
    torch.cuda.synchronize()
    B = main.batch
    req = sorted({0, 3, 7, B // 3, B // 2, (2 * B) // 3, B - 2, B - 1})
    o_ref, lse_ref = att.decode(q, cache, main.kv_indptr, main.kv_indices, main.kv_last_page_len,
                                main.num_kv_heads, requests=req)
    gu.assert_close(o, lse, o_ref, lse_ref, requests=req, label=f"run_composable full {name}")


# ---------------------------------------------------------------------------
# FP8 E4M3 cache: shared-prefix plans and the composable call with scales

K_SCALE, V_SCALE = 1.0 / 64, 1.0 / 32


@pytest.mark.parametrize("P", [16, 32, 64])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_fp8_shared_groups(P, G):
    """A shared-prefix plan over E4M3 codes (NaN codes past every group's
    last token): every request's state over its group's tokens against the
    oracle on the table expanded to one page list per request; unsplit and
    split."""
    import torch

    Hkv = 8 if G <= 4 else 4
    Hq = Hkv * G
    rows, lens = [128 // G + 3, 5], [40 * P + 7, 3 * P]
    rng = np.random.default_rng(2000 + 10 * P + G)
    gb = workloads.make_batch(lens, P, int(sum(-(-l // P) for l in lens)) + 7, Hq, Hkv, 128, rng)
    qo = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    q = workloads.normal_bf16(rng, (int(qo[-1]), Hq, 128))
    codes = workloads.host_cache_e4m3(gb, rng, poison=True)
    indptr, indices, last = _expanded(gb, qo)
    o_ref, lse_ref = att.decode_fp8(q, codes, indptr, indices, last, Hkv, k_scale=K_SCALE,
                                    v_scale=V_SCALE)
    r = shared_runner(Hq=Hq, Hkv=Hkv)
    idx = torch.from_numpy(gb.kv_indices.astype(np.int32)).cuda()
    for opts in ({}, {"fixed_chunk_pages": 3}):
        gu.say("fp8 shared", "P", P, "G", G, "rows", rows, "lens", lens, opts)
        r.plan(qo, gb.kv_indptr, idx, gb.kv_last_page_len, Hq, Hkv, 128, P,
               kv_data_type=torch.float8_e4m3fn, **opts)
        o, lse = r.run(gu.bits_to_dev(q), gu.codes_to_dev(codes), return_lse=True,
                       k_scale=K_SCALE, v_scale=V_SCALE)
        torch.cuda.synchronize()
        assert r.read_device_error() == 0
        gu.assert_close(o, lse, o_ref, lse_ref, label=f"fp8 shared P{P} G{G} {opts}")


def test_fp8_shared_unit_scales():
    """Unit scales (values up to 448): P enters the product as a bf16 high
    part plus remainder, so the plain bar holds at any magnitude."""
    import torch

    rows, lens, P = [32], [700], 16
    rng = np.random.default_rng(2100)
    gb = workloads.make_batch(lens, P, 60, 32, 8, 128, rng)
    qo = np.array([0, 32], np.int32)
    q = workloads.normal_bf16(rng, (32, 32, 128))
    codes = workloads.host_cache_e4m3(gb, rng, poison=True)
    indptr, indices, last = _expanded(gb, qo)
    o_ref, lse_ref = att.decode_fp8(q, codes, indptr, indices, last, 8, k_scale=1.0, v_scale=1.0,
                                    sm_scale=1.0 / 4096)
    r = shared_runner()
    idx = torch.from_numpy(gb.kv_indices.astype(np.int32)).cuda()
    r.plan(qo, gb.kv_indptr, idx, gb.kv_last_page_len, 32, 8, 128, P,
           kv_data_type=torch.float8_e4m3fn)
    o, lse = r.run(gu.bits_to_dev(q), gu.codes_to_dev(codes), return_lse=True, k_scale=1.0,
                   v_scale=1.0, sm_scale=1.0 / 4096)
    torch.cuda.synchronize()
    gu.assert_close(o, lse, o_ref, lse_ref, label="fp8 shared unit scales")


@pytest.mark.parametrize("side_by_side", [False, True])
@pytest.mark.parametrize("case", range(6))
def test_fp8_run_composable(case, side_by_side):
    """Prefix groups and per-request suffixes over one E4M3 cache, with
    scales, against the oracle's merge of the two exact states: the
    shared-prefix kernel and the FP8 decode kernel one after the other
    (default slot counts), and in one launch (half of the compute units per
    handle)."""
    import torch
    import paged_kv_decode_11_amd as pkd
    from oracle import merge as om

    P, Hq, Hkv, rows, plens, popts, sopts = [
        (16, 32, 8, [32], [8 * 16 + 5], {}, {}),
        (16, 32, 8, [5, 40, 1], [300, 2000, 17], {"fixed_chunk_pages": 2}, {"fixed_chunk_pages": 1}),
        (64, 8, 8, [9, 3], [700, 64], {}, {"fixed_chunk_pages": 3}),
        # KV head counts the 8 waves of a workgroup do not divide evenly
        (16, 16, 2, [33], [5000], {}, {"min_chunk_tokens": 16}),
        (32, 32, 16, [7, 2], [900, 40], {"fixed_chunk_pages": 4}, {}),
        # one-token and page-aligned prefixes, one page per chunk
        (16, 32, 8, [2, 2, 2, 2], [16, 32, 48, 1], {"fixed_chunk_pages": 1}, {}),
    ][case]
    B = int(sum(rows))
    rng = np.random.default_rng(700 + case)
    slens = rng.integers(1, 900, size=B).tolist()
    slens[0] = 1
    gb, sb, qo, q, codes = _composable_inputs(710 + case, rows, plens, slens, P, Hq, Hkv, fp8=True)
    gu.say("fp8 composable", case, "side by side", side_by_side, "rows", rows, "prefix", plens,
           "P", P, "Hq", Hq, "Hkv", Hkv)
    slots = _half_cus() if side_by_side else 0
    rp = pkd.SharedPlanRun(64, 256, 1 << 14, Hq, Hkv, num_slots=slots)
    rs = pkd.DecodePlanRun(max_batch=1024, max_nnz=1 << 14, max_qo_heads=Hq, num_slots=slots)
    _plan_both(rp, rs, gb, sb, qo, P, Hq, Hkv, popts, sopts, fp8=True)
    o, lse = pkd.run_composable(rp, rs, gu.bits_to_dev(q), gu.codes_to_dev(codes), return_lse=True,
                                k_scale=K_SCALE, v_scale=V_SCALE)
    torch.cuda.synchronize()
    assert rp.read_device_error() == 0 and rs.read_device_error() == 0
    indptr, indices, last = _expanded(gb, qo)
    o_p, l_p = att.decode_fp8(q, codes, indptr, indices, last, Hkv, k_scale=K_SCALE,
                              v_scale=V_SCALE)
    o_s, l_s = att.decode_fp8(q, codes, sb.kv_indptr, sb.kv_indices, sb.kv_last_page_len, Hkv,
                              k_scale=K_SCALE, v_scale=V_SCALE)
    o_ref, lse_ref = om.merge_rows(o_p, l_p, o_s, l_s)
    gu.assert_close(o, lse, o_ref, lse_ref, label=f"fp8 composable-{case}")


@pytest.mark.parametrize("side_by_side", [False, True])
def test_fp8_run_composable_graph_replay(side_by_side):
    """The composable call over an E4M3 cache, captured once, replays
    correctly after both handles are planned again for other lengths, in
    both forms (one launch, and the two kernels one after the other)."""
    import torch
    import paged_kv_decode_11_amd as pkd
    from oracle import merge as om

    P, Hq, Hkv, rows = 16, 32, 8, [6, 10]
    B = sum(rows)
    slots = _half_cus() if side_by_side else 0
    rp = pkd.SharedPlanRun(4, 64, 1 << 12, Hq, Hkv, num_slots=slots)
    rs = pkd.DecodePlanRun(max_batch=512, max_nnz=1 << 12, max_qo_heads=Hq, num_slots=slots)
    steps = []
    for seed in range(3):
        rng = np.random.default_rng(730 + seed)
        plens = rng.integers(1, 1500, size=2).tolist()
        slens = rng.integers(1, 600, size=B).tolist()
        steps.append(_composable_inputs(740 + seed, rows, plens, slens, P, Hq, Hkv, fp8=True))
    pool = max(s[0].num_pages for s in steps)
    cd = torch.zeros((pool, 2, P, Hkv, 128), dtype=torch.uint8, device="cuda")
    cd8 = cd.view(torch.float8_e4m3fn)
    q_buf = torch.zeros((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    o_buf = torch.zeros((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    lse_buf = torch.zeros((B, Hq), dtype=torch.float32, device="cuda")
    gb, sb, qo, q, codes = steps[0]
    _plan_both(rp, rs, gb, sb, qo, P, Hq, Hkv, fp8=True)
    run = lambda: pkd.run_composable(rp, rs, q_buf, cd8, out=o_buf, lse=lse_buf,
                                     k_scale=K_SCALE, v_scale=V_SCALE)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pkd.run_composable(rp, rs, q_buf, cd8, out=o_buf, lse=lse_buf, k_scale=K_SCALE,
                           v_scale=V_SCALE, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for n, (gb, sb, qo, q, codes) in enumerate(steps[1:] + steps[:1]):
        gu.say("fp8 composable graph step", n, "side by side", side_by_side)
        _plan_both(rp, rs, gb, sb, qo, P, Hq, Hkv, sopts={"fixed_chunk_pages": n + 1}, fp8=True)
        cd[:codes.shape[0]].copy_(torch.from_numpy(codes).cuda())
        q_buf.copy_(gu.bits_to_dev(q))
        indptr, indices, last = _expanded(gb, qo)
        o_p, l_p = att.decode_fp8(q, codes, indptr, indices, last, Hkv, k_scale=K_SCALE,
                                  v_scale=V_SCALE)
        o_s, l_s = att.decode_fp8(q, codes, sb.kv_indptr, sb.kv_indices, sb.kv_last_page_len, Hkv,
                                  k_scale=K_SCALE, v_scale=V_SCALE)
        o_ref, lse_ref = om.merge_rows(o_p, l_p, o_s, l_s)
        for _ in range(2):
            o_buf.zero_()
            g.replay()
            torch.cuda.synchronize()
            gu.assert_close(o_buf, lse_buf, o_ref, lse_ref, label=f"fp8 composable replay {n}")
