"""Decode parity on the GPU: the HIP path (through the C ABI) against the
fp64 oracle, element by element, on seeded inputs.  Bar: max abs error
<= 1e-2 on the bf16 output and <= 1e-3 on lse."""

import numpy as np
import pytest

import workloads
from oracle import attention as att
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

VARIANTS = ["dot2", "mfma", "mfma_pv"]


def _small(seed, lens, P, Hq, Hkv, poison=True, spare=9):
    rng = np.random.default_rng(seed)
    need = int(sum(-(-l // P) for l in lens))
    batch = workloads.make_batch(lens, P, need + spare, Hq, Hkv, 128, rng)
    q = workloads.host_query(batch, rng)
    cache = workloads.host_cache(batch, rng, poison=poison)
    return batch, q, cache


def _check(batch, q, cache, label, sm_scale=None, return_lse=True, r=None, **opts):
    gu.say(label, "B", batch.batch, "P", batch.page_size, "Hq", batch.num_qo_heads,
           "Hkv", batch.num_kv_heads, "T", batch.total_tokens, opts)
    o_ref, lse_ref = att.decode(q, cache, batch.kv_indptr, batch.kv_indices,
                                batch.kv_last_page_len, batch.num_kv_heads, sm_scale=sm_scale)
    o, lse = gu.decode(batch, gu.bits_to_dev(q), gu.bits_to_dev(cache), r=r, sm_scale=sm_scale,
                       return_lse=return_lse, **opts)
    return gu.assert_close(o, lse, o_ref, lse_ref, label=label)


def test_device_plan_image():
    """The uploaded plan is the host planner's image, except that the item
    rows (first-item rows and items) of a decode plan also carry the ids of
    each item's first two pages, read on the device from kv_indices."""
    import torch

    import paged_kv_decode_11_amd as pkd
    from paged_kv_decode_11_amd import _lib

    rng = np.random.default_rng(71)
    lens = [int(x) for x in rng.integers(1, 900, size=23)] + [16, 17, 1, 2000]
    need = sum(-(-n // 16) for n in lens)
    batch = workloads.make_batch(lens, 16, need + 40, 32, 8, 128, rng)
    r = gu.runner()
    gu.decode(batch, gu.bits_to_dev(workloads.host_query(batch, rng)),
              gu.bits_to_dev(workloads.host_cache(batch, rng)), r=r, fixed_chunk_pages=7)
    host = pkd.plan_host(batch.kv_indptr, batch.kv_last_page_len, 32, 8, 128, 16, r.num_slots,
                         fixed_chunk_pages=7)
    img = host["image"]
    dev = r.int_workspace.view(torch.int32)[: img.size].cpu().numpy()
    h = host["header"]
    gu.say("plan image", "ints", img.size, "items", h["ITEMS"], "slots", h["SLOTS"])
    # item rows: the first-item table, then the items (after the merge list)
    row_ints = np.concatenate([
        np.arange(h["OFF_FIRST"], h["OFF_FIRST"] + 8 * h["SLOTS"]),
        np.arange(h["OFF_ITEMS"], h["OFF_ITEMS"] + 8 * h["ITEMS"])])
    plan_id = _lib.HEADER_BASE + _lib.H["PLAN_ID"]
    same = np.ones(img.size, dtype=bool)
    same[: _lib.HEADER_BASE] = False  # device-only words
    same[plan_id] = False
    rows = row_ints.reshape(-1, 8)
    same[rows[:, 6:].ravel()] = False
    assert np.array_equal(dev[same], img[same])
    assert dev[plan_id] == r.plan_id
    fields = dev[row_ints].reshape(-1, 8)
    kv = batch.kv_indices.astype(np.int64)
    for row, f in enumerate(fields):
        if f[2] == 0:  # a slot without items
            assert f[6] == 0 and f[7] == 0, row
            continue
        assert f[6] == kv[f[1]], row
        assert f[7] == kv[f[1] + (1 if f[2] > 1 else 0)], row


@pytest.mark.parametrize("variant", VARIANTS)
def test_tiny_workload_writethrough(variant):
    spec, rng, b = workloads.workload("tiny")
    batch = b["main"]
    q = workloads.host_query(batch, rng)
    cache = workloads.host_cache(batch, rng, poison=True)
    _check(batch, q, cache, f"tiny-{variant}", variant=variant)


def test_tiny_worked_example_pages():
    rng = np.random.default_rng(0)
    batch = workloads.make_batch([37, 16, 5], 16, 64, 32, 8, 128, rng, scatter=False)
    assert batch.kv_indptr.tolist() == [0, 3, 4, 5]
    q = workloads.host_query(batch, rng)
    cache = workloads.host_cache(batch, rng, poison=True)
    _check(batch, q, cache, "worked-example")


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("fixed", [1, 2])
def test_tiny_forced_splits(fixed, variant):
    spec, rng, b = workloads.workload("tiny")
    batch = b["main"]
    q = workloads.host_query(batch, rng)
    cache = workloads.host_cache(batch, rng, poison=True)
    _check(batch, q, cache, f"tiny-split{fixed}-{variant}", fixed_chunk_pages=fixed,
           variant=variant)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("P", [1, 2, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_page_sizes_and_groups(P, G, variant):
    Hkv = 8 if G <= 4 else 4
    lens = sorted(set(workloads.edge_lengths(P) + [3 * P + 5, 77, 300]))
    batch, q, cache = _small(10 * P + G, lens, P, Hkv * G, Hkv)
    _check(batch, q, cache, f"P{P}-G{G}-{variant}", variant=variant)
    _check(batch, q, cache, f"P{P}-G{G}-{variant}-split",
           fixed_chunk_pages=1 if P >= 16 else max(1, 48 // P), variant=variant)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("Hkv", [1, 2, 3, 8, 12, 16])
def test_kv_head_counts(Hkv, variant):
    """Fewer waves than 8 per workgroup (Hkv < 8) and heads looped over
    waves (Hkv > 8)."""
    batch, q, cache = _small(50 + Hkv, [1, 40, 129, 500], 16, 4 * Hkv, Hkv)
    _check(batch, q, cache, f"Hkv{Hkv}-{variant}", variant=variant)
    _check(batch, q, cache, f"Hkv{Hkv}-{variant}-split", min_chunk_tokens=16, variant=variant)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("P", [1, 4])
@pytest.mark.parametrize("G", [2, 8])
@pytest.mark.parametrize("Hkv", [3, 12])
def test_kv_head_counts_small_pages(Hkv, G, P, variant):
    """Pages below 16 tokens (each lane addresses its own rows) with fewer
    waves than 8 (Hkv = 3) and with heads looped over waves (Hkv = 12)."""
    batch, q, cache = _small(60 + Hkv + G + P, [1, 15, 17, 70, 300], P, G * Hkv, Hkv)
    _check(batch, q, cache, f"P{P}-G{G}-Hkv{Hkv}-{variant}", variant=variant)
    _check(batch, q, cache, f"P{P}-G{G}-Hkv{Hkv}-{variant}-split", min_chunk_tokens=16,
           variant=variant)


@pytest.mark.parametrize("variant", VARIANTS)
def test_no_lse_and_custom_scale(variant):
    batch, q, cache = _small(7, [100, 33, 1], 16, 32, 8)
    _check(batch, q, cache, "no-lse", return_lse=False, variant=variant)
    _check(batch, q, cache, "scale0.3", sm_scale=0.3, variant=variant)
    _check(batch, q, cache, "scale0.3-split", sm_scale=0.3, fixed_chunk_pages=2, variant=variant)


@pytest.mark.parametrize("variant", VARIANTS)
def test_single_token_requests(variant):
    batch, q, cache = _small(8, [1] * 37, 16, 32, 8)
    _check(batch, q, cache, "ones", variant=variant)


@pytest.mark.parametrize("variant", VARIANTS)
def test_random_batches_many_splits(variant):
    rng = np.random.default_rng(99)
    for trial in range(4):
        lens = rng.integers(1, 2000, size=int(rng.integers(1, 40)))
        batch, q, cache = _small(200 + trial, lens.tolist(), 16, 32, 8)
        _check(batch, q, cache, f"random{trial}-{variant}", variant=variant)
        _check(batch, q, cache, f"random{trial}-{variant}-mct16", min_chunk_tokens=16,
               variant=variant)
        # other cost weights change only which slot takes which chunk
        _check(batch, q, cache, f"random{trial}-{variant}-a40b3", min_chunk_tokens=16, alpha=40,
               beta=3, variant=variant)


@pytest.mark.parametrize("variant", VARIANTS)
def test_few_slots_long_queues(variant):
    """A handle with 3 slots: each workgroup walks many items."""
    r = gu.runner(max_batch=64, max_nnz=1 << 14, num_slots=3)
    assert r.num_slots == 3
    batch, q, cache = _small(31, [700, 20, 1, 999, 64, 65], 16, 32, 8)
    _check(batch, q, cache, "3slots", r=r, variant=variant)
    _check(batch, q, cache, "3slots-split", r=r, fixed_chunk_pages=4, variant=variant)


@pytest.mark.parametrize("variant", VARIANTS)
def test_outputs_are_deterministic(variant):
    import torch

    batch, q, cache = _small(12, [3000, 17, 900], 16, 32, 8)
    qd, cd = gu.bits_to_dev(q), gu.bits_to_dev(cache)
    o1, l1 = gu.decode(batch, qd, cd, min_chunk_tokens=16, variant=variant)
    o2, l2 = gu.decode(batch, qd, cd, min_chunk_tokens=16, variant=variant)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_variants_agree():
    """The kernels compute the same states; they may differ only in rounding
    (fp32 arithmetic, and the probabilities' high-and-low bf16 split in the
    mfma_pv kernel)."""
    batch, q, cache = _small(13, [1, 17, 300, 2000, 4999], 16, 32, 8)
    qd, cd = gu.bits_to_dev(q), gu.bits_to_dev(cache)
    o1, l1 = gu.decode(batch, qd, cd, variant="dot2")
    for other in ("mfma", "mfma_pv"):
        o2, l2 = gu.decode(batch, qd, cd, variant=other)
        gu.check_o(gu.dev_to_f64(o2), gu.dev_to_f64(o1), f"{other}-vs-dot2")
        gu.check_lse(l2.cpu().numpy().astype(np.float64), l1.cpu().numpy().astype(np.float64),
                     f"{other}-vs-dot2")


def test_auto_variant_by_shape():
    """The default kernel for a bf16 cache: both products on the matrix
    cores for group size 8, pages below 16 tokens, or fewer than 768 KV
    tokens per slot; q.k on the matrix cores otherwise; explicit variants are
    kept."""
    import torch

    r = gu.runner(max_batch=64, max_nnz=1 << 12)
    for P, Hq, Hkv, want in ((16, 64, 8, "mfma_pv"), (64, 8, 1, "mfma_pv"), (8, 64, 8, "mfma_pv"),
                             (1, 64, 8, "mfma_pv"), (1, 32, 8, "mfma_pv"), (4, 16, 8, "mfma_pv"),
                             (16, 32, 8, "mfma_pv"), (16, 8, 8, "mfma_pv"),
                             (32, 16, 8, "mfma_pv")):
        batch, q, cache = _small(3, [40, 7], P, Hq, Hkv)
        idx = torch.from_numpy(batch.kv_indices).cuda()
        r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, Hq, Hkv, 128, P)
        assert r.planned_variant == want, (P, Hq, Hkv, r.planned_variant)
    r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, 8, 8, 128, 16, variant="mfma")
    assert r.planned_variant == "mfma"
    # about 1,000 tokens per slot (a Llama-3-8B-like layer) against about 520
    # (the skewed batch), planned only
    big = gu.runner(max_batch=64, max_nnz=1 << 15)
    rng = np.random.default_rng(5)
    for lens, Hq, want in (([4000] * 64, 32, "mfma"), ([512] * 63 + [100000], 32, "mfma_pv"),
                           ([4000] * 64, 64, "mfma_pv")):
        b = workloads.make_batch(lens, 16, sum(-(-n // 16) for n in lens) + 8, Hq, 8, 128, rng)
        big.plan(b.kv_indptr, torch.from_numpy(b.kv_indices).cuda(), b.kv_last_page_len, Hq, 8,
                 128, 16)
        per_slot = sum(lens) // big.num_slots
        assert big.planned_variant == want, (per_slot, Hq, big.planned_variant)
    r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, 8, 8, 128, 16, variant="dot2")
    assert r.planned_variant == "dot2"


@pytest.mark.parametrize("P", [1, 4, 16, 32, 64])
@pytest.mark.parametrize("G,Hkv", [(3, 2), (5, 8), (6, 4), (7, 4)])
def test_other_group_sizes(P, G, Hkv):
    """Group sizes 3, 5, 6 and 7 (Hq = 28 over Hkv = 4 is a common model
    shape), built for the kernel with both products on the matrix cores,
    which the default picks for them; unsplit and split."""
    lens = [1, 2, P, P + 1, 37, 333, 1500] if P > 1 else [1, 2, 3, 37, 333, 700]
    batch, q, cache = _small(900 + 10 * G + P, lens, P, G * Hkv, Hkv)
    _check(batch, q, cache, f"P{P}-G{G}-Hkv{Hkv}")
    _check(batch, q, cache, f"P{P}-G{G}-Hkv{Hkv}-split", min_chunk_tokens=16, variant="mfma_pv")


def test_other_group_sizes_variant_refusals():
    """Group sizes the kernels are not built for, or a kernel built only for
    1, 2, 4 and 8, are refused on the host."""
    import torch
    import paged_kv_decode_11_amd as pkd
    from paged_kv_decode_11_amd import _lib

    batch, _, _ = _small(990, [40, 3], 16, 21, 3)
    r = gu.runner()
    idx = torch.from_numpy(batch.kv_indices.astype(np.int32)).cuda()
    for variant in ("dot2", "mfma"):
        with pytest.raises(pkd.PkdError) as e:
            r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, 21, 3, 128, 16, variant=variant)
        assert e.value.code == _lib.PKD_ERR_UNSUPPORTED
    r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, 21, 3, 128, 16)
    assert r.planned_variant == "mfma_pv"
    with pytest.raises(pkd.PkdError) as e:  # group size 9
        r.plan(batch.kv_indptr, idx, batch.kv_last_page_len, 27, 3, 128, 16)
    assert e.value.code == _lib.PKD_ERR_UNSUPPORTED
