"""Seeded synthetic batches for paged GQA decode.

Everything here is input generation: request lengths, where each request's
pages sit in the pool, and N(0, 1) values rounded to bf16 for q, K and V (or
uniformly drawn FP8 E4M3 codes for an FP8 cache).
The page-table layout is the one the FlashInfer pages describe (aicassindra
"FlashInfer, in depth", section "The block-sparse page table"): a CSR triple
(kv_indptr, kv_indices, kv_last_page_len) over a pool of fixed-size pages, and
a per-layer cache of shape [pages, 2, page_size, num_kv_heads, head_dim].

Draw order for one batch, from numpy's PCG64 seeded with the workload seed:
lengths, then page placement, then q, then K/V.  Large pools are filled on
the device with torch's seeded generator instead (see ``device_cache``).
"""

from __future__ import annotations

import dataclasses
from typing import Callable, Dict, List, Optional

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)


# ---------------------------------------------------------------------------
# bf16 values
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return
    the 16-bit patterns.  NaN inputs become the canonical quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    return np.where(np.isnan(x), BF16_QNAN, rounded).astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0, 1) float32 draws rounded to bf16, as uint16 bit patterns."""
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


# ---------------------------------------------------------------------------
# page placement (the serving engine's allocator, not the attention method)
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class PagedBatch:
    """One decode batch: page table plus head configuration."""

    page_size: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    num_pages: int               # pool size (pages in each layer's cache)
    kv_lens: np.ndarray          # int64 [B]
    kv_indptr: np.ndarray        # int32 [B+1]
    kv_indices: np.ndarray       # int32 [nnz]
    kv_last_page_len: np.ndarray  # int32 [B]

    @property
    def batch(self) -> int:
        return int(self.kv_lens.shape[0])

    @property
    def nnz(self) -> int:
        return int(self.kv_indices.shape[0])

    @property
    def total_tokens(self) -> int:
        return int(self.kv_lens.sum())

    def kv_bytes_per_token(self) -> int:
        return 2 * self.num_kv_heads * self.head_dim * 2

    def cache_shape(self):
        return (self.num_pages, 2, self.page_size, self.num_kv_heads, self.head_dim)


def allocate_pages(kv_lens, page_size: int, page_ids) -> tuple:
    """Hand each request, in order, as many pages from ``page_ids`` as its
    length needs.  Returns (kv_indptr, kv_indices, kv_last_page_len)."""
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    if np.any(kv_lens < 1):
        raise ValueError("every request needs at least one token")
    pages_per_req = (kv_lens + (page_size - 1)) // page_size
    fill_of_last = ((kv_lens - 1) % page_size) + 1
    indptr = np.zeros(kv_lens.shape[0] + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(pages_per_req)
    page_ids = np.asarray(page_ids, dtype=np.int64)
    if page_ids.shape[0] < indptr[-1]:
        raise ValueError("not enough pages in the pool")
    return (indptr.astype(np.int32), page_ids[: indptr[-1]].astype(np.int32),
            fill_of_last.astype(np.int32))


def make_batch(kv_lens, page_size: int, num_pages: int, num_qo_heads: int,
               num_kv_heads: int, head_dim: int,
               rng: Optional[np.random.Generator], scatter: bool = True,
               page_ids=None) -> PagedBatch:
    """Place a batch's pages in a pool of ``num_pages``: a random permutation
    of the pool when ``scatter`` (drawn from ``rng``), else pages 0, 1, 2...
    ``page_ids`` overrides both."""
    if page_ids is None:
        page_ids = rng.permutation(num_pages) if scatter else np.arange(num_pages)
    indptr, indices, last = allocate_pages(kv_lens, page_size, page_ids)
    return PagedBatch(page_size, num_qo_heads, num_kv_heads, head_dim, num_pages,
                      np.asarray(kv_lens, dtype=np.int64), indptr, indices, last)


def host_query(batch: PagedBatch, rng: np.random.Generator) -> np.ndarray:
    """q as bf16 bits, [B, Hq, D]."""
    return normal_bf16(rng, (batch.batch, batch.num_qo_heads, batch.head_dim))


def host_cache(batch: PagedBatch, rng: np.random.Generator, poison: bool = False,
               fill_pages: str = "used") -> np.ndarray:
    """One layer's cache as bf16 bits, [pages, 2, P, Hkv, D].

    The pages the batch uses get N(0, 1) values (in ascending page order);
    other pages hold zeros, or quiet NaNs when ``poison``.  With ``poison`` the
    unfilled slots of each request's last page are NaN as well, so any read
    past kv_last_page_len shows up in the output.  ``fill_pages="all"`` fills
    the whole pool with values instead."""
    shape = batch.cache_shape()
    cache = np.full(shape, BF16_QNAN if poison else np.uint16(0), dtype=np.uint16)
    if fill_pages == "all":
        cache[...] = normal_bf16(rng, shape)
    else:
        used = np.unique(batch.kv_indices)
        cache[used] = normal_bf16(rng, (used.shape[0],) + shape[1:])
    if poison:
        last_pages = batch.kv_indices[batch.kv_indptr[1:] - 1]
        for page, fill in zip(last_pages, batch.kv_last_page_len):
            cache[page, :, int(fill):] = BF16_QNAN
    return cache


def device_cache(batch: PagedBatch, seed: int, device, chunk_pages: int = 4096,
                 used_only: bool = False):
    """One layer's cache on ``device`` as a torch bfloat16 tensor.

    The pool is filled with N(0, 1) float32 draws from torch's generator
    seeded with ``seed`` and rounded to bf16 (torch rounds to nearest even):
    every page, or with ``used_only`` only the pages the batch uses, in
    ascending page order (the others hold zeros).  Used for pools too large
    to fill with numpy."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    if used_only:
        cache = torch.zeros(batch.cache_shape(), dtype=torch.bfloat16, device=device)
        pages = torch.from_numpy(np.unique(batch.kv_indices).astype(np.int64)).to(device)
    else:
        cache = torch.empty(batch.cache_shape(), dtype=torch.bfloat16, device=device)
        pages = None
    flat = cache.view(batch.num_pages, -1)
    total = batch.num_pages if pages is None else int(pages.shape[0])
    for p0 in range(0, total, chunk_pages):
        p1 = min(total, p0 + chunk_pages)
        vals = torch.randn((p1 - p0, flat.shape[1]), generator=gen, dtype=torch.float32,
                           device=device).to(torch.bfloat16)
        if pages is None:
            flat[p0:p1].copy_(vals)
        else:
            flat.index_copy_(0, pages[p0:p1], vals)
    return cache


E4M3_NAN = np.uint8(0x7F)


def e4m3_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniformly drawn FP8 E4M3 codes (uint8) other than the two NaN codes
    0x7F and 0xFF, which are replaced by the largest finite codes of their
    sign: every exponent field equally likely, so values span 2^-9 .. 448
    before the tensor's scale."""
    c = rng.integers(0, 256, size=shape, dtype=np.uint16).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c - 1, c).astype(np.uint8)


def host_cache_e4m3(batch: PagedBatch, rng: np.random.Generator, poison: bool = False) -> np.ndarray:
    """One layer's FP8 E4M3 cache as codes, [pages, 2, P, Hkv, D] uint8: the
    used pages get ``e4m3_codes`` (in ascending page order), the others zeros,
    or NaN codes when ``poison`` -- which also fills the unused slots of each
    request's last page with NaN codes."""
    shape = batch.cache_shape()
    cache = np.full(shape, E4M3_NAN if poison else np.uint8(0), dtype=np.uint8)
    used = np.unique(batch.kv_indices)
    cache[used] = e4m3_codes(rng, (used.shape[0],) + shape[1:])
    if poison:
        last_pages = batch.kv_indices[batch.kv_indptr[1:] - 1]
        for page, fill in zip(last_pages, batch.kv_last_page_len):
            cache[page, :, int(fill):] = E4M3_NAN
    return cache


def device_cache_e4m3(batch: PagedBatch, seed: int, device, chunk_pages: int = 8192):
    """One layer's FP8 E4M3 cache on ``device`` as a torch float8_e4m3fn
    tensor, every page filled like ``e4m3_codes`` from torch's generator
    seeded with ``seed`` (for pools too large to fill with numpy)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    cache = torch.empty(batch.cache_shape(), dtype=torch.uint8, device=device)
    flat = cache.view(batch.num_pages, -1)
    for p0 in range(0, batch.num_pages, chunk_pages):
        p1 = min(batch.num_pages, p0 + chunk_pages)
        c = torch.randint(0, 256, (p1 - p0, flat.shape[1]), generator=gen, dtype=torch.int32,
                          device=device)
        c = torch.where((c & 0x7F) == 0x7F, c - 1, c)
        flat[p0:p1].copy_(c.to(torch.uint8))
    return cache.view(torch.float8_e4m3fn)


def device_query(batch: PagedBatch, seed: int, device):
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    q = torch.randn((batch.batch, batch.num_qo_heads, batch.head_dim), generator=gen,
                    dtype=torch.float32, device=device)
    return q.to(torch.bfloat16)


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    name: str
    description: str
    seed: int
    page_size: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    num_layers: int
    pool_pages: int
    build: Callable[["WorkloadSpec", np.random.Generator], Dict[str, PagedBatch]]


def _single(spec: WorkloadSpec, kv_lens, rng, scatter=True, page_ids=None) -> PagedBatch:
    return make_batch(kv_lens, spec.page_size, spec.pool_pages, spec.num_qo_heads,
                      spec.num_kv_heads, spec.head_dim, rng, scatter=scatter,
                      page_ids=page_ids)


def _build_tiny(spec, rng):
    return {"main": _single(spec, [37, 16, 5], rng)}


def _build_llama8b(spec, rng):
    lens = rng.integers(3000, 5001, size=64)
    return {"main": _single(spec, lens, rng)}


def _build_skewed(spec, rng):
    lens = np.array([512] * 63 + [100_000], dtype=np.int64)
    return {"main": _single(spec, lens, rng)}


def _build_shared_prefix(spec, rng):
    """32 requests over one 8192-token prefix (512 shared pages) plus their
    own suffix of U{64..1024} tokens.  Three page tables over one pool:
    ``main`` (each row = prefix pages + own suffix pages), ``prefix`` (every
    row = the 512 prefix pages) and ``suffix`` (own suffix pages only)."""
    return _shared_prefix(spec, rng, 32, 8192, 64, 1024)


def _build_shared_prefix_b16(spec, rng):
    """16 requests over one 8192-token prefix, each with its own 128-token
    suffix (the batch-16, prefix-8192 row of the pinghaoyang page's
    composable-format table; the page states no head shapes)."""
    return _shared_prefix(spec, rng, 16, 8192, 128, 128)


def _build_shared_prefix_b64(spec, rng):
    """The same with 64 requests (that table's batch-64 row)."""
    return _shared_prefix(spec, rng, 64, 8192, 128, 128)


def _shared_prefix(spec, rng, n_req, prefix_len, suffix_lo, suffix_hi):
    """n_req requests over one prefix_len-token prefix plus their own suffix
    of U{suffix_lo..suffix_hi} tokens, in the three page tables described
    above."""
    P = spec.page_size
    suffix = rng.integers(suffix_lo, suffix_hi + 1, size=n_req)
    perm = rng.permutation(spec.pool_pages)
    n_prefix_pages = prefix_len // P
    prefix_pages = perm[:n_prefix_pages]
    suffix_pages = perm[n_prefix_pages:]
    s_indptr, s_indices, s_last = allocate_pages(suffix, P, suffix_pages)
    rows = []
    for i in range(n_req):
        rows.append(np.concatenate([prefix_pages, s_indices[s_indptr[i]:s_indptr[i + 1]]]))
    main_lens = prefix_len + suffix
    main = PagedBatch(P, spec.num_qo_heads, spec.num_kv_heads, spec.head_dim, spec.pool_pages,
                      main_lens.astype(np.int64),
                      np.concatenate([[0], np.cumsum([r.shape[0] for r in rows])]).astype(np.int32),
                      np.concatenate(rows).astype(np.int32), s_last.astype(np.int32))
    prefix = PagedBatch(P, spec.num_qo_heads, spec.num_kv_heads, spec.head_dim, spec.pool_pages,
                        np.full(n_req, prefix_len, dtype=np.int64),
                        (np.arange(n_req + 1) * n_prefix_pages).astype(np.int32),
                        np.tile(prefix_pages, n_req).astype(np.int32),
                        np.full(n_req, P, dtype=np.int32))
    suffix_batch = PagedBatch(P, spec.num_qo_heads, spec.num_kv_heads, spec.head_dim,
                              spec.pool_pages, suffix.astype(np.int64), s_indptr, s_indices, s_last)
    return {"main": main, "prefix": prefix, "suffix": suffix_batch}


def _build_token_sparse(spec, rng):
    """page_size 1: 32 requests, each over 2048 distinct token slots drawn
    uniformly from a 65,536-slot pool and sorted ascending."""
    rows = [np.sort(rng.choice(spec.pool_pages, size=2048, replace=False)) for _ in range(32)]
    lens = np.full(32, 2048, dtype=np.int64)
    indptr = (np.arange(33) * 2048).astype(np.int32)
    return {"main": PagedBatch(1, spec.num_qo_heads, spec.num_kv_heads, spec.head_dim,
                               spec.pool_pages, lens, indptr,
                               np.concatenate(rows).astype(np.int32),
                               np.ones(32, dtype=np.int32))}


def _build_wide_gqa(spec, rng):
    """256 requests, lengths log-normal with median 2048 (sigma 1), clipped to
    [16, 32768]."""
    lens = np.clip(np.round(np.exp(rng.normal(np.log(2048.0), 1.0, size=256))), 16, 32768)
    return {"main": _single(spec, lens.astype(np.int64), rng)}


WORKLOADS: Dict[str, WorkloadSpec] = {
    s.name: s for s in [
        WorkloadSpec("tiny", "3 requests, KV lengths [37,16,5], 64-page pool", 0,
                     16, 32, 8, 128, 1, 64, _build_tiny),
        WorkloadSpec("llama8b_step", "Llama-3-8B-like step: 32 layers, batch 64, KV U[3000,5000]",
                     1, 16, 32, 8, 128, 32, 1 << 15, _build_llama8b),
        WorkloadSpec("skewed", "63 x 512 tokens + 1 x 100,000 tokens", 2,
                     16, 32, 8, 128, 1, 1 << 14, _build_skewed),
        WorkloadSpec("shared_prefix", "32 requests: 8192-token shared prefix + U[64,1024] suffix",
                     3, 16, 32, 8, 128, 1, 1 << 15, _build_shared_prefix),
        WorkloadSpec("token_sparse", "page_size 1: 32 x 2048 random token slots of 65,536", 4,
                     1, 32, 8, 128, 1, 1 << 16, _build_token_sparse),
        WorkloadSpec("wide_gqa", "batch 256, log-normal KV (median 2048), Hq 64 / Hkv 8", 5,
                     16, 64, 8, 128, 1, 1 << 20, _build_wide_gqa),
        WorkloadSpec("shared_prefix_b16", "16 requests: 8192-token shared prefix + 128 suffix", 6,
                     16, 32, 8, 128, 1, 1 << 15, _build_shared_prefix_b16),
        WorkloadSpec("shared_prefix_b64", "64 requests: 8192-token shared prefix + 128 suffix", 7,
                     16, 32, 8, 128, 1, 1 << 15, _build_shared_prefix_b64),
    ]
}


def workload(name: str, seed: Optional[int] = None) -> tuple:
    """(spec, rng, batches) for a named workload; the rng continues after the
    page placement, ready to draw q and then K/V."""
    spec = WORKLOADS[name]
    rng = np.random.Generator(np.random.PCG64(spec.seed if seed is None else seed))
    batches = spec.build(spec, rng)
    return spec, rng, batches


def random_batch(rng: np.random.Generator, batch: int, max_len: int, page_size: int,
                 num_qo_heads: int, num_kv_heads: int, head_dim: int,
                 num_pages: Optional[int] = None, min_len: int = 1) -> PagedBatch:
    """A small random batch for tests: lengths U{min_len..max_len}, pages
    scattered over a pool with some spare pages."""
    lens = rng.integers(min_len, max_len + 1, size=batch)
    need = int(((lens + page_size - 1) // page_size).sum())
    pool = num_pages if num_pages is not None else need + 7
    return make_batch(lens, page_size, pool, num_qo_heads, num_kv_heads, head_dim, rng)


def edge_lengths(page_size: int) -> List[int]:
    """Lengths around page boundaries: 1, P-1, P, P+1, 2P, 2P+1."""
    P = page_size
    return sorted({1, max(1, P - 1), P, P + 1, 2 * P, 2 * P + 1})
