"""Appending new tokens to the paged KV cache (oracle).

The pyshine FlashInfer tour, section "The Paged KV Cache Layer": after every
generated token the engine writes the new K and V rows into their page
slots, given the page table that already covers the new positions; a helper
builds, from the page indirection, each new token's request ("batch index")
and its position in that request's sequence.  A run of new tokens that
crosses into a fresh page simply continues on the next page of the
request's page list (aicassindra "FlashInfer, in depth", section "The
block-sparse page table": token t of a request sits in page
indices[indptr[i] + t // P], slot t % P).

Readings taken where the pages are silent:
* the new tokens of request i are the last a_i tokens of its sequence, so
  their positions are L_i - a_i .. L_i - 1 with L_i the request's length
  after the append (its page table: L_i = P (n_i - 1) + r_i) and a_i from a
  CSR ``append_indptr`` over the new tokens;
* K and V rows are copied bit for bit (no conversion);
* a token whose position lies outside its request's pages is not written
  (the library reports it through its device error flag).
"""

from __future__ import annotations

import numpy as np

from . import page_table as pt


def batch_indices_positions(append_indptr, kv_indptr, kv_last_page_len, page_size: int):
    """For every new token t (in append order): its request and its position
    in that request's sequence, as int32 arrays."""
    append_indptr = np.asarray(append_indptr, dtype=np.int64)
    lengths = pt.kv_lengths(kv_indptr, kv_last_page_len, page_size)
    batch, pos = [], []
    for i in range(append_indptr.shape[0] - 1):
        a = int(append_indptr[i + 1] - append_indptr[i])
        if a > lengths[i]:
            raise ValueError("a request cannot append more tokens than it holds")
        for j in range(a):
            batch.append(i)
            pos.append(int(lengths[i]) - a + j)
    return np.asarray(batch, dtype=np.int32), np.asarray(pos, dtype=np.int32)


def append(cache_bits, k_new_bits, v_new_bits, batch_indices, positions, kv_indptr, kv_indices):
    """A copy of the cache [pages, 2, P, Hkv, D] with new token t's K and V
    rows ([Hkv, D] each) written to page indices[indptr[b] + pos // P], slot
    pos % P, where b = batch_indices[t] and pos = positions[t]."""
    out = np.array(cache_bits, copy=True)
    P = out.shape[2]
    for t in range(len(batch_indices)):
        b, pos = int(batch_indices[t]), int(positions[t])
        n = int(kv_indptr[b + 1]) - int(kv_indptr[b])
        if pos < 0 or pos // P >= n:
            continue
        page = int(kv_indices[int(kv_indptr[b]) + pos // P])
        out[page, 0, pos % P] = k_new_bits[t]
        out[page, 1, pos % P] = v_new_bits[t]
    return out


def append_quantized(cache_codes, k_new_bits, v_new_bits, batch_indices, positions, kv_indptr,
                     kv_indices, k_scale: float = 1.0, v_scale: float = 1.0):
    """``append`` into an FP8 E4M3 cache: new bf16 rows are stored as
    e4m3(x / k_scale) and e4m3(x / v_scale) (nearest, ties to even,
    saturated; oracle.fp8), fused with the write as the pyshine page
    describes for quantising appends.

    The code is a rounding decision, so it is taken in the precision the
    library computes x / scale in: float32, as x times the float32 value of
    1 / scale.  The scale itself is the float32 the C interface receives, so
    it is rounded to float32 first."""
    from . import fp8
    from .attention import bf16_to_f64

    def scaled(bits, scale):
        inv = np.float32(1.0 / float(np.float32(scale)))
        with np.errstate(over="ignore"):  # a product past float32's range is inf, then saturates
            return (bf16_to_f64(bits).astype(np.float32) * inv).astype(np.float64)

    k = fp8.f64_to_e4m3(scaled(k_new_bits, k_scale))
    v = fp8.f64_to_e4m3(scaled(v_new_bits, v_scale))
    return append(cache_codes, k, v, batch_indices, positions, kv_indptr, kv_indices)
