"""Paged GQA decode attention (oracle, float64).

The definition is the one on the pinghaoyang page, section "从推理形状出发"
(starting from the inference shapes): S = Q K^T / sqrt(d), P = softmax(S),
O = P V, here with one query row per request (decode, l_q = 1).  The
attention state (O, L) over a key set I is the one in the section
"在线 Softmax 为什么允许任意切块" (why online softmax allows any split):
L_I = log sum_{i in I} exp(s_i) and O_I = sum_{i in I} exp(s_i - L_I) v_i, where
s_i is the scaled logit, so that L is the natural-log log-sum-exp of the
logits softmax sees.  Keys and values of request i are gathered through the
CSR page table (aicassindra "FlashInfer, in depth", section "The
block-sparse page table") from a cache laid out [pages, 2, P, Hkv, D] (NHD,
K at index 0, V at index 1).

Readings taken where the pages are silent (listed again in the design notes):
* the scale 1/sqrt(D) multiplies the logits, and ``lse`` is taken over the
  scaled logits, in natural log;
* query head h reads KV head h // g with g = Hq / Hkv (contiguous groups);
* bf16 inputs are widened exactly (bits << 16 as float32, then float64).
"""

from __future__ import annotations

import math

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def gather_request(cache_bits, kv_indptr, kv_indices, kv_last_page_len, i: int):
    """K and V of request ``i`` in token order, each [l_i, Hkv, D] (bf16 bits).

    Token t of the request sits in page kv_indices[indptr[i] + t // P] at
    slot t % P; only the first last_page_len[i] slots of the final page
    belong to the request."""
    P = cache_bits.shape[2]
    b, e = int(kv_indptr[i]), int(kv_indptr[i + 1])
    pages = np.asarray(kv_indices[b:e], dtype=np.int64)
    n = pages.shape[0]
    length = P * (n - 1) + int(kv_last_page_len[i])
    blocks = cache_bits[pages]                    # [n, 2, P, Hkv, D]
    k = blocks[:, 0].reshape((n * P,) + blocks.shape[3:])[:length]
    v = blocks[:, 1].reshape((n * P,) + blocks.shape[3:])[:length]
    return k, v


def attention_state(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float):
    """(o, lse) of one query row q [D] over keys K [n, D] and values V [n, D].

    An empty key set has the neutral state (o = 0, lse = -inf)."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[-1]), -math.inf
    s = sm_scale * (K @ q)
    m = float(s.max())
    lse = m + math.log(float(np.exp(s - m).sum()))
    o = np.exp(s - lse) @ V
    return o, lse


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def decode(q_bits, cache_bits, kv_indptr, kv_indices, kv_last_page_len, num_kv_heads: int,
           sm_scale=None, requests=None):
    """o [B, Hq, D] and lse [B, Hq] in float64 for every request (or only the
    listed ``requests``; other rows are left NaN)."""
    q_bits = np.asarray(q_bits)
    B, Hq, D = q_bits.shape
    if Hq % num_kv_heads:
        raise ValueError("num_qo_heads must be a multiple of num_kv_heads")
    g = Hq // num_kv_heads
    scale = default_scale(D) if sm_scale is None else float(sm_scale)
    o = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    for i in (range(B) if requests is None else requests):
        k_bits, v_bits = gather_request(cache_bits, kv_indptr, kv_indices, kv_last_page_len, i)
        K, V = bf16_to_f64(k_bits), bf16_to_f64(v_bits)
        q = bf16_to_f64(q_bits[i])
        for h in range(Hq):
            kh = h // g
            o[i, h], lse[i, h] = attention_state(q[h], K[:, kh], V[:, kh], scale)
    return o, lse


def request_state(q_bits, cache_bits, kv_indptr, kv_indices, kv_last_page_len,
                  num_kv_heads: int, i: int, t0: int, t1: int, sm_scale=None):
    """Attention states of request i over its tokens [t0, t1), for every query
    head: (o [Hq, D], lse [Hq])."""
    Hq, D = q_bits.shape[1], q_bits.shape[2]
    g = Hq // num_kv_heads
    scale = default_scale(D) if sm_scale is None else float(sm_scale)
    k_bits, v_bits = gather_request(cache_bits, kv_indptr, kv_indices, kv_last_page_len, i)
    K, V = bf16_to_f64(k_bits[t0:t1]), bf16_to_f64(v_bits[t0:t1])
    q = bf16_to_f64(q_bits[i])
    o = np.zeros((Hq, D))
    lse = np.zeros(Hq)
    for h in range(Hq):
        o[h], lse[h] = attention_state(q[h], K[:, h // g], V[:, h // g], scale)
    return o, lse


def decode_bruteforce(q_bits, cache_bits, kv_indptr, kv_indices, kv_last_page_len,
                      num_kv_heads: int, sm_scale=None):
    """The same quantity with scalar Python loops and exactly rounded sums
    (math.fsum), one token at a time.  For tiny inputs only."""
    B, Hq, D = q_bits.shape
    P = cache_bits.shape[2]
    g = Hq // num_kv_heads
    scale = default_scale(D) if sm_scale is None else float(sm_scale)

    def val(bits):
        return float(np.uint32(int(bits) << 16).view(np.float32))

    o = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    lse = [[0.0] * Hq for _ in range(B)]
    for i in range(B):
        n_pages = int(kv_indptr[i + 1]) - int(kv_indptr[i])
        length = (n_pages - 1) * P + int(kv_last_page_len[i])
        for h in range(Hq):
            kh = h // g
            qv = [val(q_bits[i, h, d]) for d in range(D)]
            logits, rows = [], []
            for t in range(length):
                page = int(kv_indices[int(kv_indptr[i]) + t // P])
                slot = t % P
                kv = [val(cache_bits[page, 0, slot, kh, d]) for d in range(D)]
                vv = [val(cache_bits[page, 1, slot, kh, d]) for d in range(D)]
                logits.append(scale * math.fsum(a * b for a, b in zip(qv, kv)))
                rows.append(vv)
            top = max(logits)
            weights = [math.exp(s - top) for s in logits]
            total = math.fsum(weights)
            lse[i][h] = top + math.log(total)
            for d in range(D):
                o[i][h][d] = math.fsum(w * r[d] for w, r in zip(weights, rows)) / total
    return np.array(o), np.array(lse)


def decode_fp8(q_bits, cache_codes, kv_indptr, kv_indices, kv_last_page_len, num_kv_heads: int,
               sm_scale=None, k_scale: float = 1.0, v_scale: float = 1.0, requests=None):
    """``decode`` over an FP8 E4M3 cache ([pages, 2, P, Hkv, D] uint8 codes)
    with per-tensor scales: the keys are e4m3(code) * k_scale, the values
    e4m3(code) * v_scale (the dequantising key and value transforms; see
    oracle.fp8 for the format and the scale contract)."""
    from . import fp8

    q_bits = np.asarray(q_bits)
    B, Hq, D = q_bits.shape
    g = Hq // num_kv_heads
    scale = default_scale(D) if sm_scale is None else float(sm_scale)
    o = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    for i in (range(B) if requests is None else requests):
        k_codes, v_codes = gather_request(cache_codes, kv_indptr, kv_indices, kv_last_page_len, i)
        K = fp8.e4m3_to_f64(k_codes) * float(k_scale)
        V = fp8.e4m3_to_f64(v_codes) * float(v_scale)
        q = bf16_to_f64(q_bits[i])
        for h in range(Hq):
            kh = h // g
            o[i, h], lse[i, h] = attention_state(q[h], K[:, kh], V[:, kh], scale)
    return o, lse
