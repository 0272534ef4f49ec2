"""Exact merge of attention states (oracle, float64).

Follows the pinghaoyang page, section "在线 Softmax 为什么允许任意切块" (why
online softmax allows any split): for states (O_I, L_I) and (O_J, L_J) over
disjoint key sets, M = max(L_I, L_J), Z = exp(L_I - M) + exp(L_J - M), and the
state over the union is L = M + log Z, O = (exp(L_I - M) O_I + exp(L_J - M) O_J) / Z.
The aicassindra page gives the same combine in its section "Load balancing
with split-KV" with natural-log LSE.

Reading for a case the pages do not cover: the empty key set has state
(O = 0, L = -inf), which is the identity of the merge; merging only empty
states gives (0, -inf).
"""

from __future__ import annotations

import math

import numpy as np


def merge_two(o_a, lse_a, o_b, lse_b):
    """Merge two states of one query row: o_* [D], lse_* scalars."""
    if lse_a == -math.inf and lse_b == -math.inf:
        return np.zeros_like(np.asarray(o_a, dtype=np.float64)), -math.inf
    M = max(lse_a, lse_b)
    wa = math.exp(lse_a - M)
    wb = math.exp(lse_b - M)
    Z = wa + wb
    o = (wa * np.asarray(o_a, dtype=np.float64) + wb * np.asarray(o_b, dtype=np.float64)) / Z
    return o, M + math.log(Z)


def merge_many(states):
    """Fold a sequence of (o, lse) states left to right."""
    it = iter(states)
    o, lse = next(it)
    o = np.asarray(o, dtype=np.float64)
    for o2, lse2 in it:
        o, lse = merge_two(o, lse, o2, lse2)
    return o, lse


def merge_rows(o_a, lse_a, o_b, lse_b):
    """Row-wise merge of batched states: o_* [..., D], lse_* [...]."""
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    out_o = np.empty(np.broadcast_shapes(o_a.shape, o_b.shape))
    out_l = np.empty(np.broadcast_shapes(lse_a.shape, lse_b.shape))
    for idx in np.ndindex(out_l.shape):
        out_o[idx], out_l[idx] = merge_two(o_a[idx], float(lse_a[idx]), o_b[idx], float(lse_b[idx]))
    return out_o, out_l
