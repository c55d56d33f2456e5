"""Brute-force dense attention in numpy fp64 (no pages, no gather).

TEST INFRASTRUCTURE ONLY (see the package docstring).  This is the second,
independent statement of the attention the pages describe, used to pin the C
oracle: keys and values arrive as plain per-sequence arrays, the causal rule is
a dense boolean mask, kv heads are widened with ``numpy.repeat`` and the
softmax / log-sum-exp come from scipy.  Readings are the same as the C oracle's
(scale 1/sqrt(D), bottom-right causal alignment, contiguous GQA groups, empty
row -> out 0 and lse -inf), written here in matrix form.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import logsumexp


def attention_one_sequence(q, k, v, *, causal=False, scale=None):
    """q [n_q, Hq, D], k/v [n_k, Hkv, D] (float64).  Returns out, lse."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, hq, d = q.shape
    n_k, hkv, _ = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    group = hq // hkv
    k_wide = np.repeat(k, group, axis=1)          # [n_k, Hq, D]
    v_wide = np.repeat(v, group, axis=1)
    scores = np.einsum("ihd,jhd->hij", q, k_wide) * scale   # [Hq, n_q, n_k]
    allowed = np.ones((n_q, n_k), dtype=bool)
    if causal:
        rows = np.arange(n_q)[:, None]
        cols = np.arange(n_k)[None, :]
        allowed = cols <= (n_k - n_q) + rows      # token i sits at position n_k - n_q + i
    scores = np.where(allowed[None], scores, -np.inf)
    empty = ~allowed.any(axis=1)                  # [n_q]
    lse = logsumexp(scores, axis=-1)              # -inf on empty rows
    with np.errstate(invalid="ignore"):
        weights = np.exp(scores - lse[..., None])
    weights = np.where(empty[None, :, None], 0.0, weights)
    out = np.einsum("hij,jhd->ihd", weights, v_wide)
    lse = np.where(empty[None, :], -np.inf, lse)
    return out, lse.transpose(1, 0)               # out [n_q, Hq, D], lse [n_q, Hq]


def attention_varlen(q, k_seqs, v_seqs, cu_seqlens_q, *, causal=False, scale=None):
    """Per-sequence dense attention over a packed [total_q, Hq, D] query."""
    q = np.asarray(q, dtype=np.float64)
    total_q, hq, d = q.shape
    out = np.zeros((total_q, hq, d))
    lse = np.zeros((total_q, hq))
    for b in range(len(cu_seqlens_q) - 1):
        s, e = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        if e <= s:
            continue
        o, l = attention_one_sequence(q[s:e], k_seqs[b], v_seqs[b], causal=causal, scale=scale)
        out[s:e] = o
        lse[s:e] = l
    return out, lse
