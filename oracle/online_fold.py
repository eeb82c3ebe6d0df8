"""Oracle: the online-softmax recurrence, key block by key block, float64 (test infrastructure).

Only tests, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg may
use this module. It does not import :mod:`oracle.attention` and shares no code
with the GPU library.

Per query row it carries three quantities -- the largest score seen so far m,
the running sum of exponentials l and the running weighted sum of values o --
and folds in one block of keys at a time, following fanfani.net
"FlashAttention", section "A pinch of math: making the softmax work in pieces"
(the two update equations for l and o, and the final division of o by l), and
mentria.ai "Exact attention, sped up by never writing the giant grid down",
card "The trick: keep a running max, and rebase as you go.":

    m_new = max(m, max of the block's scores)
    l     = exp(m - m_new) * l + sum_j exp(s_j - m_new)
    o     = exp(m - m_new) * o + sum_j exp(s_j - m_new) v_j
    m     = m_new
    at the end: O = o / l,  lse = m + ln(l)

With Nq queries and Nk keys the causal mask is aligned to the bottom right
(key j visible to query i iff j <= i + Nk - Nq). Restricted to a key range
[key_lo, key_hi) the same loop gives the partial result of that range; a row
that saw no key of it has O = 0 and lse = -inf.

A block in which a row sees no key leaves that row unchanged (the rescale
factor is 1 and the block adds nothing); a row that has seen no key yet has
m = -inf, and its first visible block sets the factor exp(m - m_new) to 0.
"""

from __future__ import annotations

import numpy as np

__all__ = ["fold_head", "attn_fwd_online_fold"]


def fold_head(q_h, k_h, v_h, scale, causal, block_k, rows=None, key_lo=0, key_hi=None):
    """One head by the recurrence over keys [key_lo, key_hi) (default all);
    returns (O [R, d], lse [R]) in float64."""
    q_h = np.asarray(q_h, dtype=np.float64)
    k_h = np.asarray(k_h, dtype=np.float64)
    v_h = np.asarray(v_h, dtype=np.float64)
    n_keys = k_h.shape[0]
    offset = n_keys - q_h.shape[0]
    key_hi = n_keys if key_hi is None else key_hi
    qi = np.arange(q_h.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    qr = q_h[qi]
    R = qr.shape[0]
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    o = np.zeros((R, v_h.shape[1]))
    for j0 in range(key_lo, key_hi, block_k):
        j1 = min(j0 + block_k, key_hi)
        s = scale * (qr @ k_h[j0:j1].T)
        if causal:
            keys = np.arange(j0, j1)
            s = np.where(keys[None, :] <= qi[:, None] + offset, s, -np.inf)
        m_blk = s.max(axis=1)
        m_new = np.maximum(m, m_blk)
        seen = np.isfinite(m_new)
        # Rows that have still seen no key keep m = -inf, l = 0, o = 0.
        base = np.where(seen, m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(m - base), 0.0)
        p = np.exp(s - base[:, None])  # hidden keys give exp(-inf) = 0
        l = alpha * l + p.sum(axis=1)
        o = alpha[:, None] * o + p @ v_h[j0:j1]
        m = m_new
    seen = l > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(seen[:, None], o / l[:, None], 0.0), m + np.log(l)


def attn_fwd_online_fold(q, k, v, scale, causal, block_k, rows=None):
    """All heads by the recurrence. q: [B,Hq,N,d]; k, v: [B,Hkv,N,d]."""
    B, Hq, N, _ = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    R = N if rows is None else len(rows)
    O = np.empty((B, Hq, R, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, Hq, R), dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            g = hq // G
            O[b, hq], lse[b, hq] = fold_head(q[b, hq], k[b, g], v[b, g], scale, causal, block_k, rows)
    return O, lse
