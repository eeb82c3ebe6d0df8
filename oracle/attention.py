"""Oracle: exact softmax attention by its definition, in float64 (test infrastructure).

Only tests, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg may
use this module. It shares no code with the GPU library.

The forward is the plain definition, with the whole score matrix of one
(batch, head) materialised:

1. scores ``S = scale * Q K^T`` -- mentria.ai "Exact attention, sped up by never
   writing the giant grid down", card "So don't load it all. Work one block at a
   time." (the score equation, with scale = 1/sqrt(d) there);
2. the mask step between scores and softmax -- fanfani.net "FlashAttention",
   section "The bottleneck was never the arithmetic" (standard pipeline: scores,
   mask, softmax, multiply by V). The mask is causal: key j is visible to query
   i iff j <= i; hidden scores are -inf;
3. the max-subtracted softmax of each row -- mentria.ai, card "But softmax
   needs the whole row at once." (the softmax equation with m = max_j x_j);
4. ``O = P V`` -- fanfani.net, same section (multiply by the values);
5. the saved per-query statistic ``lse = m + ln(l)`` (l = sum of exponentials),
   which is the pair (m, l) of fanfani.net section "The backward pass, and where
   the memory saving comes from" folded into one number: P_ij = exp(S_ij - lse_i).

Rectangular problems (Nq queries, Nk keys) align the causal mask to the
bottom right: query i sees key j iff j <= i + (Nk - Nq), so the last query sees
every key (the pages only fix the square case; this is the reading that keeps
the last query of a prefix-extended problem identical). A query row that sees
no key (possible only when Nq > Nk) has an empty softmax: its output is 0 and
its lse is -inf.

Partial results over disjoint key ranges (split keys) combine by the same
rescale step the recurrence applies to each new block (fanfani.net section "A
pinch of math: making the softmax work in pieces"): each partial (O_s, lse_s)
enters like one block whose maximum is lse_s and whose exponential sum is 1.

Variable-length batches pack B sequences along the token axis, q [Hq, Tq, d]
and k, v [Hkv, Tk, d], sequence b owning query rows cu_q[b] .. cu_q[b+1]-1 and
key rows cu_k[b] .. cu_k[b+1]-1; each sequence is an independent problem.

The backward is derived from that definition by the chain rule (the pages only
say the score blocks are recomputed from the saved statistics), for the same
problems as the forward (square, rectangular with the bottom-right mask,
variable-length batches):
``dV = P^T dO``, ``dP = dO V^T``, ``D_i = sum_j P_ij dP_ij``,
``dS = P * (dP - D)``, ``dQ = scale dS K``, ``dK = scale dS^T Q``. With grouped
K/V heads (GQA) query head hq reads K/V head ``hq // (Hq / Hkv)`` and dK, dV of
a K/V head sum over its query heads.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "kv_head",
    "attn_probs",
    "attn_fwd_head",
    "attn_fwd_materialised",
    "attn_bwd_group",
    "attn_bwd_analytic",
    "merge_partials",
    "attn_fwd_varlen",
    "attn_bwd_varlen",
]


def kv_head(hq: int, Hq: int, Hkv: int) -> int:
    """K/V head read by query head ``hq``: contiguous groups of Hq/Hkv query heads."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return hq // (Hq // Hkv)


def _scores(q_h: np.ndarray, k_h: np.ndarray, scale: float) -> np.ndarray:
    """S_ij = scale * <q_i, k_j>; rows are queries, columns keys."""
    return scale * (q_h @ k_h.T)


def _visible(rows: np.ndarray, n_keys: int, causal: bool, offset: int = 0) -> np.ndarray:
    """Boolean [len(rows), n_keys]: key j visible to query rows[r] (causal: j <= row + offset)."""
    if not causal:
        return np.ones((rows.shape[0], n_keys), dtype=bool)
    return np.arange(n_keys)[None, :] <= rows[:, None] + offset


def _softmax_rows(S: np.ndarray):
    """Max-subtracted softmax of each row; returns (P, m, l). A row with no
    finite score (no visible key) gets P = 0, m = -inf, l = 0."""
    m = S.max(axis=1)
    seen = np.isfinite(m)
    E = np.exp(S - np.where(seen, m, 0.0)[:, None])
    l = E.sum(axis=1)
    P = np.where(seen[:, None], E / np.where(seen, l, 1.0)[:, None], 0.0)
    return P, m, l


def _rows(rows, n: int) -> np.ndarray:
    return np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)


def attn_probs(q_h, k_h, scale, causal, rows=None) -> np.ndarray:
    """Attention weights P of one head (rows: query indices, default all)."""
    q_h = np.asarray(q_h, dtype=np.float64)
    k_h = np.asarray(k_h, dtype=np.float64)
    r = _rows(rows, q_h.shape[0])
    S = _scores(q_h[r], k_h, scale)
    S = np.where(_visible(r, k_h.shape[0], causal, k_h.shape[0] - q_h.shape[0]), S, -np.inf)
    P, _, _ = _softmax_rows(S)
    return P


def attn_fwd_head(q_h, k_h, v_h, scale, causal, rows=None):
    """Forward of one head: returns (O [R, d], lse [R]) for query rows ``rows``."""
    q_h = np.asarray(q_h, dtype=np.float64)
    k_h = np.asarray(k_h, dtype=np.float64)
    v_h = np.asarray(v_h, dtype=np.float64)
    r = _rows(rows, q_h.shape[0])
    S = _scores(q_h[r], k_h, scale)
    S = np.where(_visible(r, k_h.shape[0], causal, k_h.shape[0] - q_h.shape[0]), S, -np.inf)
    P, m, l = _softmax_rows(S)
    with np.errstate(divide="ignore"):
        return P @ v_h, m + np.log(l)


def attn_fwd_materialised(q, k, v, scale, causal, rows=None):
    """Forward over all heads.

    q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d]. Returns O [B, Hq, R, d] and
    lse [B, Hq, R] (float64) for query rows ``rows`` (default all Nq).
    """
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    R = N if rows is None else len(rows)
    O = np.empty((B, Hq, R, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, Hq, R), dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            g = kv_head(hq, Hq, Hkv)
            O[b, hq], lse[b, hq] = attn_fwd_head(q[b, hq], k[b, g], v[b, g], scale, causal, rows)
    return O, lse


def attn_bwd_group(q_g, k_h, v_h, do_g, scale, causal):
    """Backward of one K/V head and the G query heads that read it.

    q_g, do_g: [G, Nq, d]; k_h, v_h: [Nk, d]. Returns dq [G, Nq, d], dk [Nk, d],
    dv [Nk, d] (float64), the gradients of sum(dO * O). With Nq != Nk the
    causal mask is the forward's, aligned to the bottom right (query i sees
    key j iff j <= i + Nk - Nq). A query row that sees no key has O = 0 for
    any q, k, v: its dq is 0 and it adds nothing to dk and dv (its P row is
    0, so is its dS row).
    """
    q_g = np.asarray(q_g, dtype=np.float64)
    do_g = np.asarray(do_g, dtype=np.float64)
    k_h = np.asarray(k_h, dtype=np.float64)
    v_h = np.asarray(v_h, dtype=np.float64)
    G, Nq, _ = q_g.shape
    Nk = k_h.shape[0]
    dq = np.empty_like(q_g)
    dk = np.zeros_like(k_h)
    dv = np.zeros_like(v_h)
    vis = _visible(np.arange(Nq), Nk, causal, Nk - Nq)
    for j in range(G):
        S = np.where(vis, _scores(q_g[j], k_h, scale), -np.inf)
        P, _, _ = _softmax_rows(S)
        dv += P.T @ do_g[j]
        dP = do_g[j] @ v_h.T
        D = (P * dP).sum(axis=1)
        dS = P * (dP - D[:, None])
        dq[j] = scale * (dS @ k_h)
        dk += scale * (dS.T @ q_g[j])
    return dq, dk, dv


def attn_bwd_analytic(q, k, v, do, scale, causal):
    """Backward over all heads: q, do [B,Hq,Nq,d], k, v [B,Hkv,Nk,d]; returns
    dq [B,Hq,Nq,d], dk, dv [B,Hkv,Nk,d] (float64)."""
    B, Hq, Nq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(k.shape, dtype=np.float64)
    dv = np.empty(v.shape, dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            dq[b, hs], dk[b, g], dv[b, g] = attn_bwd_group(q[b, hs], k[b, g], v[b, g], do[b, hs], scale, causal)
    return dq, dk, dv


def merge_partials(o_parts, lse_parts):
    """Combine partial results over disjoint key ranges.

    o_parts: [S, R, d], each normalised by its own exponential sum;
    lse_parts: [S, R] natural-log statistics (-inf for a range a row saw no key
    of). Folds the S partials in order with the recurrence's rescale step:
    m_new = max(m, lse_s); l = exp(m - m_new) l + exp(lse_s - m_new);
    o = exp(m - m_new) o + exp(lse_s - m_new) O_s; then O = o / l and
    lse = m + ln l. Rows with no key in any range get O = 0, lse = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    S, R = lse_parts.shape
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    o = np.zeros(o_parts.shape[1:])
    for s_ in range(S):
        m_new = np.maximum(m, lse_parts[s_])
        seen = np.isfinite(m_new)
        base = np.where(seen, m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(m - base), 0.0)
        w = np.where(np.isfinite(lse_parts[s_]), np.exp(lse_parts[s_] - base), 0.0)
        l = alpha * l + w
        o = alpha[:, None] * o + w[:, None] * o_parts[s_]
        m = m_new
    seen = l > 0
    with np.errstate(divide="ignore"):
        return np.where(seen[:, None], o / np.where(seen, l, 1.0)[:, None], 0.0), m + np.log(l)


def attn_fwd_varlen(q, k, v, cu_q, cu_k, scale, causal):
    """Variable-length batch: q [Hq, Tq, d], k, v [Hkv, Tk, d]; sequence b owns
    query rows cu_q[b]:cu_q[b+1] and key rows cu_k[b]:cu_k[b+1]. Returns
    O [Hq, Tq, d] and lse [Hq, Tq] (float64)."""
    Hq, Tq, _ = q.shape
    Hkv = k.shape[0]
    O = np.zeros((Hq, Tq, v.shape[-1]), dtype=np.float64)
    lse = np.full((Hq, Tq), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0:
            continue
        for hq in range(Hq):
            g = kv_head(hq, Hq, Hkv)
            if k1 == k0:
                continue  # no keys: O = 0, lse = -inf
            O[hq, q0:q1], lse[hq, q0:q1] = attn_fwd_head(q[hq, q0:q1], k[g, k0:k1], v[g, k0:k1], scale, causal)
    return O, lse


def attn_bwd_varlen(q, k, v, do, cu_q, cu_k, scale, causal):
    """Backward of a variable-length batch (the packing of attn_fwd_varlen):
    q, do [Hq, Tq, d], k, v [Hkv, Tk, d]; sequence b owns query rows
    cu_q[b]:cu_q[b+1] and key rows cu_k[b]:cu_k[b+1], each sequence an
    independent problem (bottom-right causal mask when its lengths differ).
    Returns dq [Hq, Tq, d], dk, dv [Hkv, Tk, d] (float64); rows outside every
    sequence, and every row of a sequence without keys or queries, are 0."""
    Hq, Tq, _ = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0 or k1 == k0:
            continue
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            dq[hs, q0:q1], dk[g, k0:k1], dv[g, k0:k1] = attn_bwd_group(
                q[hs, q0:q1], k[g, k0:k1], v[g, k0:k1], do[hs, q0:q1], scale, causal)
    return dq, dk, dv
