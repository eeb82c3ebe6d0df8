"""Pins of the CPU oracle: facts fixed by the pages and by mathematics.

Each ``pin_*`` function takes a namespace ``ns`` holding the oracle's functions
(``attn_fwd_materialised``, ``attn_fwd_head``, ``attn_probs``, ``attn_bwd_group``,
``attn_bwd_analytic``, ``kv_head``, ``attn_fwd_online_fold``, ``fold_head``) and
raises AssertionError when the oracle disagrees with the fact. They run on the
real oracle (``test_oracle.py``) and on copies with planted mistakes
(``test_oracle_mutations.py``), which each pin set must catch.
"""

from __future__ import annotations

import json
import math
import os
import types

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.json")

TOL = 1e-12  # fp64 agreement of two exact formulations


def real_ns():
    import oracle.attention as att
    import oracle.online_fold as fold
    return make_ns(att, fold)


def make_ns(att, fold):
    return types.SimpleNamespace(
        attn_fwd_materialised=att.attn_fwd_materialised,
        attn_fwd_head=att.attn_fwd_head,
        attn_probs=att.attn_probs,
        attn_bwd_group=att.attn_bwd_group,
        attn_bwd_analytic=att.attn_bwd_analytic,
        kv_head=att.kv_head,
        attn_fwd_online_fold=fold.attn_fwd_online_fold,
        fold_head=fold.fold_head,
        merge_partials=att.merge_partials,
        attn_fwd_varlen=att.attn_fwd_varlen,
        attn_bwd_varlen=att.attn_bwd_varlen,
    )


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _maxabs(a, b):
    d = np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))
    return float(np.max(d)) if d.size else 0.0


def _close(a, b, tol, what):
    err = _maxabs(a, b)
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------------------
# Forward pins
# ---------------------------------------------------------------------------

def pin_fold_equals_definition(ns):
    """The online fold reaches exactly the full softmax (fanfani.net 'A pinch of
    math': the answer is what the full softmax gives; mentria.ai 'Same answer.
    The giant grid never existed.': o_flash = o_exact). Key block sizes 1, 7
    (does not divide N), 64 and N; GQA with two query heads per K/V head."""
    for N, d in [(1, 4), (5, 3), (64, 16), (200, 64)]:
        q = _rand((1, 2, N, d), 1)
        k = _rand((1, 1, N, d), 2)
        v = _rand((1, 1, N, d), 3)
        scale = 1.0 / math.sqrt(d)
        for causal in (False, True):
            O1, l1 = ns.attn_fwd_materialised(q, k, v, scale, causal)
            for bk in sorted({1, 7, 64, N}):
                O2, l2 = ns.attn_fwd_online_fold(q, k, v, scale, causal, bk)
                _close(O1, O2, TOL, f"O fold vs definition N={N} causal={causal} Bc={bk}")
                _close(l1, l2, TOL, f"lse fold vs definition N={N} causal={causal} Bc={bk}")


def pin_rows_sum_to_one(ns):
    """Weights are non-negative and each row sums to 1 (mentria.ai 'But softmax
    needs the whole row at once.'); hidden keys weigh exactly 0."""
    q = _rand((50, 8), 4)
    k = _rand((50, 8), 5)
    for causal in (False, True):
        P = ns.attn_probs(q, k, 0.35, causal)
        assert np.all(P >= 0.0), "negative weight"
        _close(P.sum(axis=1), np.ones(50), TOL, f"row sums causal={causal}")
        if causal:
            assert np.all(P[np.triu_indices(50, 1)] == 0.0), "hidden key has non-zero weight"


def pin_qzero_closed_form(ns):
    """Q = 0: all scores 0, so O_i = mean of V over the keys visible to i and
    lse_i = ln(#visible) (ln 256 for the tiny workload, non-causal). scale = 0
    gives the same result for any Q, K."""
    with open(GOLDEN) as f:
        gold = {c["name"]: c for c in json.load(f)["cases"]}
    N, d = 256, 64
    v = _rand((1, 2, N, d), 6)
    q0 = np.zeros((1, 2, N, d))
    k = _rand((1, 2, N, d), 7)
    qr = _rand((1, 2, N, d), 8)
    ln256 = gold["tiny_qzero_lse"]["noncausal_lse"]
    for causal in (False, True):
        if causal:
            cnt = np.arange(1, N + 1, dtype=np.float64)
            mean = np.cumsum(v, axis=2) / cnt[None, None, :, None]
            lse = np.broadcast_to(np.log(cnt), (1, 2, N))
        else:
            mean = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
            lse = np.full((1, 2, N), ln256)
        for name, (qq, sc) in {"Q=0": (q0, 0.125), "scale=0": (qr, 0.0)}.items():
            O, L = ns.attn_fwd_materialised(qq, k, v, sc, causal)
            _close(O, mean, 1e-12, f"{name} O causal={causal}")
            _close(L, lse, 1e-12, f"{name} lse causal={causal}")
            O2, L2 = ns.attn_fwd_online_fold(qq, k, v, sc, causal, 64)
            _close(O2, mean, 1e-12, f"{name} fold O causal={causal}")
            _close(L2, lse, 1e-12, f"{name} fold lse causal={causal}")


def pin_one_hot_and_large_scores(ns):
    """A dominant score returns that V row (within N e^-50); a huge score shared
    by every key gives uniform weights with no overflow -- the max subtraction of
    the safe softmax (mentria.ai 'But softmax needs the whole row at once.')."""
    N, d, L = 40, 8, 10.0
    rng = np.random.default_rng(9)
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    jstar = 17
    k[:, 0] = 0.0
    k[jstar] = 0.0
    k[jstar, 0] = L
    q = np.zeros((5, d))
    q[:, 0] = L
    scale = 0.5  # scale * L^2 = 50
    for fn in (lambda: ns.attn_fwd_head(q, k, v, scale, False),
               lambda: ns.fold_head(q, k, v, scale, False, 7)):
        O, lse = fn()
        _close(O, np.broadcast_to(v[jstar], O.shape), N * math.exp(-50.0) * 10, "one-hot row")
        _close(lse, np.full(5, 50.0), 1e-12, "one-hot lse")
    # all keys equal, huge shared score ~ 1e3 (exp would overflow without the max subtraction)
    kk = np.tile(rng.standard_normal((1, d)), (N, 1))
    qq = 1e3 * kk[:1] / float(kk[0] @ kk[0])
    for causal in (False, True):
        rows = np.array([N - 1])
        O, lse = ns.attn_fwd_head(np.repeat(qq, N, axis=0), kk, v, 1.0, causal, rows=rows)
        assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse)), "overflow with a large shared score"
        _close(O[0], v.mean(axis=0), 1e-9, "uniform weights under a large shared score")
        _close(lse, [1e3 + math.log(N)], 1e-9, "lse under a large shared score")
        O2, lse2 = ns.fold_head(np.repeat(qq, N, axis=0), kk, v, 1.0, causal, 7, rows=rows)
        assert np.all(np.isfinite(O2)), "fold overflow with a large shared score"
        _close(O2[0], v.mean(axis=0), 1e-9, "fold uniform weights")


def pin_special_rows(ns):
    """Causal row 0 sees key 0 only: O_0 = v_0, lse_0 = scale q_0.k_0. N = 1
    gives O = V. Adding c to every V entry adds c to every output (weights sum
    to 1)."""
    N, d = 33, 16
    q = _rand((1, 2, N, d), 10)
    k = _rand((1, 2, N, d), 11)
    v = _rand((1, 2, N, d), 12)
    sc = 0.25
    for fwd in (lambda *a: ns.attn_fwd_materialised(*a),
                lambda *a: ns.attn_fwd_online_fold(*a, 5)):
        O, lse = fwd(q, k, v, sc, True)
        _close(O[:, :, 0], v[:, :, 0], 1e-15, "causal row 0 output")
        _close(lse[:, :, 0], sc * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), 1e-14, "causal row 0 lse")
        O1, _ = fwd(q[:, :, :1], k[:, :, :1], v[:, :, :1], sc, False)
        _close(O1, v[:, :, :1], 1e-15, "N=1")
        for causal in (False, True):
            Oa, la = fwd(q, k, v, sc, causal)
            Ob, lb = fwd(q, k, v + 3.5, sc, causal)
            _close(Ob, Oa + 3.5, 1e-12, f"V translation causal={causal}")
            _close(lb, la, 0.0, f"lse independent of V causal={causal}")


def _brute_head(q, k, v, scale, causal):
    """Pure-Python loops from the definition (scores, mask, softmax, weighted
    sum). With len(q) queries and len(k) keys the causal mask is aligned to the
    bottom right (key j visible to query i iff j <= i + len(k) - len(q)); a
    query that sees no key gets output 0 and lse -inf."""
    n, d = len(q), len(q[0])
    O, L = [], []
    for i in range(n):
        keys = [j for j in range(len(k)) if (not causal or j <= i + len(k) - n)]
        if not keys:
            O.append([0.0] * len(v[0]))
            L.append(-math.inf)
            continue
        s = [scale * sum(q[i][c] * k[j][c] for c in range(d)) for j in keys]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = sum(w)
        O.append([sum(w[t] * v[keys[t]][c] for t in range(len(keys))) / tot for c in range(len(v[0]))])
        L.append(mx + math.log(tot))
    return O, L


def pin_brute_force(ns):
    """Tiny inputs against pure-Python loops written from the definition,
    with GQA (query heads 0,1 read K/V head 0; 2,3 read head 1)."""
    B, Hq, Hkv, N, d = 1, 4, 2, 6, 3
    q = _rand((B, Hq, N, d), 13)
    k = _rand((B, Hkv, N, d), 14)
    v = _rand((B, Hkv, N, d), 15)
    sc = 0.6
    for causal in (False, True):
        O1, l1 = ns.attn_fwd_materialised(q, k, v, sc, causal)
        O2, l2 = ns.attn_fwd_online_fold(q, k, v, sc, causal, 4)
        for hq in range(Hq):
            g = hq // 2
            Ob, Lb = _brute_head(q[0, hq].tolist(), k[0, g].tolist(), v[0, g].tolist(), sc, causal)
            for O, l, tag in ((O1, l1, "definition"), (O2, l2, "fold")):
                _close(O[0, hq], Ob, TOL, f"{tag} vs brute force O hq={hq} causal={causal}")
                _close(l[0, hq], Lb, TOL, f"{tag} vs brute force lse hq={hq} causal={causal}")


def pin_golden(ns):
    """Hand-derived worked examples (tests/golden/closed_forms.json)."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        if "q" not in c:
            continue
        q = np.array(c["q"], dtype=np.float64)[None, None]
        k = np.array(c["k"], dtype=np.float64)[None, None]
        v = np.array(c["v"], dtype=np.float64)[None, None]
        for mode, causal in (("noncausal", False), ("causal", True)):
            if mode not in c:
                continue
            exp_o = np.array(c[mode]["o"])
            exp_l = np.array(c[mode]["lse"])
            if causal and q.shape[2] != k.shape[2]:
                continue
            O, L = ns.attn_fwd_materialised(q, k, v, c["scale"], causal)
            _close(O[0, 0], exp_o, 1e-13, f"golden {c['name']} {mode} O")
            _close(L[0, 0], exp_l, 1e-13, f"golden {c['name']} {mode} lse")
            O2, L2 = ns.attn_fwd_online_fold(q, k, v, c["scale"], causal, 1)
            _close(O2[0, 0], exp_o, 1e-13, f"golden fold {c['name']} {mode} O")
            _close(L2[0, 0], exp_l, 1e-13, f"golden fold {c['name']} {mode} lse")


def pin_gqa_is_repeated_kv(ns):
    """Grouped K/V heads equal plain multi-head attention with each K/V head
    repeated for its contiguous group of query heads."""
    B, Hq, Hkv, N, d = 2, 6, 2, 20, 8
    q = _rand((B, Hq, N, d), 16)
    k = _rand((B, Hkv, N, d), 17)
    v = _rand((B, Hkv, N, d), 18)
    kr = np.repeat(k, Hq // Hkv, axis=1)
    vr = np.repeat(v, Hq // Hkv, axis=1)
    assert [ns.kv_head(h, Hq, Hkv) for h in range(Hq)] == [0, 0, 0, 1, 1, 1]
    for causal in (False, True):
        Og, lg = ns.attn_fwd_materialised(q, k, v, 0.3, causal)
        Om, lm = ns.attn_fwd_materialised(q, kr, vr, 0.3, causal)
        _close(Og, Om, 0.0, f"GQA vs repeated K/V causal={causal}")
        _close(lg, lm, 0.0, f"GQA lse vs repeated causal={causal}")


# ---------------------------------------------------------------------------
# Backward pins
# ---------------------------------------------------------------------------

def pin_bwd_finite_difference(ns):
    """Analytic gradients of L = sum(dO * O) agree with central differences of
    the forward definition (n=8, d=4, a group of two query heads)."""
    G, N, d = 2, 8, 4
    q = _rand((G, N, d), 19)
    k = _rand((N, d), 20)
    v = _rand((N, d), 21)
    do = _rand((G, N, d), 22)
    sc = 0.7

    def loss(qq, kk, vv, causal):
        return sum(float(np.sum(do[j] * ns.attn_fwd_head(qq[j], kk, vv, sc, causal)[0])) for j in range(G))

    h = 1e-6
    for causal in (False, True):
        dq, dk, dv = ns.attn_bwd_group(q, k, v, do, sc, causal)
        for arr, grad, name in ((q, dq, "dq"), (k, dk, "dk"), (v, dv, "dv")):
            num = np.zeros_like(arr)
            it = np.nditer(arr, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                a_p = arr.copy()
                a_m = arr.copy()
                a_p[idx] += h
                a_m[idx] -= h
                args_p = {"q": q, "k": k, "v": v}
                args_m = dict(args_p)
                args_p[name[1]] = a_p
                args_m[name[1]] = a_m
                num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"], causal)
                            - loss(args_m["q"], args_m["k"], args_m["v"], causal)) / (2 * h)
            _close(grad, num, 1e-7, f"finite differences {name} causal={causal}")


def pin_bwd_invariants(ns):
    """Each row of dS sums to 0, so sum_j dK_j = 0; weights sum to 1, so
    sum_j dV_j = sum_i dO_i (per head, Hq = Hkv)."""
    B, H, N, d = 1, 2, 40, 8
    q = _rand((B, H, N, d), 23)
    k = _rand((B, H, N, d), 24)
    v = _rand((B, H, N, d), 25)
    do = _rand((B, H, N, d), 26)
    for causal in (False, True):
        dq, dk, dv = ns.attn_bwd_analytic(q, k, v, do, 0.4, causal)
        _close(dk.sum(axis=2), np.zeros((B, H, d)), 1e-12, f"sum dK causal={causal}")
        _close(dv.sum(axis=2), do.sum(axis=2), 1e-12, f"sum dV causal={causal}")


def pin_bwd_qzero_causal(ns):
    """Q = 0, causal: row i weighs each visible key 1/(i+1), so
    dV_j = sum_{i >= j} dO_i / (i+1)."""
    N, d = 30, 5
    q = np.zeros((1, 1, N, d))
    k = _rand((1, 1, N, d), 27)
    v = _rand((1, 1, N, d), 28)
    do = _rand((1, 1, N, d), 29)
    _, _, dv = ns.attn_bwd_analytic(q, k, v, do, 0.5, True)
    w = do[0, 0] / np.arange(1, N + 1, dtype=np.float64)[:, None]
    expect = np.cumsum(w[::-1], axis=0)[::-1]
    _close(dv[0, 0], expect, 1e-12, "Q=0 causal dV closed form")



# ---------------------------------------------------------------------------
# Rectangular problems, split keys, variable-length batches
# ---------------------------------------------------------------------------

def _close_inf(a, b, tol, what):
    """As _close, with -inf required at exactly the same places."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    ia, ib = np.isneginf(a), np.isneginf(b)
    assert np.array_equal(ia, ib), f"{what}: -inf at different places"
    _close(np.where(ia, 0.0, a), np.where(ib, 0.0, b), tol, what)


def pin_rectangular_causal(ns):
    """Nq != Nk: brute force (bottom-right mask), the single-query closed case
    (the last query sees every key, so causal equals full attention), the
    prefix-extension identity (the rectangular problem is the last Nq rows of
    the square one whose first Nk - Nq queries are arbitrary), and rows that
    see no key (Nq > Nk): output exactly 0, lse exactly -inf."""
    sc = 0.45
    for Nq, Nk in [(1, 9), (3, 11), (5, 5), (7, 4)]:
        q = _rand((Nq, 3), 100 + Nq)
        k = _rand((Nk, 3), 200 + Nk)
        v = _rand((Nk, 2), 300 + Nk)
        for causal in (False, True):
            Ob, Lb = _brute_head(q.tolist(), k.tolist(), v.tolist(), sc, causal)
            O1, l1 = ns.attn_fwd_head(q, k, v, sc, causal)
            O2, l2 = ns.fold_head(q, k, v, sc, causal, 3)
            for O, l, tag in ((O1, l1, "definition"), (O2, l2, "fold")):
                _close(O, Ob, TOL, f"{tag} O Nq={Nq} Nk={Nk} causal={causal}")
                _close_inf(l, Lb, TOL, f"{tag} lse Nq={Nq} Nk={Nk} causal={causal}")
    q = _rand((1, 8), 7)
    k = _rand((40, 8), 8)
    v = _rand((40, 8), 9)
    Oc, lc = ns.attn_fwd_head(q, k, v, sc, True)
    On, ln = ns.attn_fwd_head(q, k, v, sc, False)
    _close(Oc, On, TOL, "one query: causal == full")
    _close(lc, ln, TOL, "one query: causal == full (lse)")
    Nq, Nk = 6, 17
    q = _rand((Nq, 5), 21)
    k = _rand((Nk, 5), 22)
    v = _rand((Nk, 4), 23)
    qfull = np.concatenate([_rand((Nk - Nq, 5), 24), q])
    Os, ls = ns.attn_fwd_head(qfull, k, v, sc, True)
    for O, l, tag in (ns.attn_fwd_head(q, k, v, sc, True) + ("definition",),
                      ns.fold_head(q, k, v, sc, True, 4) + ("fold",)):
        _close(O, Os[Nk - Nq:], TOL, f"{tag}: prefix extension O")
        _close(l, ls[Nk - Nq:], TOL, f"{tag}: prefix extension lse")
    q = _rand((9, 4), 31)
    k = _rand((3, 4), 32)
    v = _rand((3, 4), 33)
    for O, l, tag in (ns.attn_fwd_head(q, k, v, sc, True) + ("definition",),
                      ns.fold_head(q, k, v, sc, True, 2) + ("fold",)):
        assert np.all(O[:6] == 0.0) and np.all(np.isneginf(l[:6])), f"{tag}: rows without keys"
        assert np.all(np.isfinite(l[6:])), f"{tag}: rows with keys"


def pin_merge_partials(ns):
    """Split keys: partial results over disjoint key ranges (one of them empty,
    one ragged) merged by the rescale step equal the full softmax; the order of
    the partials does not matter; one partial merges to itself; two partials
    with equal lse and outputs a, b give (a + b) / 2 and lse + ln 2 (closed
    form); ranges a row sees no key of (lse -inf) add nothing, and a row with
    no key anywhere gets 0 and -inf."""
    sc = 0.3
    Nq, Nk, d = 6, 23, 5
    q = _rand((Nq, d), 41)
    k = _rand((Nk, d), 42)
    v = _rand((Nk, d), 43)
    bounds = [0, 5, 5, 12, 23]
    for causal in (False, True):
        parts = [ns.fold_head(q, k, v, sc, causal, 4, key_lo=a, key_hi=b) for a, b in zip(bounds, bounds[1:])]
        o_parts = np.stack([p[0] for p in parts])
        l_parts = np.stack([p[1] for p in parts])
        Oref, lref = ns.attn_fwd_head(q, k, v, sc, causal)
        O, l = ns.merge_partials(o_parts, l_parts)
        _close(O, Oref, TOL, f"merge == full causal={causal}")
        _close(l, lref, TOL, f"merge lse == full causal={causal}")
        perm = [3, 1, 0, 2]
        O2, l2 = ns.merge_partials(o_parts[perm], l_parts[perm])
        _close(O2, Oref, TOL, f"merge order causal={causal}")
        _close(l2, lref, TOL, f"merge order lse causal={causal}")
    O1, l1 = ns.merge_partials(o_parts[2:3], l_parts[2:3])
    _close(O1, o_parts[2], TOL, "single partial O")
    _close(l1, l_parts[2], TOL, "single partial lse")
    a = _rand((3, 4), 44)
    b = _rand((3, 4), 45)
    lse = np.array([0.3, -2.0, 5.0])
    O, l = ns.merge_partials(np.stack([a, b]), np.stack([lse, lse]))
    _close(O, (a + b) / 2, TOL, "equal-lse closed form O")
    _close(l, lse + math.log(2.0), TOL, "equal-lse closed form lse")
    lp = np.array([[-np.inf, 1.0], [-np.inf, -np.inf]])
    op = np.stack([np.zeros((2, 4)), np.zeros((2, 4))])
    op[0, 1] = 7.0
    O, l = ns.merge_partials(op, lp)
    assert np.all(O[0] == 0.0) and np.isneginf(l[0]), "no key anywhere"
    _close(O[1], op[0, 1], TOL, "empty ranges add nothing")
    _close(l[1], 1.0, TOL, "empty ranges add nothing (lse)")


def pin_varlen(ns):
    """Variable-length batch (sequences packed along the token axis, GQA):
    every sequence against brute force on its own rows, including a sequence
    with no queries, one with no keys (outputs 0, lse -inf) and a rectangular
    causal one."""
    sc = 0.5
    cu_q = [0, 3, 3, 8, 10]
    cu_k = [0, 5, 9, 9, 16]
    Hq, Hkv, d = 4, 2, 3
    q = _rand((Hq, cu_q[-1], d), 51)
    k = _rand((Hkv, cu_k[-1], d), 52)
    v = _rand((Hkv, cu_k[-1], d), 53)
    for causal in (False, True):
        O, l = ns.attn_fwd_varlen(q, k, v, cu_q, cu_k, sc, causal)
        for b in range(len(cu_q) - 1):
            q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
            for hq in range(Hq):
                g = hq // 2
                if k1 == k0:
                    assert np.all(O[hq, q0:q1] == 0.0) and np.all(np.isneginf(l[hq, q0:q1])), "no keys"
                    continue
                if q1 == q0:
                    continue
                Ob, Lb = _brute_head(q[hq, q0:q1].tolist(), k[g, k0:k1].tolist(), v[g, k0:k1].tolist(), sc, causal)
                _close(O[hq, q0:q1], Ob, TOL, f"varlen O seq={b} hq={hq} causal={causal}")
                _close_inf(l[hq, q0:q1], Lb, TOL, f"varlen lse seq={b} hq={hq} causal={causal}")

def _num_grad(loss, arrays, h=1e-6):
    """Central differences of loss() with respect to every element of every
    array in `arrays` (edited in place and restored)."""
    out = []
    for arr in arrays:
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            x0 = arr[idx]
            arr[idx] = x0 + h
            lp = loss()
            arr[idx] = x0 - h
            lm = loss()
            arr[idx] = x0
            num[idx] = (lp - lm) / (2 * h)
        out.append(num)
    return out


def pin_bwd_rectangular(ns):
    """Nq != Nk (bottom-right causal mask), a group of two query heads: the
    analytic gradients of L = sum(dO * O) agree with central differences of
    the forward definition; with Nq > Nk the first Nq - Nk query rows see no
    key (O = 0 for any input), so their dq is exactly 0; sum_j dK_j = 0."""
    sc = 0.6
    for Nq, Nk in ((5, 9), (9, 5)):
        G, d = 2, 3
        q = _rand((G, Nq, d), 61)
        k = _rand((Nk, d), 62)
        v = _rand((Nk, d), 63)
        do = _rand((G, Nq, d), 64)
        for causal in (False, True):
            dq, dk, dv = ns.attn_bwd_group(q, k, v, do, sc, causal)

            def loss():
                return sum(float(np.sum(do[j] * ns.attn_fwd_head(q[j], k, v, sc, causal)[0])) for j in range(G))

            for got, num, name in zip((dq, dk, dv), _num_grad(loss, [q, k, v]), ("dq", "dk", "dv")):
                _close(got, num, 1e-7, f"rectangular Nq={Nq} Nk={Nk} {name} causal={causal}")
            _close(dk.sum(axis=0), np.zeros(d), 1e-12, f"rectangular sum dK Nq={Nq} Nk={Nk} causal={causal}")
            if causal and Nq > Nk:
                assert np.all(dq[:, : Nq - Nk] == 0.0), "rows without keys have dq = 0"


def pin_bwd_varlen(ns):
    """Variable-length batch (GQA, sequences with no queries, no keys, fewer
    and more queries than keys): the analytic gradients agree with central
    differences of the packed forward definition; per sequence and K/V head
    sum_j dK_j = 0 and sum_j dV_j = the sum of dO over the group's query rows
    that see a key; rows of sequences without keys or queries are 0."""
    sc = 0.5
    cu_q = [0, 3, 3, 8, 10, 14]
    cu_k = [0, 5, 9, 9, 16, 18]
    Hq, Hkv, d = 4, 2, 3
    G = Hq // Hkv
    q = _rand((Hq, cu_q[-1], d), 65)
    k = _rand((Hkv, cu_k[-1], d), 66)
    v = _rand((Hkv, cu_k[-1], d), 67)
    do = _rand((Hq, cu_q[-1], d), 68)
    for causal in (False, True):
        dq, dk, dv = ns.attn_bwd_varlen(q, k, v, do, cu_q, cu_k, sc, causal)

        def loss():
            return float(np.sum(do * ns.attn_fwd_varlen(q, k, v, cu_q, cu_k, sc, causal)[0]))

        for got, num, name in zip((dq, dk, dv), _num_grad(loss, [q, k, v]), ("dq", "dk", "dv")):
            _close(got, num, 1e-7, f"varlen {name} causal={causal}")
        for b in range(len(cu_q) - 1):
            q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
            nq, nk = q1 - q0, k1 - k0
            for g in range(Hkv):
                _close(dk[g, k0:k1].sum(axis=0), np.zeros(d), 1e-12, f"varlen sum dK seq={b} g={g}")
                seen = np.arange(nq) + (nk - nq if causal else nk) >= 0 if nk else np.zeros(nq, bool)
                expect = do[g * G:(g + 1) * G, q0:q1][:, seen].sum(axis=(0, 1)) if nk else np.zeros(d)
                _close(dv[g, k0:k1].sum(axis=0), expect, 1e-12, f"varlen sum dV seq={b} g={g} causal={causal}")
            if nk == 0:
                assert np.all(dq[:, q0:q1] == 0.0), f"seq {b} without keys: dq = 0"
            if nq == 0:
                assert np.all(dk[:, k0:k1] == 0.0) and np.all(dv[:, k0:k1] == 0.0), f"seq {b} without queries"


FWD_PINS = [
    pin_fold_equals_definition,
    pin_rows_sum_to_one,
    pin_qzero_closed_form,
    pin_one_hot_and_large_scores,
    pin_special_rows,
    pin_brute_force,
    pin_golden,
    pin_gqa_is_repeated_kv,
    pin_rectangular_causal,
    pin_merge_partials,
    pin_varlen,
]
BWD_PINS = [
    pin_bwd_finite_difference,
    pin_bwd_invariants,
    pin_bwd_qzero_causal,
    pin_bwd_rectangular,
    pin_bwd_varlen,
]
ALL_PINS = FWD_PINS + BWD_PINS
