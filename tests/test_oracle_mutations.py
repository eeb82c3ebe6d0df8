"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutation edits the oracle's source text in memory (a dropped term, a wrong
sign or index, a transposed operand, a dropped rescale ...), loads that copy as
a fresh module and runs the pins against it. The committed oracle is never
changed. CPU only.
"""

import os
import types
import warnings

import numpy as np
import pytest

from oracle_pins import ALL_PINS, BWD_PINS, FWD_PINS, make_ns

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ATT = os.path.join(ROOT, "oracle", "attention.py")
FOLD = os.path.join(ROOT, "oracle", "online_fold.py")

MUTATIONS = [
    # (id, file, old text, new text)
    ("scores_transposed", ATT, "return scale * (q_h @ k_h.T)", "return scale * (k_h @ q_h.T)"),
    ("scores_no_scale", ATT, "return scale * (q_h @ k_h.T)", "return (q_h @ k_h.T)"),
    ("mask_reversed", ATT, "<= rows[:, None]", ">= rows[:, None]"),
    ("mask_off_by_one", ATT, "<= rows[:, None]", "< rows[:, None] + 2"),
    ("softmax_no_max", ATT, "E = np.exp(S - np.where(seen, m, 0.0)[:, None])", "E = np.exp(S)"),
    ("softmax_wrong_axis", ATT, "l = E.sum(axis=1)", "l = E.sum(axis=0)"),
    ("lse_dropped_log", ATT, "return P @ v_h, m + np.log(l)", "return P @ v_h, m"),
    ("pv_transposed", ATT, "return P @ v_h, m + np.log(l)", "return P.T @ v_h, m + np.log(l)"),
    ("gqa_interleaved", ATT, "return hq // (Hq // Hkv)", "return hq % Hkv"),
    ("bwd_dropped_D", ATT, "D = (P * dP).sum(axis=1)", "D = 0.0 * (P * dP).sum(axis=1)"),
    ("bwd_D_sign", ATT, "dS = P * (dP - D[:, None])", "dS = P * (dP + D[:, None])"),
    ("bwd_dq_no_scale", ATT, "dq[j] = scale * (dS @ k_h)", "dq[j] = (dS @ k_h)"),
    ("bwd_dk_transposed", ATT, "dk += scale * (dS.T @ q_g[j])", "dk += scale * (dS @ q_g[j])"),
    ("bwd_dv_transposed", ATT, "dv += P.T @ do_g[j]", "dv += P @ do_g[j]"),
    ("bwd_dp_wrong_operand", ATT, "dP = do_g[j] @ v_h.T", "dP = do_g[j] @ k_h.T"),
    ("fold_no_rescale_l", FOLD, "l = alpha * l + p.sum(axis=1)", "l = l + p.sum(axis=1)"),
    ("fold_no_rescale_o", FOLD, "o = alpha[:, None] * o + p @ v_h[j0:j1]", "o = o + p @ v_h[j0:j1]"),
    ("fold_keeps_block_max", FOLD, "        m = m_new\n", "        m = m_blk\n"),
    ("fold_no_final_divide", FOLD, "np.where(seen[:, None], o / l[:, None], 0.0)", "np.where(seen[:, None], o, 0.0)"),
    ("fold_mask_strict", FOLD, "keys[None, :] <= qi[:, None]", "keys[None, :] < qi[:, None]"),
    ("offset_sign", ATT, "<= rows[:, None] + offset", "<= rows[:, None] - offset"),
    ("offset_top_left", ATT, "causal, k_h.shape[0] - q_h.shape[0]), S, -np.inf)\n    P, m, l",
     "causal, 0), S, -np.inf)\n    P, m, l"),
    ("empty_row_uniform", ATT, "P = np.where(seen[:, None], E / np.where(seen, l, 1.0)[:, None], 0.0)",
     "P = np.where(seen[:, None], E / np.where(seen, l, 1.0)[:, None], 1.0 / S.shape[1])"),
    ("merge_no_rescale", ATT, "l = alpha * l + w", "l = l + w"),
    ("merge_unweighted", ATT, "w = np.where(np.isfinite(lse_parts[s_]), np.exp(lse_parts[s_] - base), 0.0)",
     "w = np.where(np.isfinite(lse_parts[s_]), 1.0, 0.0)"),
    ("merge_no_divide", ATT, "o / np.where(seen, l, 1.0)[:, None], 0.0), m + np.log(l)",
     "o, 0.0), m + np.log(l)"),
    ("varlen_key_rows", ATT, "attn_fwd_head(q[hq, q0:q1], k[g, k0:k1], v[g, k0:k1]",
     "attn_fwd_head(q[hq, q0:q1], k[g, q0:q1], v[g, q0:q1]"),
    ("fold_offset_dropped", FOLD, "<= qi[:, None] + offset", "<= qi[:, None]"),
    ("fold_range_from_zero", FOLD, "range(key_lo, key_hi, block_k)", "range(0, key_hi, block_k)"),
    ("bwd_offset_dropped", ATT, "vis = _visible(np.arange(Nq), Nk, causal, Nk - Nq)",
     "vis = _visible(np.arange(Nq), Nk, causal, 0)"),
    ("bwd_offset_sign", ATT, "vis = _visible(np.arange(Nq), Nk, causal, Nk - Nq)",
     "vis = _visible(np.arange(Nq), Nk, causal, Nq - Nk)"),
    ("bwd_varlen_key_rows", ATT, "q[hs, q0:q1], k[g, k0:k1], v[g, k0:k1], do[hs, q0:q1]",
     "q[hs, q0:q1], k[g, q0:q1], v[g, q0:q1], do[hs, q0:q1]"),
    ("bwd_varlen_heads_interleaved", ATT, "            hs = slice(g * G, (g + 1) * G)\n            dq[hs, q0:q1]",
     "            hs = slice(g, Hq, Hkv)\n            dq[hs, q0:q1]"),
    ("bwd_varlen_do_rows", ATT, "v[g, k0:k1], do[hs, q0:q1], scale, causal)",
     "v[g, k0:k1], do[hs, k0:k0 + (q1 - q0)], scale, causal)"),
    ("fold_wrong_scale", FOLD, "s = scale * (qr @ k_h[j0:j1].T)", "s = scale * scale * (qr @ k_h[j0:j1].T)"),
]


def _load(path, old=None, new=None, name="mut"):
    with open(path) as f:
        src = f.read()
    if old is not None:
        assert src.count(old) == 1, f"mutation anchor not found exactly once in {path}: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType(name)
    mod.__dict__["__name__"] = name
    exec(compile(src, path + ":" + name, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("mid,path,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(mid, path, old, new):
    att = _load(ATT, *((old, new) if path == ATT else (None, None)), name="att_" + mid)
    fold = _load(FOLD, *((old, new) if path == FOLD else (None, None)), name="fold_" + mid)
    ns = make_ns(att, fold)
    failed = []
    with warnings.catch_warnings(), np.errstate(all="ignore"):
        warnings.simplefilter("ignore")
        for pin in ALL_PINS:
            try:
                pin(ns)
            except Exception as e:  # AssertionError, or a shape error the mistake causes
                failed.append((pin.__name__, type(e).__name__))
    assert failed, f"planted mistake {mid} passed every pin"


def test_unmutated_copy_passes():
    """The in-memory loading used above, without a mutation, passes every pin."""
    ns = make_ns(_load(ATT, name="att_clean"), _load(FOLD, name="fold_clean"))
    for pin in ALL_PINS:
        pin(ns)
