"""GPU parity of the general backward (Nq != Nk with the bottom-right causal
mask, variable-length batches) against the fp64 oracle's analytic gradients,
through the C ABI.

The backward consumes the GPU forward's own O and lse (flash_attn_fwd_kv /
flash_attn_fwd_varlen), as a caller would. Small shapes are compared element
by element on dQ, dK and dV (several 32-row tiles and 64-key blocks, ragged
tails, GQA and MQA, every head dim, both masks); query rows that see no key
must have dQ exactly 0. The chunked-prefill and variable-length workloads run
in full and are compared on whole sampled K/V head groups, plus invariants
that hold at any size."""

import math

import numpy as np
import pytest

import oracle
from online_softmax_flash_amd.inputs import make_kv_inputs, make_varlen_inputs, varlen_lengths
from online_softmax_flash_amd.workloads import KV_WORKLOADS
from parity_util import announce, assert_close, from_dev, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import online_softmax_flash_amd as fa  # noqa: E402


def run_kv(inp, scale, causal):
    q, k, v, do = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    o, lse = fa.attention_forward_kv(q, k, v, scale, causal, num_splits=1)
    dq, dk, dv = fa.attention_backward_kv(q, k, v, o, lse, do, scale, causal)
    torch.cuda.synchronize()
    return dq, dk, dv


BWD_KV_SMALL = [
    # B, Hq, Hkv, Nq, Nk, d
    (1, 4, 2, 5, 130, 64),
    (2, 4, 2, 70, 200, 128),
    (1, 2, 1, 200, 70, 128),   # more queries than keys: the first 130 rows see no key when causal
    (1, 2, 2, 129, 300, 256),
    (1, 8, 1, 33, 64, 128),
    (1, 2, 2, 300, 300, 64),   # square through the general entry point
    (1, 3, 3, 1, 257, 128),    # one query
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", BWD_KV_SMALL, ids=["x".join(map(str, s)) for s in BWD_KV_SMALL])
def test_bwd_kv_small_parity(shape, causal):
    B, Hq, Hkv, Nq, Nk, d = shape
    announce(f"bwd kv small shape={shape} causal={causal} seed=81")
    inp = make_kv_inputs(B, Hq, Hkv, Nq, Nk, d, seed=81, with_dout=True)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = (from_dev(x) for x in run_kv(inp, scale, causal))
    rq, rk, rv = oracle.attn_bwd_analytic(inp.q, inp.k, inp.v, inp.do, scale, causal)
    assert_close(dq, rq, "bf16", f"dQ {shape} causal={causal}")
    assert_close(dk, rk, "bf16", f"dK {shape} causal={causal}")
    assert_close(dv, rv, "bf16", f"dV {shape} causal={causal}")
    if causal and Nq > Nk:
        assert np.all(dq[:, :, : Nq - Nk] == 0.0), "rows that see no key have dQ = 0"


VARLEN = [
    # cu_q, cu_k: a sequence without queries, one without keys, a one-token
    # sequence, more queries than keys, ragged tails
    ([0, 3, 3, 70, 71, 200, 260], [0, 100, 164, 164, 400, 650, 690]),
    ([0, 40, 90], [0, 40, 90]),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", range(len(VARLEN)))
def test_bwd_varlen_small_parity(case, causal, d):
    cu_q, cu_k = VARLEN[case]
    Hq, Hkv = 4, 2
    announce(f"bwd varlen small cu_q={cu_q} cu_k={cu_k} causal={causal} d={d} seed=82")
    inp = make_varlen_inputs(Hq, Hkv, cu_q, cu_k, d, seed=82, with_dout=True)
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    cq = torch.tensor(cu_q, dtype=torch.int32, device="cuda")
    ck = torch.tensor(cu_k, dtype=torch.int32, device="cuda")
    mq, mk = int(np.diff(cu_q).max()), int(np.diff(cu_k).max())
    o, lse = fa.attention_forward_varlen(q, k, v, cq, ck, mq, mk, scale, causal, num_splits=1)
    dq, dk, dv = fa.attention_backward_varlen(q, k, v, o, lse, do, cq, ck, mq, mk, scale, causal)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd_varlen(inp.q, inp.k, inp.v, inp.do, cu_q, cu_k, scale, causal)
    what = f"varlen case={case} causal={causal} d={d}"
    assert_close(from_dev(dq), rq, "bf16", f"dQ {what}")
    assert_close(from_dev(dk), rk, "bf16", f"dK {what}")
    assert_close(from_dev(dv), rv, "bf16", f"dV {what}")


def test_bwd_kv_repeatable():
    """No atomics: two runs of the general backward give identical bits."""
    B, Hq, Hkv, Nq, Nk, d = 1, 8, 2, 300, 1000, 128
    announce(f"bwd kv repeat shape={(B, Hq, Hkv, Nq, Nk, d)} seed=83")
    inp = make_kv_inputs(B, Hq, Hkv, Nq, Nk, d, seed=83, with_dout=True)
    a = run_kv(inp, 1.0 / math.sqrt(d), True)
    b = run_kv(inp, 1.0 / math.sqrt(d), True)
    for x, y, what in zip(a, b, ("dQ", "dK", "dV")):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), f"{what} differs between runs"


def _group_invariants(dk_h, dv_h, do_rows, N, what):
    """sum_j dK_j = 0 and sum_j dV_j = sum of dO over the query rows (all of
    which see a key); bound: bf16 rounding of N stored rows on top of the
    fp32 sums."""
    for arr, expect, name in ((dk_h, np.zeros(dk_h.shape[-1]), "sum dK"), (dv_h, do_rows, "sum dV")):
        got = arr.sum(axis=0)
        tol = 8.0 * math.sqrt(N) * 2.0 ** -9 * float(np.sqrt(np.mean(arr ** 2))) + 1e-3
        err = float(np.max(np.abs(got - expect)))
        assert err <= tol, f"{what} {name}: {err:.3e} > {tol:.3e}"


def test_bwd_chunk_2k_8k_full_size():
    """The chunked-prefill workload (B=1, Hq=32, Hkv=8, 2048 queries on 8192
    keys, d=128, causal, seed 6) in full; two whole K/V head groups against
    the oracle, invariants on every group."""
    w = KV_WORKLOADS["chunk_2k_8k"]
    announce(f"bwd kv full chunk_2k_8k shape=({w.B},{w.Hq},{w.Hkv},{w.Nq},{w.Nk},{w.d}) seed={w.seed}")
    inp = make_kv_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.seed, with_dout=True)
    dq, dk, dv = (from_dev(x) for x in run_kv(inp, w.scale, w.causal))
    for x in (dq, dk, dv):
        assert np.all(np.isfinite(x))
    G = w.Hq // w.Hkv
    rng = np.random.default_rng(2100 + w.seed)
    for g in rng.choice(w.Hkv, size=2, replace=False):
        g = int(g)
        hs = slice(g * G, (g + 1) * G)
        rq, rk, rv = oracle.attn_bwd_group(inp.q[0, hs], inp.k[0, g], inp.v[0, g], inp.do[0, hs], w.scale, w.causal)
        assert_close(dq[0, hs], rq, "bf16", f"chunk_2k_8k dQ g={g}")
        assert_close(dk[0, g], rk, "bf16", f"chunk_2k_8k dK g={g}")
        assert_close(dv[0, g], rv, "bf16", f"chunk_2k_8k dV g={g}")
    do = inp.do.astype(np.float64)
    for g in range(w.Hkv):
        _group_invariants(dk[0, g], dv[0, g], do[0, g * G:(g + 1) * G].sum(axis=(0, 1)), w.Nk, f"chunk_2k_8k g={g}")


def test_bwd_varlen_mix_full_size():
    """The variable-length workload (16 sequences of 64-4096 tokens, Hq=32,
    Hkv=8, d=128, causal, seed 7) in full; one K/V head group of four
    sequences against the oracle, invariants on every sequence and group."""
    w = KV_WORKLOADS["varlen_mix"]
    lens = varlen_lengths(w.B, w.Nq_lo, w.Nq, w.lengths_seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    announce(f"bwd varlen full varlen_mix B={w.B} Tq={int(cu[-1])} seed={w.seed}")
    inp = make_varlen_inputs(w.Hq, w.Hkv, cu, cu, w.d, w.seed, with_dout=True)
    q, k, v, do = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    cq = torch.tensor(cu, dtype=torch.int32, device="cuda")
    mx = int(np.diff(cu).max())
    o, lse = fa.attention_forward_varlen(q, k, v, cq, cq, mx, mx, w.scale, w.causal, num_splits=1)
    dq, dk, dv = (from_dev(x) for x in fa.attention_backward_varlen(q, k, v, o, lse, do, cq, cq, mx, mx, w.scale,
                                                                    w.causal))
    for x in (dq, dk, dv):
        assert np.all(np.isfinite(x))
    G = w.Hq // w.Hkv
    rng = np.random.default_rng(2101)
    dof = inp.do.astype(np.float64)
    for b in range(w.B):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        for g in range(w.Hkv):
            _group_invariants(dk[g, t0:t1], dv[g, t0:t1], dof[g * G:(g + 1) * G, t0:t1].sum(axis=(0, 1)), t1 - t0,
                              f"varlen_mix seq={b} g={g}")
    for b in rng.choice(w.B, size=4, replace=False):
        b = int(b)
        t0, t1 = int(cu[b]), int(cu[b + 1])
        g = int(rng.integers(w.Hkv))
        hs = slice(g * G, (g + 1) * G)
        rq, rk, rv = oracle.attn_bwd_group(inp.q[hs, t0:t1], inp.k[g, t0:t1], inp.v[g, t0:t1], inp.do[hs, t0:t1],
                                           w.scale, w.causal)
        # dV of a K/V head sums P^T dO over its 4 query heads: in these short
        # causal sequences its first keys reach |dV| = 12, where one bf16
        # rounding step of the stored value alone exceeds 2e-2; the bound
        # adds that rounding (2^-8 |ref|).
        assert_close(dq[hs, t0:t1], rq, "bf16", f"varlen_mix dQ seq={b} g={g}", storage_rounding=True)
        assert_close(dk[g, t0:t1], rk, "bf16", f"varlen_mix dK seq={b} g={g}", storage_rounding=True)
        assert_close(dv[g, t0:t1], rv, "bf16", f"varlen_mix dV seq={b} g={g}", storage_rounding=True)


@pytest.mark.parametrize("n_seq", [64, 300])
def test_bwd_varlen_many_sequences(n_seq):
    """Many short sequences (0-150 queries, 0-200 keys each, seeded), causal:
    every gradient against the oracle."""
    rng = np.random.default_rng(1100 + n_seq)
    lq = rng.integers(0, 151, size=n_seq)
    lk = rng.integers(0, 201, size=n_seq)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    Hq, Hkv, d = 4, 2, 64
    announce(f"bwd varlen many sequences n_seq={n_seq} Tq={int(cu_q[-1])} Tk={int(cu_k[-1])} seed=84")
    inp = make_varlen_inputs(Hq, Hkv, cu_q, cu_k, d, seed=84, with_dout=True)
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    cq = torch.tensor(cu_q, dtype=torch.int32, device="cuda")
    ck = torch.tensor(cu_k, dtype=torch.int32, device="cuda")
    mq, mk = int(lq.max()), int(lk.max())
    o, lse = fa.attention_forward_varlen(q, k, v, cq, ck, mq, mk, scale, True, num_splits=1)
    dq, dk, dv = fa.attention_backward_varlen(q, k, v, o, lse, do, cq, ck, mq, mk, scale, True)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_bwd_varlen(inp.q, inp.k, inp.v, inp.do, cu_q, cu_k, scale, True)
    # In short causal sequences the first keys take most of the weight of many
    # queries: |dV| reaches 7 (159 elements above 4 at n_seq = 64), where one
    # bf16 rounding step of the stored value is up to 0.031; the bound adds
    # that rounding (2^-8 |ref|), as for the variable-length workload.
    assert_close(from_dev(dq), rq, "bf16", f"dQ n_seq={n_seq}", storage_rounding=True)
    assert_close(from_dev(dk), rk, "bf16", f"dK n_seq={n_seq}", storage_rounding=True)
    assert_close(from_dev(dv), rv, "bf16", f"dV n_seq={n_seq}", storage_rounding=True)


ORDER = [(8, 8, 128, True), (4, 2, 64, False)]


@pytest.mark.parametrize("Hq,Hkv,d,causal", ORDER, ids=["h8-d128-causal", "gqa-d64-noncausal"])
def test_varlen_sequence_order_invariance(Hq, Hkv, d, causal):
    """The kernels take the sequences of a variable-length batch (up to 64)
    longest first, whatever order the batch lists them in. Listing the same
    sequences in another order must leave every sequence's O, lse, dQ, dK and
    dV bit for bit unchanged: the work items differ only in the order they run
    in. Lengths with ties, an empty sequence and several multi-block ones;
    queries and keys of different lengths when not causal."""
    rng = np.random.default_rng(91)
    lq = np.array([300, 17, 300, 0, 129, 64, 1000, 65, 300, 1, 511, 96], dtype=np.int64)
    lk = lq.copy() if causal else rng.integers(1, 700, size=lq.size)
    scale = 1.0 / math.sqrt(d)
    announce(f"varlen order invariance Hq={Hq} Hkv={Hkv} d={d} causal={causal} seed=92")
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    inp = make_varlen_inputs(Hq, Hkv, cu_q, cu_k, d, seed=92, with_dout=True)

    def run(order):
        sq = [slice(int(cu_q[s]), int(cu_q[s + 1])) for s in order]
        sk = [slice(int(cu_k[s]), int(cu_k[s + 1])) for s in order]
        q = np.concatenate([inp.q[:, x] for x in sq], axis=1)
        do = np.concatenate([inp.do[:, x] for x in sq], axis=1)
        k = np.concatenate([inp.k[:, x] for x in sk], axis=1)
        v = np.concatenate([inp.v[:, x] for x in sk], axis=1)
        cq = torch.tensor(np.concatenate([[0], np.cumsum(lq[order])]), dtype=torch.int32, device="cuda")
        ck = torch.tensor(np.concatenate([[0], np.cumsum(lk[order])]), dtype=torch.int32, device="cuda")
        qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
        mq, mk = int(lq.max()), int(lk.max())
        o, lse = fa.attention_forward_varlen(qd, kd, vd, cq, ck, mq, mk, scale, causal, num_splits=1)
        dq, dk, dv = fa.attention_backward_varlen(qd, kd, vd, o, lse, dod, cq, ck, mq, mk, scale, causal)
        torch.cuda.synchronize()
        out = {}
        oq = np.concatenate([[0], np.cumsum(lq[order])])
        ok = np.concatenate([[0], np.cumsum(lk[order])])
        for i, s in enumerate(order):
            a, b = int(oq[i]), int(oq[i + 1])
            c, e = int(ok[i]), int(ok[i + 1])
            out[int(s)] = (o[:, a:b].view(torch.int16).cpu(), lse[:, a:b].cpu(), dq[:, a:b].view(torch.int16).cpu(),
                           dk[:, c:e].view(torch.int16).cpu(), dv[:, c:e].view(torch.int16).cpu())
        return out

    base = run(np.arange(lq.size))
    for order in (np.arange(lq.size)[::-1].copy(), rng.permutation(lq.size), np.argsort(-lq, kind="stable")):
        got = run(order)
        for s in range(lq.size):
            for name, x, y in zip(("O", "lse", "dQ", "dK", "dV"), base[s], got[s]):
                assert torch.equal(x, y), f"sequence {s}: {name} depends on the batch order {order.tolist()}"
