"""GPU parity of the general forward (rectangular problems with the bottom-right
causal mask, split keys with the combine step, variable-length batches)
against the fp64 oracle, through the C ABI.

Small shapes are compared element by element (several 32-row tiles and 64-key
blocks, ragged tails, GQA and MQA, every head dim, split counts 1, 3 and the
library's choice); rows that see no key must be exactly 0 with lse -inf. The
decode, chunked-prefill and variable-length workloads run in the launch
configuration the benchmark times and are compared on sampled rows."""

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


def check_rows(O, L, O_ref, L_ref, what):
    """Rows the oracle gives no key (lse -inf) must be exactly 0 / -inf; the rest to the bf16 bounds."""
    O, L, O_ref, L_ref = (np.asarray(x, np.float64) for x in (O, L, O_ref, L_ref))
    empty = np.isneginf(L_ref)
    assert np.array_equal(np.isneginf(L), empty), f"{what}: rows without keys differ"
    assert np.all(O[empty] == 0.0), f"{what}: rows without keys are not 0"
    if np.any(~empty):
        assert_close(O[~empty], O_ref[~empty], "bf16", f"{what} O")
        assert_close(L[~empty], L_ref[~empty], "bf16", f"{what} lse", lse=True)


KV_SMALL = [
    # B, Hq, Hkv, Nq, Nk, d
    (1, 8, 1, 1, 300, 64),
    (2, 4, 2, 5, 130, 128),
    (1, 2, 2, 200, 200, 128),
    (1, 4, 1, 100, 37, 64),
    (1, 2, 1, 70, 1000, 256),
    (2, 8, 8, 33, 64, 128),
    (1, 16, 2, 3, 4099, 128),
]


@pytest.mark.parametrize("splits", [1, 3, 0])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", KV_SMALL, ids=["x".join(map(str, s)) for s in KV_SMALL])
def test_kv_small_parity(shape, causal, splits):
    B, Hq, Hkv, Nq, Nk, d = shape
    announce(f"kv small shape={shape} causal={causal} splits={splits} seed=31")
    inp = make_kv_inputs(B, Hq, Hkv, Nq, Nk, d, seed=31)
    scale = 1.0 / math.sqrt(d)
    q, k, v = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v))
    o, lse = fa.attention_forward_kv(q, k, v, scale, causal, num_splits=splits)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attn_fwd_materialised(inp.q, inp.k, inp.v, scale, causal)
    check_rows(from_dev(o), from_dev(lse), O_ref, L_ref, f"{shape} causal={causal} splits={splits}")


# Uniform batches at d = 128 whose row blocks see 4096 keys or more on
# average, with 1024 packed rows or more and one split, run in eight-wave
# workgroups (256 rows per block of keys): ragged rows and keys here.
KV_EIGHT = [
    # B, Hq, Hkv, Nq, Nk
    (1, 4, 1, 300, 4500),
    (2, 8, 2, 257, 4300),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", KV_EIGHT, ids=["x".join(map(str, s)) for s in KV_EIGHT])
def test_kv_eight_wave_parity(shape, causal):
    B, Hq, Hkv, Nq, Nk = shape
    d = 128
    announce(f"kv eight-wave shape={shape} causal={causal} seed=33")
    inp = make_kv_inputs(B, Hq, Hkv, Nq, Nk, d, seed=33)
    scale = 1.0 / math.sqrt(d)
    q, k, v = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v))
    o, lse = fa.attention_forward_kv(q, k, v, scale, causal, num_splits=1)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attn_fwd_materialised(inp.q, inp.k, inp.v, scale, causal)
    check_rows(from_dev(o), from_dev(lse), O_ref, L_ref, f"{shape} causal={causal} eight waves")


def test_kv_split_matches_unsplit():
    """Split keys change only the rounding order: lse to fp32 rounding, O to one bf16 step."""
    B, Hq, Hkv, Nq, Nk, d = 2, 8, 2, 2, 5000, 128
    announce(f"kv split vs unsplit shape={(B, Hq, Hkv, Nq, Nk, d)} seed=32")
    inp = make_kv_inputs(B, Hq, Hkv, Nq, Nk, d, seed=32)
    q, k, v = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v))
    o1, l1 = fa.attention_forward_kv(q, k, v, 1.0 / math.sqrt(d), True, num_splits=1)
    for s in (2, 7, 40):
        o2, l2 = fa.attention_forward_kv(q, k, v, 1.0 / math.sqrt(d), True, num_splits=s)
        torch.cuda.synchronize()
        assert float((l1 - l2).abs().max()) <= 1e-5, f"lse splits={s}"
        assert float((o1.float() - o2.float()).abs().max()) <= 8e-3, f"O splits={s}"


def test_kv_square_equals_oracle_like_square_kernel():
    """Nq == Nk with one split is the square problem: same oracle bounds as flash_attn_fwd."""
    B, Hq, Hkv, N, d = 1, 4, 2, 300, 128
    announce(f"kv square shape={(B, Hq, Hkv, N, d)} seed=33")
    inp = make_kv_inputs(B, Hq, Hkv, N, N, d, seed=33)
    q, k, v = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v))
    for causal in (False, True):
        o, lse = fa.attention_forward_kv(q, k, v, 1.0 / math.sqrt(d), causal, num_splits=1)
        o_sq, lse_sq = fa.attention_forward(q, k, v, 1.0 / math.sqrt(d), causal)
        torch.cuda.synchronize()
        O_ref, L_ref = oracle.attn_fwd_materialised(inp.q, inp.k, inp.v, 1.0 / math.sqrt(d), causal)
        check_rows(from_dev(o), from_dev(lse), O_ref, L_ref, f"square causal={causal}")
        assert float((lse - lse_sq).abs().max()) <= 1e-4, "lse of the two kernels"


VARLEN = [
    # cu_q, cu_k: empty query range, key-less sequence, one-token sequence, ragged tails
    ([0, 3, 3, 70, 71, 200], [0, 100, 164, 164, 400, 650]),
    ([0, 40, 90], [0, 40, 90]),
]


@pytest.mark.parametrize("splits", [1, 2, 0])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", range(len(VARLEN)))
def test_varlen_small_parity(case, causal, splits):
    cu_q, cu_k = VARLEN[case]
    Hq, Hkv, d = 4, 2, 128
    announce(f"varlen small cu_q={cu_q} cu_k={cu_k} causal={causal} splits={splits} seed=34")
    inp = make_varlen_inputs(Hq, Hkv, cu_q, cu_k, d, seed=34)
    q, k, v = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v))
    cq = torch.tensor(cu_q, dtype=torch.int32, device="cuda")
    ck = torch.tensor(cu_k, dtype=torch.int32, device="cuda")
    mq = int(np.diff(cu_q).max())
    mk = int(np.diff(cu_k).max())
    o, lse = fa.attention_forward_varlen(q, k, v, cq, ck, mq, mk, 1.0 / math.sqrt(d), causal, num_splits=splits)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attn_fwd_varlen(inp.q, inp.k, inp.v, cu_q, cu_k, 1.0 / math.sqrt(d), causal)
    check_rows(from_dev(o), from_dev(lse), O_ref, L_ref, f"varlen case={case} causal={causal} splits={splits}")


def _kv_full(name):
    w = KV_WORKLOADS[name]
    if w.lengths_seed:
        lens = varlen_lengths(w.B, w.Nq_lo, w.Nq, w.lengths_seed)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        inp = make_varlen_inputs(w.Hq, w.Hkv, cu, cu, w.d, w.seed)
        return w, inp, cu
    return w, make_kv_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.seed), None


@pytest.mark.parametrize("name", ["decode_32k", "chunk_2k_8k", "chunk_wide_2k_8k"])
def test_kv_full_size_sampled(name):
    w, inp, _ = _kv_full(name)
    announce(f"kv full {name} shape=({w.B},{w.Hq},{w.Hkv},{w.Nq},{w.Nk},{w.d}) seed={w.seed}")
    q, k, v = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v))
    o, lse = fa.attention_forward_kv(q, k, v, w.scale, w.causal, num_splits=w.num_splits)
    torch.cuda.synchronize()
    O, L = from_dev(o), from_dev(lse)
    rng = np.random.default_rng(900 + w.seed)
    G = w.Hq // w.Hkv
    for p in rng.choice(w.B * w.Hq, size=6, replace=False):
        b, hq = divmod(int(p), w.Hq)
        rows = np.unique(np.concatenate([[0, w.Nq - 1], rng.choice(w.Nq, size=min(8, w.Nq), replace=False)]))
        O_ref, L_ref = oracle.attn_fwd_head(inp.q[b, hq], inp.k[b, hq // G], inp.v[b, hq // G], w.scale, w.causal,
                                            rows=rows)
        check_rows(O[b, hq, rows], L[b, hq, rows], O_ref, L_ref, f"{name} b={b} hq={hq}")


def test_varlen_full_size_sampled():
    w, inp, cu = _kv_full("varlen_mix")
    announce(f"varlen full varlen_mix B={w.B} Tq={int(cu[-1])} seed={w.seed}")
    q, k, v = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v))
    cq = torch.tensor(cu, dtype=torch.int32, device="cuda")
    mx = int(np.diff(cu).max())
    o, lse = fa.attention_forward_varlen(q, k, v, cq, cq, mx, mx, w.scale, w.causal, num_splits=w.num_splits)
    torch.cuda.synchronize()
    O, L = from_dev(o), from_dev(lse)
    rng = np.random.default_rng(901)
    G = w.Hq // w.Hkv
    for b in range(w.B):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        hq = int(rng.integers(w.Hq))
        rows = np.unique(np.concatenate([[0, t1 - t0 - 1], rng.choice(t1 - t0, size=min(4, t1 - t0), replace=False)]))
        O_ref, L_ref = oracle.attn_fwd_head(inp.q[hq, t0:t1], inp.k[hq // G, t0:t1], inp.v[hq // G, t0:t1], w.scale,
                                            w.causal, rows=rows)
        check_rows(O[hq, t0 + rows], L[hq, t0 + rows], O_ref, L_ref, f"varlen_mix seq={b} hq={hq}")


def test_kv_decode_very_long_cache():
    """One decode step over a 262144-key cache (MQA: 8 query heads on one K/V
    head, d = 128) with the library's split count, against the oracle on every
    row, and the same step with one split."""
    B, Hq, Hkv, Nq, Nk, d = 1, 8, 1, 1, 262144, 128
    announce(f"kv very long cache shape={(B, Hq, Hkv, Nq, Nk, d)} seed=35")
    inp = make_kv_inputs(B, Hq, Hkv, Nq, Nk, d, seed=35)
    q, k, v = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v))
    O_ref, L_ref = oracle.attn_fwd_materialised(inp.q, inp.k, inp.v, 1.0 / math.sqrt(d), True)
    for splits in (0, 1):
        o, lse = fa.attention_forward_kv(q, k, v, 1.0 / math.sqrt(d), True, num_splits=splits)
        torch.cuda.synchronize()
        check_rows(from_dev(o), from_dev(lse), O_ref, L_ref, f"very long cache splits={splits}")


def test_kv_two_grid_rows():
    """A grid of more than 65536 workgroups, laid out over two grid rows: 64
    sequences x 8 K/V heads x 256 splits of a 1000-key cache (split 16 on
    hold no key), every row against the oracle."""
    B, Hq, Hkv, Nq, Nk, d = 64, 8, 8, 1, 1000, 128
    announce(f"kv two grid rows shape={(B, Hq, Hkv, Nq, Nk, d)} splits=256 seed=36")
    inp = make_kv_inputs(B, Hq, Hkv, Nq, Nk, d, seed=36)
    q, k, v = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v))
    O_ref, L_ref = oracle.attn_fwd_materialised(inp.q, inp.k, inp.v, 1.0 / math.sqrt(d), True)
    o, lse = fa.attention_forward_kv(q, k, v, 1.0 / math.sqrt(d), True, num_splits=256)
    torch.cuda.synchronize()
    check_rows(from_dev(o), from_dev(lse), O_ref, L_ref, "two grid rows")


MANY = [(64, 4, 2), (64, 16, 8), (256, 4, 2), (300, 4, 2)]


@pytest.mark.parametrize("n_seq,Hq,Hkv", MANY, ids=["64-compact", "64-compact-xcd-heads", "256-compact", "300-full-grid"])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_many_sequences(n_seq, Hq, Hkv, causal):
    """Many short sequences (0-150 queries, 0-200 keys each, seeded): the
    compact grid of the sequences' row blocks (64 sequences: ranked longest
    first; 256: found by a prefix sum over four chunks of 64, the largest
    batch that takes the compact grid; 8 K/V heads: the order that gives each
    XCD its own heads) and the full grid of max_seqlen row blocks per
    sequence (300 sequences); every row against the oracle."""
    rng = np.random.default_rng(1000 + n_seq)
    lq = rng.integers(0, 151, size=n_seq)
    lk = rng.integers(0, 201, size=n_seq)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    d = 64
    announce(f"varlen many sequences n_seq={n_seq} Hq={Hq} Hkv={Hkv} Tq={int(cu_q[-1])} Tk={int(cu_k[-1])} "
             f"causal={causal} seed=37")
    inp = make_varlen_inputs(Hq, Hkv, cu_q, cu_k, d, seed=37)
    q, k, v = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v))
    cq = torch.tensor(cu_q, dtype=torch.int32, device="cuda")
    ck = torch.tensor(cu_k, dtype=torch.int32, device="cuda")
    mq, mk = int(lq.max()), int(lk.max())
    o, lse = fa.attention_forward_varlen(q, k, v, cq, ck, mq, mk, 1.0 / math.sqrt(d), causal, num_splits=1)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attn_fwd_varlen(inp.q, inp.k, inp.v, cu_q, cu_k, 1.0 / math.sqrt(d), causal)
    check_rows(from_dev(o), from_dev(lse), O_ref, L_ref, f"varlen n_seq={n_seq} causal={causal}")
