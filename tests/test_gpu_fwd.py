"""GPU forward parity against the fp64 oracle, through the C ABI.

Small shapes (several tiles, ragged tails, GQA, every head dim, both mask
modes, bf16 and the fp32 check mode) are compared element by element on every
output. The full-size workloads run in the launch configuration the benchmark
times and are compared on sampled query rows that the oracle computes one by
one, plus properties that hold at any size."""

import math

import numpy as np
import pytest

import oracle
from online_softmax_flash_amd.inputs import make_inputs
from online_softmax_flash_amd.workloads import WORKLOADS
from parity_util import announce, assert_close, from_dev, sample_rows, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import online_softmax_flash_amd as fa  # noqa: E402


def run_fwd(inp, scale, causal):
    q, k, v = (to_dev(x, inp.dtype) for x in (inp.q, inp.k, inp.v))
    o, lse = fa.attention_forward(q, k, v, scale, causal)
    torch.cuda.synchronize()
    return o, lse


SMALL = [
    # B, Hq, Hkv, N, d
    (1, 2, 2, 1, 64),
    (1, 2, 1, 17, 64),
    (2, 4, 2, 255, 128),
    (1, 2, 2, 300, 128),
    (1, 4, 1, 1000, 64),
    (1, 2, 2, 130, 256),
    (1, 3, 3, 384, 256),
    (2, 2, 2, 129, 128),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=["x".join(map(str, s)) for s in SMALL])
def test_fwd_small_full_parity(shape, causal, dtype):
    B, Hq, Hkv, N, d = shape
    announce(f"fwd small shape={shape} causal={causal} dtype={dtype} seed=11")
    inp = make_inputs(B, Hq, Hkv, N, d, seed=11, dtype=dtype)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_fwd(inp, scale, causal)
    O_ref, L_ref = oracle.attn_fwd_materialised(inp.q, inp.k, inp.v, scale, causal)
    assert_close(from_dev(o), O_ref, dtype, f"O {shape} causal={causal}")
    assert_close(from_dev(lse), L_ref, dtype, f"lse {shape} causal={causal}", lse=True)


def test_fwd_tiny_workload_and_qzero():
    """Tiny fp32 workload (B=1, H=2, N=256, d=64, non-causal, seed 0), and the
    same shape with Q = 0: O = mean of V, lse = ln 256."""
    w = WORKLOADS["tiny_f32"]
    for qz in (False, True):
        announce(f"fwd tiny_f32 q_zero={qz}")
        inp = make_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, seed=w.seed, dtype="f32", q_zero=qz)
        o, lse = run_fwd(inp, w.scale, False)
        O_ref, L_ref = oracle.attn_fwd_materialised(inp.q, inp.k, inp.v, w.scale, False)
        assert_close(from_dev(o), O_ref, "f32", f"tiny O q_zero={qz}")
        assert_close(from_dev(lse), L_ref, "f32", f"tiny lse q_zero={qz}", lse=True)
        if qz:
            mean_v = inp.v.astype(np.float64).mean(axis=2, keepdims=True)
            assert_close(from_dev(o), np.broadcast_to(mean_v, o.shape), "f32", "Q=0 closed form")
            assert np.max(np.abs(from_dev(lse) - math.log(256))) <= 1e-5 * math.log(256)


def test_fwd_scale_zero_uniform():
    """scale = 0: uniform weights over the visible keys (prefix means when causal)."""
    inp = make_inputs(1, 2, 2, 200, 64, seed=12, dtype="f32")
    announce("fwd scale=0 causal")
    o, lse = run_fwd(inp, 0.0, True)
    cnt = np.arange(1, 201, dtype=np.float64)
    mean = np.cumsum(inp.v.astype(np.float64), axis=2) / cnt[None, None, :, None]
    assert_close(from_dev(o), mean, "f32", "scale=0 prefix means")
    assert np.max(np.abs(from_dev(lse) - np.log(cnt)[None, None])) <= 1e-5 * math.log(200)


FULL = [(n, c) for n in ("fwd_2k", "long_8k", "long_16k", "gqa_4k", "wide_4k", "bwd_4k", "short_256", "short_512")
        for c in WORKLOADS[n].causal]


@pytest.mark.parametrize("name,causal", FULL, ids=[f"{n}-{'causal' if c else 'full'}" for n, c in FULL])
def test_fwd_full_size_sampled(name, causal):
    w = WORKLOADS[name]
    announce(f"fwd full {name} causal={causal} shape=({w.B},{w.Hq},{w.Hkv},{w.N},{w.d}) seed={w.seed}")
    inp = make_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, seed=w.seed, dtype=w.dtype, heavy_frac=w.heavy_frac)
    o, lse = run_fwd(inp, w.scale, causal)
    o_h = o.float().cpu().numpy()
    lse_h = lse.cpu().numpy()
    assert np.all(np.isfinite(o_h)) and np.all(np.isfinite(lse_h))
    rng = np.random.default_rng(1000 + w.seed)
    G = w.Hq // w.Hkv
    worst = 0.0
    for b, hq, rows in sample_rows(rng, w.B, w.Hq, w.N, 6, 48, inp.heavy_rows):
        g = hq // G
        O_ref, L_ref = oracle.attn_fwd_head(inp.q[b, hq], inp.k[b, g], inp.v[b, g], w.scale, causal, rows=rows)
        mx, _ = assert_close(o_h[b, hq, rows], O_ref, "bf16", f"{name} O b={b} hq={hq}")
        assert_close(lse_h[b, hq, rows], L_ref, "bf16", f"{name} lse b={b} hq={hq}", lse=True)
        worst = max(worst, mx)
    if causal:
        # Row 0 sees key 0 only: O_0 = v_0 exactly, lse_0 = scale * q_0 . k_0.
        for b in range(w.B):
            for hq in range(w.Hq):
                g = hq // G
                assert np.array_equal(o_h[b, hq, 0], inp.v[b, g, 0]), f"row 0 b={b} hq={hq}"
        s0 = w.scale * np.einsum("bhd,bhd->bh", inp.q[:, :, 0].astype(np.float64),
                                 np.repeat(inp.k[:, :, 0], G, axis=1).astype(np.float64))
        assert np.max(np.abs(lse_h[:, :, 0] - s0)) <= 1e-5 * (1 + np.abs(s0).max())
    print(f"{name} causal={causal}: worst sampled max-abs {worst:.3e}")


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_fwd_2k_every_element(causal):
    """The B=4, H=32, N=2048, d=128 workload (seed 1) compared on every
    element of O and lse: 1024 work items on one persistent workgroup per
    compute unit, so every workgroup runs several items (the mirrored item
    order of odd rounds, the next item's first K/V block copied into the
    stage the last block freed, its query rows read behind the last block's
    score products)."""
    w = WORKLOADS["fwd_2k"]
    announce(f"fwd every element fwd_2k causal={causal} seed={w.seed}")
    inp = make_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, seed=w.seed, dtype=w.dtype)
    o, lse = run_fwd(inp, w.scale, causal)
    O_ref, L_ref = oracle.attn_fwd_materialised(inp.q, inp.k, inp.v, w.scale, causal)
    assert_close(from_dev(o), O_ref, "bf16", f"fwd_2k O causal={causal}")
    assert_close(from_dev(lse), L_ref, "bf16", f"fwd_2k lse causal={causal}", lse=True)


MULTI_ROUND = [
    # B, Hq, Hkv, N, d: 4 query blocks of 256 x 128 heads = 512 items, two
    # rounds over 256 persistent workgroups; ragged N; GQA and MQA-like groups.
    (2, 64, 64, 1000, 64),
    (2, 64, 16, 1000, 128),
    (2, 64, 64, 1024, 128),
    (1, 128, 8, 777, 64),
    # d = 64 on a long sequence takes 16-wave workgroups (512 rows): 5 query
    # blocks x 128 heads = 640 items, three rounds; ragged N; GQA.
    (1, 128, 16, 2100, 64),
]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("shape", MULTI_ROUND, ids=["x".join(map(str, s)) for s in MULTI_ROUND])
def test_fwd_multi_round_every_element(shape, causal):
    """More work items than compute units at d <= 128: each persistent
    workgroup runs a second item (and the hand-off between items), compared
    element by element against the oracle."""
    B, Hq, Hkv, N, d = shape
    announce(f"fwd multi-round shape={shape} causal={causal} seed=13")
    inp = make_inputs(B, Hq, Hkv, N, d, seed=13)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_fwd(inp, scale, causal)
    O_ref, L_ref = oracle.attn_fwd_materialised(inp.q, inp.k, inp.v, scale, causal)
    assert_close(from_dev(o), O_ref, "bf16", f"O {shape} causal={causal}")
    assert_close(from_dev(lse), L_ref, "bf16", f"lse {shape} causal={causal}", lse=True)


def test_fwd_repeatable_and_allocation_free():
    """Two runs give identical bits; a call allocates no device memory."""
    w = WORKLOADS["fwd_2k"]
    announce("fwd repeat/alloc fwd_2k causal")
    inp = make_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, seed=w.seed)
    q, k, v = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v))
    o1, l1 = fa.attention_forward(q, k, v, w.scale, True)
    o2 = torch.empty_like(q)
    l2 = torch.empty_like(l1)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    fa.flash_attn_fwd(q, k, v, o2, l2, w.scale, True)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    assert free1 == free0, f"device free memory changed by {free0 - free1} bytes during a call"


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fwd_very_long_single_head(d):
    """One head at N = 65536 (the longest sequence in any test; 2^32 scores per
    head, never stored), causal and full, on sampled rows including the first
    and last, plus a query block boundary in the ragged layout N - 1."""
    N = 65536 - 1  # ragged: not a multiple of any tile size
    announce(f"fwd very long N={N} d={d} seed=61")
    inp = make_inputs(1, 1, 1, N, d, seed=61)
    scale = 1.0 / math.sqrt(d)
    for causal in (True, False):
        o, lse = run_fwd(inp, scale, causal)
        o_h = o.float().cpu().numpy()
        lse_h = lse.cpu().numpy()
        rows = np.array([0, 1, 255, 256, 32767, 40000, N - 2, N - 1])
        O_ref, L_ref = oracle.attn_fwd_head(inp.q[0, 0], inp.k[0, 0], inp.v[0, 0], scale, causal, rows=rows)
        assert_close(o_h[0, 0, rows], O_ref, "bf16", f"N={N} d={d} causal={causal} O")
        assert_close(lse_h[0, 0, rows], L_ref, "bf16", f"N={N} d={d} causal={causal} lse", lse=True)


@pytest.mark.parametrize("case", ["jump", "overflow"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_fwd_late_maximum_jump(d, case):
    """Running maximum that jumps in a later, unmasked key block. Key 150 (the
    third 64-key block) is set to alpha * q_900, so query 900 and the rows
    whose queries align with it score far above everything in the first two
    blocks: by about 8 to 17 (alpha = 1) and by 170 to 240 (alpha = 16, or 8
    at d = 256) in log2 units, where a weight taken against the earlier
    maximum would overflow fp32. The kernels must raise their reference
    maximum as the block maximum dictates; compared element by element
    against the oracle, both masks."""
    alpha = 1.0 if case == "jump" else (16.0 if d <= 128 else 8.0)
    B, H, N = 1, 2, 1024
    announce(f"fwd late max jump d={d} alpha={alpha} seed=71")
    inp = make_inputs(B, H, H, N, d, seed=71)
    k = inp.k.copy()
    k[:, :, 150, :] = alpha * inp.q[:, :, 900, :]  # power-of-two multiple of bf16 values: exact
    scale = 1.0 / math.sqrt(d)
    q_d, k_d, v_d = (to_dev(x, "bf16") for x in (inp.q, k, inp.v))
    for causal in (False, True):
        o, lse = fa.attention_forward(q_d, k_d, v_d, scale, causal)
        torch.cuda.synchronize()
        O_ref, L_ref = oracle.attn_fwd_materialised(inp.q, k, inp.v, scale, causal)
        assert np.abs(L_ref[:, :, 900]).min() > (100.0 if alpha > 1 else 5.0)
        assert_close(from_dev(o), O_ref, "bf16", f"O d={d} alpha={alpha} causal={causal}")
        assert_close(from_dev(lse), L_ref, "bf16", f"lse d={d} alpha={alpha} causal={causal}", lse=True)
