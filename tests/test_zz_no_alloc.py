"""flash_attn_fwd_kv_noalloc: the general forward with its split partials in
the library's static scratch (no workspace argument, no device allocation),
called through the C ABI and compared bit for bit with flash_attn_fwd_kv on a
caller-owned workspace (same kernels, same split count), on two calls in a
row, the second smaller than the first, so that the second runs over the
first one's leftover partials. Also checked against the oracle on sampled
rows, and for unchanged free device memory around every call after the
first (the first call on a device is its set-up: the HIP runtime maps the
library's static scratch onto the device when its address is first looked
up)."""

import math

import numpy as np
import pytest

import oracle
from online_softmax_flash_amd.inputs import make_kv_inputs
from parity_util import announce, assert_close, from_dev, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import online_softmax_flash_amd as fa  # noqa: E402

CASES = [
    # B, Hq, Hkv, Nq, Nk, d, causal, num_splits (0: the library's choice)
    (8, 32, 8, 1, 32768, 128, True, 0),   # a decode step over a 32768-key cache
    (2, 16, 4, 3, 5000, 64, True, 7),     # smaller, ragged, explicit split count
]


def _run_pair(case, seed):
    B, Hq, Hkv, Nq, Nk, d, causal, splits = case
    inp = make_kv_inputs(B, Hq, Hkv, Nq, Nk, d, seed)
    q, k, v = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v))
    scale = 1.0 / math.sqrt(d)
    used = splits or fa.flash_attn_fwd_kv_num_splits(B, Hq, Hkv, Nq, Nk, d)
    assert used > 1  # the scratch is in use
    o_ref, lse_ref = torch.empty_like(q), torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    n = fa.flash_attn_fwd_kv_workspace_bytes(B * Hq * Nq, d, used)
    assert 0 < n <= (32 << 20)
    ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    fa.flash_attn_fwd_kv(q, k, v, o_ref, lse_ref, scale, causal, used, ws)
    o, lse = torch.empty_like(q), torch.empty_like(lse_ref)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    fa.flash_attn_fwd_kv_noalloc(q, k, v, o, lse, scale, causal, splits)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    return inp, (o, lse), (o_ref, lse_ref), free0 - free1


def test_noalloc_matches_workspace_entry_point_twice():
    # The two cases in a row (the second smaller), then the first again.
    for i, case in enumerate(CASES + CASES[:1]):
        B, Hq, Hkv, Nq, Nk, d, causal, splits = case
        announce(f"fwd_kv_noalloc call {i + 1} case={case} seed={40 + i}")
        inp, (o, lse), (o_ref, lse_ref), grown = _run_pair(case, 40 + i)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"O differs, case {case}"
        assert torch.equal(lse, lse_ref), f"lse differs, case {case}"
        if i > 0:
            assert grown == 0, f"free device memory changed by {grown} bytes during call {i + 1}"
        G = Hq // Hkv
        o_h, lse_h = from_dev(o), from_dev(lse)
        for b, hq in ((0, 0), (B - 1, Hq - 1)):
            O_r, L_r = oracle.attn_fwd_head(inp.q[b, hq], inp.k[b, hq // G], inp.v[b, hq // G], 1.0 / math.sqrt(d),
                                            causal)
            assert_close(o_h[b, hq], O_r, "bf16", f"noalloc O b={b} hq={hq}")
            assert_close(lse_h[b, hq], L_r, "bf16", f"noalloc lse b={b} hq={hq}", lse=True)
