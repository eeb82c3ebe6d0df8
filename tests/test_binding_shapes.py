"""The Python binding checks every tensor's full shape before it passes a
pointer to the C ABI (which cannot see buffer sizes): a mis-shaped or short
caller-allocated tensor raises ValueError on the host instead of becoming an
out-of-bounds access on the GPU. CPU only: the tensors here live on the host,
so a call whose shapes all agree stops at the device check, which comes after
the shape checks; nothing reaches the library."""

import pytest

torch = pytest.importorskip("torch")
import online_softmax_flash_amd as fa  # noqa: E402

B, HQ, HKV, N, D = 2, 4, 2, 24, 64


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def fwd_args():
    return dict(q=bf(B, HQ, N, D), k=bf(B, HKV, N, D), v=bf(B, HKV, N, D), o=bf(B, HQ, N, D), lse=f32(B, HQ, N))


def bwd_args():
    a = fwd_args()
    a.update(dout=bf(B, HQ, N, D), dq=bf(B, HQ, N, D), dk=bf(B, HKV, N, D), dv=bf(B, HKV, N, D))
    return a


# One wrong shape per argument: a shorter sequence, a wrong head count, a
# wrong head dim, or a missing axis.
BAD = {
    "k": [(B, HKV, N - 1, D), (B, HKV, N, 32)],
    "v": [(B, HKV, N - 1, D), (B, HKV + 1, N, D), (B, HKV, N, 2 * D)],
    "o": [(B, HQ, N - 1, D), (B, HQ - 1, N, D), (B, HQ, N, 32)],
    "lse": [(B, HQ, N - 1), (B, HQ, N, 1), (B * HQ * N,)],
    "dout": [(B, HQ, N - 1, D), (1, HQ, N, D)],
    "dq": [(B, HQ, N, D // 2), (B, HQ, N + 1, D)],
    "dk": [(B, HKV, N - 1, D), (B, HQ, N, D)],
    "dv": [(B, HKV, N, D + 8), (B, HKV - 1, N, D)],
}


def _mk(name, shape):
    return f32(*shape) if name == "lse" else bf(*shape)


@pytest.mark.parametrize("fn", ["flash_attn_fwd", "flash_attn_naive_fwd"])
def test_forward_wrappers_check_shapes(fn):
    extra = {"workspace": torch.zeros(256, dtype=torch.uint8)} if fn == "flash_attn_naive_fwd" else {}
    call = getattr(fa, fn)
    for name in ("k", "v", "o", "lse"):
        for shape in BAD[name]:
            a = fwd_args()
            a[name] = _mk(name, shape)
            with pytest.raises(ValueError, match=rf"{name}: shape"):
                call(**a, scale=0.1, causal=True, **extra)
    with pytest.raises(ValueError, match="on the GPU"):
        call(**fwd_args(), scale=0.1, causal=True, **extra)


@pytest.mark.parametrize("fn", ["flash_attn_bwd", "flash_attn_bwd_f32"])
def test_backward_wrappers_check_shapes(fn):
    call = getattr(fa, fn)
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    for name in ("k", "v", "o", "lse", "dout", "dq", "dk", "dv"):
        for shape in BAD[name]:
            a = bwd_args()
            a[name] = _mk(name, shape)
            with pytest.raises(ValueError, match=rf"{name}: shape"):
                call(**a, workspace=ws, scale=0.1, causal=True)
    with pytest.raises(ValueError, match="on the GPU"):
        call(**bwd_args(), workspace=ws, scale=0.1, causal=True)


def test_kv_wrapper_checks_shapes():
    NQ, NK = 5, 40

    def args():
        return dict(q=bf(B, HQ, NQ, D), k=bf(B, HKV, NK, D), v=bf(B, HKV, NK, D), o=bf(B, HQ, NQ, D),
                    lse=f32(B, HQ, NQ))

    bad = {"k": (B, HKV, NK, 32), "v": (B, HKV, NK - 1, D), "o": (B, HQ, NQ + 1, D), "lse": (B, HQ, NK)}
    for name, shape in bad.items():
        a = args()
        a[name] = _mk(name, shape)
        with pytest.raises(ValueError, match=": shape"):
            fa.flash_attn_fwd_kv(**a, scale=0.1, causal=True)
    with pytest.raises(ValueError, match="on the GPU"):
        fa.flash_attn_fwd_kv(**args(), scale=0.1, causal=True)


def test_varlen_wrapper_checks_shapes():
    TQ, TK = 30, 50
    cu = torch.tensor([0, 10, 30], dtype=torch.int32)
    cuk = torch.tensor([0, 20, 50], dtype=torch.int32)

    def args():
        return dict(q=bf(HQ, TQ, D), k=bf(HKV, TK, D), v=bf(HKV, TK, D), o=bf(HQ, TQ, D), lse=f32(HQ, TQ),
                    cu_seqlens_q=cu, cu_seqlens_k=cuk)

    bad = {"k": (HKV, TK - 1, D), "v": (HKV, TK, 2 * D), "o": (HQ - 1, TQ, D), "lse": (HQ, TQ + 1)}
    for name, shape in bad.items():
        a = args()
        a[name] = _mk(name, shape)
        with pytest.raises(ValueError, match=": shape"):
            fa.flash_attn_fwd_varlen(**a, max_seqlen_q=20, max_seqlen_k=30, scale=0.1, causal=True)
    a = args()
    a["cu_seqlens_k"] = torch.tensor([0, 50], dtype=torch.int32)  # B+1 entries must agree
    with pytest.raises(ValueError, match="cu_seqlens_k has"):
        fa.flash_attn_fwd_varlen(**a, max_seqlen_q=20, max_seqlen_k=30, scale=0.1, causal=True)
    with pytest.raises(ValueError, match="on the GPU"):
        fa.flash_attn_fwd_varlen(**args(), max_seqlen_q=20, max_seqlen_k=30, scale=0.1, causal=True)
