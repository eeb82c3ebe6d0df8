"""Helpers shared by the GPU parity tests: device upload, error metrics, tolerances."""

from __future__ import annotations

import numpy as np

# bf16 storage with fp32 accumulation: elementwise max-abs and mean-abs of O
# (and of dQ, dK, dV) against the fp64 oracle.
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
# lse carries no bf16 rounding (fp32 output): absolute bound.
BF16_LSE_ABS = 1e-3
# fp32 check mode: normwise relative, max|diff| / max|ref|.
F32_REL = 1e-5


def to_dev(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def from_dev(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    return float(d.max()), float(d.mean())


def assert_close(got, ref, dtype, what, lse=False, ref_scale=None, storage_rounding=False):
    """Compare against the oracle. fp32 mode is normwise: max|diff| over
    max|ref| of this output. ``ref_scale`` replaces max|ref| only for an
    output that is exactly zero in exact arithmetic (dQ and dK when N = 1),
    which is then judged against the size of the terms that cancel in it.
    ``storage_rounding`` (bf16 only, for workloads whose outputs reach
    magnitudes where one bf16 rounding step exceeds the absolute bound:
    half an ulp is 2^-8 |x| at worst, 0.031 for |x| in [8, 16)) adds the
    storage rounding of each reference value to the absolute bound:
    |got - ref| <= 2e-2 + 2^-8 |ref| elementwise."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    mx, mean = errors(got, ref)
    if dtype == "f32":
        scale = max(float(np.abs(ref).max()) if ref_scale is None else ref_scale, 1e-30)
        assert mx <= F32_REL * scale, f"{what}: max|diff| {mx:.3e} > {F32_REL:.0e} * max|ref| ({scale:.3e})"
    elif lse:
        assert mx <= BF16_LSE_ABS, f"{what}: lse max-abs {mx:.3e} > {BF16_LSE_ABS}"
    elif storage_rounding:
        excess = np.abs(got - ref) - (BF16_MAX_ABS + 2.0 ** -8 * np.abs(ref))
        assert float(excess.max()) <= 0.0, f"{what}: |diff| exceeds 2e-2 + 2^-8 |ref| by {float(excess.max()):.3e}"
        assert mean <= BF16_MEAN_ABS, f"{what}: mean-abs {mean:.3e} > {BF16_MEAN_ABS}"
    else:
        assert mx <= BF16_MAX_ABS, f"{what}: max-abs {mx:.3e} > {BF16_MAX_ABS}"
        assert mean <= BF16_MEAN_ABS, f"{what}: mean-abs {mean:.3e} > {BF16_MEAN_ABS}"
    return mx, mean


def announce(msg: str) -> None:
    """Name the case about to run on the GPU, unbuffered and past pytest's capture."""
    import sys
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def sample_rows(rng, B, Hq, N, n_heads, n_rows, heavy=None):
    """Pick (b, hq) pairs and, per pair, query rows to check one by one.

    Always includes rows 0, 1 and N-1 and every heavy (scaled-up) row of the
    pair; the rest are uniform without replacement."""
    pairs = [(int(x) // Hq, int(x) % Hq) for x in rng.choice(B * Hq, size=min(n_heads, B * Hq), replace=False)]
    out = []
    for b, hq in pairs:
        rows = set(int(r) for r in rng.choice(N, size=min(n_rows, N), replace=False))
        rows |= {0, min(1, N - 1), N - 1}
        if heavy is not None:
            base = (b * Hq + hq) * N
            hv = heavy[(heavy >= base) & (heavy < base + N)] - base
            rows |= set(int(r) for r in hv)
        out.append((b, hq, np.array(sorted(rows), dtype=np.int64)))
    return out
