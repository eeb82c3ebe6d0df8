"""Seeded synthetic inputs for the attention hot path.

This module holds no attention arithmetic. It draws the tensors that both the
GPU path and the CPU oracle consume, so that the two sides see the very same
values:

* Q ``[B, Hq, N, d]``, K ``[B, Hkv, N, d]``, V ``[B, Hkv, N, d]`` and, for the
  backward, dO ``[B, Hq, N, d]`` are i.i.d. standard normal float32 draws from
  ``numpy.random.default_rng(seed)``, taken in that order.
* Optionally a fraction of the flattened query rows (B*Hq*N rows) is chosen
  without replacement after the draws above and multiplied by a power of two,
  so the scaling is exact. It forces large jumps of the running maximum.
* For bf16 workloads every value is rounded fp32 -> bf16 with
  round-to-nearest-even; the arrays stay float32 (holding bf16-representable
  values) and :func:`bf16_bits` gives the raw 16-bit patterns.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "bf16_round",
    "bf16_bits",
    "bits_to_f32",
    "AttnInputs",
    "make_inputs",
    "make_kv_inputs",
    "make_varlen_inputs",
]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bf16. Inputs must
    be finite (the generators only produce finite values).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Raw bf16 bit patterns (uint16) of float32 values already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("bf16_bits: values are not bf16-representable; call bf16_round first")
    return (u >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """float32 values of raw bf16 bit patterns (uint16)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class AttnInputs:
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray | None
    dtype: str
    seed: int
    heavy_rows: np.ndarray | None  # flattened (b*Hq + hq)*N + i indices scaled up


def make_inputs(
    B: int,
    Hq: int,
    Hkv: int,
    N: int,
    d: int,
    seed: int,
    dtype: str = "bf16",
    heavy_frac: float = 0.0,
    heavy_scale: float = 8.0,
    with_dout: bool = False,
    q_zero: bool = False,
) -> AttnInputs:
    """Draw one workload's tensors.

    ``dtype`` is ``"bf16"`` (values rounded to bf16, RNE) or ``"f32"``.
    ``heavy_frac`` selects ``(B*Hq*N) * heavy_frac`` query rows (rounded down)
    and multiplies them by ``heavy_scale`` (a power of two).
    ``q_zero`` replaces Q by zeros after all draws (the draws stay identical).
    """
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, N, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, N, d), dtype=np.float32)
    do = rng.standard_normal((B, Hq, N, d), dtype=np.float32) if with_dout else None
    heavy = None
    if heavy_frac > 0.0:
        rows = B * Hq * N
        count = int(rows * heavy_frac)
        heavy = np.sort(rng.choice(rows, size=count, replace=False))
        q.reshape(rows, d)[heavy] *= np.float32(heavy_scale)
    if q_zero:
        q[...] = 0.0
    if dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
        if do is not None:
            do = bf16_round(do)
    return AttnInputs(q=q, k=k, v=v, do=do, dtype=dtype, seed=seed, heavy_rows=heavy)


def make_kv_inputs(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, seed: int,
                   with_dout: bool = False) -> AttnInputs:
    """Rectangular problem: Q ``[B, Hq, Nq, d]``, K and V ``[B, Hkv, Nk, d]``
    (and dO shaped like Q when ``with_dout``), i.i.d. standard normal float32
    draws in that order, rounded to bf16."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Nq, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    do = bf16_round(rng.standard_normal((B, Hq, Nq, d), dtype=np.float32)) if with_dout else None
    return AttnInputs(q=bf16_round(q), k=bf16_round(k), v=bf16_round(v), do=do, dtype="bf16", seed=seed,
                      heavy_rows=None)


def make_varlen_inputs(Hq: int, Hkv: int, cu_q, cu_k, d: int, seed: int, with_dout: bool = False) -> AttnInputs:
    """Variable-length batch packed along the token axis: Q ``[Hq, Tq, d]``,
    K and V ``[Hkv, Tk, d]`` with Tq = cu_q[-1], Tk = cu_k[-1] (and dO shaped
    like Q when ``with_dout``); i.i.d. standard normal float32 draws in that
    order, rounded to bf16."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Hq, int(cu_q[-1]), d), dtype=np.float32)
    k = rng.standard_normal((Hkv, int(cu_k[-1]), d), dtype=np.float32)
    v = rng.standard_normal((Hkv, int(cu_k[-1]), d), dtype=np.float32)
    do = bf16_round(rng.standard_normal((Hq, int(cu_q[-1]), d), dtype=np.float32)) if with_dout else None
    return AttnInputs(q=bf16_round(q), k=bf16_round(k), v=bf16_round(v), do=do, dtype="bf16", seed=seed,
                      heavy_rows=None)


def varlen_lengths(n_seq: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Sequence lengths of a variable-length batch: log-uniform integers in
    [lo, hi] (many short sequences, a few long ones), seeded."""
    rng = np.random.default_rng(seed)
    return np.exp(rng.uniform(np.log(lo), np.log(hi + 1), size=n_seq)).astype(np.int64).clip(lo, hi)
