"""The named synthetic workloads of the attention hot path (shapes, seeds, modes).

Each entry is data only: shapes, seed, dtype, which mask modes are run and how
the inputs are drawn (see :mod:`online_softmax_flash_amd.inputs`). The scale is
always 1/sqrt(d), the scaled dot product of the score definition.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str  # "bf16" or "f32"
    causal: tuple  # mask modes exercised
    seed: int
    heavy_frac: float = 0.0
    backward: bool = False
    note: str = ""
    bound: str = "mfma"  # what limits the forward at this shape: "mfma" or "hbm" (short sequences)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def fwd_flops(self, causal: bool) -> float:
        """Credited forward flops: 4*B*Hq*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.Hq * self.N * self.N * self.d
        return f / 2.0 if causal else f

    def bwd_flops(self, causal: bool) -> float:
        """Credited backward flops (five N^2*d contractions): 10*B*Hq*N^2*d, halved causal."""
        f = 10.0 * self.B * self.Hq * self.N * self.N * self.d
        return f / 2.0 if causal else f

    def min_fwd_bytes(self) -> int:
        """Smallest possible forward HBM traffic: read Q, K, V once, write O and lse once."""
        e = 2 if self.dtype == "bf16" else 4
        qo = self.B * self.Hq * self.N * self.d * e
        kv = self.B * self.Hkv * self.N * self.d * e
        lse = self.B * self.Hq * self.N * 4
        return 2 * qo + 2 * kv + lse


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32", 1, 2, 2, 256, 64, "f32", (False,), 0,
                 note="tiny oracle check, fp32 check mode; also run with Q=0"),
        Workload("fwd_2k", 4, 32, 32, 2048, 128, "bf16", (False, True), 1),
        Workload("long_8k", 1, 32, 32, 8192, 128, "bf16", (True,), 2, heavy_frac=0.01,
                 note="1% of query rows scaled x8"),
        Workload("long_16k", 1, 32, 32, 16384, 128, "bf16", (True,), 2, heavy_frac=0.01,
                 note="1% of query rows scaled x8"),
        Workload("gqa_4k", 2, 32, 8, 4096, 128, "bf16", (True,), 3),
        Workload("wide_4k", 2, 16, 16, 4096, 256, "bf16", (False,), 3),
        Workload("bwd_4k", 2, 16, 16, 4096, 128, "bf16", (True,), 4, backward=True),
        # Short sequences: N/2 flop per byte, below the MI355X ridge (about 315
        # flop/B), so the forward is bound by HBM bandwidth there.
        Workload("short_256", 16, 32, 32, 256, 128, "bf16", (False,), 5, bound="hbm",
                 note="HBM-bound line: minimum traffic Q+K+V+O+lse over time"),
        Workload("short_512", 16, 32, 32, 512, 128, "bf16", (False,), 5, bound="hbm",
                 note="HBM-bound line: minimum traffic Q+K+V+O+lse over time"),
    ]
}

# The workload the headline throughput is quoted on.
HEADLINE = "long_8k"


@dataclass(frozen=True)
class KvWorkload:
    """Rectangular or variable-length problems of the general forward (bottom-right
    causal mask), with the key range split over workgroups (num_splits = 0: the
    library's choice). ``lengths_seed`` > 0 makes it a variable-length batch of
    B sequences, query and key lengths drawn by inputs.varlen_lengths in
    [Nq_lo, Nq] and [Nk_lo, Nk]."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    seed: int
    num_splits: int = 0
    Nq_lo: int = 0
    Nk_lo: int = 0
    lengths_seed: int = 0
    note: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def lengths(self):
        """Per-sequence (query, key) lengths."""
        if not self.lengths_seed:
            return [(self.Nq, self.Nk)] * self.B
        from .inputs import varlen_lengths
        lens = varlen_lengths(self.B, self.Nq_lo, self.Nq, self.lengths_seed)
        return [(int(n), int(n)) for n in lens]

    def visible_pairs(self) -> int:
        """(query, key) pairs the mask keeps, summed over sequences (one head)."""
        tot = 0
        for nq, nk in self.lengths():
            if not self.causal:
                tot += nq * nk
            else:
                # query i sees min(nk, max(0, i + nk - nq + 1)) keys
                for i in range(nq):
                    tot += min(nk, max(0, i + nk - nq + 1))
        return tot

    def fwd_flops(self) -> float:
        """Credited flops: 4*d per visible (query, key) pair and query head."""
        return 4.0 * self.d * self.Hq * self.visible_pairs()

    def min_bytes(self) -> int:
        """Smallest HBM traffic: read Q, K, V once, write O (bf16) and lse once."""
        tq = sum(nq for nq, _ in self.lengths())
        tk = sum(nk for _, nk in self.lengths())
        return 2 * (2 * self.Hq * tq * self.d) + 2 * (2 * self.Hkv * tk * self.d) + 4 * self.Hq * tq


KV_WORKLOADS = {
    w.name: w
    for w in [
        KvWorkload("decode_32k", 8, 32, 8, 1, 32768, 128, True, 5,
                   note="one decode step: 8 sequences, 32 query heads on 8 K/V heads, 32768 cached keys"),
        KvWorkload("chunk_2k_8k", 1, 32, 8, 2048, 8192, 128, True, 6,
                   note="chunked prefill: the last 2048 queries of an 8192-token causal prefix"),
        KvWorkload("chunk_wide_2k_8k", 1, 16, 16, 2048, 8192, 256, True, 9,
                   note="chunked prefill at d = 256: the last 2048 queries of an 8192-token causal prefix"),
        KvWorkload("varlen_mix", 16, 32, 8, 4096, 4096, 128, True, 7, Nq_lo=64, Nk_lo=64, lengths_seed=8,
                   note="16 sequences, log-uniform lengths in [64, 4096], queries = keys per sequence"),
    ]
}
