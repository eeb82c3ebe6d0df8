"""The seeded input generator: determinism, bf16 rounding, heavy-row selection. CPU only."""

import numpy as np
import torch

from online_softmax_flash_amd.inputs import bf16_bits, bf16_round, bits_to_f32, make_inputs


def test_same_seed_same_bytes():
    a = make_inputs(1, 4, 2, 64, 16, seed=7, heavy_frac=0.05, with_dout=True)
    b = make_inputs(1, 4, 2, 64, 16, seed=7, heavy_frac=0.05, with_dout=True)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.do, b.do)):
        assert x.tobytes() == y.tobytes()
    c = make_inputs(1, 4, 2, 64, 16, seed=8)
    assert a.q.tobytes() != c.q.tobytes()


def test_bf16_round_ties_to_even_and_matches_torch():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)  # bf16 spacing at 1.0
    x = np.array([one + ulp / 2, one + 3 * ulp / 2, -(one + ulp / 2), one + ulp / 2 + 2.0 ** -20],
                 dtype=np.float32)
    r = bf16_round(x)
    assert r[0] == one  # tie -> even (1.0)
    assert r[1] == one + 2 * ulp  # tie -> even (1 + 2ulp)
    assert r[2] == -one
    assert r[3] == one + ulp  # above the tie -> up
    rng = np.random.default_rng(0)
    y = (rng.standard_normal(100000) * 10.0 ** rng.integers(-20, 20, 100000)).astype(np.float32)
    t = torch.from_numpy(y).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bf16_round(y), t)
    assert np.array_equal(bits_to_f32(bf16_bits(bf16_round(y))), bf16_round(y))


def test_heavy_rows_selection():
    B, Hq, N, d = 1, 8, 128, 4
    plain = make_inputs(B, Hq, 8, N, d, seed=2, dtype="f32")
    heavy = make_inputs(B, Hq, 8, N, d, seed=2, dtype="f32", heavy_frac=0.01)
    rows = B * Hq * N
    assert heavy.heavy_rows.shape == (rows // 100,)
    assert len(np.unique(heavy.heavy_rows)) == rows // 100
    qp = plain.q.reshape(rows, d)
    qh = heavy.q.reshape(rows, d)
    mask = np.zeros(rows, dtype=bool)
    mask[heavy.heavy_rows] = True
    assert np.array_equal(qh[mask], 8.0 * qp[mask])
    assert np.array_equal(qh[~mask], qp[~mask])


def test_bf16_workload_is_representable():
    w = make_inputs(2, 2, 1, 16, 8, seed=3, with_dout=True)
    for x in (w.q, w.k, w.v, w.do):
        assert x.dtype == np.float32
        assert np.array_equal(bf16_round(x), x)
