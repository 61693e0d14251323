"""Host-side logic of bench.py (no GPU): the max-affine fit of the expert-time profile."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _grid():
    G = np.repeat([1, 4, 16, 64], 10)
    n = np.tile([1, 2, 4, 16, 64, 256, 512, 1024, 2048, 4096], 4)
    N = G * n
    keep = N <= 65536
    return G[keep].astype(float), N[keep].astype(float)


def test_max_affine_fit_recovers_exact_model():
    G, N = _grid()
    t = np.maximum(30.0 + 12.0 * G, 90.0 + 0.07 * N)
    a, b, c, beta, mx, rms = bench.fit_max_affine(np.stack([G, N, t], 1))
    assert np.allclose([a, b, c, beta], [30.0, 12.0, 90.0, 0.07], rtol=1e-6)
    assert mx < 1e-9 and rms < 1e-9


def test_max_affine_fit_bounds_noisy_misfit():
    G, N = _grid()
    rng = np.random.default_rng(0)
    t = np.maximum(40.0 + 6.0 * G, 95.0 + 0.033 * N) * (1 + rng.uniform(-0.05, 0.05, G.shape))
    a, b, c, beta, mx, rms = bench.fit_max_affine(np.stack([G, N, t], 1))
    # the minimax fit can do no worse than the generating model's own misfit (5%)
    assert mx <= 0.052
    assert abs(b / beta - 6.0 / 0.033) / (6.0 / 0.033) < 0.2


def test_prefill_schedule_fills_hand_worked():
    """The schedule model's fills on cases worked out by hand (host arithmetic, no GPU)."""
    from token_dispatch_expert_amd import traffic as tr
    K = 64
    # one gated expert of 256 rows, 16 column blocks of 128: no streaming role, one round of 16
    # items in runs of 2 per XCD, so each XCD fetches the one A tile and 2 B tiles
    r = tr.prefill_schedule_fills([256], K, 2048, True)
    assert r["streaming_cus"] == 0 and r["tile_items"] == 16
    assert r["tile_fills"] == 8 * 256 * K * 2 + 16 * 256 * K * 2
    assert r["algorithmic"] == 256 * K * 2 + 2 * 2048 * K * 2
    # one plain expert of 300 rows: 19 fragments dealt 10 + 9 (160 and 140 rows) to two row
    # tiles; 8 column blocks of 256, items (row tile, column block) with the row tiles inner, so
    # each XCD's run of 2 holds both row tiles of one block
    r = tr.prefill_schedule_fills([300, 0, 0], K, 2048, False)
    assert r["tile_items"] == 16
    assert r["tile_fills"] == 8 * (300 + 256) * K * 2
    # only small experts: every CU streams, no tile fills
    r = tr.prefill_schedule_fills([8, 16, 0], K, 2048, True)
    assert r["streaming_cus"] == 256 and r["tile_fills"] == 0
    assert r["fills"] == r["streamed"] == 2 * (2 * 2048 * K * 2)
