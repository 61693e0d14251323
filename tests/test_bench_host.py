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
