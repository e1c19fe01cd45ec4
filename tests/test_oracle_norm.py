"""Pins of the RMS normalisation oracle (oracle/norm.py): PyTorch's own
rms_norm in float64, a row worked by hand, and the closed forms of constant
rows and scaled rows."""

import numpy as np
import torch

from oracle import norm


def test_matches_torch_rms_norm_in_float64():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 384))
    x[:, 5] *= 40
    g = 1 + 0.1 * rng.standard_normal(384)
    for eps in (0.0, 1e-6, 1e-2):
        eps = float(np.float32(eps))
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (384,), torch.from_numpy(g), eps).numpy()
        np.testing.assert_allclose(norm.rmsnorm(x, g, eps), ref, rtol=1e-14, atol=0)


def test_a_row_worked_by_hand():
    # x = [3, 4]: mean of squares 12.5, rms sqrt(12.5) = 3.5355339...; g = [1, 2]
    y = norm.rmsnorm(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), 0.0)
    np.testing.assert_allclose(y, [[3 / 12.5 ** 0.5, 8 / 12.5 ** 0.5]], rtol=1e-15)
    np.testing.assert_allclose(y, [[0.848528137423857, 2.262741699796952]], rtol=1e-14)


def test_constant_rows_and_scale_invariance():
    g = np.linspace(0.5, 1.5, 64)
    for c in (1.0, -3.0, 1e-20, 1e30):
        y = norm.rmsnorm(np.full((1, 64), c), g, 0.0)
        np.testing.assert_allclose(y[0], np.sign(c) * g, rtol=1e-15)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 64))
    for a in (0.001, 7.0, 2.0 ** 40):
        np.testing.assert_allclose(norm.rmsnorm(a * x, g, 0.0), norm.rmsnorm(x, g, 0.0), rtol=1e-14)


def test_eps_bounds_small_rows():
    # a row far below sqrt(eps) is scaled by about 1 / sqrt(eps) instead of being blown up to unit RMS
    x = np.full((1, 16), 1e-6)
    y = norm.rmsnorm(x, np.ones(16), 1e-2)
    np.testing.assert_allclose(y, x / np.sqrt(1e-12 + float(np.float32(1e-2))), rtol=1e-15)
