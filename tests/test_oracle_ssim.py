"""Pins of the oracle's L1 + D-SSIM loss (CPU only).

The loss passage of "Scaling 3D Gaussian Splatting with Distributed Compute" weights an L1 term
and a D-SSIM term by lambda but prints neither formula nor constants; the oracle takes SSIM with
an 11x11 Gaussian window (sigma 1.5), C1 = 0.01^2, C2 = 0.03^2, over the window positions wholly
inside the image.  None of these pins re-types the oracle's arithmetic:
  - identical images give SSIM 1 and a zero D-SSIM gradient (SSIM's maximum);
  - constant images give the closed form (2ab + C1) / (a^2 + b^2 + C1);
  - a brute-force per-position SSIM from centred weighted statistics (sum w (x - mu)^2, not
    sum w x^2 - mu^2) with the window from scipy's Gaussian window routine;
  - symmetry in its two images; lambda = 0 reduces to the L1 oracle;
  - central finite differences of the loss pin every gradient entry sampled, at the borders
    and in the interior, for several lambdas.
"""
from __future__ import annotations

import numpy as np
import pytest
from scipy.signal import windows

import oracle

C1, C2 = 0.01 ** 2, 0.03 ** 2


def _pair(H, W, seed):
    rng = np.random.default_rng(seed)
    x = rng.random((H, W, 3))
    # target correlated with x plus a smooth ramp, so every statistic is non-trivial
    ramp = np.linspace(0.0, 0.3, W)[None, :, None] * np.linspace(1.0, 0.5, H)[:, None, None]
    y = np.clip(0.6 * x + 0.3 * rng.random((H, W, 3)) + ramp, 0.0, 1.0)
    return x, y


def test_identical_images_give_one_and_zero_ssim_gradient():
    x, _ = _pair(17, 21, 1)
    L, l1, ssim, g = oracle.loss_l1_dssim(x, x, lam=1.0)
    assert ssim == pytest.approx(1.0, abs=1e-12)
    assert l1 == 0.0 and L == pytest.approx(0.0, abs=1e-12)
    assert np.abs(g).max() < 1e-12


@pytest.mark.parametrize("a,b", [(0.25, 0.75), (0.9, 0.1), (0.5, 0.5), (0.0, 0.3)])
def test_constant_images_closed_form(a, b):
    H, W = 14, 19
    x = np.full((H, W, 3), a)
    y = np.full((H, W, 3), b)
    L, l1, ssim, _ = oracle.loss_l1_dssim(x, y, lam=0.2)
    expect = (2 * a * b + C1) / (a * a + b * b + C1)
    assert ssim == pytest.approx(expect, rel=1e-12, abs=1e-12)
    assert l1 == pytest.approx(abs(a - b), abs=1e-13)
    assert L == pytest.approx(0.8 * abs(a - b) + 0.2 * (1 - expect), rel=1e-12, abs=1e-14)


def _ssim_bruteforce(x, y):
    """Mean SSIM from centred weighted statistics, position by position, in Python loops."""
    g = windows.gaussian(11, 1.5)
    w = np.outer(g, g)
    w /= w.sum()
    H, W, _ = x.shape
    total, count = 0.0, 0
    for c in range(3):
        for r in range(H - 10):
            for s in range(W - 10):
                px = x[r:r + 11, s:s + 11, c]
                py = y[r:r + 11, s:s + 11, c]
                mx = float((w * px).sum())
                my = float((w * py).sum())
                vx = float((w * (px - mx) ** 2).sum())
                vy = float((w * (py - my) ** 2).sum())
                cv = float((w * (px - mx) * (py - my)).sum())
                total += ((2 * mx * my + C1) * (2 * cv + C2)) / ((mx * mx + my * my + C1) * (vx + vy + C2))
                count += 1
    return total / count


@pytest.mark.parametrize("H,W,seed", [(11, 11, 2), (13, 16, 3), (19, 12, 4)])
def test_bruteforce_centred_statistics(H, W, seed):
    x, y = _pair(H, W, seed)
    _, _, ssim, _ = oracle.loss_l1_dssim(x, y)
    assert ssim == pytest.approx(_ssim_bruteforce(x, y), rel=1e-11)


def test_symmetric_in_its_images():
    x, y = _pair(15, 18, 5)
    assert oracle.loss_l1_dssim(x, y)[2] == pytest.approx(oracle.loss_l1_dssim(y, x)[2], rel=1e-13)


def test_lambda_zero_is_the_l1_loss():
    x, y = _pair(16, 16, 6)
    L, l1, _, g = oracle.loss_l1_dssim(x, y, lam=0.0)
    L1, g1 = oracle.loss_l1(x, y)
    assert L == pytest.approx(L1, rel=1e-14) and l1 == pytest.approx(L1, rel=1e-14)
    np.testing.assert_allclose(g, g1, rtol=0, atol=1e-18)


def test_image_smaller_than_window_is_nan():
    x, y = _pair(10, 30, 7)
    assert np.isnan(oracle.loss_l1_dssim(x, y)[0])


@pytest.mark.parametrize("lam", [1.0, 0.2])
def test_gradient_matches_finite_differences(lam):
    H, W = 15, 17
    x, y = _pair(H, W, 8)
    _, _, _, g = oracle.loss_l1_dssim(x, y, lam=lam)
    rng = np.random.default_rng(9)
    picks = [(0, 0, 0), (H - 1, W - 1, 2), (0, W - 1, 1), (H - 1, 0, 0), (7, 8, 1), (5, 10, 2)]
    picks += [tuple(int(v) for v in (rng.integers(H), rng.integers(W), rng.integers(3))) for _ in range(14)]
    h = 1e-6
    for (r, s, c) in picks:
        xp = x.copy()
        xm = x.copy()
        xp[r, s, c] += h
        xm[r, s, c] -= h
        fd = (oracle.loss_l1_dssim(xp, y, lam=lam)[0] - oracle.loss_l1_dssim(xm, y, lam=lam)[0]) / (2 * h)
        assert g[r, s, c] == pytest.approx(fd, rel=1e-5, abs=1e-10), (r, s, c)
