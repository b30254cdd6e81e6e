"""Pins of the oracle's adaptive density control (CPU only): a hand-built scene whose every
Gaussian's fate and every output value follows by hand (pruned, kept, cloned, split under a
rotation about z, a Gaussian never seen), the statistic's closed form, the decision in the logit
domain against the sigmoid, and the count identity on a random scene."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle

LOG16 = math.log(1.6)


def _scene():
    """Six Gaussians at SH degree 0 (14 rows)."""
    n = 6
    p = np.zeros((14, n), dtype=np.float32)
    p[0:3] = np.arange(3 * n, dtype=np.float32).reshape(3, n) * 0.1
    p[3:6] = -6.0                                  # small: scale 2.5e-3 <= 0.01
    p[6] = 1.0                                     # identity rotation
    p[10] = 2.0                                    # opacity 0.88
    p[11:14] = 0.3
    p[10, 0] = -6.0                                # G0: opacity 0.0025 < 0.005 -> pruned
    p[3:6, 3] = (-1.0, -2.0, -1.5)                 # G3: largest scale e^-1 -> split
    p[6:10, 3] = (2 * math.cos(math.pi / 4), 0.0, 0.0, 2 * math.sin(math.pi / 4))  # 90 deg about z, |q| = 2
    p[3:6, 5] = -1.0                               # G5: big and transparent -> pruned, no children
    p[10, 5] = -7.0
    acc = np.array([1.0, 1e-4, 3e-3, 9e-4, 0.0, 1.0], dtype=np.float32)
    cnt = np.array([2.0, 2.0, 3.0, 3.0, 0.0, 2.0], dtype=np.float32)
    # G1: 5e-5 < 2e-4 keep; G2: 1e-3 clone (small); G3: 3e-4 split; G4: never seen -> keep
    z = np.zeros((2, 3, n), dtype=np.float32)
    z[0, :, 3] = (1.0, 0.0, 0.0)
    z[1, :, 3] = (0.0, -2.0, 0.5)
    return p, acc, cnt, z


def test_hand_built_scene():
    p, acc, cnt, z = _scene()
    m = np.full_like(p, 0.25)
    v = np.full_like(p, 0.5)
    out, mo, vo, codes = oracle.densify(p, m, v, acc, cnt, z)
    assert codes.tolist() == [oracle.DENS_PRUNE, oracle.DENS_KEEP, oracle.DENS_CLONE, oracle.DENS_SPLIT,
                              oracle.DENS_KEEP, oracle.DENS_PRUNE]
    assert out.shape == (14, 6)  # 3 kept + 1 clone + 2 children
    np.testing.assert_array_equal(out[:, 0], p[:, 1])
    np.testing.assert_array_equal(out[:, 1], p[:, 2])
    np.testing.assert_array_equal(out[:, 2], p[:, 4])
    np.testing.assert_array_equal(out[:, 3], p[:, 2])
    # children of G3: scales (e^-1, e^-2, e^-1.5); the rotation takes x to y and y to -x
    s = np.exp(np.array([-1.0, -2.0, -1.5]))
    mu = p[0:3, 3].astype(np.float64)
    np.testing.assert_allclose(out[0:3, 4], mu + np.array([0.0, s[0], 0.0]), rtol=0, atol=1e-7)
    np.testing.assert_allclose(out[0:3, 5], mu + np.array([2.0 * s[1], 0.0, 0.5 * s[2]]), rtol=0, atol=1e-7)
    for c in (4, 5):
        np.testing.assert_allclose(out[3:6, c], p[3:6, 3].astype(np.float64) - LOG16, rtol=0, atol=1e-12)
        np.testing.assert_array_equal(out[6:, c], p[6:, 3])
    # moments: kept columns keep theirs, the three new ones start at zero
    assert (mo[:, :3] == 0.25).all() and (vo[:, :3] == 0.5).all()
    assert (mo[:, 3:] == 0).all() and (vo[:, 3:] == 0).all()


def test_view_statistic_closed_form():
    W, H = 64, 48
    g2 = np.zeros((9, 3))
    g2[0, 0], g2[1, 0] = 3.0 / (W / 2), 4.0 / (H / 2)   # -> |(3, 4)| = 5
    g2[0, 1] = 1.0                                      # not seen by the view
    g2[1, 2] = -2.0 / (H / 2)
    radii = np.array([[2, 0, 1], [2, 0, 1]])
    norm, seen = oracle.densify_view_stats(g2, radii, W, H)
    np.testing.assert_allclose(norm, [5.0, 0.0, 2.0], rtol=1e-15)
    np.testing.assert_array_equal(seen, [1.0, 0.0, 1.0])


def test_decisions_match_the_plain_criteria_and_the_count_identity():
    rng = np.random.default_rng(11)
    n = 20000
    p = np.zeros((14, n), dtype=np.float32)
    p[3:6] = rng.normal(-4.6, 0.8, (3, n))
    p[6] = 1.0
    p[10] = rng.normal(-2.0, 2.0, n)
    acc = rng.uniform(0, 1e-3, n).astype(np.float32)
    cnt = rng.integers(0, 4, n).astype(np.float32)
    codes = oracle.densify_codes(p, acc, cnt, extent=1.0)
    opac = 1.0 / (1.0 + np.exp(-p[10].astype(np.float64)))
    g = np.where(cnt > 0, acc.astype(np.float64) / np.maximum(cnt, 1), 0.0)
    big = np.exp(p[3:6].astype(np.float64)).max(0) > 0.01
    far = (np.abs(opac - 0.005) > 1e-6) & (np.abs(g - 2e-4) > 1e-9) & (np.abs(np.exp(p[3:6].max(0)) - 0.01) > 1e-8)
    want = np.where(opac < 0.005, 3, np.where(g >= 2e-4, np.where(big, 2, 1), 0))
    np.testing.assert_array_equal(codes[far], want[far])
    assert far.mean() > 0.99 and len(set(codes.tolist())) == 4
    z = rng.standard_normal((2, 3, n)).astype(np.float32)
    out, _, _, _ = oracle.densify(p, np.zeros_like(p), np.zeros_like(p), acc, cnt, z)
    k = np.bincount(codes, minlength=4)
    assert out.shape[1] == n - k[3] - k[2] + k[1] + 2 * k[2]
