"""Finite-difference pins of the oracle's gradients (backward blend and preprocess
backward).  The discrete structure -- culling, tile lists, sorted order and every per-pixel
skip / clamp / termination decision -- is frozen at the base point, so the loss is a smooth
function of the parameters and central differences in double must match the analytic
gradient of the branch the forward took."""
import math

import numpy as np
import pytest

import oracle
from gaussian_splatting_differentiable_preprocess_amd import inputs

# grad2d row -> proj row
G2P = [0, 1, 4, 5, 6, 3, 7, 8, 9]


def _scene(seed, n, deg, W):
    """A compact cluster (radius 0.15 at distance 3) so pixels stack enough layers to hit
    the transmittance cut-off."""
    params = inputs.small_scene(seed, n, deg, logscale_mean=-1.9, logscale_std=0.3,
                                radius=0.15).astype(np.float64)
    params[10] += 2.0
    cam = inputs.lookat_camera((3.0, 0.4, 0.3), W, W)
    return params, cam


def _frozen(params, deg, cam, W):
    c = cam.flat()
    proj, radii, tiles = oracle.preprocess(params, deg, c, W, W)
    keys, vals = oracle.bin_sort(proj, radii, W, W)
    rg = oracle.ranges(keys, oracle.n_tiles(W, W))
    dec = oracle.render_forward(proj, vals, rg, W, W, record_decisions=True)["decisions"]
    return proj, vals, rg, dec


EPS = np.finfo(np.float64).eps


def _check(fd, an, what, noise):
    """|fd - an| <= 1e-6 |an| + noise, where noise = 64 eps sum|terms of L| / h bounds the
    rounding error of a central difference of L in double."""
    err = np.abs(fd - an)
    bad = err > 1e-6 * np.abs(an) + noise
    assert not bad.any(), (what, np.argwhere(bad)[:5], fd[bad][:5], an[bad][:5], noise)


@pytest.mark.parametrize("deg", [0, 3])
def test_fd_backward_blend(deg):
    W = 32
    params, cam = _scene(30 + deg, 20, deg, W)
    proj, vals, rg, _ = _frozen(params, deg, cam, W)
    # centre a third of the Gaussians on pixel centres with opacity 0.9997: alpha = o G is
    # clamped at 0.99 on those pixels
    k = params.shape[1] // 3
    proj[0, :k] = np.floor(proj[0, :k]) + 0.5
    proj[1, :k] = np.floor(proj[1, :k]) + 0.5
    proj[3, :k] = 0.9997
    dec = oracle.render_forward(proj, vals, rg, W, W, record_decisions=True)["decisions"]
    G = np.random.default_rng(1).uniform(-1, 1, (W, W, 3))
    bg = (0.2, 0.1, 0.4)
    an = oracle.render_backward(proj, vals, rg, W, W, G, bg, decisions=dec)
    assert (dec == oracle.DEC_BLEND_CLAMPED).any() and (dec == oracle.DEC_STOP).any()

    def L(pr):
        return float((oracle.render_forward(pr, vals, rg, W, W, bg, decisions=dec)["image"] * G).sum())

    Labs = float(np.abs(oracle.render_forward(proj, vals, rg, W, W, bg, decisions=dec)["image"] * G).sum())
    vis = np.nonzero(proj[3] > 0)[0]
    fd = np.zeros((9, vis.size))
    hs = np.zeros((9, vis.size))
    for k, i in enumerate(vis):
        for r in range(9):
            f = G2P[r]
            h = 1e-6 * max(1.0, abs(proj[f, i]))
            hs[r, k] = h
            pp, pm = proj.copy(), proj.copy()
            pp[f, i] += h
            pm[f, i] -= h
            fd[r, k] = (L(pp) - L(pm)) / (2 * h)
    for r in range(9):
        _check(fd[r], an[r, vis], oracle.GRAD2D_FIELDS[r], 64 * EPS * Labs / hs[r])


@pytest.mark.parametrize("deg", [0, 1, 2, 3])
def test_fd_preprocess_backward_linear_functional(deg):
    """L = sum_f sum_i w[f][i] proj_f(params)_i, so dL/dproj = w exactly and the chain rule
    through the per-Gaussian preprocess is isolated."""
    W = 64
    params, cam = _scene(40 + deg, 16, deg, W)
    c = cam.flat()
    w = np.random.default_rng(2).normal(size=(9, params.shape[1]))
    an = oracle.preprocess_backward(params, deg, c, W, W, w)
    proj0, _, _ = oracle.preprocess(params, deg, c, W, W)
    mg = oracle.preprocess_margins(params, deg, c, W, W)
    assert (mg[2][proj0[3] > 0] > 1e-3).all()  # no colour clamp near switching

    def L(p):
        pr, _, _ = oracle.preprocess(p, deg, c, W, W)
        return float(sum((w[r] * pr[G2P[r]]).sum() for r in range(9)))

    Labs = float(sum(np.abs(w[r] * proj0[G2P[r]]).sum() for r in range(9)))
    R = params.shape[0]
    vis = np.nonzero(proj0[3] > 0)[0]
    for r in range(R):
        fd = np.zeros(vis.size)
        hs = np.maximum(1.0, np.abs(params[r, vis])) * 1e-6
        for k, i in enumerate(vis):
            h = hs[k]
            pp, pm = params.copy(), params.copy()
            pp[r, i] += h
            pm[r, i] -= h
            fd[k] = (L(pp) - L(pm)) / (2 * h)
        _check(fd, an[r, vis], f"row {r}", 64 * EPS * Labs / hs)


@pytest.mark.parametrize("deg", [0, 3])
def test_fd_full_step(deg):
    W = 32
    params, cam = _scene(50 + deg, 12, deg, W)
    c = cam.flat()
    proj, vals, rg, dec = _frozen(params, deg, cam, W)
    mg = oracle.preprocess_margins(params, deg, c, W, W)
    assert (mg[2][proj[3] > 0] > 1e-3).all()
    G = np.random.default_rng(3).uniform(-1, 1, (W, W, 3))
    g2 = oracle.render_backward(proj, vals, rg, W, W, G, decisions=dec)
    an = oracle.preprocess_backward(params, deg, c, W, W, g2)

    def L(p):
        pr, _, _ = oracle.preprocess(p, deg, c, W, W)
        return float((oracle.render_forward(pr, vals, rg, W, W, decisions=dec)["image"] * G).sum())

    Labs = float(np.abs(oracle.render_forward(proj, vals, rg, W, W, decisions=dec)["image"] * G).sum())
    vis = np.nonzero(proj[3] > 0)[0]
    for r in range(params.shape[0]):
        fd = np.zeros(vis.size)
        hs = np.maximum(1.0, np.abs(params[r, vis])) * 1e-6
        for k, i in enumerate(vis):
            h = hs[k]
            pp, pm = params.copy(), params.copy()
            pp[r, i] += h
            pm[r, i] -= h
            fd[k] = (L(pp) - L(pm)) / (2 * h)
        _check(fd, an[r, vis], f"row {r}", 64 * EPS * Labs / hs)


def test_fd_unfrozen_when_margins_are_wide():
    """Without freezing anything: a two-Gaussian scene whose decisions all sit far from
    their thresholds gives the same derivative as the frozen one."""
    W = 32
    cam = inputs.lookat_camera((3.0, 0.0, 0.0), W, W)
    c = cam.flat()
    p = np.zeros((14, 2))
    p[0:3, 0], p[0:3, 1] = [0.0, 0.03, -0.02], [-0.2, -0.05, 0.04]
    p[3:6, 0], p[3:6, 1] = [-2.2, -2.0, -2.4], [-2.0, -2.3, -2.1]
    p[6:10, 0], p[6:10, 1] = [0.9, 0.1, -0.2, 0.3], [0.8, -0.3, 0.1, 0.2]
    p[10] = [0.3, -0.2]
    p[11:14, 0], p[11:14, 1] = [0.2, 0.5, 0.8], [0.7, 0.3, 0.1]
    G = np.random.default_rng(4).uniform(-1, 1, (W, W, 3))
    out = oracle.train_step_reference(p, 0, c, W, W, upstream=G)
    fwd = oracle.render_forward(out["proj"], out["vals"], out["ranges"], W, W, margins=[1e-3, 1e-3, 1e-3])
    assert not fwd["borderline"].any()

    def L(q):
        return oracle.train_step_reference(q, 0, c, W, W, upstream=G)["loss"]

    for r in range(14):
        for i in range(2):
            h = 1e-6 * max(1.0, abs(p[r, i]))
            pp, pm = p.copy(), p.copy()
            pp[r, i] += h
            pm[r, i] -= h
            fd = (L(pp) - L(pm)) / (2 * h)
            an = out["grads"][r, i]
            Labs = float(np.abs(out["image"] * G).sum())
            assert abs(fd - an) <= 1e-6 * abs(an) + 64 * EPS * Labs / h, (r, i, fd, an)
