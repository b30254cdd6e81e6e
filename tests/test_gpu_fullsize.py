"""Parity at the full workload sizes, in the launch configuration the bench times.

gyroid_4m_2048 (4M Gaussians, SH degree 3, 2048x2048): the oracle runs the whole step for one
orbit view on the seeded inputs; the GPU runs each stage on the oracle's inputs to it and the
whole step from the parameters, and every output is compared element by element.

bumps_18m_2048 (18.18M Gaussians): the oracle's preprocess and sort run over every Gaussian and
the GPU's sort of the oracle's records must match bit for bit; the blends are compared on a
sample of tiles (the heaviest ones and a seeded random set), both sides given the same lists
with every other tile emptied.  Set GSMI_FULLSIZE_18M=0 to skip it (its scene takes about a
minute to draw on the host).

gyroid_4m_1024 and gyroid_4m_2048 with the L1 loss against a seeded target: the fused image pass
and the preprocess backward from its staged sums -- the launch configuration the bench times --
on the oracle's records and lists and end to end.

Elsewhere upstream dL/dI is the seeded U(-1, 1) field of the configuration."""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from gaussian_splatting_differentiable_preprocess_amd import inputs
from parity_util import (BORDER_FRACTION, FWD_MARGINS, GRAD_REL_L2, IMG_MAX_ABS, GpuStep, oracle_pipeline,
                         preprocess_borderline, proj_from_splat, records_from_oracle, rel_l2, say)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

BG = (0.0, 0.0, 0.0)


def _compare_forward(g, o, P, label):
    bl = o["borderline"]
    err = np.abs(g["image"] - o["image"]).max(axis=-1)
    say(f"[fullsize] {label} forward: {int(bl.sum())} borderline of {P}; max err non-borderline {err[~bl].max():.3g}")
    assert bl.sum() <= max(1.0, BORDER_FRACTION * P), bl.sum()
    assert err[~bl].max() <= IMG_MAX_ABS
    np.testing.assert_array_equal(g["last_contrib"][~bl], o["last_contrib"][~bl])
    np.testing.assert_array_equal(g["n_examined"][~bl], o["n_examined"][~bl])


def test_gyroid_4m_2048_full_step():
    cfg = inputs.CONFIGS["gyroid_4m_2048"]
    W = H = cfg.res
    say("[fullsize] gyroid_4m_2048: drawing the scene")
    params = inputs.gaussian_params(cfg)
    cam = inputs.cameras_for(cfg)[0]
    up = inputs.upstream_gradient(cfg, W, H)
    R, n = params.shape
    say("[fullsize] oracle step (all Gaussians, all pixels)")
    o = oracle_pipeline(params, cfg.sh_degree, cam.flat(), W, H, BG, upstream=up, margins=FWD_MARGINS)
    K = o["keys"].size
    say(f"[fullsize] K = {K}; GPU preprocess")
    g = GpuStep(params, cfg.sh_degree, cam, W, H, k_capacity=K + 4096)
    splat, tiles, _ = g.preprocess()
    gp, gr = proj_from_splat(splat)
    bl = preprocess_borderline(params, cfg.sh_degree, cam.flat(), W, H, o["proj"][0], o["proj"][1], o["radii"])
    same = (gr[0] > 0) & (o["radii"][0] > 0) & ~bl
    assert ((gr[0] > 0) != (o["radii"][0] > 0))[~bl].sum() == 0
    np.testing.assert_array_equal(gr[:, same], o["radii"][:, same])
    for f in (0, 1, 2, 3):  # u, v, depth, opacity
        assert (np.abs(gp[f, same] - o["proj"][f, same]) <= 1e-5 * np.abs(o["proj"][f, same])).all(), f
    say("[fullsize] GPU sort of the oracle's records")
    g.load_proj(*records_from_oracle(o["p32"], o["radii"], o["tiles"], W, H))
    Kg, keys, vals, rg = g.bin_and_sort()
    assert Kg == K
    np.testing.assert_array_equal(keys, o["keys"])
    np.testing.assert_array_equal(vals, o["vals"])
    np.testing.assert_array_equal(rg.reshape(-1, 2), o["ranges"])
    say("[fullsize] GPU forward and backward on the oracle's lists")
    fwd = g.forward(BG)
    _compare_forward(fwd, o["fwd"], W * H, "stage")
    g.set_upstream(o["dl32"])
    g2, grads = g.backward()
    errs = [rel_l2(g2[r, :n], o["grad2d"][r]) for r in range(9)]
    say("[fullsize] backward blend rel-L2 per row: " + " ".join(f"{e:.2g}" for e in errs))
    assert max(errs) <= GRAD_REL_L2
    e = rel_l2(grads, o["grads"])
    say(f"[fullsize] preprocess backward (chained) rel-L2 {e:.3g}")
    assert e <= GRAD_REL_L2
    e_iso = rel_l2(g.preprocess_backward(o["grad2d"]), o["grads"])
    assert e_iso <= GRAD_REL_L2
    say("[fullsize] GPU step end to end from the parameters")
    e2 = GpuStep(params, cfg.sh_degree, cam, W, H, k_capacity=K + 4096)
    e2.preprocess()
    e2.bin_and_sort()
    f2 = e2.forward(BG)
    err = np.abs(f2["image"] - o["fwd"]["image"]).max(axis=-1)
    ok = ~o["fwd"]["borderline"]
    frac_bad = float((err[ok] > IMG_MAX_ABS).mean())
    e2.set_upstream(up)
    g2e, grads_e = e2.backward()
    ee = rel_l2(grads_e, o["grads"])
    say(f"[fullsize] e2e: image frac > 1e-4 {frac_bad:.3g}, grads rel-L2 {ee:.3g}")
    assert frac_bad <= 1e-3 and ee <= 1e-2


@pytest.mark.parametrize("name", ["gyroid_4m_1024", "gyroid_4m_2048"])
def test_gyroid_4m_fused_step_with_l1(name):
    """The step as the bench runs it: the fused image pass (forward, L1 against a target and
    backward blend in one persistent kernel, gs_render_step) and the preprocess backward from
    the staged sums, at 1024^2 and 2048^2.  Stage parity on the oracle's records and lists,
    then the whole step from the parameters."""
    cfg = inputs.CONFIGS[name]
    W = H = cfg.res
    say(f"[fullsize] {name}: drawing the scene")
    params = inputs.gaussian_params(cfg)
    cam = inputs.cameras_for(cfg)[7]
    target = np.random.default_rng(cfg.index).uniform(0, 1, (H, W, 3)).astype(np.float32)
    R, n = params.shape
    say(f"[fullsize] {name}: oracle step with the L1 loss")
    o = oracle_pipeline(params, cfg.sh_degree, cam.flat(), W, H, BG, target=target, margins=FWD_MARGINS)
    K = o["keys"].size
    say(f"[fullsize] {name}: K = {K}; fused pass on the oracle's records and lists")
    g = GpuStep(params, cfg.sh_degree, cam, W, H, k_capacity=K + 4096)
    g.load_proj(*records_from_oracle(o["p32"], o["radii"], o["tiles"], W, H))
    g.load_lists(o["vals"], o["ranges"])
    r = g.step(BG, target)
    assert r["stall"] == 0
    _compare_forward(r, o["fwd"], W * H, "fused")
    assert r["loss"] == pytest.approx(o["loss"], rel=1e-5)
    errs = [rel_l2(r["grad2d"][k, :n], o["grad2d"][k]) for k in range(9)]
    say("[fullsize] fused backward blend rel-L2 per row: " + " ".join(f"{e:.2g}" for e in errs))
    assert max(errs) <= GRAD_REL_L2
    e = rel_l2(g.preprocess_backward_staged(), o["grads"])
    say(f"[fullsize] preprocess backward from the staged sums rel-L2 {e:.3g}")
    assert e <= GRAD_REL_L2
    say(f"[fullsize] {name}: the whole step from the parameters")
    e2 = GpuStep(params, cfg.sh_degree, cam, W, H, k_capacity=K + 4096)
    e2.preprocess()
    e2.bin_and_sort()
    r2 = e2.step(BG, target)
    assert r2["stall"] == 0
    err = np.abs(r2["image"] - o["fwd"]["image"]).max(axis=-1)
    frac_bad = float((err[~o["fwd"]["borderline"]] > IMG_MAX_ABS).mean())
    ee = rel_l2(e2.preprocess_backward_staged(), o["grads"])
    say(f"[fullsize] e2e fused: image frac > 1e-4 {frac_bad:.3g}, loss {r2['loss']:.7g} vs {o['loss']:.7g}, "
        f"grads rel-L2 {ee:.3g}")
    assert frac_bad <= 1e-3 and ee <= 1e-2
    assert r2["loss"] == pytest.approx(o["loss"], rel=1e-4)


@pytest.mark.skipif(os.environ.get("GSMI_FULLSIZE_18M", "1") == "0", reason="GSMI_FULLSIZE_18M=0")
def test_bumps_18m_2048_sort_and_sampled_tiles():
    cfg = inputs.CONFIGS["bumps_18m_2048"]
    W = H = cfg.res
    say("[fullsize] bumps_18m_2048: drawing the scene")
    params = inputs.gaussian_params(cfg)
    cam = inputs.cameras_for(cfg)[0]
    up = inputs.upstream_gradient(cfg, W, H)
    R, n = params.shape
    c = cam.flat()
    say("[fullsize] oracle preprocess and sort (all Gaussians)")
    proj, radii, tiles = oracle.preprocess(params, cfg.sh_degree, c, W, H)
    from parity_util import proj_f32
    p32 = proj_f32(proj)
    okeys, ovals = oracle.bin_sort(p32, radii, W, H)
    T = oracle.n_tiles(W, H)
    orng = oracle.ranges(okeys, T).reshape(-1, 2)
    K = okeys.size
    say(f"[fullsize] K = {K}; GPU sort of the oracle's records")
    g = GpuStep(params, cfg.sh_degree, cam, W, H, k_capacity=K + 4096)
    g.load_proj(*records_from_oracle(p32, radii, tiles, W, H))
    Kg, keys, vals, rg = g.bin_and_sort()
    assert Kg == K
    np.testing.assert_array_equal(keys, okeys)
    np.testing.assert_array_equal(vals, ovals)
    np.testing.assert_array_equal(rg.reshape(-1, 2), orng)
    # sampled tiles: the 8 longest lists and 24 seeded random non-empty ones
    lens = orng[:, 1].astype(np.int64) - orng[:, 0]
    nonempty = np.flatnonzero(lens > 0)
    pick = set(np.argsort(-lens)[:8].tolist())
    pick |= set(np.random.default_rng(inputs.seed_for(cfg, 4)).choice(nonempty, 24, replace=False).tolist())
    mask = np.zeros(T, bool)
    mask[sorted(pick)] = True
    srng = np.where(mask[:, None], orng, 0).astype(np.uint32)
    say(f"[fullsize] {mask.sum()} sampled tiles, {int(lens[mask].sum())} list entries; oracle blends")
    ofwd = oracle.render_forward(p32, ovals, srng, W, H, BG, margins=FWD_MARGINS)
    dl32 = up.astype(np.float32)
    og2 = oracle.render_backward(p32, ovals, srng, W, H, dl32.astype(np.float64), BG)
    g.load_lists(ovals, srng)
    fwd = g.forward(BG)
    tile_of_px = ((np.arange(H)[:, None] // 16) * ((W + 15) // 16) + np.arange(W)[None, :] // 16)
    sel = mask[tile_of_px]
    sub = {k: fwd[k][sel] for k in ("image", "last_contrib", "n_examined")}
    osub = {k: ofwd[k][sel] for k in ("image", "last_contrib", "n_examined", "borderline")}
    _compare_forward(sub, osub, int(sel.sum()), "sampled")
    g.set_upstream(dl32)
    g2, _ = g.backward()
    errs = [rel_l2(g2[r, :n], og2[r]) for r in range(9)]
    say("[fullsize] sampled backward blend rel-L2 per row: " + " ".join(f"{e:.2g}" for e in errs))
    assert max(errs) <= GRAD_REL_L2
