"""GPU parity of adaptive density control against the oracle on the same seeded inputs:
  - gs_densify: decision codes, the output count and the order of the output bit-exact; copied
    columns and moments bit-exact; split children's means within 1e-6 and log-scales within
    2e-7 (float32 rounding of the same expressions);
  - the capacity error when the output does not fit, with the required count;
  - gs_densify_stats after a whole GPU step against the oracle's statistic from its own step
    (end-to-end bar: relative L2 1e-2; the visibility counts equal wherever the preprocess
    decisions agree)."""
import numpy as np
import pytest
import torch

import oracle
from gaussian_splatting_differentiable_preprocess_amd import gsmi, inputs
from parity_util import rel_l2, say

pytestmark = pytest.mark.gpu


def _inputs(n, deg, seed):
    rng = np.random.default_rng(seed)
    if n == 262144:
        params = inputs.gaussian_params(inputs.CONFIGS["torus_262k_512"])
    else:
        params = inputs.small_scene(seed, n, deg, logscale_mean=-4.6, logscale_std=0.8)
    R = params.shape[0]
    params = params.copy()
    params[10] = rng.normal(-2.0, 2.0, n).astype(np.float32)   # some below the opacity floor
    acc = rng.uniform(0, 1e-3, n).astype(np.float32)
    cnt = rng.integers(0, 4, n).astype(np.float32)
    z = rng.standard_normal((2, 3, n)).astype(np.float32)
    m = (1e-3 * rng.standard_normal((R, n))).astype(np.float32)
    v = (1e-6 * rng.random((R, n))).astype(np.float32)
    return params, m, v, acc, cnt, z


def _gpu_densify(params, m, v, acc, cnt, z, deg, ld_out, opts):
    R, n = params.shape
    dev = torch.device("cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    po = torch.full((R, max(ld_out, 1)), float("nan"), device=dev)
    mo = torch.full_like(po, float("nan"))
    vo = torch.full_like(po, float("nan"))
    codes = torch.full((n,), -1, dtype=torch.int32, device=dev)
    ws = torch.empty(gsmi.densify_workspace(n), dtype=torch.uint8, device=dev)
    n_out = gsmi.densify(gsmi.make_scene(n, n, deg), t(params), t(m), t(v), t(acc), t(cnt), t(z), opts, po, mo, vo,
                         ld_out, ws, codes=codes)
    torch.cuda.synchronize()
    return n_out, po.cpu().numpy()[:, :n_out], mo.cpu().numpy()[:, :n_out], vo.cpu().numpy()[:, :n_out], \
        codes.cpu().numpy()


@pytest.mark.parametrize("n,deg,seed", [(1, 0, 1), (257, 1, 2), (5000, 3, 3), (262144, 3, 4)])
def test_densify_parity(n, deg, seed):
    params, m, v, acc, cnt, z = _inputs(n, deg, seed)
    opts = dict(grad_threshold=2e-4, percent_dense=0.01, extent=1.0, min_opacity=0.005, split_factor=1.6)
    say(f"[densify] n={n} deg={deg}: oracle")
    want, wm, wv, wcodes = oracle.densify(params, m, v, acc, cnt, z, **opts)
    n_out, got, gm, gv, codes = _gpu_densify(params, m, v, acc, cnt, z, deg, 3 * n, gsmi.densify_opts(**opts))
    k = np.bincount(wcodes, minlength=4)
    say(f"[densify]   kept {k[0]}, cloned {k[1]}, split {k[2]}, pruned {k[3]} -> {n_out} (oracle {want.shape[1]})")
    np.testing.assert_array_equal(codes, wcodes)
    assert n_out == want.shape[1]
    n_copy = int(k[0] + 2 * k[1])  # kept columns and clone copies are copies of the inputs
    np.testing.assert_array_equal(got[:, :n_copy], want[:, :n_copy].astype(np.float32))
    np.testing.assert_array_equal(gm, wm.astype(np.float32))
    np.testing.assert_array_equal(gv, wv.astype(np.float32))
    ch = slice(n_copy, n_out)
    np.testing.assert_allclose(got[0:3, ch], want[0:3, ch], rtol=0, atol=1e-6)
    np.testing.assert_allclose(got[3:6, ch], want[3:6, ch], rtol=0, atol=2e-6)
    np.testing.assert_array_equal(got[6:, ch], want[6:, ch].astype(np.float32))


def test_densify_capacity_error_reports_the_count():
    params, m, v, acc, cnt, z = _inputs(3000, 2, 7)
    want = oracle.densify(params, m, v, acc, cnt, z)[0].shape[1]
    with pytest.raises(gsmi.GsCapacityError) as e:
        _gpu_densify(params, m, v, acc, cnt, z, 2, want - 1, gsmi.densify_opts())
    assert e.value.required == want
    n_out = _gpu_densify(params, m, v, acc, cnt, z, 2, want, gsmi.densify_opts())[0]
    assert n_out == want


def test_densify_stats_after_a_step():
    """Torus scene (262,144 Gaussians, SH 3), orbit view 0 at 512x512, L1 against the target
    set's image: the GPU's fused step then gs_densify_stats, twice (two accumulated views), against
    the oracle's statistic from its own step."""
    from test_gpu_parity import _case

    params, deg, cam, W, H, tgt, _ = _case("torus_262k_512_v0")
    say("[densify] stats: oracle step")
    o = oracle.train_step_reference(params, deg, cam.flat(), W, H, target=tgt)
    want, seen = oracle.densify_view_stats(o["grad2d"], o["radii"], W, H)
    R, n = params.shape
    buf = gsmi.StepBuffers(n, n, deg, W, H, k_capacity=4 * n)
    p = torch.from_numpy(params).cuda()
    c = gsmi.make_camera(cam)
    acc = torch.zeros(n, device="cuda")
    cnt = torch.zeros(n, device="cuda")
    for _ in range(2):
        gsmi.preprocess(buf.scene, p, c, buf.proj)
        K = gsmi.bin_and_sort(buf.scene, c, buf.proj, buf.ws, buf.k_capacity, buf.vals, buf.ranges)
        gsmi.render_plan(buf.scene, c, buf.proj, buf.ranges, buf.render_ws, k=K)
        gsmi.render_step(buf.scene, c, buf.proj, buf.vals, buf.ranges, (0.0, 0.0, 0.0), torch.from_numpy(tgt).cuda(),
                         buf.image, buf.T_final, buf.last, buf.loss, buf.dLdI, buf.render_ws, k=K)
        gsmi.densify_stats(buf.scene, c, buf.proj, buf.render_ws, acc, cnt)
    torch.cuda.synchronize()
    a = acc.cpu().numpy() / 2
    k = cnt.cpu().numpy() / 2
    mism = int((k != seen).sum())
    e = rel_l2(a, want)
    say(f"[densify]   statistic rel-L2 {e:.3g}; {int(seen.sum())} seen, {mism} visibility mismatches")
    assert mism <= max(2, 1e-3 * n)
    assert e <= 1e-2


@pytest.mark.slow
def test_densify_full_size_gyroid_4m():
    """The 4M-Gaussian gyroid scene (SH 3) with seeded statistics that send every outcome to
    hundreds of thousands of Gaussians: codes, count and order bit-exact, every output column
    compared."""
    cfg = inputs.CONFIGS["gyroid_4m_2048"]
    say("[densify] gyroid_4m: drawing the scene")
    params = inputs.gaussian_params(cfg)
    n = params.shape[1]
    rng = np.random.default_rng(99)
    params[10] = rng.normal(-2.0, 2.0, n).astype(np.float32)
    acc = rng.uniform(0, 1e-3, n).astype(np.float32)
    cnt = rng.integers(0, 4, n).astype(np.float32)
    z = rng.standard_normal((2, 3, n)).astype(np.float32)
    m = np.zeros_like(params)
    v = np.zeros_like(params)
    opts = dict(extent=0.35)  # 0.01 x extent near the scene's typical largest scale: clones and splits
    say("[densify] gyroid_4m: oracle")
    want, wm, wv, wcodes = oracle.densify(params, m, v, acc, cnt, z, **opts)
    n_out, got, gm, gv, codes = _gpu_densify(params, m, v, acc, cnt, z, 3, 2 * n, gsmi.densify_opts(**opts))
    k = np.bincount(wcodes, minlength=4)
    say(f"[densify]   kept {k[0]}, cloned {k[1]}, split {k[2]}, pruned {k[3]} -> {n_out}")
    assert min(k) > 1000
    np.testing.assert_array_equal(codes, wcodes)
    assert n_out == want.shape[1]
    n_copy = int(k[0] + 2 * k[1])
    np.testing.assert_array_equal(got[:, :n_copy], want[:, :n_copy].astype(np.float32))
    assert (gm == 0).all() and (gv == 0).all()
    ch = slice(n_copy, n_out)
    np.testing.assert_allclose(got[0:3, ch], want[0:3, ch], rtol=0, atol=4e-6)
    np.testing.assert_allclose(got[3:6, ch], want[3:6, ch], rtol=0, atol=2e-6)
    np.testing.assert_array_equal(got[6:, ch], want[6:, ch].astype(np.float32))


def test_densify_non_finite_inputs():
    """Every comparison with NaN is false on both sides: a NaN statistic never densifies, a NaN
    logit never prunes, three NaN log-scales neither clone nor split, and a NaN among the
    log-scales is skipped by the largest-scale test."""
    params, m, v, acc, cnt, z = _inputs(600, 1, 11)
    acc[0:50] = np.nan
    params[10, 50:100] = np.nan
    params[3:6, 100:150] = np.nan
    params[4, 150:200] = np.nan
    acc[100:200] = 5e-3  # dense: only the largest-scale test decides
    cnt[100:200] = 1.0
    want, wm, wv, wcodes = oracle.densify(params, m, v, acc, cnt, z)
    keep_or_prune = (wcodes == oracle.DENS_KEEP) | (wcodes == oracle.DENS_PRUNE)
    assert keep_or_prune[0:50].all() and keep_or_prune[100:150].all()
    assert (wcodes[50:100] != oracle.DENS_PRUNE).all()
    assert (wcodes[150:200] != oracle.DENS_KEEP).any()
    n_out, got, gm, gv, codes = _gpu_densify(params, m, v, acc, cnt, z, 1, 3 * 600, gsmi.densify_opts())
    np.testing.assert_array_equal(codes, wcodes)
    assert n_out == want.shape[1]
    k = np.bincount(wcodes, minlength=4)
    n_copy = int(k[0] + 2 * k[1])
    np.testing.assert_array_equal(got[:, :n_copy], want[:, :n_copy].astype(np.float32))
