"""GPU parity of the L1 + D-SSIM loss (gs_loss_l1_dssim) against the CPU oracle on the same seeded
images: the three loss values within relative 1e-5, dL/dimage within relative L2 1e-3 (the
gradient bar) and within 1e-3 of its largest entry elementwise.  Sizes cover the smallest image
the 11x11 window fits, ragged strips and row blocks of the kernels' 256-column x 64-row
workgroups, and the full 2048x2048 image the step renders."""
import numpy as np
import pytest
import torch

import oracle
from gaussian_splatting_differentiable_preprocess_amd import gsmi
from parity_util import GRAD_REL_L2, rel_l2, say

pytestmark = pytest.mark.gpu


def _images(H, W, seed, same=False):
    """A smooth image with texture and a target that differs by a shifted field and noise, both in
    [0, 1] like rendered and ground-truth images."""
    rng = np.random.default_rng(seed)
    yy, xx = np.mgrid[0:H, 0:W].astype(np.float64)
    img = np.zeros((H, W, 3))
    tgt = np.zeros((H, W, 3))
    for c in range(3):
        f = rng.uniform(0.01, 0.2, 4)
        ph = rng.uniform(0, 2 * np.pi, 4)
        base = 0.5 + 0.25 * np.sin(f[0] * xx + ph[0]) * np.cos(f[1] * yy + ph[1])
        img[..., c] = base + 0.1 * rng.standard_normal((H, W))
        tgt[..., c] = base + 0.15 * np.sin(f[2] * xx + f[3] * yy + ph[2]) + 0.05 * rng.standard_normal((H, W))
    img = np.clip(img, 0, 1).astype(np.float32)
    tgt = img.copy() if same else np.clip(tgt, 0, 1).astype(np.float32)
    return img, tgt


def _gpu(img, tgt, lam):
    H, W, _ = img.shape
    dev = torch.device("cuda")
    ti = torch.from_numpy(img).to(dev)
    tt = torch.from_numpy(tgt).to(dev)
    loss = torch.full((3,), float("nan"), device=dev)
    dl = torch.full_like(ti, float("nan"))
    ws = torch.empty(gsmi.loss_l1_dssim_workspace(W, H), dtype=torch.uint8, device=dev)
    gsmi.loss_l1_dssim(W, H, ti, tt, lam, loss, dl, ws)
    torch.cuda.synchronize()
    return loss.cpu().numpy().astype(np.float64), dl.cpu().numpy()


def _compare(img, tgt, lam):
    L, l1, ssim, want = oracle.loss_l1_dssim(img.astype(np.float64), tgt.astype(np.float64), lam=lam)
    got, dl = _gpu(img, tgt, lam)
    assert np.isfinite(dl).all()
    np.testing.assert_allclose(got, [L, l1, ssim], rtol=1e-5, atol=1e-7)
    err = rel_l2(dl, want)
    scale = np.abs(want).max()
    worst = np.abs(dl - want).max()
    say(f"[ssim] {img.shape[1]}x{img.shape[0]} lambda {lam}: L {got[0]:.7g} vs {L:.7g}, SSIM {got[2]:.7g} "
        f"vs {ssim:.7g}, dL/dI rel-L2 {err:.3g}, max-abs {worst:.3g} of {scale:.3g}")
    assert err < GRAD_REL_L2
    assert worst <= 1e-3 * scale


@pytest.mark.parametrize("H,W,seed", [(11, 11, 1), (33, 17, 2), (70, 100, 3), (270, 300, 4), (523, 530, 5)])
@pytest.mark.parametrize("lam", [0.2, 1.0])
def test_loss_l1_dssim_parity(H, W, seed, lam):
    img, tgt = _images(H, W, seed)
    _compare(img, tgt, lam)


def test_lambda_zero_matches_l1_call():
    img, tgt = _images(64, 80, 6)
    got, dl = _gpu(img, tgt, 0.0)
    dev = torch.device("cuda")
    n = img.size
    loss = torch.zeros(1, device=dev)
    g = torch.empty(n, device=dev)
    ws = torch.empty(gsmi.loss_l1_workspace(n), dtype=torch.uint8, device=dev)
    gsmi.loss_l1(n, torch.from_numpy(img).to(dev), torch.from_numpy(tgt).to(dev), loss, g, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dl.reshape(-1), g.cpu().numpy())
    assert got[0] == pytest.approx(float(loss.item()), rel=1e-6)


def test_identical_images():
    img, tgt = _images(90, 75, 7, same=True)
    got, dl = _gpu(img, tgt, 0.2)
    assert got[1] == 0.0
    assert got[2] == pytest.approx(1.0, abs=1e-5)
    assert np.abs(dl).max() < 1e-9  # SSIM's maximum: only rounding remains


def test_repeatable():
    img, tgt = _images(200, 260, 8)
    a = _gpu(img, tgt, 0.2)
    b = _gpu(img, tgt, 0.2)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_full_size_2048():
    say("[ssim] 2048x2048: drawing images")
    img, tgt = _images(2048, 2048, 9)
    _compare(img, tgt, 0.2)


def test_train_step_with_dssim_end_to_end():
    """The whole step with the L1 + D-SSIM loss from the same parameters on both sides (torus
    scene, 262,144 Gaussians at SH degree 3, orbit view 0 at 512x512, targets from the second
    seeded set): the loss, and the image and parameter gradients under the flip rule.  A flipped
    pixel's image difference also moves dL/dI of its neighbours through the SSIM windows, by the
    window weights (a Gaussian of sigma 1.5 applied twice); those continuous changes stay in the
    compared set and within its bar."""
    from parity_util import FWD_MARGINS, check_e2e, gpu_e2e, oracle_pipeline, preprocess_borderline
    from test_gpu_parity import _case

    params, deg, cam, W, H, tgt, _ = _case("torus_262k_512_v0")
    say("[ssim] torus_262k_512 view 0: oracle step with L1 + D-SSIM")
    o = oracle_pipeline(params, deg, cam.flat(), W, H, (0.0, 0.0, 0.0), target=tgt, margins=FWD_MARGINS, dssim=0.2)
    e = gpu_e2e(params, deg, cam, W, H, (0.0, 0.0, 0.0), target=tgt, dssim=0.2)
    assert abs(e["K"] - o["keys"].size) <= 4
    say(f"[ssim]   loss {e['loss'][0]:.7g} vs {o['loss']:.7g}")
    assert e["loss"][0] == pytest.approx(o["loss"], rel=1e-4)
    bl = preprocess_borderline(params, deg, cam.flat(), W, H, o["proj"][0], o["proj"][1], o["radii"])
    check_e2e("torus_262k_512 L1 + D-SSIM", o, e, W, H, (0.0, 0.0, 0.0), e["grads"], o["grads"], target=tgt,
              pre_bl=bl, grad2d_g=e["grad2d"], grad2d_o=o["grad2d"])
