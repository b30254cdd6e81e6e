"""The L1 loss without allocation (gs_loss_l1_noalloc) against gs_loss_l1 with a workspace, through
the C ABI: two calls in a row, the second with a smaller input, both bit-identical to the
workspace call (the same kernels and a fixed summation order); sizes beyond the static scratch are
refused."""
import numpy as np
import pytest
import torch

from gaussian_splatting_differentiable_preprocess_amd import gsmi

pytestmark = pytest.mark.gpu


def _noalloc(count, image, target, loss, dl):
    """The C-ABI call itself (its status code, not the binding's exception)."""
    return gsmi.load().gs_loss_l1_noalloc(int(count), gsmi._ptr(image), gsmi._ptr(target), gsmi._ptr(loss),
                                          gsmi._ptr(dl), gsmi._stream())


def _case(H, W, seed):
    rng = np.random.default_rng(seed)
    img = torch.from_numpy(rng.uniform(0, 1, (H, W, 3)).astype(np.float32)).cuda()
    tgt = torch.from_numpy(rng.uniform(0, 1, (H, W, 3)).astype(np.float32)).cuda()
    tgt.view(-1)[::97] = img.view(-1)[::97]  # ties: sign(0) = 0
    return img, tgt


def _with_workspace(img, tgt):
    n = img.numel()
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    dl = torch.empty_like(img)
    ws = torch.empty(gsmi.loss_l1_workspace(n), dtype=torch.uint8, device="cuda")
    gsmi.loss_l1(n, img, tgt, loss, dl, ws)
    return loss, dl


def test_no_alloc_loss_matches_the_workspace_call_twice():
    for H, W, seed in ((2048, 2048, 1), (333, 517, 2)):  # the second call smaller
        print(f"[noalloc] {W}x{H}", flush=True)
        img, tgt = _case(H, W, seed)
        n = img.numel()
        loss = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
        dl = torch.full_like(img, float("nan"))
        assert _noalloc(n, img, tgt, loss, dl) == gsmi.GS_OK, gsmi.last_error()
        gsmi.loss_l1_noalloc(n, img, tgt, loss, dl)  # the binding, a second call on the same scratch
        loss_w, dl_w = _with_workspace(img, tgt)
        torch.cuda.synchronize()
        assert torch.equal(loss, loss_w), (loss.item(), loss_w.item())
        assert torch.equal(dl, dl_w)
        want = float(np.abs(img.cpu().numpy().astype(np.float64) - tgt.cpu().numpy()).mean())
        assert abs(loss.item() - want) <= 1e-6 * want


def test_no_alloc_loss_refuses_sizes_beyond_its_scratch():
    img, tgt = _case(16, 16, 3)
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    dl = torch.empty_like(img)
    assert _noalloc((1 << 28) + 1, img, tgt, loss, dl) == gsmi.GS_ERR_CAPACITY
    assert "static scratch" in gsmi.last_error()
    assert _noalloc(-1, img, tgt, loss, dl) == gsmi.GS_ERR_INVALID_ARGUMENT
    assert _noalloc(0, None, None, loss, None) == gsmi.GS_OK  # empty: the loss is 0
    torch.cuda.synchronize()
    assert loss.item() == 0.0
