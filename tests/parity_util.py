"""Helpers for the GPU parity tests: run each stage of the step through the C ABI on seeded
inputs and compare with the CPU oracle fed the same inputs."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from gaussian_splatting_differentiable_preprocess_amd import gsmi

# tolerances: floating point per the stated bars, integer work bit-exact
IMG_MAX_ABS = 1e-4
GRAD_REL_L2 = 1e-3
PROJ_RTOL = 1e-5
# Borderline margins for threshold decisions with identical inputs.  float32 evaluation of
# o exp(power) at the 1/255 threshold (power ~ -5.5, three rounded products, one fma chain,
# v_exp) is off by ~3e-6 relative at most; T after up to a few hundred float32 products by
# ~1e-5 relative.  Pixels with a decision inside these bands are flagged and excluded.
FWD_MARGINS = (1e-5, 3e-5, 1e-6)   # alpha (relative), T (relative), power (absolute)
BORDER_FRACTION = 1e-3             # sanity bound on the flagged share of pixels
# preprocess: |u| <= 2048 px carries ~1e-4 px of float32 error = 6e-6 tile units
TILE_EDGE_MARGIN = 2e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))


def to_t(x, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def proj_f32(proj):
    """The oracle's projected record as float32 values (the record is 12 float32 scalars); the
    oracle's later stages and the GPU stages under test both read these values."""
    return np.asarray(proj, np.float64).astype(np.float32).astype(np.float64)


def pack_rects(rect):
    """Oracle tile rects [4][n] (x0, x1, y0, y1) -> the packed form [n][2] uint32
    (x0 | y0 << 16, x1 | y1 << 16)."""
    r = np.asarray(rect, np.uint32)
    return np.stack([r[0] | (r[2] << 16), r[1] | (r[3] << 16)], axis=1).astype(np.uint32)


def records_from_oracle(proj, radii, tiles, W, H):
    """Oracle projection (planar [10][n], radii [2][n], tiles [n]) -> the GPU's 48-byte records
    ([n][12] float32: u, v, radius bits x2, conic a b c, opacity, r g b, depth), tiles, depth
    keys (float bits, all-ones when culled) and the oracle's tile rects, packed.  A layout
    conversion: every value is the oracle's."""
    p = np.asarray(proj, np.float64)
    radii = np.asarray(radii, np.int32)
    n = p.shape[1]
    rec = np.zeros((n, 12), np.float32)
    rec[:, 0], rec[:, 1] = p[0], p[1]
    rec[:, 2], rec[:, 3] = radii[0].view(np.float32), radii[1].view(np.float32)
    rec[:, 4], rec[:, 5], rec[:, 6], rec[:, 7] = p[4], p[5], p[6], p[3]
    rec[:, 8], rec[:, 9], rec[:, 10], rec[:, 11] = p[7], p[8], p[9], p[2]
    vis = (radii[0] > 0) & (radii[1] > 0)
    dkey = np.where(vis, rec[:, 11].view(np.uint32), np.uint32(0xFFFFFFFF)).astype(np.uint32)
    return rec, np.asarray(tiles, np.uint32), dkey, pack_rects(oracle.tile_rects(proj, radii, W, H))


def oracle_pipeline(params, deg, cam_flat, W, H, bg, target=None, upstream=None, margins=None):
    """The oracle's whole step from the seeded inputs alone: preprocess, then every later stage
    on the float32 record values; the loss on the float32 image; dL/dI rounded to float32 for
    the backward (the form the GPU stages under test are given)."""
    proj, radii, tiles = oracle.preprocess(params, deg, cam_flat, W, H)
    p32 = proj_f32(proj)
    keys, vals = oracle.bin_sort(p32, radii, W, H)
    rg = oracle.ranges(keys, oracle.n_tiles(W, H))
    fwd = oracle.render_forward(p32, vals, rg, W, H, bg, margins=margins)
    img32 = fwd["image"].astype(np.float32)
    if upstream is not None:
        loss, dLdI = None, np.asarray(upstream, np.float64)
    else:
        loss, dLdI = oracle.loss_l1(img32.astype(np.float64), target)
    dl32 = dLdI.astype(np.float32)
    g2 = oracle.render_backward(p32, vals, rg, W, H, dl32.astype(np.float64), bg)
    grads = oracle.preprocess_backward(params, deg, cam_flat, W, H, g2)
    return dict(proj=proj, p32=p32, radii=radii, tiles=tiles, keys=keys, vals=vals, ranges=rg.reshape(-1, 2),
                fwd=fwd, img32=img32, loss=loss, dLdI=dLdI, dl32=dl32, grad2d=g2, grads=grads)


def proj_from_splat(splat, depth_key=None):
    """GPU records [n, 12] float32 -> oracle layout proj [10][n] float64, radii [2][n]."""
    s = np.asarray(splat, np.float32)
    proj = np.zeros((10, s.shape[0]))
    proj[0], proj[1] = s[:, 0], s[:, 1]
    proj[2] = s[:, 11]
    proj[3] = s[:, 7]
    proj[4], proj[5], proj[6] = s[:, 4], s[:, 5], s[:, 6]
    proj[7], proj[8], proj[9] = s[:, 8], s[:, 9], s[:, 10]
    radii = np.stack([s[:, 2].view(np.int32), s[:, 3].view(np.int32)]).astype(np.int32)
    return proj, radii


class GpuStep:
    """Runs the stages of one training step on the GPU for numpy inputs."""

    def __init__(self, params, deg, cam, W, H, k_capacity=None):
        import torch
        self.deg, self.W, self.H = deg, W, H
        self.R, self.ld = params.shape
        self.n = self.ld
        self.cam = gsmi.make_camera(cam)
        self.scene = gsmi.make_scene(self.n, self.ld, deg)
        self.params = to_t(params.astype(np.float32))
        self.proj = gsmi.alloc_proj(max(1, self.ld))
        self.T = gsmi.n_tiles(W, H)
        self.kcap = k_capacity
        self.torch = torch

    def load_proj(self, rec, tiles, dkey, rect):
        """Puts oracle-derived records, tiles and depth keys in the GPU projection buffers."""
        n = rec.shape[0]
        self.proj.splat[:n].copy_(to_t(np.ascontiguousarray(rec, np.float32)))
        self.proj.tiles[:n].copy_(to_t(np.ascontiguousarray(tiles, np.uint32).view(np.int32)))
        self.proj.depth_key[:n].copy_(to_t(np.ascontiguousarray(dkey, np.uint32).view(np.int32)))
        self.proj.rect[:n].copy_(to_t(np.ascontiguousarray(rect, np.uint32).view(np.int32)))
        self.torch.cuda.synchronize()

    def load_lists(self, vals, ranges):
        """Puts oracle-derived sorted lists (vals [K], ranges [T][2]) on the GPU."""
        torch = self.torch
        vals = np.ascontiguousarray(vals, np.uint32)
        self.vals = torch.empty(max(1, vals.size), dtype=torch.int32, device="cuda")
        if vals.size:
            self.vals[: vals.size].copy_(to_t(vals.view(np.int32)))
        self.ranges = to_t(np.ascontiguousarray(np.asarray(ranges, np.uint32).reshape(-1, 2)).view(np.int32))
        self.K = int(vals.size)

    def loss_on(self, image, target):
        """GPU L1 loss of a given float32 image."""
        self.image = to_t(np.ascontiguousarray(image, np.float32))
        return self.loss(target)

    def preprocess(self):
        gsmi.preprocess(self.scene, self.params, self.cam, self.proj)
        self.torch.cuda.synchronize()
        splat = self.proj.splat.cpu().numpy()[: self.n]
        tiles = self.proj.tiles.cpu().numpy().view(np.uint32)[: self.n]
        dkey = self.proj.depth_key.cpu().numpy().view(np.uint32)[: self.n]
        self.last_rect = self.proj.rect.cpu().numpy().view(np.uint32)[: self.n]  # [n][2], packed
        return splat, tiles, dkey

    def bin_and_sort(self, k_capacity=None):
        torch = self.torch
        kcap = k_capacity if k_capacity is not None else (self.kcap or int(self.proj.tiles[: self.n].sum().item()) + 16)
        self.vals = torch.empty(max(kcap, 1), dtype=torch.int32, device="cuda")
        self.keys = torch.empty(max(kcap, 1), dtype=torch.int64, device="cuda")
        self.ranges = torch.empty((self.T, 2), dtype=torch.int32, device="cuda")
        ws = torch.empty(gsmi.bin_and_sort_workspace(self.n, kcap, self.W, self.H), dtype=torch.uint8, device="cuda")
        K = gsmi.bin_and_sort(self.scene, self.cam, self.proj, ws, kcap, self.vals, self.ranges, self.keys)
        torch.cuda.synchronize()
        self.K = K
        return (K, self.keys.cpu().numpy().view(np.uint64)[:K], self.vals.cpu().numpy().view(np.uint32)[:K],
                self.ranges.cpu().numpy().view(np.uint32))

    def forward(self, bg=(0.0, 0.0, 0.0), ranges=None):
        torch = self.torch
        H, W = self.H, self.W
        self.bg = bg
        rg = self.ranges if ranges is None else to_t(np.asarray(ranges, np.uint32).view(np.int32))
        nb = gsmi.render_workspace(W, H, self.n, max(1, int(self.vals.numel())))
        self.render_ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        self.image = torch.empty((H, W, 3), dtype=torch.float32, device="cuda")
        self.T_final = torch.empty((H, W), dtype=torch.float32, device="cuda")
        self.last = torch.empty((H, W), dtype=torch.int32, device="cuda")
        self.nex = torch.empty((H, W), dtype=torch.int32, device="cuda")
        self.bcount = torch.zeros(3, dtype=torch.int64, device="cuda")
        gsmi.render_forward(self.cam, self.n, self.proj.splat, self.vals, rg, bg, self.image, self.T_final,
                            self.last, self.render_ws, self.nex, self.bcount)
        torch.cuda.synchronize()
        return dict(image=self.image.cpu().numpy(), T_final=self.T_final.cpu().numpy(),
                    last_contrib=self.last.cpu().numpy().view(np.uint32),
                    n_examined=self.nex.cpu().numpy().view(np.uint32), blend_count=self.bcount.cpu().tolist())

    def loss(self, target):
        torch = self.torch
        self.target = to_t(target.astype(np.float32))
        self.dLdI = torch.empty((self.H, self.W, 3), dtype=torch.float32, device="cuda")
        lossv = torch.zeros(1, dtype=torch.float32, device="cuda")
        cnt = 3 * self.H * self.W
        ws = torch.empty(gsmi.loss_l1_workspace(cnt), dtype=torch.uint8, device="cuda")
        gsmi.loss_l1(cnt, self.image, self.target, lossv, self.dLdI, ws)
        torch.cuda.synchronize()
        return float(lossv.item()), self.dLdI.cpu().numpy()

    def set_upstream(self, g):
        self.dLdI = to_t(g.astype(np.float32))

    def backward(self, ranges=None):
        torch = self.torch
        self.grad2d = torch.empty((self.ld, 9), dtype=torch.float32, device="cuda")
        self.grads = torch.empty((self.R, self.ld), dtype=torch.float32, device="cuda")
        rg = self.ranges if ranges is None else to_t(np.asarray(ranges, np.uint32).view(np.int32))
        gsmi.render_backward(self.scene, self.params, self.cam, self.proj, self.vals, rg, self.bg, self.T_final,
                             self.last, self.dLdI, self.grad2d, self.render_ws, self.grads)
        torch.cuda.synchronize()
        return np.ascontiguousarray(self.grad2d.cpu().numpy().T), self.grads.cpu().numpy()  # grad2d as [9][ld]

    def step(self, bg, target, ranges=None):
        """The fused image pass (forward, L1 loss and backward blend in one kernel) on the loaded
        records and lists: the forward's outputs, the loss, dL/dI, grad2d gathered from the staged
        sums ([9][ld]) and the workspace's stall word."""
        torch = self.torch
        H, W = self.H, self.W
        self.bg = bg
        rg = self.ranges if ranges is None else to_t(np.asarray(ranges, np.uint32).view(np.int32))
        nb = gsmi.render_workspace(W, H, self.n, max(1, int(self.vals.numel())))
        self.render_ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        self.image = torch.empty((H, W, 3), dtype=torch.float32, device="cuda")
        self.T_final = torch.empty((H, W), dtype=torch.float32, device="cuda")
        self.last = torch.empty((H, W), dtype=torch.int32, device="cuda")
        self.nex = torch.empty((H, W), dtype=torch.int32, device="cuda")
        self.bcount = torch.zeros(3, dtype=torch.int64, device="cuda")
        self.target = to_t(np.asarray(target, np.float32))
        self.dLdI = torch.empty((H, W, 3), dtype=torch.float32, device="cuda")
        lossv = torch.zeros(1, dtype=torch.float32, device="cuda")
        g2 = torch.empty((max(1, self.ld), 9), dtype=torch.float32, device="cuda")
        gsmi.render_plan(self.scene, self.cam, self.proj, rg, self.render_ws)
        gsmi.render_step(self.scene, self.cam, self.proj, self.vals, rg, bg, self.target, self.image, self.T_final,
                         self.last, lossv, self.dLdI, self.render_ws, grad2d=g2, n_examined=self.nex,
                         blend_count=self.bcount)
        torch.cuda.synchronize()
        stall = int(self.render_ws[:64].cpu().numpy().view(np.uint32)[8])
        return dict(image=self.image.cpu().numpy(), T_final=self.T_final.cpu().numpy(),
                    last_contrib=self.last.cpu().numpy().view(np.uint32),
                    n_examined=self.nex.cpu().numpy().view(np.uint32), blend_count=self.bcount.cpu().tolist(),
                    loss=float(lossv.item()), dLdI=self.dLdI.cpu().numpy(),
                    grad2d=np.ascontiguousarray(g2.cpu().numpy()[: self.ld].T), stall=stall)

    def preprocess_backward_staged(self, adam=None):
        """The preprocess backward from the sums the last step left staged: dL/dparams."""
        torch = self.torch
        grads = torch.empty((self.R, self.ld), dtype=torch.float32, device="cuda")
        gsmi.preprocess_backward_staged(self.scene, self.params, self.cam, self.proj, self.render_ws, grads, adam)
        torch.cuda.synchronize()
        return grads.cpu().numpy()

    def preprocess_backward(self, grad2d):
        torch = self.torch
        g2 = to_t(np.ascontiguousarray(np.asarray(grad2d, np.float32).T))  # [9][ld] -> [ld][9]
        grads = torch.empty((self.R, self.ld), dtype=torch.float32, device="cuda")
        gsmi.preprocess_backward(self.scene, self.params, self.cam, g2, grads)
        torch.cuda.synchronize()
        return grads.cpu().numpy()


def preprocess_borderline(params, deg, cam_flat, W, H, u, v, radii):
    """Gaussians whose integer outputs may legitimately differ between float32 evaluations:
    3 sqrt(S2_ii) within 1e-5 (relative) of an integer, or a box edge (u +- r)/16 within 1e-4
    tile of a tile boundary."""
    mg = oracle.preprocess_margins(params, deg, cam_flat, W, H)
    bl = np.zeros(params.shape[1], bool)
    for a in (mg[0], mg[1]):
        frac = np.abs(a - np.round(a))
        bl |= (a > 0) & (frac <= 1e-5 * np.maximum(a, 1.0))
    for c, r in ((u, radii[0]), (u, -radii[0]), (v, radii[1]), (v, -radii[1])):
        x = (c + r) / 16.0
        bl |= np.abs(x - np.round(x)) <= TILE_EDGE_MARGIN
    return bl
