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
# A pixel is flagged when one of its walk's decisions lies in a band around a threshold; the
# alpha decisions near 1/255 lie on the rims of the Gaussians' footprints, so the flagged pixels
# grow with the composited pairs (measured 3e-6 to 7.5e-6 per composited pair from the 16K sphere
# to the 18.18M scene): bound them at 4e-5 per composited pair.
BORDER_PER_COMPOSITED = 4e-5


def border_bound(n_blended):
    """The most borderline-flagged pixels allowed for a forward whose pixels composited n_blended
    entries."""
    return max(8.0, BORDER_PER_COMPOSITED * float(np.asarray(n_blended, np.int64).sum()))
# preprocess: |u| <= 2048 px carries ~1e-4 px of float32 error = 6e-6 tile units
TILE_EDGE_MARGIN = 2e-5
# End to end, both sides run the whole step from the parameters, so their float32 records differ
# in the last bits and a decision at a threshold can flip; the flipped pixels and the Gaussians
# they reach are counted, bounded and left out of the element-wise bars (e2e_exclusion).
FLIP_FRACTION = 5e-3               # bound on the flipped share of pixels
EXCLUDED_FRACTION = 0.1            # bound on the excluded share of visible Gaussians
ALPHA_MIN = 1.0 / 255.0
CANDIDATE_ALPHA_REL = 1e-3         # "may be composited": o e^power >= (1/255)(1 - 1e-3)


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


def oracle_pipeline(params, deg, cam_flat, W, H, bg, target=None, upstream=None, margins=None, dssim=None):
    """The oracle's whole step from the seeded inputs alone: preprocess, then every later stage
    on the float32 record values; the loss (L1, or L1 + D-SSIM weighted by `dssim`) on the float32
    image; dL/dI rounded to float32 for the backward (the form the GPU stages under test are
    given)."""
    big = params.shape[1] >= 1 << 20  # progress lines for the full-size runs
    proj, radii, tiles = oracle.preprocess(params, deg, cam_flat, W, H)
    p32 = proj_f32(proj)
    keys, vals = oracle.bin_sort(p32, radii, W, H)
    rg = oracle.ranges(keys, oracle.n_tiles(W, H))
    if big:
        say(f"[oracle]   preprocess and sort done (K = {keys.size}); forward")
    fwd = oracle.render_forward(p32, vals, rg, W, H, bg, margins=margins, walk=True)
    img32 = fwd["image"].astype(np.float32)
    if upstream is not None:
        loss, dLdI = None, np.asarray(upstream, np.float64)
    elif dssim is not None:
        loss, _, _, dLdI = oracle.loss_l1_dssim(img32.astype(np.float64), target, dssim)
    else:
        loss, dLdI = oracle.loss_l1(img32.astype(np.float64), target)
    dl32 = dLdI.astype(np.float32)
    if big:
        say("[oracle]   forward done; backward blend")
    g2 = oracle.render_backward(p32, vals, rg, W, H, dl32.astype(np.float64), bg)
    if big:
        say("[oracle]   backward blend done; preprocess backward")
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
        self.render_ws = gsmi.new_render_ws(W, H, self.n, max(1, int(self.vals.numel())))
        self.image = torch.empty((H, W, 3), dtype=torch.float32, device="cuda")
        self.T_final = torch.empty((H, W), dtype=torch.float32, device="cuda")
        self.last = torch.empty((H, W), dtype=torch.int32, device="cuda")
        self.nex = torch.empty((H, W), dtype=torch.int32, device="cuda")
        self.bcount = torch.zeros(4, dtype=torch.int64, device="cuda")
        gsmi.render_forward(self.cam, self.n, self.proj.splat, self.vals, rg, bg, self.image, self.T_final,
                            self.last, self.render_ws, self.nex, self.bcount, k=self.K)
        gsmi.render_status(self.render_ws)
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
                             self.last, self.dLdI, self.grad2d, self.render_ws, self.grads, k=self.K)
        gsmi.render_status(self.render_ws)
        return np.ascontiguousarray(self.grad2d.cpu().numpy().T), self.grads.cpu().numpy()  # grad2d as [9][ld]

    def step(self, bg, target, ranges=None):
        """The fused image pass (forward, L1 loss and backward blend in one kernel) on the loaded
        records and lists: the forward's outputs, the loss, dL/dI, grad2d gathered from the staged
        sums ([9][ld]) and the workspace's stall word."""
        torch = self.torch
        H, W = self.H, self.W
        self.bg = bg
        rg = self.ranges if ranges is None else to_t(np.asarray(ranges, np.uint32).view(np.int32))
        self.render_ws = gsmi.new_render_ws(W, H, self.n, max(1, int(self.vals.numel())))
        self.image = torch.empty((H, W, 3), dtype=torch.float32, device="cuda")
        self.T_final = torch.empty((H, W), dtype=torch.float32, device="cuda")
        self.last = torch.empty((H, W), dtype=torch.int32, device="cuda")
        self.nex = torch.empty((H, W), dtype=torch.int32, device="cuda")
        self.bcount = torch.zeros(4, dtype=torch.int64, device="cuda")
        self.target = to_t(np.asarray(target, np.float32))
        self.dLdI = torch.empty((H, W, 3), dtype=torch.float32, device="cuda")
        lossv = torch.zeros(1, dtype=torch.float32, device="cuda")
        g2 = torch.empty((max(1, self.ld), 9), dtype=torch.float32, device="cuda")
        gsmi.render_plan(self.scene, self.cam, self.proj, rg, self.render_ws, k=self.K)
        gsmi.render_step(self.scene, self.cam, self.proj, self.vals, rg, bg, self.target, self.image, self.T_final,
                         self.last, lossv, self.dLdI, self.render_ws, grad2d=g2, n_examined=self.nex,
                         blend_count=self.bcount, k=self.K)
        flags, _ = gsmi.render_status(self.render_ws, raise_error=False)
        stall = flags & gsmi.RENDER_FLAG_STALL
        assert not flags & gsmi.RENDER_FLAG_CAPACITY, "the render workspace is short of the lists"
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

    def loss_dssim(self, target, lam):
        """GPU L1 + D-SSIM loss of the current image: (L, mean L1, mean SSIM), dL/dI."""
        torch = self.torch
        self.target = to_t(np.asarray(target, np.float32))
        self.dLdI = torch.empty((self.H, self.W, 3), dtype=torch.float32, device="cuda")
        lossv = torch.zeros(3, dtype=torch.float32, device="cuda")
        ws = torch.empty(gsmi.loss_l1_dssim_workspace(self.W, self.H), dtype=torch.uint8, device="cuda")
        gsmi.loss_l1_dssim(self.W, self.H, self.image, self.target, lam, lossv, self.dLdI, ws)
        torch.cuda.synchronize()
        return lossv.cpu().numpy(), self.dLdI.cpu().numpy()

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



def tile_of_pixels(W, H):
    """[H][W] tile index of every pixel."""
    TX = (W + 15) // 16
    return (np.arange(H)[:, None] // 16) * TX + (np.arange(W)[None, :] // 16)


def _hits(rec, ids, xs, ys):
    """bool [pixels][ids]: o e^power >= (1/255)(1 - 1e-3) with power <= 1e-3 at pixel centres
    (xs, ys), in float64 from float32 records rec [10][n] (oracle layout)."""
    u, v, o = rec[0, ids], rec[1, ids], rec[3, ids]
    A, B, C = rec[4, ids], rec[5, ids], rec[6, ids]
    dx = xs[:, None] - u[None, :]
    dy = ys[:, None] - v[None, :]
    power = -0.5 * (A * dx * dx + C * dy * dy) - B * dx * dy
    oG = o * np.exp(np.minimum(power, 1.0))
    return (power <= 1e-3) & (oG >= ALPHA_MIN * (1.0 - CANDIDATE_ALPHA_REL))


def _groups(tiles):
    order = np.argsort(tiles, kind="stable")
    st = tiles[order]
    cuts = np.flatnonzero(np.diff(st)) + 1
    return order, [(int(st[a]), order[a:b]) for a, b in zip(np.r_[0, cuts], np.r_[cuts, st.size])]


def may_composite(rec, vals, ranges, W, H, pix, prefix, chunk=1 << 15):
    """Gaussians that may be composited at the pixels `pix` (flat indices): per pixel, the entries
    of its tile's list at positions < prefix[pixel] that pass _hits there.  When the two sides'
    records agree to float32 rounding this holds every entry either side composites there."""
    out = np.zeros(rec.shape[1], bool)
    if pix.size == 0:
        return out
    ranges = np.asarray(ranges, np.int64).reshape(-1, 2)
    vals = np.asarray(vals, np.int64)
    TX = (W + 15) // 16
    py, px = pix // W, pix % W
    pre = np.asarray(prefix, np.int64)
    for t, sel in _groups((py // 16) * TX + px // 16)[1]:
        s, e = ranges[t]
        L = int(min(e - s, pre[sel].max()))
        xs, ys, ps = px[sel] + 0.5, py[sel] + 0.5, pre[sel]
        for c0 in range(0, L, chunk):
            ids = vals[s + c0: s + min(L, c0 + chunk)]
            pos = c0 + np.arange(ids.size)
            hit = _hits(rec, ids, xs, ys) & (pos[None, :] < ps[:, None])
            out[ids[hit.any(axis=0)]] = True
    return out



def stage_exclusion(o, g, W, H, target=None):
    """The Gaussians a stage comparison of gradients leaves out: those that may be composited at a
    pixel where the two forwards legitimately differ -- the oracle flags it borderline, or its
    integer outputs differ (only at borderline pixels, which the forward tests assert) -- or,
    with an L1 loss computed on each side's own image, where the sign of image - target differs
    in a channel.  Both sides walk the same records and lists there, so the backward of such a
    pixel follows different decisions on each side.
      o  the oracle's step (oracle_pipeline); g  the GPU forward's image, last_contrib, n_examined
    Returns (excluded bool [n], report)."""
    fo = o["fwd"]
    flip = fo["borderline"] | (np.asarray(g["last_contrib"]) != fo["last_contrib"]) | \
        (np.asarray(g["n_examined"]) != fo["n_examined"])
    n_sign = 0
    if target is not None:
        t = np.asarray(target, np.float64)
        sflip = (np.sign(np.asarray(g["image"], np.float64) - t) != np.sign(o["img32"].astype(np.float64) - t)).any(-1)
        n_sign = int((sflip & ~flip).sum())
        flip = flip | sflip
    pix = np.flatnonzero(flip.reshape(-1))
    prefix = np.maximum(np.asarray(g["n_examined"], np.int64), fo["n_examined"].astype(np.int64)).reshape(-1)[pix]
    ex = may_composite(o["p32"], o["vals"], o["ranges"], W, H, pix, prefix)
    rep = dict(pixels=int(flip.sum()), sign=n_sign, excluded=int(ex.sum()), visible=int((o["radii"][0] > 0).sum()))
    assert rep["excluded"] <= max(8, EXCLUDED_FRACTION * rep["visible"]), rep
    return ex, rep


def e2e_exclusion(o, g, W, H, bg, target=None, ssim_reach=0, pre_bl=None):
    """The flipped pixels and excluded Gaussians of an end-to-end run.
      o  the oracle's step (oracle_pipeline: its walk hashes over its own records and lists)
      g  the GPU's own run: image, last_contrib, n_examined, vals [K], ranges [T][2], radii [2][n],
         tiles [n], rec (its float32 records in the oracle's layout [10][n])
    The oracle walks the GPU's records and lists too.  A pixel is flipped when that walk composites
    other Gaussians, or in another order, or stops elsewhere than the oracle's walk over its own
    records (the two records differ in their last bits, so an entry near a threshold can land on
    either side); when the GPU's float32 walk may differ from that walk on the same records (the
    stage-borderline flag, or differing integer outputs); or, for an L1 loss, when the sign of
    image - target differs in a channel (the pixel's dL/dI then differs).  With the D-SSIM loss a
    flipped pixel's image difference reaches every pixel within `ssim_reach`, so the flipped set
    is dilated by that much first.  A Gaussian is excluded when its preprocess is borderline or
    its integer preprocess outputs differ, or when it may be composited at a flipped pixel on
    either side.  Returns (excluded bool [n], flipped pixels bool [H][W] before the dilation,
    report)."""
    fo = o["fwd"]
    f2 = oracle.render_forward(g["rec"], g["vals"], np.asarray(g["ranges"]).reshape(-1, 2), W, H, bg,
                               margins=FWD_MARGINS, walk=True)
    walk = fo["walk"] != f2["walk"]
    stage = f2["borderline"]
    gint = (np.asarray(g["last_contrib"]) != f2["last_contrib"]) | (np.asarray(g["n_examined"]) != f2["n_examined"])
    flip = walk | stage | gint
    img_flip = flip.copy()
    if ssim_reach and flip.any():
        from scipy.ndimage import binary_dilation
        flip = binary_dilation(flip, structure=np.ones((2 * ssim_reach + 1, 2 * ssim_reach + 1), bool))
    n_sign = 0
    if target is not None:
        t = np.asarray(target, np.float64)
        sflip = (np.sign(np.asarray(g["image"], np.float64) - t) != np.sign(o["img32"].astype(np.float64) - t)).any(-1)
        n_sign = int(sflip.sum())
        flip |= sflip
    pix = np.flatnonzero(flip.reshape(-1))
    prefix = np.maximum(np.asarray(g["n_examined"], np.int64), fo["n_examined"].astype(np.int64)).reshape(-1)[pix]
    ex = may_composite(o["p32"], o["vals"], o["ranges"], W, H, pix, prefix)
    ex |= may_composite(g["rec"], g["vals"], g["ranges"], W, H, pix, prefix)
    pre = (np.asarray(g["radii"]) != o["radii"]).any(axis=0) | (np.asarray(g["tiles"]) != o["tiles"])
    if pre_bl is not None:
        pre |= pre_bl
    ex |= pre
    rep = dict(pixels=W * H, flipped=int(img_flip.sum()), walk=int(walk.sum()), stage=int(stage.sum()),
               gpu_int=int(gint.sum()), sign=n_sign, reach=int(flip.sum()), excluded=int(ex.sum()),
               pre=int(pre.sum()), visible=int((o["radii"][0] > 0).sum()))
    return ex, img_flip, rep

def check_e2e(label, o, g, W, H, bg, grads_g, grads_o, target=None, ssim_reach=0, pre_bl=None, grad2d_g=None,
              grad2d_o=None):
    """Asserts the end-to-end bars under the flip rule (image max-abs 1e-4 off the flipped pixels,
    gradients rel-L2 1e-3 per parameter group and overall off the excluded Gaussians) and the
    bounds on the flipped and excluded shares; prints every share.  Returns the report."""
    ex, flip, rep = e2e_exclusion(o, g, W, H, bg, target, ssim_reach, pre_bl)
    keep = ~ex
    err = np.abs(np.asarray(g["image"], np.float64) - o["fwd"]["image"]).max(axis=-1)
    img_err = float(err[~flip].max()) if (~flip).any() else 0.0
    gg, go = np.asarray(grads_g), np.asarray(grads_o)
    e_all = rel_l2(gg[:, keep], go[:, keep])
    groups = {"mean": slice(0, 3), "scale": slice(3, 6), "rot": slice(6, 10), "opacity": slice(10, 11),
              "sh": slice(11, None)}
    e_grp = {k: rel_l2(gg[sl][:, keep], go[sl][:, keep]) for k, sl in groups.items()}
    rep.update(image_err=img_err, grads_rel=e_all, grads_rel_unexcluded=rel_l2(gg, go))
    msg = (f"[e2e] {label}: {rep['flipped']} flipped px of {rep['pixels']} ({rep['walk']} walks differ, "
           f"{rep['stage']} stage-borderline, {rep['gpu_int']} GPU integer outputs differ; "
           f"{rep['sign']} L1 sign; {rep['reach']} px reached), {rep['excluded']} of {rep['visible']} visible "
           f"Gaussians excluded ({rep['pre']} by the preprocess); image max-abs elsewhere {img_err:.3g}; grads rel-L2 "
           f"on the rest {e_all:.3g} (" + ", ".join(f"{k} {v:.2g}" for k, v in e_grp.items()) +
           f"), unexcluded {rep['grads_rel_unexcluded']:.3g}")
    if grad2d_g is not None:
        e2 = max(rel_l2(np.asarray(grad2d_g)[r][keep], np.asarray(grad2d_o)[r][keep]) for r in range(9))
        msg += f"; grad2d worst row on the rest {e2:.3g}"
        rep["grad2d_rel"] = e2
    say(msg)
    assert rep["flipped"] <= max(4, FLIP_FRACTION * rep["pixels"]), (label, rep)
    assert rep["excluded"] <= max(8, EXCLUDED_FRACTION * rep["visible"]), (label, rep)
    assert img_err <= IMG_MAX_ABS, (label, img_err)
    assert e_all <= GRAD_REL_L2, (label, e_all)
    for k, v in e_grp.items():
        assert v <= GRAD_REL_L2, (label, k, v)
    if grad2d_g is not None:
        assert rep["grad2d_rel"] <= GRAD_REL_L2, (label, rep["grad2d_rel"])
    return rep



def gpu_e2e(params, deg, cam, W, H, bg, target=None, upstream=None, fused=False, dssim=None, k_capacity=None):
    """The GPU's whole step from the parameters: preprocess, bin/sort, then the fused image pass
    (fused, L1 against target) or the separate forward, loss (L1, L1 + D-SSIM, or the given
    upstream dL/dI) and backward blend, then the preprocess backward.  Returns what the flip rule
    and the bars read: image, last_contrib, n_examined, vals, ranges, radii, tiles, rec (its
    records in the oracle's layout), grad2d [9][n], grads [R][n], and the loss."""
    g = GpuStep(params, deg, cam, W, H, k_capacity=k_capacity)
    splat, tiles, _ = g.preprocess()
    rec, radii = proj_from_splat(splat)
    K, _, vals, rg = g.bin_and_sort()
    out = dict(rec=rec.astype(np.float32).astype(np.float64), radii=radii, tiles=tiles, vals=vals,
               ranges=rg.reshape(-1, 2), K=K)
    if fused:
        r = g.step(bg, target)
        assert r["stall"] == 0
        out.update(image=r["image"], last_contrib=r["last_contrib"], n_examined=r["n_examined"], loss=r["loss"],
                   grad2d=r["grad2d"], blend_count=r["blend_count"])
        out["grads"] = g.preprocess_backward_staged()
        return out
    f = g.forward(bg)
    out.update(image=f["image"], last_contrib=f["last_contrib"], n_examined=f["n_examined"],
               blend_count=f["blend_count"])
    if upstream is not None:
        g.set_upstream(np.asarray(upstream, np.float32))
        out["loss"] = None
    elif dssim is not None:
        out["loss"], _ = g.loss_dssim(target, dssim)
    else:
        out["loss"], _ = g.loss(target)
    out["grad2d"], out["grads"] = g.backward()
    return out
