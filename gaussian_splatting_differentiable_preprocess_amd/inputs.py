"""Seeded synthetic inputs for the training step: isosurface-shaped Gaussian scenes and
pinhole cameras on a structured orbit.

This module is shared by the GPU path's callers and by the CPU oracle's tests, and it holds
none of the rendering method's arithmetic: it only draws scene parameters (means on an
implicit surface, log-scales, quaternions, opacity logits, SH coefficients), builds
world-to-camera matrices with a look-at construction, and draws upstream gradients.

What the inputs stand in for:
  * "Toward Distributed 3D Gaussian Splatting for High-Resolution Isosurface Visualization",
    sections III (Method Overview) and IV (Results): isosurface point clouds extracted from
    volume data are used directly as Gaussian initialisations, and synthetic camera views
    sit on a structured orbit (448 views; 512^2, 1024^2, 2048^2 images; Kingsnake ~4M and
    Miranda ~18.18M Gaussians).  The volumes themselves are not available, so analytic
    implicit surfaces (sphere, torus, gyroid, a sum of Gaussian bumps) stand in for them.
  * "Scaling 3D Gaussian Splatting with Distributed Compute", the parameter list (mean,
    covariance from scale and rotation, SH colour, opacity) and the SH-degree-3 accounting
    (16 coefficients per channel, 59 learnable scalars per Gaussian).

Parameter storage is planar: ``params[row][ld]`` float32 with rows
    0-2 mean, 3-5 log-scale, 6-9 quaternion (w, x, y, z), 10 opacity logit,
    11 + 3k + ch  SH coefficient k of colour channel ch,   k < (d+1)^2.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

NEAR_PLANE = 0.01
FOV_DEG = 50.0


def rows_for_degree(sh_degree: int) -> int:
    """Learnable scalars per Gaussian: 3 mean + 3 scale + 4 rotation + 1 opacity + 3(d+1)^2."""
    return 11 + 3 * (sh_degree + 1) ** 2


@dataclasses.dataclass(frozen=True)
class SceneConfig:
    name: str
    index: int            # 1-based index used in the seed formula
    surface: str
    n: int
    logscale_mean: float
    logscale_std: float
    sh_degree: int
    views: str            # "single", "orbit8" or "orbit448"
    res: int
    loss: str             # "upstream" (seeded dL/dI) or "l1"
    bound_radius: float   # radius of a sphere holding the surface; camera distance = 3x this


CONFIGS = {
    "sphere_16k_256": SceneConfig("sphere_16k_256", 1, "sphere", 16384, -4.5, 0.3, 0,
                                  "single", 256, "upstream", 1.0),
    "torus_262k_512": SceneConfig("torus_262k_512", 2, "torus", 262144, -4.5, 0.3, 3,
                                  "orbit8", 512, "l1", 1.3),
    "gyroid_4m_1024": SceneConfig("gyroid_4m_1024", 3, "gyroid", 4_000_000, -6.0, 0.4, 3,
                                  "orbit448", 1024, "l1", math.pi * math.sqrt(3.0)),
    "gyroid_4m_2048": SceneConfig("gyroid_4m_2048", 4, "gyroid", 4_000_000, -6.0, 0.4, 3,
                                  "orbit448", 2048, "l1", math.pi * math.sqrt(3.0)),
    "bumps_18m_2048": SceneConfig("bumps_18m_2048", 5, "bumps", 18_180_000, -6.5, 0.4, 3,
                                  "orbit448", 2048, "l1", math.sqrt(3.0)),
}

STREAM_SCENE, STREAM_TARGET, STREAM_UPSTREAM, STREAM_FIELD = 0, 1, 2, 3


def seed_for(cfg: SceneConfig, stream: int) -> int:
    return 20260000 + 100 * cfg.index + stream


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------------------
# Surface samplers: return (points[n,3], unit normals[n,3]) in float64.
# --------------------------------------------------------------------------------------

def sample_sphere(rng, n):
    p = rng.normal(size=(n, 3))
    p /= np.linalg.norm(p, axis=1, keepdims=True)
    return p, p.copy()


def sample_torus(rng, n, big_r=1.0, small_r=0.3):
    """Area-uniform samples of a torus about z: u uniform, v by rejection with weight
    (R + r cos v) / (R + r)."""
    us = np.empty(0)
    vs = np.empty(0)
    while vs.size < n:
        m = 2 * (n - vs.size) + 1024
        v = rng.uniform(0.0, 2.0 * math.pi, m)
        w = rng.uniform(0.0, 1.0, m)
        keep = w <= (big_r + small_r * np.cos(v)) / (big_r + small_r)
        vs = np.concatenate([vs, v[keep]])
    vs = vs[:n]
    us = rng.uniform(0.0, 2.0 * math.pi, n)
    ring = big_r + small_r * np.cos(vs)
    p = np.stack([ring * np.cos(us), ring * np.sin(us), small_r * np.sin(vs)], axis=1)
    nrm = np.stack([np.cos(vs) * np.cos(us), np.cos(vs) * np.sin(us), np.sin(vs)], axis=1)
    return p, nrm


def _gyroid(x):
    sx, cx = np.sin(x[:, 0]), np.cos(x[:, 0])
    sy, cy = np.sin(x[:, 1]), np.cos(x[:, 1])
    sz, cz = np.sin(x[:, 2]), np.cos(x[:, 2])
    f = sx * cy + sy * cz + sz * cx
    g = np.stack([cx * cy - sz * sx, cy * cz - sx * sy, cz * cx - sy * sz], axis=1)
    return f, g


def sample_gyroid(rng, n, iters=16, tol=1e-7):
    """Uniform seeds in [-pi, pi]^3 Newton-projected onto sin x cos y + sin y cos z +
    sin z cos x = 0 (x <- x - f grad f / |grad f|^2, at most `iters` steps; a point stops once
    |f| < 1e-13); a seed is kept when |f| < tol and it stays inside the box."""
    pts = []
    got = 0
    while got < n:
        m = int(1.6 * (n - got)) + 4096
        x = rng.uniform(-math.pi, math.pi, (m, 3))
        active = np.arange(m)
        for _ in range(iters):
            xa = x[active]
            f, g = _gyroid(xa)
            keep = np.abs(f) >= 1e-13
            active, xa, f, g = active[keep], xa[keep], f[keep], g[keep]
            if active.size == 0:
                break
            g2 = np.einsum("ij,ij->i", g, g)
            step = np.where(g2 > 1e-30, f / np.maximum(g2, 1e-30), 0.0)
            x[active] = xa - step[:, None] * g
        f, g = _gyroid(x)
        ok = (np.abs(f) < tol) & np.all(np.abs(x) <= math.pi, axis=1) & np.all(np.isfinite(x), axis=1)
        pts.append(x[ok])
        got += int(ok.sum())
    p = np.concatenate(pts)[:n]
    _, g = _gyroid(p)
    return p, g / np.linalg.norm(g, axis=1, keepdims=True)


def _bump_field(centres, widths, amps):
    """phi(x) = sum_m a_m exp(-|x - c_m|^2 / (2 w_m^2)) evaluated with torch (CPU threads or
    a GPU when present) because 18M points x 64 bumps is too slow in numpy."""
    import torch

    dev = "cuda" if torch.cuda.is_available() else "cpu"
    c = torch.tensor(centres, dtype=torch.float64, device=dev)
    inv2w2 = torch.tensor(1.0 / (2.0 * widths ** 2), dtype=torch.float64, device=dev)
    a = torch.tensor(amps, dtype=torch.float64, device=dev)

    def field(x_np):
        x = torch.as_tensor(x_np, device=dev)
        d = x[:, None, :] - c[None, :, :]
        e = a * torch.exp(-(d * d).sum(-1) * inv2w2)
        phi = e.sum(1)
        grad = (-2.0 * (e * inv2w2)[:, :, None] * d).sum(1)
        return phi, grad

    return field, dev


def sample_bumps(rng, field_rng, n, iters=16):
    """Multi-level isosurface of a seeded sum of 64 Gaussian bumps in [-1,1]^3: levels
    {0.25, 0.5, 0.75} x the field's maximum over a 128^3 grid; an equal share of points per
    level, each Newton-projected from uniform seeds in [-1,1]^3."""
    import torch

    centres = field_rng.uniform(-0.8, 0.8, (64, 3))
    widths = field_rng.uniform(0.08, 0.25, 64)
    amps = field_rng.uniform(0.5, 1.0, 64)
    field, dev = _bump_field(centres, widths, amps)
    g1 = np.linspace(-1.0, 1.0, 128)
    gmax = 0.0
    for zi in range(128):
        xx, yy = np.meshgrid(g1, g1, indexing="ij")
        grid = np.stack([xx.ravel(), yy.ravel(), np.full(xx.size, g1[zi])], axis=1)
        gmax = max(gmax, float(field(grid)[0].max()))
    levels = [0.25 * gmax, 0.5 * gmax, 0.75 * gmax]
    per = [n // 3 + (1 if i < n % 3 else 0) for i in range(3)]
    pts, nrms = [], []
    for level, want in zip(levels, per):
        got = 0
        while got < want:
            m = min(4 * (want - got) + 4096, 2_000_000)
            x = torch.as_tensor(rng.uniform(-1.0, 1.0, (m, 3)), device=dev)
            for _ in range(iters):
                phi, g = field(x)
                g2 = (g * g).sum(1)
                step = torch.where(g2 > 1e-30, (phi - level) / g2.clamp_min(1e-30), torch.zeros_like(g2))
                x = x - step[:, None] * g
                x = torch.nan_to_num(x, nan=10.0, posinf=10.0, neginf=-10.0)
            phi, g = field(x)
            ok = ((phi - level).abs() < 1e-7 * gmax) & (x.abs() <= 1.0).all(1)
            ok &= (g * g).sum(1) > 1e-20
            xs, gs = x[ok], g[ok]
            take = min(want - got, xs.shape[0])
            pts.append(xs[:take].cpu().numpy())
            nrms.append((gs[:take] / gs[:take].norm(dim=1, keepdim=True)).cpu().numpy())
            got += take
    return np.concatenate(pts), np.concatenate(nrms)


# --------------------------------------------------------------------------------------
# Gaussian parameters
# --------------------------------------------------------------------------------------

def gaussian_params(cfg: SceneConfig, stream: int = STREAM_SCENE, n: int | None = None,
                    ld: int | None = None) -> np.ndarray:
    """Planar float32 parameters [R][ld] for the configuration's scene (stream 0) or its
    target set (stream 1).  ``n`` overrides the Gaussian count (smaller test scenes with the
    same distributions)."""
    n = cfg.n if n is None else n
    ld = n if ld is None else ld
    rng = rng_for(seed_for(cfg, stream))
    if cfg.surface == "sphere":
        p, nrm = sample_sphere(rng, n)
    elif cfg.surface == "torus":
        p, nrm = sample_torus(rng, n)
    elif cfg.surface == "gyroid":
        p, nrm = sample_gyroid(rng, n)
    elif cfg.surface == "bumps":
        p, nrm = sample_bumps(rng, rng_for(seed_for(cfg, STREAM_FIELD)), n)
    else:
        raise ValueError(cfg.surface)
    return draw_attributes(rng, p, nrm, cfg.logscale_mean, cfg.logscale_std, cfg.sh_degree, ld)


def draw_attributes(rng, points, normals, logscale_mean, logscale_std, sh_degree, ld=None):
    """Means = surface point + N(0, 0.005) along the normal; log-scales iid
    N(mean, std) per axis; quaternions = normalised N(0, I4); opacity logits N(0, 1);
    SH DC ~ U(0, 1) per channel; higher SH ~ N(0, 0.05)."""
    n = points.shape[0]
    ld = n if ld is None else ld
    rows = rows_for_degree(sh_degree)
    out = np.zeros((rows, ld), dtype=np.float32)
    eps = rng.normal(0.0, 0.005, n)
    out[0:3, :n] = (points + eps[:, None] * normals).T
    out[3:6, :n] = rng.normal(logscale_mean, logscale_std, (3, n))
    q = rng.normal(size=(4, n))
    out[6:10, :n] = q / np.linalg.norm(q, axis=0, keepdims=True)
    out[10, :n] = rng.normal(0.0, 1.0, n)
    out[11:14, :n] = rng.uniform(0.0, 1.0, (3, n))
    if sh_degree > 0:
        out[14:rows, :n] = rng.normal(0.0, 0.05, (rows - 14, n))
    return out


# --------------------------------------------------------------------------------------
# Cameras
# --------------------------------------------------------------------------------------

@dataclasses.dataclass
class Camera:
    viewmat: np.ndarray   # float32 [3,4] row-major world->camera [R|t], x right, y down, z forward
    fx: float
    fy: float
    cx: float
    cy: float
    width: int
    height: int
    near: float = NEAR_PLANE

    def flat(self) -> np.ndarray:
        """17 float64 values: viewmat (12), fx, fy, cx, cy, near -- each the float32 value."""
        v = np.concatenate([self.viewmat.astype(np.float32).ravel(),
                            np.array([self.fx, self.fy, self.cx, self.cy, self.near], np.float32)])
        return v.astype(np.float64)


def lookat_camera(position, width, height, fov_deg=FOV_DEG) -> Camera:
    """Camera at `position` looking at the origin, world up +z: forward f = -c/|c|,
    right = normalise(f x z), down = f x right."""
    c = np.asarray(position, dtype=np.float64)
    f = -c / np.linalg.norm(c)
    r = np.cross(f, np.array([0.0, 0.0, 1.0]))
    r /= np.linalg.norm(r)
    d = np.cross(f, r)
    rot = np.stack([r, d, f])
    t = -rot @ c
    vm = np.concatenate([rot, t[:, None]], axis=1).astype(np.float32)
    focal = (width / 2.0) / math.tan(math.radians(fov_deg / 2.0))
    return Camera(vm, float(np.float32(focal)), float(np.float32(focal)),
                  width / 2.0, height / 2.0, width, height)


def orbit_positions(kind: str, distance: float):
    if kind == "single":
        return [(distance, 0.0, 0.0)]
    if kind == "orbit8":
        out = []
        for j in range(8):
            phi = math.radians(45.0 * j)
            th = math.radians(20.0 if j % 2 == 0 else -20.0)
            out.append((distance * math.cos(th) * math.cos(phi),
                        distance * math.cos(th) * math.sin(phi), distance * math.sin(th)))
        return out
    if kind == "orbit448":
        out = []
        for k in range(14):
            th = math.radians(-65.0 + 10.0 * k)
            for j in range(32):
                phi = math.radians(11.25 * j + 5.625 * (k % 2))
                out.append((distance * math.cos(th) * math.cos(phi),
                            distance * math.cos(th) * math.sin(phi), distance * math.sin(th)))
        return out
    raise ValueError(kind)


def cameras_for(cfg: SceneConfig, res: int | None = None):
    res = cfg.res if res is None else res
    return [lookat_camera(p, res, res) for p in orbit_positions(cfg.views, 3.0 * cfg.bound_radius)]


def upstream_gradient(cfg: SceneConfig, width: int, height: int) -> np.ndarray:
    """Seeded dL/dpixel ~ U(-1, 1), float32 [H][W][3] (the configuration without a loss)."""
    rng = rng_for(seed_for(cfg, STREAM_UPSTREAM))
    return rng.uniform(-1.0, 1.0, (height, width, 3)).astype(np.float32)


def small_scene(seed: int, n: int, sh_degree: int, logscale_mean=-3.0, logscale_std=0.3,
                radius=1.0) -> np.ndarray:
    """A small random scene (points on a sphere of `radius`) for tests that need a few tens
    to a few thousand Gaussians."""
    rng = rng_for(seed)
    p, nrm = sample_sphere(rng, n)
    return draw_attributes(rng, p * radius, nrm, logscale_mean, logscale_std, sh_degree)
