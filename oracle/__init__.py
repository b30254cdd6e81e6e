"""CPU oracle for one 3D Gaussian Splatting training step -- TEST INFRASTRUCTURE.

Only the test-suite, the smoke check and the bench's CPU-baseline leg import this package.
The product path (the HIP library and its binding) never imports, links or runs it.

The arithmetic lives in ``oracle.c`` (plain C, IEEE double); this module compiles it with
gcc into ``liboracle.so`` next to the source and wraps each function with numpy arrays.
Function-by-function citations of the pages are in ``oracle.c``.

Parity status: every function is pinned by tests under ``tests/`` (closed forms,
invariants, brute force, finite differences, a library Adam); the absolute images are not
pinned by the pages, which print no rendered values.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIBRARY names a prebuilt copy of the library to load instead (the host-sanitizer test
# builds one with AddressSanitizer and UndefinedBehaviorSanitizer); such a copy is never rebuilt.
_LIB_OVERRIDE = os.environ.get("ORACLE_LIBRARY")
_LIB = _LIB_OVERRIDE or os.path.join(_HERE, "liboracle.so")

PROJ_FIELDS = ("u", "v", "depth", "opacity", "A", "B", "C", "r", "g", "b")
GRAD2D_FIELDS = ("u", "v", "A", "B", "C", "opacity", "r", "g", "b")
DEC_SKIP, DEC_BLEND, DEC_BLEND_CLAMPED, DEC_STOP, DEC_NONE = 0, 1, 2, 3, 4


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    if _LIB_OVERRIDE:
        return _LIB
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-D_GNU_SOURCE", "-ffp-contract=off", "-fno-fast-math",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.or_rows_for_degree.argtypes = [i32]
        L.or_set_num_threads.argtypes = [i32]
        L.or_get_max_threads.restype = i32
        L.or_sh_basis.argtypes = [i32, dbl, dbl, dbl, P]
        L.or_quat_to_rot.argtypes = [P, P]
        L.or_preprocess.argtypes = [i64, i32, P, P, i32, i32, P, P, P]
        L.or_preprocess_margins.argtypes = [i64, i32, P, P, i32, i32, P]
        L.or_tile_rects.argtypes = [i64, P, P, i32, i32, P]
        L.or_count_intersections.argtypes = [i64, P, P, i32, i32]
        L.or_count_intersections.restype = i64
        L.or_bin_sort.argtypes = [i64, P, P, i32, i32, P, P]
        L.or_bin_sort.restype = i64
        L.or_ranges.argtypes = [i64, P, i32, P]
        L.or_render_forward.argtypes = [i32, i32, P, i64, P, P, P, P, P, P, P, P, P, P, P, i64, i32, P]
        L.or_render_bruteforce.argtypes = [i32, i32, P, i64, P, P, P, P, P, P]
        L.or_loss_l1.argtypes = [i64, P, P, P]
        L.or_loss_l1.restype = dbl
        L.or_loss_l1_dssim.argtypes = [i32, i32, P, P, dbl, P, P]
        L.or_loss_l1_dssim.restype = dbl
        L.or_render_backward.argtypes = [i32, i32, P, i64, P, P, P, P, P, P, i64]
        L.or_preprocess_backward.argtypes = [i64, i32, P, P, i32, i32, P, P]
        L.or_adam.argtypes = [i64, P, P, P, P, i32, dbl, dbl, dbl, dbl]
        L.or_debug_gaussian.argtypes = [i32, P, P, i32, i32, P]
        _lib = L
    return _lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def set_num_threads(n):
    """OpenMP threads of the oracle's parallel loops."""
    lib().or_set_num_threads(int(n))


def max_threads():
    return lib().or_get_max_threads()


def rows_for_degree(d):
    return lib().or_rows_for_degree(d)


def sh_basis(deg, x, y, z):
    out = np.zeros(16)
    lib().or_sh_basis(deg, x, y, z, _p(out))
    return out


def quat_to_rot(q):
    q = _f64(q)
    out = np.zeros(9)
    lib().or_quat_to_rot(_p(q), _p(out))
    return out.reshape(3, 3)


def debug_gaussian(param_col, sh_degree, cam_flat, W, H):
    """Intermediates of the preprocess for one Gaussian (its R parameters)."""
    p = _f64(param_col).reshape(-1)
    out = np.zeros(63)
    lib().or_debug_gaussian(sh_degree, _p(p), _p(_f64(cam_flat)), W, H, _p(out))
    return dict(visible=bool(out[0]), s=out[1:4], o=out[4], R=out[5:14].reshape(3, 3),
                Sigma=out[14:23].reshape(3, 3), p_cam=out[23:26], J=out[26:32].reshape(2, 3),
                V=out[32:41].reshape(3, 3), S2=out[41:45].reshape(2, 2), Q=out[45:49].reshape(2, 2),
                u=out[49], v=out[50], rx=int(out[51]), ry=int(out[52]), tiles=int(out[53]),
                dir=out[54:57], raw=out[57:60], rgb=out[60:63])


def preprocess(params, sh_degree, cam_flat, W, H):
    """params [R][n] -> (proj [10][n] float64, radii [2][n] int32, tiles [n] uint32)."""
    params = _f64(params)
    n = params.shape[1]
    cam = _f64(cam_flat)
    proj = np.zeros((10, n))
    radii = np.zeros((2, n), np.int32)
    tiles = np.zeros(n, np.uint32)
    lib().or_preprocess(n, sh_degree, _p(params), _p(cam), W, H, _p(proj), _p(radii), _p(tiles))
    return proj, radii, tiles


def preprocess_margins(params, sh_degree, cam_flat, W, H):
    """[3][n]: 3 sqrt(S2_00), 3 sqrt(S2_11), min |raw colour| (0 for culled)."""
    params = _f64(params)
    n = params.shape[1]
    out = np.zeros((3, n))
    lib().or_preprocess_margins(n, sh_degree, _p(params), _p(_f64(cam_flat)), W, H, _p(out))
    return out


def tile_rects(proj, radii, W, H):
    """-> int32 [4][n]: x0, x1, y0, y1 of each Gaussian's tile rect [x0, x1) x [y0, y1) (all 0
    if culled); u, v are read as float32 (the binning decision)."""
    proj = _f64(proj)
    radii = np.ascontiguousarray(radii, np.int32)
    n = proj.shape[1]
    out = np.zeros((4, n), np.int32)
    lib().or_tile_rects(n, _p(proj), _p(radii), W, H, _p(out))
    return out


def bin_sort(proj, radii, W, H):
    """-> (keys uint64 [K], vals uint32 [K]).  u, v, depth are read as float32."""
    proj = _f64(proj)
    radii = np.ascontiguousarray(radii, np.int32)
    n = proj.shape[1]
    K = lib().or_count_intersections(n, _p(proj), _p(radii), W, H)
    keys = np.zeros(max(K, 1), np.uint64)
    vals = np.zeros(max(K, 1), np.uint32)
    K2 = lib().or_bin_sort(n, _p(proj), _p(radii), W, H, _p(keys), _p(vals))
    assert K2 == K
    return keys[:K], vals[:K]


def ranges(keys, n_tiles):
    keys = np.ascontiguousarray(keys, np.uint64)
    out = np.zeros(2 * n_tiles, np.uint32)
    lib().or_ranges(keys.size, _p(keys), n_tiles, _p(out))
    return out.reshape(n_tiles, 2)


def render_forward(proj, vals, rng, W, H, bg=(0.0, 0.0, 0.0), margins=None,
                   record_decisions=False, decisions=None, walk=False):
    """Tiled forward.  Returns dict(image [H][W][3], T_final, last_contrib, n_examined,
    borderline, n_blended), with record_decisions 'decisions' (int8 [H*W][maxlen]) and with walk
    'walk' (uint64 [H][W]: a hash of the Gaussians each pixel composited, in order, and the one
    that stopped it)."""
    proj = _f64(proj)
    n = proj.shape[1]
    vals = np.ascontiguousarray(vals, np.uint32)
    rng = np.ascontiguousarray(rng, np.uint32).reshape(-1)
    bgv = _f64(bg)
    img = np.zeros((H, W, 3))
    Tf = np.zeros((H, W))
    last = np.zeros((H, W), np.uint32)
    ex = np.zeros((H, W), np.uint32)
    bl = np.zeros((H, W), np.uint8)
    nb = np.zeros((H, W), np.uint32)
    mg = _f64(margins) if margins is not None else None
    lens = rng[1::2].astype(np.int64) - rng[0::2].astype(np.int64)
    stride = int(max(1, lens.max() if lens.size else 1))
    dec, mode = None, 0
    if record_decisions:
        dec = np.full((H * W, stride), DEC_NONE, np.int8)
        mode = 1
    elif decisions is not None:
        dec = np.ascontiguousarray(decisions, np.int8)
        stride = dec.shape[1]
        mode = 2
    vals_arg = vals if vals.size else np.zeros(1, np.uint32)
    wh = np.zeros((H, W), np.uint64) if walk else None
    lib().or_render_forward(W, H, _p(bgv), n, _p(proj), _p(vals_arg), _p(rng), _p(img), _p(Tf),
                            _p(last), _p(ex), _p(bl), _p(nb), _p(mg), _p(dec), stride, mode, _p(wh))
    out = dict(image=img, T_final=Tf, last_contrib=last, n_examined=ex, borderline=bl.astype(bool),
               n_blended=nb)
    if walk:
        out["walk"] = wh
    if record_decisions:
        out["decisions"] = dec
    return out


def render_bruteforce(proj, radii, W, H, bg=(0.0, 0.0, 0.0)):
    proj = _f64(proj)
    n = proj.shape[1]
    radii = np.ascontiguousarray(radii, np.int32)
    img = np.zeros((H, W, 3))
    Tf = np.zeros((H, W))
    last = np.zeros((H, W), np.uint32)
    ex = np.zeros((H, W), np.uint32)
    lib().or_render_bruteforce(W, H, _p(_f64(bg)), n, _p(proj), _p(radii), _p(img), _p(Tf),
                               _p(last), _p(ex))
    return dict(image=img, T_final=Tf, last_contrib=last, n_examined=ex)


def loss_l1(image, target):
    image = _f64(image)
    target = _f64(target)
    g = np.zeros_like(image)
    L = lib().or_loss_l1(image.size, _p(image), _p(target), _p(g))
    return L, g


def loss_l1_dssim(image, target, lam=0.2):
    """L1 + D-SSIM loss of an [H][W][3] image -> (L, mean L1, mean SSIM, dL/dimage float64)."""
    image = _f64(image)
    target = _f64(target)
    H, W = image.shape[0], image.shape[1]
    assert image.shape == (H, W, 3) and target.shape == image.shape
    g = np.zeros_like(image)
    parts = np.zeros(2)
    L = lib().or_loss_l1_dssim(W, H, _p(image), _p(target), float(lam), _p(parts), _p(g))
    return L, float(parts[0]), float(parts[1]), g


def render_backward(proj, vals, rng, W, H, dLdI, bg=(0.0, 0.0, 0.0), decisions=None):
    """-> grad2d [9][n] float64 (u, v, A, B, C, opacity, r, g, b)."""
    proj = _f64(proj)
    n = proj.shape[1]
    vals = np.ascontiguousarray(vals, np.uint32)
    rng = np.ascontiguousarray(rng, np.uint32).reshape(-1)
    g = _f64(dLdI)
    out = np.zeros((9, n))
    dec, stride = None, 0
    if decisions is not None:
        dec = np.ascontiguousarray(decisions, np.int8)
        stride = dec.shape[1]
    vals_arg = vals if vals.size else np.zeros(1, np.uint32)
    lib().or_render_backward(W, H, _p(_f64(bg)), n, _p(proj), _p(vals_arg), _p(rng), _p(g),
                             _p(out), _p(dec), stride)
    return out


def preprocess_backward(params, sh_degree, cam_flat, W, H, grad2d):
    params = _f64(params)
    n = params.shape[1]
    out = np.zeros_like(params)
    lib().or_preprocess_backward(n, sh_degree, _p(params), _p(_f64(cam_flat)), W, H,
                                 _p(_f64(grad2d)), _p(out))
    return out


def adam(theta, grad, m, v, t, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8):
    """In-place on float64 arrays (copies are returned for convenience)."""
    theta = _f64(theta).copy()
    m = _f64(m).copy()
    v = _f64(v).copy()
    g = _f64(grad)
    lib().or_adam(theta.size, _p(theta), _p(g), _p(m), _p(v), t, lr, b1, b2, eps)
    return theta, m, v


def n_tiles(W, H):
    return ((W + 15) // 16) * ((H + 15) // 16)


def train_step_reference(params, sh_degree, cam_flat, W, H, target=None, upstream=None,
                         m=None, v=None, t=1, lr=1e-3, bg=(0.0, 0.0, 0.0), dssim_lambda=None):
    """The whole step in the oracle: preprocess -> bin/sort -> ranges -> forward -> loss
    (L1 against `target`, L1 + D-SSIM when `dssim_lambda` is given, or the given upstream
    dL/dI) -> backward -> preprocess backward -> Adam.  Returns a dict with every
    intermediate."""
    proj, radii, tiles = preprocess(params, sh_degree, cam_flat, W, H)
    keys, vals = bin_sort(proj, radii, W, H)
    rg = ranges(keys, n_tiles(W, H))
    fwd = render_forward(proj, vals, rg, W, H, bg)
    if upstream is not None:
        dLdI = _f64(upstream)
        loss = float((dLdI * fwd["image"]).sum())
    elif dssim_lambda is not None:
        loss, _, _, dLdI = loss_l1_dssim(fwd["image"], target, dssim_lambda)
    else:
        loss, dLdI = loss_l1(fwd["image"], target)
    g2 = render_backward(proj, vals, rg, W, H, dLdI, bg)
    grads = preprocess_backward(params, sh_degree, cam_flat, W, H, g2)
    out = dict(proj=proj, radii=radii, tiles=tiles, keys=keys, vals=vals, ranges=rg, loss=loss,
               dLdI=dLdI, grad2d=g2, grads=grads, **fwd)
    if m is not None:
        out["params_new"], out["m_new"], out["v_new"] = adam(params, grads, m, v, t, lr)
    return out


def adam_batch_hparams(lr, beta1, beta2, eps, batch):
    """Adam's hyper-parameters for `batch` views per optimizer step ("Scaling 3D Gaussian
    Splatting with Distributed Compute", the batch-size passage): the learning rate scales as
    sqrt(BS), epsilon as 1/sqrt(BS), and each momentum coefficient is decayed linearly,
    beta <- 1 - BS (1 - beta), which takes beta1 = 0.9 to zero at BS = 10 as the page says.
    Returns (lr, beta1, beta2, eps)."""
    s = math.sqrt(batch)
    return lr * s, 1.0 - batch * (1.0 - beta1), 1.0 - batch * (1.0 - beta2), eps / s


def train_batch_reference(params, sh_degree, cam_flats, W, H, targets, m, v, t, lr=1e-3, beta1=0.9,
                          beta2=0.999, eps=1e-8, bg=(0.0, 0.0, 0.0), dssim_lambda=None):
    """One optimizer step over a batch of views (the batch-size passage of the same page): the
    loss is the mean of the views' losses, so the gradient is the mean of their gradients, and
    one Adam step with the batch-scaled hyper-parameters follows.  Returns (params_new, m_new,
    v_new, grads)."""
    grads = None
    for c, tgt in zip(cam_flats, targets):
        g = train_step_reference(params, sh_degree, c, W, H, target=tgt, bg=bg, dssim_lambda=dssim_lambda)["grads"]
        grads = g if grads is None else grads + g
    grads = grads / len(cam_flats)
    lr_b, b1_b, b2_b, eps_b = adam_batch_hparams(lr, beta1, beta2, eps, len(cam_flats))
    p_new, m_new, v_new = adam(params, grads, m, v, t, lr_b, b1_b, b2_b, eps_b)
    return p_new, m_new, v_new, grads


# ------------------------------------------------------------------------------------------
# Adaptive density control: clone, split, prune
# ------------------------------------------------------------------------------------------
# "Scaling 3D Gaussian Splatting with Distributed Compute" names adaptive density control
# (pruning and densifying, growing N) and its intervals in steps, and prints none of its rules.
# The reading taken is 3D-GS's: the statistic is each Gaussian's view-space 2D mean gradient
# norm in normalised device units, averaged over the views that saw it; a Gaussian at or above
# the gradient threshold is cloned when its largest scale is at most percent_dense x the scene
# extent and split in two otherwise; Gaussians below the minimum opacity are removed.  The
# decisions are taken on float32 values in forms both sides evaluate exactly: the averaged
# statistic (one float32 division), the largest log-scale against log(percent_dense x extent),
# and the opacity logit against logit(min_opacity).
DENS_KEEP, DENS_CLONE, DENS_SPLIT, DENS_PRUNE = 0, 1, 2, 3


def densify_view_stats(grad2d, radii, W, H):
    """One view's contribution to the densification statistics: the norm of (dL/du W/2,
    dL/dv H/2) -- the mean's gradient in normalised device units -- and 1, for every Gaussian
    the view sees (radius > 0); 0 and 0 elsewhere."""
    vis = np.asarray(radii)[0] > 0
    g = _f64(grad2d)
    norm = np.sqrt((g[0] * (0.5 * W)) ** 2 + (g[1] * (0.5 * H)) ** 2)
    return np.where(vis, norm, 0.0), vis.astype(np.float64)


def densify_thresholds(grad_threshold, percent_dense, extent, min_opacity):
    """The three float32 thresholds the decisions compare against."""
    return (np.float32(grad_threshold), np.float32(math.log(percent_dense * extent)),
            np.float32(math.log(min_opacity / (1.0 - min_opacity))))


def densify_codes(params, grad_acc, count, grad_threshold=2e-4, percent_dense=0.01, extent=1.0,
                  min_opacity=0.005):
    """Per Gaussian: prune when its opacity is below min_opacity; otherwise, when its averaged
    statistic reaches grad_threshold, clone (largest scale <= percent_dense x extent) or split."""
    p = np.asarray(params, dtype=np.float32)
    acc = np.asarray(grad_acc, dtype=np.float32)
    cnt = np.asarray(count, dtype=np.float32)
    t_grad, t_lscale, t_logit = densify_thresholds(grad_threshold, percent_dense, extent, min_opacity)
    seen = cnt > 0
    g = np.zeros_like(acc)
    g[seen] = acc[seen] / cnt[seen]                      # one float32 division
    largest = np.fmax(np.fmax(p[3], p[4]), p[5])         # largest log-scale (a NaN one skipped)
    codes = np.full(p.shape[1], DENS_KEEP, dtype=np.int32)
    dense = g >= t_grad
    codes[dense & (largest <= t_lscale)] = DENS_CLONE
    codes[dense & (largest > t_lscale)] = DENS_SPLIT
    codes[p[10] < t_logit] = DENS_PRUNE
    # every comparison with NaN is false: a NaN statistic never densifies, a NaN logit never
    # prunes, and three NaN log-scales neither clone nor split
    return codes


def _rotations(q):
    """Rotation matrices [n][3][3] of the quaternions q [4][n] = (w, x, y, z) after normalising."""
    w, x, y, z = np.asarray(q, dtype=np.float64) / np.linalg.norm(q, axis=0)
    return np.stack([
        np.stack([1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)], -1),
        np.stack([2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)], -1),
        np.stack([2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)], -1)], 1)


def densify(params, m, v, grad_acc, count, z, grad_threshold=2e-4, percent_dense=0.01, extent=1.0,
            min_opacity=0.005, split_factor=1.6):
    """One densification.  Output Gaussians, in this order: the kept ones (neither pruned nor
    split) in index order; a copy of each cloned one in index order; the first child of each
    split one in index order; the second children likewise.  A split Gaussian's child k takes
    mean mu + R(q) (s * z[k]) with s = exp(log-scale) and z[k] the standard normal draw given
    for it (z: [2][3][n]), log-scale minus log(split_factor), and the parent's rotation,
    opacity and colour.  Kept Gaussians keep their Adam moments; new ones start at zero.
    Returns (params, m, v) as float64 [R][n_out], and the codes."""
    P = _f64(params)
    codes = densify_codes(params, grad_acc, count, grad_threshold, percent_dense, extent, min_opacity)
    kept = np.nonzero((codes == DENS_KEEP) | (codes == DENS_CLONE))[0]
    clones = np.nonzero(codes == DENS_CLONE)[0]
    splits = np.nonzero(codes == DENS_SPLIT)[0]
    zz = _f64(z)
    Rq = _rotations(P[6:10, splits])                     # [n_split][3][3]
    s = np.exp(P[3:6, splits])                           # [3][n_split]
    children = []
    for k in range(2):
        c = P[:, splits].copy()
        d = s * zz[k][:, splits]                         # s * z[k], [3][n_split]
        c[0:3] = P[0:3, splits] + np.einsum("nij,jn->in", Rq, d)
        c[3:6] = P[3:6, splits] - math.log(split_factor)
        children.append(c)
    out = np.concatenate([P[:, kept], P[:, clones], children[0], children[1]], axis=1)
    R = P.shape[0]
    n_new = out.shape[1] - kept.size
    m_out = np.concatenate([_f64(m)[:, kept], np.zeros((R, n_new))], axis=1)
    v_out = np.concatenate([_f64(v)[:, kept], np.zeros((R, n_new))], axis=1)
    return out, m_out, v_out, codes
