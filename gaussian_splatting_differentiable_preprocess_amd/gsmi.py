"""Thin ctypes binding of libgsmi.so (the C ABI in include/gsmi.h).

Argument marshalling only: every step of the path runs in the library's HIP kernels.  torch
supplies device memory (tensors' data pointers) and the current HIP stream.  The library must be
built (``python -m gaussian_splatting_differentiable_preprocess_amd.build``); there is no
fallback path -- a missing library raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; GSMI_LIBRARY selects another build of the same ABI
LIB_PATH = os.environ.get("GSMI_LIBRARY", os.path.join(_PKG, "libgsmi.so"))

GS_OK, GS_ERR_INVALID_ARGUMENT, GS_ERR_CAPACITY, GS_ERR_HIP, GS_ERR_UNSUPPORTED, GS_ERR_INCOMPLETE = 0, -1, -2, -3, -4, -5
# bits of gs_render_status's flags
RENDER_FLAG_STALL, RENDER_FLAG_CAPACITY = 1, 2
TILE = 16
SPLAT_FLOATS = 12  # 48-byte record: u, v, radius_x, radius_y | A, B, C, opacity | r, g, b, depth

EXPORTS = (
    "gs_version", "gs_last_error", "gs_preprocess", "gs_bin_and_sort_workspace", "gs_bin_and_sort",
    "gs_bin_and_sort_count",
    "gs_render_workspace", "gs_render_workspace_capacity", "gs_render_forward", "gs_loss_l1_workspace", "gs_loss_l1",
    "gs_loss_l1_noalloc",
    "gs_loss_l1_dssim_workspace", "gs_loss_l1_dssim", "gs_render_backward",
    "gs_render_plan", "gs_render_step", "gs_render_init", "gs_render_status", "gs_preprocess_backward", "gs_preprocess_backward_staged",
    "gs_preprocess_backward_staged_next", "gs_adam_step",
    "gs_preprocess_backward_accumulate", "gs_adam_batch", "gs_densify_stats", "gs_densify_workspace", "gs_densify",
)


class GsError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"gsmi error {code}: {msg}")
        self.code = code


class GsCapacityError(GsError):
    def __init__(self, code, msg, required):
        super().__init__(code, msg)
        self.required = required


class GsCamera(ctypes.Structure):
    _fields_ = [("viewmat", ctypes.c_float * 12), ("fx", ctypes.c_float), ("fy", ctypes.c_float),
                ("cx", ctypes.c_float), ("cy", ctypes.c_float), ("width", ctypes.c_int32),
                ("height", ctypes.c_int32), ("near_plane", ctypes.c_float)]


class GsScene(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("ld", ctypes.c_int64), ("sh_degree", ctypes.c_int32)]


class GsProj(ctypes.Structure):
    _fields_ = [("splat", ctypes.c_void_p), ("tiles", ctypes.c_void_p), ("depth_key", ctypes.c_void_p),
                ("rect", ctypes.c_void_p)]


class GsAdam(ctypes.Structure):
    _fields_ = [("m", ctypes.c_void_p), ("v", ctypes.c_void_p), ("step", ctypes.c_int32),
                ("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double)]


_lib = None


class GsDensifyOpts(ctypes.Structure):
    _fields_ = [("grad_threshold", ctypes.c_double), ("percent_dense", ctypes.c_double),
                ("extent", ctypes.c_double), ("min_opacity", ctypes.c_double), ("split_factor", ctypes.c_double)]


def densify_opts(grad_threshold=2e-4, percent_dense=0.01, extent=1.0, min_opacity=0.005,
                 split_factor=1.6) -> GsDensifyOpts:
    return GsDensifyOpts(grad_threshold, percent_dense, extent, min_opacity, split_factor)


def load(path: str = LIB_PATH):
    """Loads libgsmi.so and declares every export; raises if the library is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m "
                           "gaussian_splatting_differentiable_preprocess_amd.build`")
    L = ctypes.CDLL(path)
    P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    SP, CP, AP = ctypes.POINTER(GsScene), ctypes.POINTER(GsCamera), ctypes.POINTER(GsAdam)
    L.gs_version.restype = ctypes.c_int
    L.gs_last_error.restype = ctypes.c_char_p
    L.gs_preprocess.argtypes = [SP, P, CP, GsProj, P]
    L.gs_bin_and_sort_workspace.argtypes = [i64, i64, i32, i32, ctypes.POINTER(sz)]
    L.gs_bin_and_sort.argtypes = [SP, CP, GsProj, P, sz, i64, P, P, P, ctypes.POINTER(i64), P]
    L.gs_bin_and_sort_count.argtypes = [P, sz, ctypes.POINTER(i64), P]
    L.gs_render_workspace.argtypes = [i32, i32, i64, i64, ctypes.POINTER(sz)]
    L.gs_render_workspace_capacity.argtypes = [i32, i32, i64, sz, ctypes.POINTER(i64)]
    L.gs_render_forward.argtypes = [CP, i64, P, P, P, i64, ctypes.POINTER(ctypes.c_float), P, P, P, P, P, P, sz, P]
    L.gs_loss_l1_workspace.argtypes = [i64, ctypes.POINTER(sz)]
    L.gs_loss_l1.argtypes = [i64, P, P, P, P, P, sz, P]
    L.gs_loss_l1_noalloc.argtypes = [i64, P, P, P, P, P]
    L.gs_loss_l1_dssim_workspace.argtypes = [i32, i32, ctypes.POINTER(sz)]
    L.gs_loss_l1_dssim.argtypes = [i32, i32, P, P, ctypes.c_float, P, P, P, sz, P]
    L.gs_render_backward.argtypes = [SP, P, CP, GsProj, P, P, i64, ctypes.POINTER(ctypes.c_float), P, P, P,
                                     P, P, AP, P, sz, P]
    L.gs_render_plan.argtypes = [SP, CP, GsProj, P, i64, P, sz, P]
    L.gs_render_step.argtypes = [SP, CP, GsProj, P, P, i64, ctypes.POINTER(ctypes.c_float), P, P, P, P, P, P, P, P, P,
                                 P, sz, P]
    L.gs_render_init.argtypes = [P, sz, P]
    L.gs_render_status.argtypes = [P, sz, ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(i64), P]
    L.gs_preprocess_backward.argtypes = [SP, P, CP, P, P, AP, P]
    L.gs_preprocess_backward_staged.argtypes = [SP, P, CP, GsProj, P, sz, P, AP, P]
    L.gs_preprocess_backward_staged_next.argtypes = [SP, P, CP, GsProj, P, sz, P, AP, CP, GsProj, P]
    L.gs_adam_step.argtypes = [i64, P, P, AP, P]
    L.gs_preprocess_backward_accumulate.argtypes = [SP, P, CP, GsProj, P, sz, P, i32, ctypes.c_float, AP, P]
    L.gs_adam_batch.argtypes = [AP, i32, AP]
    L.gs_densify_stats.argtypes = [SP, CP, GsProj, P, sz, P, P, P]
    L.gs_densify_workspace.argtypes = [i64, ctypes.POINTER(sz)]
    L.gs_densify.argtypes = [SP, P, P, P, P, P, P, ctypes.POINTER(GsDensifyOpts), P, P, P, i64,
                             ctypes.POINTER(i64), P, P, sz, P]
    for name in EXPORTS:
        if name not in ("gs_version", "gs_last_error"):
            getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def last_error() -> str:
    return load().gs_last_error().decode()


def _check(rc, required=None):
    if rc != GS_OK:
        msg = last_error()
        if rc == GS_ERR_CAPACITY:
            raise GsCapacityError(rc, msg, required)
        raise GsError(rc, msg)


def _k(k, vals):
    """The intersection count passed to the render calls: the caller's K, or when none is given the
    length of the vals buffer, which bounds it."""
    return int(vals.numel()) if k is None else int(k)


# ------------------------------------------------------------------------------------------
# marshalling helpers
# ------------------------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_camera(cam) -> GsCamera:
    """From inputs.Camera (or anything with viewmat, fx, fy, cx, cy, width, height, near)."""
    c = GsCamera()
    vm = np.asarray(cam.viewmat, dtype=np.float32).reshape(12)
    for k in range(12):
        c.viewmat[k] = float(vm[k])
    c.fx, c.fy, c.cx, c.cy = float(cam.fx), float(cam.fy), float(cam.cx), float(cam.cy)
    c.width, c.height = int(cam.width), int(cam.height)
    c.near_plane = float(getattr(cam, "near", 0.01))
    return c


def make_scene(n, ld, sh_degree) -> GsScene:
    return GsScene(int(n), int(ld), int(sh_degree))


def n_tiles(width, height):
    return ((width + TILE - 1) // TILE) * ((height + TILE - 1) // TILE)


@dataclasses.dataclass
class Proj:
    splat: "object"      # float32 [ld, 12] (48-byte records)
    tiles: "object"      # int32 [ld] (uint32 values)
    depth_key: "object"  # int32 [ld] (uint32 values)
    rect: "object"       # int32 [ld, 2] (packed x0 | y0 << 16, x1 | y1 << 16)

    def c(self) -> GsProj:
        return GsProj(self.splat.data_ptr(), self.tiles.data_ptr(), self.depth_key.data_ptr(), self.rect.data_ptr())


def alloc_proj(ld, device="cuda") -> Proj:
    import torch
    return Proj(torch.empty((ld, SPLAT_FLOATS), dtype=torch.float32, device=device),
                torch.empty(ld, dtype=torch.int32, device=device),
                torch.empty(ld, dtype=torch.int32, device=device),
                torch.empty((ld, 2), dtype=torch.int32, device=device))


# ------------------------------------------------------------------------------------------
# the C-ABI calls
# ------------------------------------------------------------------------------------------

def version() -> int:
    return load().gs_version()


def preprocess(scene: GsScene, params, cam: GsCamera, proj: Proj, stream=None):
    _check(load().gs_preprocess(ctypes.byref(scene), _ptr(params), ctypes.byref(cam), proj.c(), _stream(stream)))


def bin_and_sort_workspace(n, k_capacity, width, height) -> int:
    out = ctypes.c_size_t(0)
    _check(load().gs_bin_and_sort_workspace(int(n), int(k_capacity), int(width), int(height), ctypes.byref(out)))
    return out.value


def bin_and_sort(scene: GsScene, cam: GsCamera, proj: Proj, workspace, k_capacity, vals, ranges,
                 keys=None, stream=None, wait=True):
    """Returns K.  Raises GsCapacityError (with .required) if K > k_capacity.  With wait=False
    the sort is only enqueued (no host synchronisation) and None is returned; bin_and_sort_count
    reads K (and reports an overflow) later."""
    k = ctypes.c_int64(0)
    rc = load().gs_bin_and_sort(ctypes.byref(scene), ctypes.byref(cam), proj.c(), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), int(k_capacity),
                                _ptr(vals), _ptr(ranges), _ptr(keys), ctypes.byref(k) if wait else None,
                                _stream(stream))
    _check(rc, required=k.value)
    return k.value if wait else None


def bin_and_sort_count(workspace, stream=None) -> int:
    """K of the last bin_and_sort on `workspace` (waits for the stream).  Raises GsCapacityError
    if that call overflowed its capacity."""
    k = ctypes.c_int64(0)
    rc = load().gs_bin_and_sort_count(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                      ctypes.byref(k), _stream(stream))
    _check(rc, required=k.value)
    return k.value


def _bg(bg):
    arr = (ctypes.c_float * 3)(*[float(x) for x in bg])
    return arr


def render_workspace(width, height, n, k_capacity) -> int:
    out = ctypes.c_size_t(0)
    _check(load().gs_render_workspace(int(width), int(height), int(n), int(k_capacity), ctypes.byref(out)))
    return out.value


def render_workspace_capacity(width, height, n, nbytes) -> int:
    out = ctypes.c_int64(0)
    _check(load().gs_render_workspace_capacity(int(width), int(height), int(n), int(nbytes), ctypes.byref(out)))
    return out.value


def _nbytes(t):
    return t.numel() * t.element_size()


def render_forward(cam: GsCamera, n, splat, vals, ranges, bg, image, T_final, last_contrib, render_ws,
                   n_examined=None, blend_count=None, stream=None, k=None):
    if blend_count is not None and (blend_count.numel() < 4 or blend_count.element_size() != 8):
        raise ValueError("blend_count must be a device int64 tensor of at least 4 elements")
    _check(load().gs_render_forward(ctypes.byref(cam), int(n), _ptr(splat), _ptr(vals), _ptr(ranges), _k(k, vals),
                                    _bg(bg),
                                    _ptr(image), _ptr(T_final), _ptr(last_contrib), _ptr(n_examined),
                                    _ptr(blend_count), _ptr(render_ws), _nbytes(render_ws), _stream(stream)))


def loss_l1_workspace(count) -> int:
    out = ctypes.c_size_t(0)
    _check(load().gs_loss_l1_workspace(int(count), ctypes.byref(out)))
    return out.value


def loss_l1(count, image, target, loss, dL_dimage, workspace, stream=None):
    _check(load().gs_loss_l1(int(count), _ptr(image), _ptr(target), _ptr(loss), _ptr(dL_dimage),
                             _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def loss_l1_noalloc(count, image, target, loss, dL_dimage, stream=None):
    """gs_loss_l1 without a workspace (the library's static scratch; see gs_loss_l1_noalloc)."""
    _check(load().gs_loss_l1_noalloc(int(count), _ptr(image), _ptr(target), _ptr(loss), _ptr(dL_dimage),
                                     _stream(stream)))


def loss_l1_dssim_workspace(width, height) -> int:
    out = ctypes.c_size_t(0)
    _check(load().gs_loss_l1_dssim_workspace(int(width), int(height), ctypes.byref(out)))
    return out.value


def loss_l1_dssim(width, height, image, target, lam, loss, dL_dimage, workspace, stream=None):
    """loss: device float[3] <- (L, mean L1, mean SSIM); dL_dimage [H][W][3]."""
    _check(load().gs_loss_l1_dssim(int(width), int(height), _ptr(image), _ptr(target), float(lam), _ptr(loss),
                                   _ptr(dL_dimage), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def make_adam(m, v, step, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8) -> GsAdam:
    return GsAdam(m.data_ptr(), v.data_ptr(), int(step), float(lr), float(beta1), float(beta2), float(eps))


def render_backward(scene: GsScene, params, cam: GsCamera, proj: Proj, vals, ranges, bg, T_final,
                    last_contrib, dL_dimage, grad2d, render_ws, grads=None, adam: GsAdam | None = None,
                    stream=None, k=None):
    _check(load().gs_render_backward(ctypes.byref(scene), _ptr(params), ctypes.byref(cam), proj.c(), _ptr(vals),
                                     _ptr(ranges), _k(k, vals), _bg(bg), _ptr(T_final), _ptr(last_contrib), _ptr(dL_dimage),
                                     _ptr(grad2d), _ptr(grads), ctypes.byref(adam) if adam is not None else None,
                                     _ptr(render_ws), _nbytes(render_ws), _stream(stream)))


def render_plan(scene: GsScene, cam: GsCamera, proj: Proj, ranges, render_ws, stream=None, k=None):
    """Prepares render_ws for render_step over the lists of these ranges (k intersections; when not
    given, the largest count the workspace holds is assumed and only the device check applies)."""
    if k is None:
        k = render_workspace_capacity(cam.width, cam.height, scene.n, _nbytes(render_ws))
    _check(load().gs_render_plan(ctypes.byref(scene), ctypes.byref(cam), proj.c(), _ptr(ranges), int(k),
                                 _ptr(render_ws), _nbytes(render_ws), _stream(stream)))


def render_step(scene: GsScene, cam: GsCamera, proj: Proj, vals, ranges, bg, target, image, T_final, last_contrib,
                loss, dL_dimage, render_ws, grad2d=None, n_examined=None, blend_count=None, stream=None, k=None):
    """Forward blend, L1 loss and backward blend of one step in one fused kernel (after
    render_plan on the same render_ws); the gradient sums stay staged in render_ws for
    preprocess_backward_staged (and go to grad2d if given)."""
    if blend_count is not None and (blend_count.numel() < 4 or blend_count.element_size() != 8):
        raise ValueError("blend_count must be a device int64 tensor of at least 4 elements")
    _check(load().gs_render_step(ctypes.byref(scene), ctypes.byref(cam), proj.c(), _ptr(vals), _ptr(ranges),
                                 _k(k, vals), _bg(bg),
                                 _ptr(target), _ptr(image), _ptr(T_final), _ptr(last_contrib), _ptr(n_examined),
                                 _ptr(blend_count), _ptr(loss), _ptr(dL_dimage), _ptr(grad2d), _ptr(render_ws),
                                 _nbytes(render_ws), _stream(stream)))


def render_init(render_ws, stream=None):
    """Clears a new render workspace's status words."""
    _check(load().gs_render_init(_ptr(render_ws), _nbytes(render_ws), _stream(stream)))


def new_render_ws(width, height, n, k_capacity, device="cuda"):
    """A render workspace for up to k_capacity intersections, its status words cleared."""
    import torch
    ws = torch.empty(render_workspace(width, height, n, k_capacity), dtype=torch.uint8, device=device)
    render_init(ws)
    return ws


def render_status(render_ws, stream=None, raise_error=True):
    """The render workspace's device-side status since the last read: (flags, required
    intersections); the status words are cleared.  Synchronises the stream.  Raises
    GsCapacityError / GsError for a flagged workspace unless raise_error is False."""
    flags = ctypes.c_uint32(0)
    req = ctypes.c_int64(0)
    rc = load().gs_render_status(_ptr(render_ws), _nbytes(render_ws), ctypes.byref(flags), ctypes.byref(req),
                                 _stream(stream))
    if raise_error:
        _check(rc, required=req.value)
    return flags.value, req.value


def preprocess_backward(scene: GsScene, params, cam: GsCamera, grad2d, grads=None, adam: GsAdam | None = None,
                        stream=None):
    _check(load().gs_preprocess_backward(ctypes.byref(scene), _ptr(params), ctypes.byref(cam), _ptr(grad2d),
                                         _ptr(grads), ctypes.byref(adam) if adam is not None else None,
                                         _stream(stream)))


def preprocess_backward_staged(scene: GsScene, params, cam: GsCamera, proj: Proj, render_ws, grads=None,
                               adam: GsAdam | None = None, stream=None):
    """The preprocess backward from the sums a render_backward(grad2d=None) left in render_ws."""
    _check(load().gs_preprocess_backward_staged(ctypes.byref(scene), _ptr(params), ctypes.byref(cam), proj.c(),
                                                _ptr(render_ws), _nbytes(render_ws), _ptr(grads),
                                                ctypes.byref(adam) if adam is not None else None,
                                                _stream(stream)))


def preprocess_backward_staged_next(scene: GsScene, params, cam: GsCamera, proj: Proj, render_ws, next_cam: GsCamera,
                                    next_proj: Proj, grads=None, adam: GsAdam | None = None, stream=None):
    """preprocess_backward_staged, then the preprocess of next_cam on the updated parameters into
    next_proj (which may be proj), in one pass."""
    _check(load().gs_preprocess_backward_staged_next(ctypes.byref(scene), _ptr(params), ctypes.byref(cam), proj.c(),
                                                     _ptr(render_ws), _nbytes(render_ws), _ptr(grads),
                                                     ctypes.byref(adam) if adam is not None else None,
                                                     ctypes.byref(next_cam), next_proj.c(), _stream(stream)))


def preprocess_backward_accumulate(scene: GsScene, params, cam: GsCamera, proj: Proj, render_ws, grads_acc, first,
                                   scale, adam: GsAdam | None = None, stream=None):
    _check(load().gs_preprocess_backward_accumulate(
        ctypes.byref(scene), _ptr(params), ctypes.byref(cam), proj.c(), _ptr(render_ws), _nbytes(render_ws),
        _ptr(grads_acc), int(bool(first)), float(scale), ctypes.byref(adam) if adam is not None else None,
        _stream(stream)))


def adam_batch(adam: GsAdam, batch) -> GsAdam:
    out = GsAdam()
    _check(load().gs_adam_batch(ctypes.byref(adam), int(batch), ctypes.byref(out)))
    return out


def densify_stats(scene: GsScene, cam: GsCamera, proj: Proj, render_ws, grad_acc, count, stream=None):
    _check(load().gs_densify_stats(ctypes.byref(scene), ctypes.byref(cam), proj.c(), _ptr(render_ws),
                                   _nbytes(render_ws), _ptr(grad_acc), _ptr(count), _stream(stream)))


def densify_workspace(n) -> int:
    out = ctypes.c_size_t(0)
    _check(load().gs_densify_workspace(int(n), ctypes.byref(out)))
    return out.value


def densify(scene: GsScene, params, m, v, grad_acc, count, z, opts: GsDensifyOpts, params_out, m_out, v_out,
            ld_out, workspace, codes=None, stream=None) -> int:
    """One clone / split / prune pass; returns the new Gaussian count (GsCapacityError when it
    exceeds ld_out)."""
    n_out = ctypes.c_int64(0)
    rc = load().gs_densify(ctypes.byref(scene), _ptr(params), _ptr(m), _ptr(v), _ptr(grad_acc), _ptr(count), _ptr(z),
                           ctypes.byref(opts), _ptr(params_out), _ptr(m_out), _ptr(v_out), int(ld_out),
                           ctypes.byref(n_out), _ptr(codes), _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check(rc, required=n_out.value)
    return n_out.value


def adam_step(count, params, grads, adam: GsAdam, stream=None):
    _check(load().gs_adam_step(int(count), _ptr(params), _ptr(grads), ctypes.byref(adam), _stream(stream)))


# ------------------------------------------------------------------------------------------
# buffers for one training step and the step itself (a sequence of the calls above)
# ------------------------------------------------------------------------------------------

class StepBuffers:
    """Device buffers for training steps of one scene at one image size (allocated once with
    torch; the library allocates nothing)."""

    def __init__(self, n, ld, sh_degree, width, height, k_capacity, device="cuda"):
        import torch
        self.n, self.ld, self.deg, self.W, self.H = n, ld, sh_degree, width, height
        self.R = 11 + 3 * (sh_degree + 1) ** 2
        self.T = n_tiles(width, height)
        f32, i32 = torch.float32, torch.int32
        self.proj = alloc_proj(ld, device)
        self.k_capacity = int(k_capacity)
        self.vals = torch.empty(max(1, self.k_capacity), dtype=i32, device=device)
        self.ranges = torch.empty((self.T, 2), dtype=i32, device=device)
        self.ws = torch.empty(bin_and_sort_workspace(n, self.k_capacity, width, height), dtype=torch.uint8,
                              device=device)
        self.render_ws = new_render_ws(width, height, n, self.k_capacity, device)
        self.image = torch.empty((height, width, 3), dtype=f32, device=device)
        self.T_final = torch.empty((height, width), dtype=f32, device=device)
        self.last = torch.empty((height, width), dtype=i32, device=device)
        self.dLdI = torch.empty((height, width, 3), dtype=f32, device=device)
        self.loss = torch.zeros(3, dtype=f32, device=device)  # (L, mean L1, mean SSIM) with D-SSIM
        self.loss_ws = torch.empty(loss_l1_workspace(3 * width * height), dtype=torch.uint8, device=device)
        self.dssim_ws = None  # allocated on the first L1 + D-SSIM step
        self.grad2d = torch.empty((ld, 9), dtype=f32, device=device)
        self.scene = make_scene(n, ld, sh_degree)

    def grow(self, k_capacity, device="cuda"):
        import torch
        self.k_capacity = int(k_capacity)
        self.vals = torch.empty(max(1, self.k_capacity), dtype=torch.int32, device=device)
        self.ws = torch.empty(bin_and_sort_workspace(self.n, self.k_capacity, self.W, self.H), dtype=torch.uint8,
                              device=device)
        self.render_ws = new_render_ws(self.W, self.H, self.n, self.k_capacity, device)


def train_step(buf: StepBuffers, params, m, v, step, cam: GsCamera, target=None, upstream=None,
               bg=(0.0, 0.0, 0.0), lr=1e-3, fused_adam=True, grads=None, blend_count=None, dssim_lambda=None):
    """One fwd + bwd + Adam step for one view: preprocess -> bin/sort -> forward -> L1, or
    L1 + D-SSIM weighted by `dssim_lambda`, or the given upstream dL/dI -> backward (+ Adam).
    Returns K."""
    preprocess(buf.scene, params, cam, buf.proj)
    while True:
        try:
            K = bin_and_sort(buf.scene, cam, buf.proj, buf.ws, buf.k_capacity, buf.vals, buf.ranges)
            break
        except GsCapacityError as e:
            buf.grow(int(e.required * 1.25) + 1024)
    render_forward(cam, buf.n, buf.proj.splat, buf.vals, buf.ranges, bg, buf.image, buf.T_final, buf.last,
                   buf.render_ws, blend_count=blend_count, k=K)
    if upstream is not None:
        dLdI = upstream
    elif dssim_lambda is not None:
        if buf.dssim_ws is None:
            import torch
            buf.dssim_ws = torch.empty(loss_l1_dssim_workspace(buf.W, buf.H), dtype=torch.uint8,
                                       device=buf.image.device)
        loss_l1_dssim(buf.W, buf.H, buf.image, target, dssim_lambda, buf.loss, buf.dLdI, buf.dssim_ws)
        dLdI = buf.dLdI
    else:
        loss_l1(3 * buf.W * buf.H, buf.image, target, buf.loss, buf.dLdI, buf.loss_ws)
        dLdI = buf.dLdI
    adam = make_adam(m, v, step, lr)
    if fused_adam:
        render_backward(buf.scene, params, cam, buf.proj, buf.vals, buf.ranges, bg, buf.T_final, buf.last, dLdI,
                        buf.grad2d, buf.render_ws, grads, adam, k=K)
    else:
        render_backward(buf.scene, params, cam, buf.proj, buf.vals, buf.ranges, bg, buf.T_final, buf.last, dLdI,
                        buf.grad2d, buf.render_ws, grads, k=K)
        adam_step(buf.R * buf.ld, params, grads, adam)
    return K


def train_batch(buf: StepBuffers, params, m, v, step, cams, targets, grads_acc, bg=(0.0, 0.0, 0.0), lr=1e-3,
                beta1=0.9, beta2=0.999, eps=1e-8, dssim_lambda=None, blend_count=None):
    """One optimizer step over a batch of views ("Scaling 3D Gaussian Splatting with Distributed
    Compute", the batch-size passage): per view preprocess -> bin/sort -> image pass (the fused
    forward + L1 + backward, or forward, L1 + D-SSIM and backward as three calls) -> preprocess
    backward adding 1/BS of the view's gradient into grads_acc; the last view's backward runs the
    Adam update on the batch mean with gs_adam_batch's hyper-parameters.  `step` counts
    optimizer steps (batches).  Returns the views' intersection counts."""
    B = len(cams)
    if B < 1 or len(targets) != B:
        raise ValueError("one target per camera, at least one camera")
    adam = adam_batch(make_adam(m, v, step, lr, beta1, beta2, eps), B)
    ks = []
    for j, (cam, tgt) in enumerate(zip(cams, targets)):
        preprocess(buf.scene, params, cam, buf.proj)
        while True:
            try:
                K = bin_and_sort(buf.scene, cam, buf.proj, buf.ws, buf.k_capacity, buf.vals, buf.ranges)
                break
            except GsCapacityError as e:
                buf.grow(int(e.required * 1.25) + 1024)
        if dssim_lambda is None:
            render_plan(buf.scene, cam, buf.proj, buf.ranges, buf.render_ws, k=K)
            render_step(buf.scene, cam, buf.proj, buf.vals, buf.ranges, bg, tgt, buf.image, buf.T_final, buf.last,
                        buf.loss, buf.dLdI, buf.render_ws, blend_count=blend_count, k=K)
        else:
            if buf.dssim_ws is None:
                import torch
                buf.dssim_ws = torch.empty(loss_l1_dssim_workspace(buf.W, buf.H), dtype=torch.uint8,
                                           device=buf.image.device)
            render_forward(cam, buf.n, buf.proj.splat, buf.vals, buf.ranges, bg, buf.image, buf.T_final, buf.last,
                           buf.render_ws, blend_count=blend_count, k=K)
            loss_l1_dssim(buf.W, buf.H, buf.image, tgt, dssim_lambda, buf.loss, buf.dLdI, buf.dssim_ws)
            render_backward(buf.scene, None, cam, buf.proj, buf.vals, buf.ranges, bg, buf.T_final, buf.last,
                            buf.dLdI, None, buf.render_ws, k=K)
        preprocess_backward_accumulate(buf.scene, params, cam, buf.proj, buf.render_ws, grads_acc, j == 0, 1.0 / B,
                                       adam if j == B - 1 else None)
        ks.append(K)
    return ks
