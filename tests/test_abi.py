"""The C-ABI library loads and exports every symbol include/gsmi.h declares; argument checks
and workspace queries (host-only, no HIP call) behave as documented.  No compute call here."""
import ctypes
import os
import re

import pytest

from gaussian_splatting_differentiable_preprocess_amd import gsmi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared():
    src = open(os.path.join(ROOT, "include", "gsmi.h")).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(gs_\w+)\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    L = gsmi.load()
    names = declared()
    assert len(names) == len(gsmi.EXPORTS) and set(names) == set(gsmi.EXPORTS)
    for name in names:
        assert hasattr(L, name), name
    assert gsmi.version() == 9


def test_sort_count_arguments_checked_on_the_host():
    """gs_bin_and_sort_count rejects a null, short or misaligned workspace and a null k_out
    before any HIP call."""
    L = gsmi.load()
    k = ctypes.c_int64(0)
    assert L.gs_bin_and_sort_count(None, 4096, ctypes.byref(k), None) == gsmi.GS_ERR_INVALID_ARGUMENT
    assert "null" in gsmi.last_error()
    assert L.gs_bin_and_sort_count(ctypes.c_void_p(256), 4096, None, None) == gsmi.GS_ERR_INVALID_ARGUMENT
    assert L.gs_bin_and_sort_count(ctypes.c_void_p(256), 8, ctypes.byref(k), None) == gsmi.GS_ERR_INVALID_ARGUMENT
    assert "small" in gsmi.last_error()
    assert L.gs_bin_and_sort_count(ctypes.c_void_p(260), 4096, ctypes.byref(k), None) == gsmi.GS_ERR_INVALID_ARGUMENT
    assert "aligned" in gsmi.last_error()


def test_invalid_arguments_rejected_before_any_gpu_call():
    L = gsmi.load()
    cam = gsmi.GsCamera()
    cam.fx = cam.fy = 100.0
    cam.width = cam.height = 64
    cam.near_plane = 0.01
    cam.viewmat[0] = cam.viewmat[5] = cam.viewmat[10] = 1.0
    bad = [
        (gsmi.make_scene(10, 5, 0), cam, "ld"),
        (gsmi.make_scene(-1, 5, 0), cam, "n ="),
        (gsmi.make_scene(10, 10, 4), cam, "sh_degree"),
    ]
    for sc, c, msg in bad:
        rc = L.gs_preprocess(ctypes.byref(sc), None, ctypes.byref(c), gsmi.GsProj(), None)
        assert rc == gsmi.GS_ERR_INVALID_ARGUMENT and msg in gsmi.last_error()
    sc = gsmi.make_scene(10, 10, 0)
    assert L.gs_preprocess(ctypes.byref(sc), None, None, gsmi.GsProj(), None) == gsmi.GS_ERR_INVALID_ARGUMENT
    c2 = gsmi.GsCamera.from_buffer_copy(cam)
    c2.fx = float("nan")
    assert L.gs_preprocess(ctypes.byref(sc), None, ctypes.byref(c2), gsmi.GsProj(), None) == -1
    c3 = gsmi.GsCamera.from_buffer_copy(cam)
    c3.width = 0
    assert L.gs_preprocess(ctypes.byref(sc), None, ctypes.byref(c3), gsmi.GsProj(), None) == -1
    # null params with n > 0
    proj = gsmi.GsProj(16, 16, 16, 16)
    assert L.gs_preprocess(ctypes.byref(sc), None, ctypes.byref(cam), proj, None) == -1
    # misaligned record buffer, missing or misaligned tile rects
    assert L.gs_preprocess(ctypes.byref(sc), ctypes.c_void_p(64), ctypes.byref(cam), gsmi.GsProj(8, 16, 16, 16),
                           None) == -1
    assert "aligned" in gsmi.last_error()
    assert L.gs_preprocess(ctypes.byref(sc), ctypes.c_void_p(64), ctypes.byref(cam), gsmi.GsProj(16, 16, 16, None),
                           None) == -1
    assert "rect" in gsmi.last_error()
    assert L.gs_preprocess(ctypes.byref(sc), ctypes.c_void_p(64), ctypes.byref(cam), gsmi.GsProj(16, 16, 16, 20),
                           None) == -1
    assert "rect" in gsmi.last_error()
    # Adam with a bad step / null moments
    ad = gsmi.GsAdam(None, None, 1, 1e-3, 0.9, 0.999, 1e-8)
    assert L.gs_adam_step(10, ctypes.c_void_p(64), ctypes.c_void_p(64), ctypes.byref(ad), None) == -1
    ad = gsmi.GsAdam(64, 64, 0, 1e-3, 0.9, 0.999, 1e-8)
    assert L.gs_adam_step(10, ctypes.c_void_p(64), ctypes.c_void_p(64), ctypes.byref(ad), None) == -1
    assert L.gs_adam_step(10, ctypes.c_void_p(64), ctypes.c_void_p(64), None, None) == -1
    # bin_and_sort: workspace too small, null k_out
    k = ctypes.c_int64(0)
    rc = L.gs_bin_and_sort(ctypes.byref(sc), ctypes.byref(cam), proj, ctypes.c_void_p(256), 16, 100,
                           ctypes.c_void_p(64), ctypes.c_void_p(64), None, ctypes.byref(k), None)
    assert rc == -1 and "workspace" in gsmi.last_error()


def test_workspace_queries():
    a = gsmi.bin_and_sort_workspace(4_000_000, 8_000_000, 2048, 2048)
    b = gsmi.bin_and_sort_workspace(4_000_000, 16_000_000, 2048, 2048)
    # 16 bytes per intersection of capacity (two ping-pong key/value pairs)
    assert b - a >= 16 * 8_000_000 and b - a < 16 * 8_000_000 + 8 * 1024 * 1024
    assert gsmi.bin_and_sort_workspace(0, 0, 1, 1) > 0
    assert gsmi.loss_l1_workspace(3 * 2048 * 2048) >= 4 * (3 * 2048 * 2048) // 4096
    with pytest.raises(gsmi.GsError):
        gsmi.bin_and_sort_workspace(-1, 0, 16, 16)
    # render workspace: a fixed part for the tiles and Gaussians plus, per 512 intersections of
    # capacity, one 4 KiB state slot, one work item, eight 2 KiB chunks of composited masks (8
    # bytes per pixel of a tile per 64 entries) and 512 staged 36-byte gradient sums; and for
    # the split tiles (lists of at least 65536 entries, in forward segments of at least 2048),
    # per forward segment three 4 KiB per-pixel arrays and an item, and per split tile 4 KiB of
    # pixel state and 20 bytes
    r0 = gsmi.render_workspace(2048, 2048, 4_000_000, 0)
    k = 512 * 1000
    r1 = gsmi.render_workspace(2048, 2048, 4_000_000, k)
    fsegs = k // 2048 + k // 65536  # (the fixed part holds 2 segments and 1 split tile)
    splits = k // 65536
    expect = 1000 * (4096 + 8 + 8 * 2048 + 512 * 36) + fsegs * (3 * 4096 + 8) + splits * (16 * 256 + 20)
    assert abs((r1 - r0) - expect) <= 6 * 256, (r1 - r0, expect)
    assert r0 >= 16384 * (4096 + 8 + 2048 + 4) + 4 * 4_000_000
    with pytest.raises(gsmi.GsError):
        gsmi.render_workspace(0, 16, 10, 10)
    # the capacity query inverts the size query: never below the capacity asked for, and no
    # more than one 512-entry segment above it
    for W, H in ((17, 33), (64, 64), (1024, 1024), (2048, 2048)):
        for n in (1, 120, 3000, 262144, 4_000_000):
            for k in (0, 1, 255, 256, 257, 12_345, 6_800_000, 10_300_000):
                got = gsmi.render_workspace_capacity(W, H, n, gsmi.render_workspace(W, H, n, k))
                assert k <= got < k + 1024, (W, H, n, k, got)
    with pytest.raises(gsmi.GsError):
        gsmi.render_workspace_capacity(64, 64, 10, 100)


def test_loss_l1_dssim_checks_its_arguments():
    L = gsmi.load()
    need = gsmi.loss_l1_dssim_workspace(2048, 2048)
    # nine float32 partials per window position plus the per-workgroup sums
    assert 36 * 2038 * 2038 <= need < 36 * 2038 * 2038 + 64 * 1024
    assert gsmi.loss_l1_dssim_workspace(11, 11) >= 36
    for W, H in ((10, 64), (64, 10), (0, 0)):
        with pytest.raises(gsmi.GsError):
            gsmi.loss_l1_dssim_workspace(W, H)
    P = ctypes.c_void_p(256)
    f = ctypes.c_float
    ws = gsmi.loss_l1_dssim_workspace(64, 64)
    assert L.gs_loss_l1_dssim(64, 10, P, P, f(0.2), P, P, P, ws, None) == -1 and "window" in gsmi.last_error()
    for lam in (-0.1, 1.5, float("nan"), float("inf")):
        assert L.gs_loss_l1_dssim(64, 64, P, P, f(lam), P, P, P, ws, None) == -1
        assert "lambda" in gsmi.last_error()
    for k in range(5):
        args = [P, P, P, P, P]
        args[k] = None
        assert L.gs_loss_l1_dssim(64, 64, args[0], args[1], f(0.2), args[2], args[3], args[4], ws, None) == -1
        assert "null" in gsmi.last_error()
    assert L.gs_loss_l1_dssim(64, 64, P, P, f(0.2), P, P, P, ws - 1, None) == -1
    assert "workspace" in gsmi.last_error()


def test_adam_batch_scaling_and_checks():
    import math
    m = ctypes.c_void_p(256)
    base = gsmi.GsAdam(256, 256, 3, 1e-3, 0.9, 0.999, 1e-8)
    for bs in (1, 2, 4, 10):
        a = gsmi.adam_batch(base, bs)
        assert a.lr == pytest.approx(1e-3 * math.sqrt(bs), rel=1e-15)
        assert a.eps == pytest.approx(1e-8 / math.sqrt(bs), rel=1e-15)
        assert a.beta1 == pytest.approx(1 - bs * 0.1, abs=1e-15)
        assert a.beta2 == pytest.approx(1 - bs * 0.001, abs=1e-15)
        assert a.step == 3 and a.m == 256 and a.v == 256
    assert gsmi.adam_batch(base, 10).beta1 == pytest.approx(0.0, abs=1e-15)
    for bs in (0, -1, 11):
        with pytest.raises(gsmi.GsError):
            gsmi.adam_batch(base, bs)
    del m


def test_preprocess_backward_accumulate_checks_its_arguments():
    L = gsmi.load()
    cam = gsmi.GsCamera()
    cam.fx = cam.fy = 100.0
    cam.width = cam.height = 64
    cam.near_plane = 0.01
    cam.viewmat[0] = cam.viewmat[5] = cam.viewmat[10] = 1.0
    sc = gsmi.make_scene(10, 10, 0)
    proj = gsmi.GsProj(256, 256, 256, 256)
    P = ctypes.c_void_p(256)
    ws = gsmi.render_workspace(64, 64, 10, 1000)
    f = ctypes.c_float
    call = lambda grads, first, scale, adam=None, nbytes=ws: L.gs_preprocess_backward_accumulate(
        ctypes.byref(sc), P, ctypes.byref(cam), proj, P, nbytes, grads, first, f(scale), adam, None)
    assert call(None, 0, 0.5) == -1 and "grads_acc" in gsmi.last_error()
    assert call(None, 1, 0.5) == -1 and "grads_acc" in gsmi.last_error()
    assert call(P, 2, 0.5) == -1 and "first" in gsmi.last_error()
    assert call(P, 0, float("nan")) == -1 and "scale" in gsmi.last_error()
    assert call(P, 0, 0.5, nbytes=16) == -1 and "workspace" in gsmi.last_error()
    bad = gsmi.GsAdam(None, None, 1, 1e-3, 0.9, 0.999, 1e-8)
    assert call(P, 1, 1.0, ctypes.byref(bad)) == -1


def test_densify_checks_its_arguments():
    L = gsmi.load()
    sc = gsmi.make_scene(1000, 1000, 0)
    P = ctypes.c_void_p(256)
    Q = ctypes.c_void_p(512)
    ws = gsmi.densify_workspace(1000)
    assert ws >= 4 * 3 * 4 and gsmi.densify_workspace(18_180_000) >= 12 * (18_180_000 // 256)
    n_out = ctypes.c_int64(-5)
    ok = gsmi.densify_opts()

    def call(opts=ok, outs=(Q, Q, Q), ld_out=3000, nbytes=ws, ins=(P, P, P, P, P, P), wsp=P):
        return L.gs_densify(ctypes.byref(sc), *ins, ctypes.byref(opts), *outs, ld_out, ctypes.byref(n_out), None,
                            wsp, nbytes, None)
    for bad in (gsmi.densify_opts(percent_dense=0), gsmi.densify_opts(extent=-1), gsmi.densify_opts(min_opacity=1.0),
                gsmi.densify_opts(split_factor=0), gsmi.densify_opts(grad_threshold=float("nan"))):
        assert call(opts=bad) == -1 and "options" in gsmi.last_error()
    for k in range(6):
        ins = [P] * 6
        ins[k] = None
        assert call(ins=tuple(ins)) == -1 and "null" in gsmi.last_error()
    assert call(outs=(None, Q, Q)) == -1 and "output" in gsmi.last_error()
    assert call(outs=(P, Q, Q)) == -1 and "alias" in gsmi.last_error()
    assert call(nbytes=ws - 1) == -1 and "workspace" in gsmi.last_error()
    assert call(ld_out=-1) == -1
    assert L.gs_densify(ctypes.byref(sc), P, P, P, P, P, P, None, Q, Q, Q, 10, ctypes.byref(n_out), None, P, ws,
                        None) == -1
    # an empty scene needs no pointers and yields zero Gaussians without a GPU call
    e = gsmi.make_scene(0, 0, 0)
    assert L.gs_densify(ctypes.byref(e), None, None, None, None, None, None, ctypes.byref(ok), None, None, None, 0,
                        ctypes.byref(n_out), None, None, 0, None) == 0 and n_out.value == 0
    # statistics: null accumulators, short render workspace
    cam = gsmi.GsCamera()
    cam.fx = cam.fy = 100.0
    cam.width = cam.height = 64
    cam.near_plane = 0.01
    cam.viewmat[0] = cam.viewmat[5] = cam.viewmat[10] = 1.0
    proj = gsmi.GsProj(256, 256, 256, 256)
    rws = gsmi.render_workspace(64, 64, 1000, 1000)
    assert L.gs_densify_stats(ctypes.byref(sc), ctypes.byref(cam), proj, P, rws, None, P, None) == -1
    assert L.gs_densify_stats(ctypes.byref(sc), ctypes.byref(cam), proj, P, 16, P, P, None) == -1
    assert "workspace" in gsmi.last_error()


def test_render_calls_reject_a_missing_or_short_workspace():
    L = gsmi.load()
    cam = gsmi.GsCamera()
    cam.fx = cam.fy = 100.0
    cam.width = cam.height = 64
    cam.near_plane = 0.01
    cam.viewmat[0] = cam.viewmat[5] = cam.viewmat[10] = 1.0
    bg = (ctypes.c_float * 3)(0, 0, 0)
    p = ctypes.c_void_p(4096)
    need = gsmi.render_workspace(64, 64, 10, 0)
    for ws, nb in ((None, need), (p, 16), (ctypes.c_void_p(4096 + 64), need)):
        rc = L.gs_render_forward(ctypes.byref(cam), 10, p, p, p, 0, bg, p, p, p, None, None, ws, nb, None)
        assert rc == gsmi.GS_ERR_INVALID_ARGUMENT
    sc = gsmi.make_scene(10, 10, 0)
    proj = gsmi.GsProj(4096, 4096, 4096, 4096)
    rc = L.gs_render_backward(ctypes.byref(sc), None, ctypes.byref(cam), proj, p, p, 0, bg, p, p, p, p, None, None,
                              p, 16, None)
    assert rc == gsmi.GS_ERR_INVALID_ARGUMENT and "workspace" in gsmi.last_error()
    # the preprocess backward from staged sums: the same workspace checks, and params, tiles
    # and an output required
    ad = gsmi.GsAdam(4096, 4096, 1, 1e-3, 0.9, 0.999, 1e-8)
    for ws, nb in ((None, need), (p, 16), (ctypes.c_void_p(4096 + 64), need)):
        rc = L.gs_preprocess_backward_staged(ctypes.byref(sc), p, ctypes.byref(cam), proj, ws, nb, None,
                                             ctypes.byref(ad), None)
        assert rc == gsmi.GS_ERR_INVALID_ARGUMENT and "workspace" in gsmi.last_error()
    rc = L.gs_preprocess_backward_staged(ctypes.byref(sc), None, ctypes.byref(cam), proj, p, need, None,
                                         ctypes.byref(ad), None)
    assert rc == gsmi.GS_ERR_INVALID_ARGUMENT and "params" in gsmi.last_error()
    rc = L.gs_preprocess_backward_staged(ctypes.byref(sc), p, ctypes.byref(cam), gsmi.GsProj(4096, None, 4096, 4096),
                                         p, need, None, ctypes.byref(ad), None)
    assert rc == gsmi.GS_ERR_INVALID_ARGUMENT and "tiles" in gsmi.last_error()
    rc = L.gs_preprocess_backward_staged(ctypes.byref(sc), p, ctypes.byref(cam), proj, p, need, None, None, None)
    assert rc == gsmi.GS_ERR_INVALID_ARGUMENT and "grads" in gsmi.last_error()
    # the same with the next view's preprocess fused in: also the next camera and outputs
    nxt = gsmi.GsCamera()
    ctypes.pointer(nxt)[0] = cam
    rc = L.gs_preprocess_backward_staged_next(ctypes.byref(sc), p, ctypes.byref(cam), proj, p, 16, None,
                                              ctypes.byref(ad), ctypes.byref(nxt), proj, None)
    assert rc == gsmi.GS_ERR_INVALID_ARGUMENT and "workspace" in gsmi.last_error()
    rc = L.gs_preprocess_backward_staged_next(ctypes.byref(sc), p, ctypes.byref(cam), proj, p, need, None,
                                              ctypes.byref(ad), None, proj, None)
    assert rc == gsmi.GS_ERR_INVALID_ARGUMENT
    rc = L.gs_preprocess_backward_staged_next(ctypes.byref(sc), p, ctypes.byref(cam), proj, p, need, None,
                                              ctypes.byref(ad), ctypes.byref(nxt), gsmi.GsProj(4096, 4096, None, 4096),
                                              None)
    assert rc == gsmi.GS_ERR_INVALID_ARGUMENT and "depth_key" in gsmi.last_error()
    rc = L.gs_preprocess_backward_staged_next(ctypes.byref(sc), p, ctypes.byref(cam), proj, p, need, None,
                                              None, ctypes.byref(nxt), proj, None)
    assert rc == gsmi.GS_ERR_INVALID_ARGUMENT and "grads" in gsmi.last_error()


def test_fused_step_checks_its_arguments():
    """gs_render_step rejects a missing or short workspace, a missing target or loss output and
    a missing tiles array before any HIP call."""
    L = gsmi.load()
    cam = gsmi.GsCamera()
    cam.fx = cam.fy = 100.0
    cam.width = cam.height = 64
    cam.near_plane = 0.01
    cam.viewmat[0] = cam.viewmat[5] = cam.viewmat[10] = 1.0
    bg = (ctypes.c_float * 3)(0, 0, 0)
    p = ctypes.c_void_p(4096)
    need = gsmi.render_workspace(64, 64, 10, 0)
    sc = gsmi.make_scene(10, 10, 0)
    proj = gsmi.GsProj(4096, 4096, 4096, 4096)

    def call(proj=proj, target=p, loss=p, ws=p, nb=need, ranges=p):
        return L.gs_render_step(ctypes.byref(sc), ctypes.byref(cam), proj, p, ranges, 0, bg, target, p, p, p, None,
                                None, loss, p, None, ws, nb, None)

    assert call(ws=None) == gsmi.GS_ERR_INVALID_ARGUMENT and "null" in gsmi.last_error()
    for ws, nb in ((p, 16), (ctypes.c_void_p(4096 + 64), need)):
        assert call(ws=ws, nb=nb) == gsmi.GS_ERR_INVALID_ARGUMENT and "workspace" in gsmi.last_error()
    assert call(target=None) == gsmi.GS_ERR_INVALID_ARGUMENT and "null" in gsmi.last_error()
    assert call(loss=None) == gsmi.GS_ERR_INVALID_ARGUMENT and "null" in gsmi.last_error()
    assert call(proj=gsmi.GsProj(4096, None, 4096, 4096)) == gsmi.GS_ERR_INVALID_ARGUMENT
    assert "tiles" in gsmi.last_error()
    assert call(ranges=ctypes.c_void_p(4096 + 4)) == gsmi.GS_ERR_INVALID_ARGUMENT
    assert "aligned" in gsmi.last_error()


def test_render_plan_checks_its_arguments():
    """gs_render_plan rejects a missing or short workspace, missing ranges or tiles and
    misaligned ranges before any HIP call."""
    L = gsmi.load()
    cam = gsmi.GsCamera()
    cam.fx = cam.fy = 100.0
    cam.width = cam.height = 64
    cam.near_plane = 0.01
    cam.viewmat[0] = cam.viewmat[5] = cam.viewmat[10] = 1.0
    p = ctypes.c_void_p(4096)
    need = gsmi.render_workspace(64, 64, 10, 0)
    sc = gsmi.make_scene(10, 10, 0)
    proj = gsmi.GsProj(4096, 4096, 4096, 4096)
    call = lambda proj=proj, ranges=p, ws=p, nb=need: L.gs_render_plan(ctypes.byref(sc), ctypes.byref(cam), proj,
                                                                        ranges, 0, ws, nb, None)
    assert call(ws=None) == gsmi.GS_ERR_INVALID_ARGUMENT and "null" in gsmi.last_error()
    assert call(ranges=None) == gsmi.GS_ERR_INVALID_ARGUMENT and "null" in gsmi.last_error()
    for ws, nb in ((p, 16), (ctypes.c_void_p(4096 + 64), need)):
        assert call(ws=ws, nb=nb) == gsmi.GS_ERR_INVALID_ARGUMENT and "workspace" in gsmi.last_error()
    assert call(proj=gsmi.GsProj(4096, None, 4096, 4096)) == gsmi.GS_ERR_INVALID_ARGUMENT
    assert "tiles" in gsmi.last_error()
    assert call(ranges=ctypes.c_void_p(4096 + 4)) == gsmi.GS_ERR_INVALID_ARGUMENT
    assert "aligned" in gsmi.last_error()


def test_render_calls_report_a_workspace_short_of_the_intersections():
    """A render workspace sized for fewer intersections than the lists hold is a capacity error
    (GS_ERR_CAPACITY, nothing enqueued, the message naming the size needed) on every call that
    fills or reads it, never a silently partial result; k itself is range-checked."""
    L = gsmi.load()
    cam = gsmi.GsCamera()
    cam.fx = cam.fy = 100.0
    cam.width = cam.height = 64
    cam.near_plane = 0.01
    cam.viewmat[0] = cam.viewmat[5] = cam.viewmat[10] = 1.0
    bg = (ctypes.c_float * 3)(0, 0, 0)
    p = ctypes.c_void_p(4096)
    n = 100
    nb = gsmi.render_workspace(64, 64, n, 1000)
    cap = gsmi.render_workspace_capacity(64, 64, n, nb)
    assert 1000 <= cap < 1000 + 256
    need = gsmi.render_workspace(64, 64, n, 5000)
    sc = gsmi.make_scene(n, n, 0)
    proj = gsmi.GsProj(4096, 4096, 4096, 4096)
    ad = gsmi.GsAdam(4096, 4096, 1, 1e-3, 0.9, 0.999, 1e-8)
    calls = {
        "forward": lambda k: L.gs_render_forward(ctypes.byref(cam), n, p, p, p, k, bg, p, p, p, None, None, p, nb, None),
        "plan": lambda k: L.gs_render_plan(ctypes.byref(sc), ctypes.byref(cam), proj, p, k, p, nb, None),
        "step": lambda k: L.gs_render_step(ctypes.byref(sc), ctypes.byref(cam), proj, p, p, k, bg, p, p, p, p, None,
                                           None, p, p, None, p, nb, None),
        "backward": lambda k: L.gs_render_backward(ctypes.byref(sc), p, ctypes.byref(cam), proj, p, p, k, bg, p, p,
                                                   p, None, None, ctypes.byref(ad), p, nb, None),
    }
    for name, call in calls.items():
        assert call(5000) == gsmi.GS_ERR_CAPACITY, name
        msg = gsmi.last_error()
        assert f"needs {need} bytes" in msg and str(cap) in msg, (name, msg)
        assert call(cap + 1) == gsmi.GS_ERR_CAPACITY, name
        assert call(-1) == gsmi.GS_ERR_INVALID_ARGUMENT and "k =" in gsmi.last_error(), name
        assert call(1 << 33) == gsmi.GS_ERR_INVALID_ARGUMENT, name


def test_render_status_checks_its_arguments():
    """gs_render_status needs an aligned workspace of at least its header, and clears its outputs
    before any HIP call."""
    L = gsmi.load()
    flags = ctypes.c_uint32(7)
    req = ctypes.c_int64(7)
    assert L.gs_render_status(None, 4096, ctypes.byref(flags), ctypes.byref(req), None) == gsmi.GS_ERR_INVALID_ARGUMENT
    assert flags.value == 0 and req.value == 0
    assert L.gs_render_status(ctypes.c_void_p(4096), 16, None, None, None) == gsmi.GS_ERR_INVALID_ARGUMENT
    assert L.gs_render_status(ctypes.c_void_p(4096 + 64), 4096, None, None, None) == gsmi.GS_ERR_INVALID_ARGUMENT
    assert "workspace" in gsmi.last_error()
    for ws, nb in ((None, 4096), (ctypes.c_void_p(4096), 16), (ctypes.c_void_p(4096 + 64), 4096)):
        assert L.gs_render_init(ws, nb, None) == gsmi.GS_ERR_INVALID_ARGUMENT
