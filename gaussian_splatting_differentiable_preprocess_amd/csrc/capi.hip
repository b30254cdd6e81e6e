// C ABI of libgsmi.so: argument validation, launch geometry and error reporting around the
// kernels.  Every function checks its arguments before touching HIP, enqueues on the
// caller's stream and returns a gs_status; no exception crosses the boundary.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "gsmi_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(GS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

int ok() {
  g_err[0] = '\0';
  return GS_OK;
}

bool finite(float x) { return std::isfinite(x); }

int check_camera(const gs_camera* c) {
  if (!c) return fail(GS_ERR_INVALID_ARGUMENT, "camera is null");
  for (int k = 0; k < 12; ++k)
    if (!finite(c->viewmat[k])) return fail(GS_ERR_INVALID_ARGUMENT, "camera viewmat[%d] not finite", k);
  if (!(finite(c->fx) && c->fx > 0.f && finite(c->fy) && c->fy > 0.f))
    return fail(GS_ERR_INVALID_ARGUMENT, "camera focal lengths must be finite and > 0");
  if (!(finite(c->cx) && finite(c->cy))) return fail(GS_ERR_INVALID_ARGUMENT, "camera principal point not finite");
  if (!(finite(c->near_plane) && c->near_plane > 0.f))
    return fail(GS_ERR_INVALID_ARGUMENT, "camera near_plane must be finite and > 0");
  if (c->width < 1 || c->height < 1 || c->width > 32768 || c->height > 32768)
    return fail(GS_ERR_INVALID_ARGUMENT, "camera size %dx%d outside [1, 32768]", c->width, c->height);
  return GS_OK;
}

int check_scene(const gs_scene* s) {
  if (!s) return fail(GS_ERR_INVALID_ARGUMENT, "scene is null");
  if (s->n < 0 || s->n > 2147483647LL) return fail(GS_ERR_INVALID_ARGUMENT, "scene n = %lld out of range", (long long)s->n);
  if (s->ld < s->n || s->ld < 0) return fail(GS_ERR_INVALID_ARGUMENT, "scene ld = %lld < n", (long long)s->ld);
  if (s->sh_degree < 0 || s->sh_degree > 3)
    return fail(GS_ERR_INVALID_ARGUMENT, "sh_degree = %d not in [0, 3]", s->sh_degree);
  return GS_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_proj(const gs_proj& p, bool need_aux, int64_t n) {
  if (n == 0) return GS_OK;
  if (!p.splat) return fail(GS_ERR_INVALID_ARGUMENT, "proj.splat is null");
  if (!aligned16(p.splat)) return fail(GS_ERR_INVALID_ARGUMENT, "proj.splat must be 16-byte aligned");
  if (need_aux && (!p.tiles || !p.depth_key || !p.rect))
    return fail(GS_ERR_INVALID_ARGUMENT, "proj.tiles / proj.depth_key / proj.rect is null");
  if (need_aux && (reinterpret_cast<uintptr_t>(p.rect) & 7u))
    return fail(GS_ERR_INVALID_ARGUMENT, "proj.rect must be 8-byte aligned");
  return GS_OK;
}

int check_adam(const gs_adam* a) {
  if (!a) return GS_OK;
  if (!a->m || !a->v) return fail(GS_ERR_INVALID_ARGUMENT, "adam m / v is null");
  if (a->step < 1) return fail(GS_ERR_INVALID_ARGUMENT, "adam step must be >= 1");
  if (!(std::isfinite(a->lr) && std::isfinite(a->eps) && a->beta1 >= 0.0 && a->beta1 < 1.0 && a->beta2 >= 0.0 &&
        a->beta2 < 1.0))
    return fail(GS_ERR_INVALID_ARGUMENT, "adam hyper-parameters out of range");
  return GS_OK;
}

gsmi::AdamCoef adam_coef(const gs_adam& a) {
  gsmi::AdamCoef c;
  c.lr = (float)a.lr;
  c.b1 = (float)a.beta1;
  c.omb1 = (float)(1.0 - a.beta1);
  c.b2 = (float)a.beta2;
  c.omb2 = (float)(1.0 - a.beta2);
  c.eps = (float)a.eps;
  c.inv_bc1 = (float)(1.0 / (1.0 - std::pow(a.beta1, (double)a.step)));
  c.inv_bc2 = (float)(1.0 / (1.0 - std::pow(a.beta2, (double)a.step)));
  return c;
}

int64_t n_tiles(const gs_camera& c) {
  return (int64_t)((c.width + GS_TILE - 1) / GS_TILE) * ((c.height + GS_TILE - 1) / GS_TILE);
}

// k intersections must fit the render workspace's capacity; the message names the size that fits
int check_render_capacity(const gs_camera& c, int64_t n, int64_t k, const gsmi::RenderWs& ws, size_t bytes) {
  if (k < 0 || k > 4294967295LL) return fail(GS_ERR_INVALID_ARGUMENT, "k = %lld out of range", (long long)k);
  if ((uint64_t)k > ws.staging_cap) {
    const size_t need = gsmi::render_ws_bytes((int)n_tiles(c), n, k);
    return fail(GS_ERR_CAPACITY, "render workspace of %zu bytes holds %llu intersections, %lld given: it needs %zu bytes",
                bytes, (unsigned long long)ws.staging_cap, (long long)k, need);
  }
  return GS_OK;
}

}  // namespace

namespace gsmi {

int fail_status(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok_status() { return ok(); }

int hip_status(hipError_t e, const char* where) { return hip_fail(e, where); }

CamK make_cam(const gs_camera& c) {
  CamK k{};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 3; ++j) k.R[3 * i + j] = c.viewmat[4 * i + j];
    k.t[i] = c.viewmat[4 * i + 3];
  }
  k.fx = c.fx;
  k.fy = c.fy;
  k.cx = c.cx;
  k.cy = c.cy;
  k.near_plane = c.near_plane;
  k.limx = (float)(1.3 * (0.5 * c.width) / c.fx);
  k.limy = (float)(1.3 * (0.5 * c.height) / c.fy);
  for (int j = 0; j < 3; ++j) {
    double acc = 0.0;
    for (int i = 0; i < 3; ++i) acc -= (double)k.R[3 * i + j] * (double)k.t[i];
    k.pos[j] = (float)acc;
  }
  k.W = c.width;
  k.H = c.height;
  k.TX = (c.width + kTile - 1) / kTile;
  k.TY = (c.height + kTile - 1) / kTile;
  return k;
}

}  // namespace gsmi

using namespace gsmi;

extern "C" {

int gs_version(void) { return GSMI_VERSION; }

const char* gs_last_error(void) { return g_err; }

int gs_preprocess(const gs_scene* scene, const float* params, const gs_camera* cam, gs_proj out,
                  hipStream_t stream) {
  int st;
  if ((st = check_scene(scene)) || (st = check_camera(cam)) || (st = check_proj(out, true, scene->n))) return st;
  if (!params && scene->n > 0) return fail(GS_ERR_INVALID_ARGUMENT, "params is null");
  const hipError_t e = launch_preprocess(*scene, params, make_cam(*cam), out, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "gs_preprocess");
}

int gs_bin_and_sort_workspace(int64_t n, int64_t k_capacity, int32_t width, int32_t height, size_t* bytes) {
  if (!bytes) return fail(GS_ERR_INVALID_ARGUMENT, "bytes is null");
  if (n < 0 || k_capacity < 0 || width < 1 || height < 1 || k_capacity > 4294967295LL)
    return fail(GS_ERR_INVALID_ARGUMENT, "invalid sizes");
  *bytes = bin_layout(n, k_capacity, width, height).total;
  return ok();
}

int gs_bin_and_sort(const gs_scene* scene, const gs_camera* cam, gs_proj proj, void* workspace,
                    size_t workspace_bytes, int64_t k_capacity, uint32_t* vals, uint32_t* ranges,
                    uint64_t* keys, int64_t* k_out, hipStream_t stream) {
  int st;
  if ((st = check_scene(scene)) || (st = check_camera(cam)) || (st = check_proj(proj, true, scene->n))) return st;
  if (!workspace || !vals || !ranges) return fail(GS_ERR_INVALID_ARGUMENT, "workspace / vals / ranges is null");
  if (k_capacity < 0 || k_capacity > 4294967295LL) return fail(GS_ERR_INVALID_ARGUMENT, "k_capacity out of range");
  const BinLayout L = bin_layout(scene->n, k_capacity, cam->width, cam->height);
  if (workspace_bytes < L.total)
    return fail(GS_ERR_INVALID_ARGUMENT, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(GS_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  hipError_t e = launch_bin_sort(scene->n, k_capacity, make_cam(*cam), proj, ws, L, vals, ranges, keys,
                                 /*keep_ranges_on_overflow=*/k_out != nullptr, stream);
  if (e != hipSuccess) return hip_fail(e, "gs_bin_and_sort");
  if (!k_out) return ok();
  BinInfo info{};
  e = hipMemcpyAsync(&info, ws + L.info, sizeof(BinInfo), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "gs_bin_and_sort (count readback)");
  *k_out = (int64_t)info.K;
  if ((int64_t)info.K > k_capacity)
    return fail(GS_ERR_CAPACITY, "%llu intersections exceed k_capacity %lld", info.K, (long long)k_capacity);
  return ok();
}

int gs_bin_and_sort_count(const void* workspace, size_t workspace_bytes, int64_t* k_out, hipStream_t stream) {
  if (!workspace || !k_out) return fail(GS_ERR_INVALID_ARGUMENT, "workspace / k_out is null");
  if (workspace_bytes < sizeof(BinInfo)) return fail(GS_ERR_INVALID_ARGUMENT, "workspace too small");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(GS_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  BinInfo info{};
  hipError_t e = hipMemcpyAsync(&info, workspace, sizeof(BinInfo), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "gs_bin_and_sort_count");
  *k_out = (int64_t)info.K;
  if (info.K > info.kcap)
    return fail(GS_ERR_CAPACITY, "%llu intersections exceeded the capacity %llu of the last gs_bin_and_sort",
                info.K, info.kcap);
  return ok();
}

int gs_render_workspace(int32_t width, int32_t height, int64_t n, int64_t k_capacity, size_t* bytes) {
  if (!bytes || width <= 0 || height <= 0 || n < 0 || k_capacity < 0)
    return fail(GS_ERR_INVALID_ARGUMENT, "invalid arguments");
  const int T = ((width + GS_TILE - 1) / GS_TILE) * ((height + GS_TILE - 1) / GS_TILE);
  *bytes = render_ws_bytes(T, n, k_capacity);
  return ok();
}

int gs_render_workspace_capacity(int32_t width, int32_t height, int64_t n, size_t bytes,
                                 int64_t* k_capacity) {
  if (!k_capacity || width <= 0 || height <= 0 || n < 0) return fail(GS_ERR_INVALID_ARGUMENT, "invalid arguments");
  const int T = ((width + GS_TILE - 1) / GS_TILE) * ((height + GS_TILE - 1) / GS_TILE);
  RenderWs ws;
  if (!render_ws_layout(reinterpret_cast<void*>(uintptr_t(256)), bytes, T, n, &ws))
    return fail(GS_ERR_INVALID_ARGUMENT, "workspace smaller than the size for k_capacity 0");
  *k_capacity = (int64_t)ws.staging_cap;
  return ok();
}

int gs_render_forward(const gs_camera* cam, int64_t n, const gs_splat* splat, const uint32_t* vals,
                      const uint32_t* ranges, int64_t k, const float* bg, float* image, float* T_final,
                      uint32_t* last_contrib, uint32_t* n_examined, uint64_t* blend_count,
                      void* render_ws, size_t render_ws_bytes, hipStream_t stream) {
  int st;
  if ((st = check_camera(cam))) return st;
  if (n < 0) return fail(GS_ERR_INVALID_ARGUMENT, "n < 0");
  if ((!splat && n > 0) || !vals || !ranges || !bg || !image || !T_final || !last_contrib || !render_ws)
    return fail(GS_ERR_INVALID_ARGUMENT, "a required pointer is null");
  RenderWs ws;
  if (!render_ws_layout(render_ws, render_ws_bytes, (int)n_tiles(*cam), n, &ws))
    return fail(GS_ERR_INVALID_ARGUMENT, "render workspace too small or not 256-byte aligned");
  if ((st = check_render_capacity(*cam, n, k, ws, render_ws_bytes))) return st;
  if (!aligned16(splat)) return fail(GS_ERR_INVALID_ARGUMENT, "splat must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(ranges) & 7u) return fail(GS_ERR_INVALID_ARGUMENT, "ranges must be 8-byte aligned");
  if (!(finite(bg[0]) && finite(bg[1]) && finite(bg[2]))) return fail(GS_ERR_INVALID_ARGUMENT, "bg not finite");
  const hipError_t e = launch_blend_forward(make_cam(*cam), n, splat, vals, ranges, bg[0], bg[1], bg[2], image,
                                            T_final, last_contrib, n_examined, blend_count, ws, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "gs_render_forward");
}

int gs_loss_l1_workspace(int64_t count, size_t* bytes) {
  if (!bytes || count < 0) return fail(GS_ERR_INVALID_ARGUMENT, "invalid arguments");
  *bytes = loss_workspace_bytes(count);
  return ok();
}

int gs_loss_l1(int64_t count, const float* image, const float* target, float* loss, float* dL_dimage,
               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (count < 0) return fail(GS_ERR_INVALID_ARGUMENT, "count < 0");
  if (!loss || !workspace || (count > 0 && (!image || !target || !dL_dimage)))
    return fail(GS_ERR_INVALID_ARGUMENT, "a required pointer is null");
  if (workspace_bytes < loss_workspace_bytes(count))
    return fail(GS_ERR_INVALID_ARGUMENT, "loss workspace too small");
  const hipError_t e = launch_loss_l1(count, image, target, loss, dL_dimage, workspace, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "gs_loss_l1");
}

int gs_loss_l1_dssim_workspace(int32_t width, int32_t height, size_t* bytes) {
  if (!bytes) return fail(GS_ERR_INVALID_ARGUMENT, "bytes is null");
  if (width < 11 || height < 11) return fail(GS_ERR_INVALID_ARGUMENT, "image smaller than the 11x11 SSIM window");
  *bytes = ssim_workspace_bytes(width, height);
  return ok();
}

int gs_loss_l1_dssim(int32_t width, int32_t height, const float* image, const float* target, float lambda,
                     float* loss, float* dL_dimage, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  if (width < 11 || height < 11) return fail(GS_ERR_INVALID_ARGUMENT, "image smaller than the 11x11 SSIM window");
  if (!(lambda >= 0.f && lambda <= 1.f)) return fail(GS_ERR_INVALID_ARGUMENT, "lambda must be in [0, 1]");
  if (!image || !target || !loss || !dL_dimage || !workspace)
    return fail(GS_ERR_INVALID_ARGUMENT, "a required pointer is null");
  if (workspace_bytes < ssim_workspace_bytes(width, height))
    return fail(GS_ERR_INVALID_ARGUMENT, "D-SSIM workspace too small");
  const hipError_t e =
      launch_loss_l1_dssim(width, height, image, target, lambda, loss, dL_dimage, workspace, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "gs_loss_l1_dssim");
}

}  // extern "C"

namespace {
// The preprocess backward from grad2d, or (grad2d null) from the sums staged in ws.
int run_preprocess_backward(const gs_scene* scene, float* params, const gs_camera* cam, const float* grad2d,
                            const gsmi::RenderWs* ws, const uint32_t* tiles, float* grads, const gs_adam* adam,
                            hipStream_t stream, const char* who, const float* gacc = nullptr,
                            float gscale = 1.0f, const gs_camera* next_cam = nullptr,
                            const gs_proj* next = nullptr) {
  PrebwdArgs a{};
  a.gacc = gacc;
  a.gscale = gscale;
  a.n = scene->n;
  a.ld = scene->ld;
  a.deg = scene->sh_degree;
  a.params = params;
  a.grad2d = grad2d;
  if (!grad2d) {
    a.staging = ws->staging;
    a.goff = ws->goff;
    a.goff_blk = ws->goff_blk;
    a.tiles = tiles;
    a.staging_cap = ws->staging_cap;
  }
  a.grads = grads;
  if (adam) {
    a.m = adam->m;
    a.v = adam->v;
    const AdamCoef c = adam_coef(*adam);
    a.lr = c.lr;
    a.b1 = c.b1;
    a.omb1 = c.omb1;
    a.b2 = c.b2;
    a.omb2 = c.omb2;
    a.eps = c.eps;
    a.inv_bc1 = c.inv_bc1;
    a.inv_bc2 = c.inv_bc2;
  }
  hipError_t e;
  if (next_cam) {
    const CamK cn = make_cam(*next_cam);
    const NextOut nx{reinterpret_cast<float4*>(next->splat), next->tiles, next->depth_key,
                     reinterpret_cast<uint2*>(next->rect)};
    e = launch_preprocess_backward(a, make_cam(*cam), stream, &cn, &nx);
  } else {
    e = launch_preprocess_backward(a, make_cam(*cam), stream);
  }
  return e == hipSuccess ? ok() : hip_fail(e, who);
}
}  // namespace

extern "C" {

int gs_preprocess_backward(const gs_scene* scene, float* params, const gs_camera* cam,
                           const float* grad2d, float* grads, const gs_adam* adam, hipStream_t stream) {
  int st;
  if ((st = check_scene(scene)) || (st = check_camera(cam)) || (st = check_adam(adam))) return st;
  if (scene->n > 0 && (!params || !grad2d)) return fail(GS_ERR_INVALID_ARGUMENT, "params / grad2d is null");
  if (scene->n > 0 && !grads && !adam)
    return fail(GS_ERR_INVALID_ARGUMENT, "grads is null and no adam update requested");
  return run_preprocess_backward(scene, params, cam, grad2d, nullptr, nullptr, grads, adam, stream,
                                 "gs_preprocess_backward");
}

int gs_preprocess_backward_staged(const gs_scene* scene, float* params, const gs_camera* cam, gs_proj proj,
                                  const void* render_ws, size_t render_ws_bytes, float* grads,
                                  const gs_adam* adam, hipStream_t stream) {
  int st;
  if ((st = check_scene(scene)) || (st = check_camera(cam)) || (st = check_adam(adam))) return st;
  if (scene->n > 0 && !params) return fail(GS_ERR_INVALID_ARGUMENT, "params is null");
  if (scene->n > 0 && !proj.tiles) return fail(GS_ERR_INVALID_ARGUMENT, "proj.tiles is null");
  if (scene->n > 0 && !grads && !adam)
    return fail(GS_ERR_INVALID_ARGUMENT, "grads is null and no adam update requested");
  RenderWs ws;
  if (!render_ws || !render_ws_layout(const_cast<void*>(render_ws), render_ws_bytes, (int)n_tiles(*cam), scene->n, &ws))
    return fail(GS_ERR_INVALID_ARGUMENT, "render workspace too small or not 256-byte aligned");
  return run_preprocess_backward(scene, params, cam, nullptr, &ws, proj.tiles, grads, adam, stream,
                                 "gs_preprocess_backward_staged");
}

int gs_preprocess_backward_staged_next(const gs_scene* scene, float* params, const gs_camera* cam, gs_proj proj,
                                       const void* render_ws, size_t render_ws_bytes, float* grads,
                                       const gs_adam* adam, const gs_camera* next_cam, gs_proj next,
                                       hipStream_t stream) {
  int st;
  if ((st = check_scene(scene)) || (st = check_camera(cam)) || (st = check_adam(adam)) ||
      (st = check_camera(next_cam)) || (st = check_proj(next, true, scene->n)))
    return st;
  if (scene->n > 0 && !params) return fail(GS_ERR_INVALID_ARGUMENT, "params is null");
  if (scene->n > 0 && !proj.tiles) return fail(GS_ERR_INVALID_ARGUMENT, "proj.tiles is null");
  if (scene->n > 0 && !grads && !adam)
    return fail(GS_ERR_INVALID_ARGUMENT, "grads is null and no adam update requested");
  RenderWs ws;
  if (!render_ws || !render_ws_layout(const_cast<void*>(render_ws), render_ws_bytes, (int)n_tiles(*cam), scene->n, &ws))
    return fail(GS_ERR_INVALID_ARGUMENT, "render workspace too small or not 256-byte aligned");
  return run_preprocess_backward(scene, params, cam, nullptr, &ws, proj.tiles, grads, adam, stream,
                                 "gs_preprocess_backward_staged_next", nullptr, 1.0f, next_cam, &next);
}

int gs_preprocess_backward_accumulate(const gs_scene* scene, float* params, const gs_camera* cam, gs_proj proj,
                                      const void* render_ws, size_t render_ws_bytes, float* grads_acc,
                                      int32_t first, float scale, const gs_adam* adam, hipStream_t stream) {
  int st;
  if ((st = check_scene(scene)) || (st = check_camera(cam)) || (st = check_adam(adam))) return st;
  if (!std::isfinite(scale)) return fail(GS_ERR_INVALID_ARGUMENT, "scale not finite");
  if (first != 0 && first != 1) return fail(GS_ERR_INVALID_ARGUMENT, "first must be 0 or 1");
  if (scene->n > 0 && !params) return fail(GS_ERR_INVALID_ARGUMENT, "params is null");
  if (scene->n > 0 && !proj.tiles) return fail(GS_ERR_INVALID_ARGUMENT, "proj.tiles is null");
  if (scene->n > 0 && !grads_acc && !(first && adam))
    return fail(GS_ERR_INVALID_ARGUMENT, "grads_acc is null");
  RenderWs ws;
  if (!render_ws || !render_ws_layout(const_cast<void*>(render_ws), render_ws_bytes, (int)n_tiles(*cam), scene->n, &ws))
    return fail(GS_ERR_INVALID_ARGUMENT, "render workspace too small or not 256-byte aligned");
  // not first: add to the accumulated rows; with adam the total goes through Adam and the
  // accumulator is left as it was
  return run_preprocess_backward(scene, params, cam, nullptr, &ws, proj.tiles, adam ? nullptr : grads_acc, adam,
                                 stream, "gs_preprocess_backward_accumulate", first ? nullptr : grads_acc, scale);
}

int gs_adam_batch(const gs_adam* adam, int32_t batch, gs_adam* out) {
  if (!adam || !out) return fail(GS_ERR_INVALID_ARGUMENT, "adam / out is null");
  if (batch < 1) return fail(GS_ERR_INVALID_ARGUMENT, "batch must be >= 1");
  gs_adam r = *adam;
  const double s = std::sqrt((double)batch);
  r.lr = adam->lr * s;
  r.eps = adam->eps / s;
  r.beta1 = 1.0 - (double)batch * (1.0 - adam->beta1);
  r.beta2 = 1.0 - (double)batch * (1.0 - adam->beta2);
  if (!(r.beta1 >= 0.0 && r.beta2 >= 0.0))
    return fail(GS_ERR_INVALID_ARGUMENT, "batch %d takes a momentum coefficient below zero", batch);
  int st;
  if ((st = check_adam(&r))) return st;
  *out = r;
  return ok();
}

int gs_densify_stats(const gs_scene* scene, const gs_camera* cam, gs_proj proj, const void* render_ws,
                     size_t render_ws_bytes, float* grad_acc, float* count, hipStream_t stream) {
  int st;
  if ((st = check_scene(scene)) || (st = check_camera(cam))) return st;
  if (scene->n > 0 && (!proj.splat || !proj.tiles || !grad_acc || !count))
    return fail(GS_ERR_INVALID_ARGUMENT, "a required pointer is null");
  RenderWs ws;
  if (!render_ws || !render_ws_layout(const_cast<void*>(render_ws), render_ws_bytes, (int)n_tiles(*cam), scene->n, &ws))
    return fail(GS_ERR_INVALID_ARGUMENT, "render workspace too small or not 256-byte aligned");
  const hipError_t e = launch_densify_stats(scene->n, proj.splat, proj.tiles, ws, 0.5f * (float)cam->width,
                                            0.5f * (float)cam->height, grad_acc, count, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "gs_densify_stats");
}

int gs_densify_workspace(int64_t n, size_t* bytes) {
  if (!bytes || n < 0) return fail(GS_ERR_INVALID_ARGUMENT, "invalid arguments");
  *bytes = densify_workspace_bytes(n);
  return ok();
}

int gs_densify(const gs_scene* scene, const float* params, const float* m, const float* v, const float* grad_acc,
               const float* count, const float* z, const gs_densify_opts* opts, float* params_out, float* m_out,
               float* v_out, int64_t ld_out, int64_t* n_out, int32_t* codes, void* workspace,
               size_t workspace_bytes, hipStream_t stream) {
  int st;
  if ((st = check_scene(scene))) return st;
  if (!opts || !n_out) return fail(GS_ERR_INVALID_ARGUMENT, "opts / n_out is null");
  if (!(opts->percent_dense > 0.0 && opts->extent > 0.0 && opts->min_opacity > 0.0 && opts->min_opacity < 1.0 &&
        opts->split_factor > 0.0 && std::isfinite(opts->grad_threshold) && std::isfinite(opts->percent_dense) &&
        std::isfinite(opts->extent) && std::isfinite(opts->split_factor)))
    return fail(GS_ERR_INVALID_ARGUMENT, "densify options out of range");
  if (ld_out < 0) return fail(GS_ERR_INVALID_ARGUMENT, "ld_out < 0");
  if (scene->n > 0 && (!params || !m || !v || !grad_acc || !count || !z || !workspace))
    return fail(GS_ERR_INVALID_ARGUMENT, "a required pointer is null");
  if (ld_out > 0 && (!params_out || !m_out || !v_out))
    return fail(GS_ERR_INVALID_ARGUMENT, "an output pointer is null");
  if (scene->n > 0 && workspace_bytes < densify_workspace_bytes(scene->n))
    return fail(GS_ERR_INVALID_ARGUMENT, "densify workspace too small");
  if (scene->n > 0 && (params_out == params || m_out == m || v_out == v))
    return fail(GS_ERR_INVALID_ARGUMENT, "outputs must not alias inputs");
  *n_out = 0;
  if (scene->n == 0) return ok();
  DensifyLaunch d{};
  d.n = scene->n;
  d.ld = scene->ld;
  d.ld_out = ld_out;
  d.R = rows_for_degree(scene->sh_degree);
  d.params = params;
  d.m = m;
  d.v = v;
  d.grad_acc = grad_acc;
  d.count = count;
  d.z = z;
  d.t_grad = (float)opts->grad_threshold;
  d.t_lscale = (float)std::log(opts->percent_dense * opts->extent);
  d.t_logit = (float)std::log(opts->min_opacity / (1.0 - opts->min_opacity));
  d.log_split = (float)std::log(opts->split_factor);
  d.params_out = params_out;
  d.m_out = m_out;
  d.v_out = v_out;
  d.codes = codes;
  d.ws = workspace;
  uint32_t tot[3] = {0, 0, 0};
  const hipError_t e = launch_densify(d, tot, stream);
  if (e != hipSuccess) return hip_fail(e, "gs_densify");
  *n_out = (int64_t)tot[0] + tot[1] + 2 * (int64_t)tot[2];
  if (*n_out > ld_out) return fail(GS_ERR_CAPACITY, "%lld Gaussians after densification exceed ld_out %lld",
                                   (long long)*n_out, (long long)ld_out);
  return ok();
}

int gs_render_backward(const gs_scene* scene, float* params, const gs_camera* cam, gs_proj proj,
                       const uint32_t* vals, const uint32_t* ranges, int64_t k, const float* bg,
                       const float* T_final, const uint32_t* last_contrib, const float* dL_dimage,
                       float* grad2d, float* grads, const gs_adam* adam, void* render_ws,
                       size_t render_ws_bytes, hipStream_t stream) {
  int st;
  if ((st = check_scene(scene)) || (st = check_camera(cam)) || (st = check_proj(proj, false, scene->n)) ||
      (st = check_adam(adam)))
    return st;
  if (!vals || !ranges || !bg || !T_final || !last_contrib || !dL_dimage || !render_ws)
    return fail(GS_ERR_INVALID_ARGUMENT, "a required pointer is null");
  RenderWs ws;
  if (!render_ws_layout(render_ws, render_ws_bytes, (int)n_tiles(*cam), scene->n, &ws))
    return fail(GS_ERR_INVALID_ARGUMENT, "render workspace too small or not 256-byte aligned");
  if ((st = check_render_capacity(*cam, scene->n, k, ws, render_ws_bytes))) return st;
  if (scene->n > 0 && !proj.tiles) return fail(GS_ERR_INVALID_ARGUMENT, "proj.tiles is null");
  if (scene->n > 0 && (grads || adam) && !params) return fail(GS_ERR_INVALID_ARGUMENT, "params is null");
  if (reinterpret_cast<uintptr_t>(ranges) & 7u) return fail(GS_ERR_INVALID_ARGUMENT, "ranges must be 8-byte aligned");
  if (!(finite(bg[0]) && finite(bg[1]) && finite(bg[2]))) return fail(GS_ERR_INVALID_ARGUMENT, "bg not finite");
  const CamK ck = make_cam(*cam);
  const hipError_t e = launch_blend_backward(ck, scene->n, proj.splat, proj.tiles, vals, ranges, bg[0], bg[1],
                                             bg[2], T_final, last_contrib, dL_dimage, grad2d, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "gs_render_backward (blend)");
  if (!grads && !adam) return ok();  // backward blend only
  return run_preprocess_backward(scene, params, cam, grad2d, &ws, proj.tiles, grads, adam, stream,
                                 "gs_render_backward (preprocess backward)");
}

int gs_render_plan(const gs_scene* scene, const gs_camera* cam, gs_proj proj, const uint32_t* ranges, int64_t k,
                   void* render_ws, size_t render_ws_bytes, hipStream_t stream) {
  int st;
  if ((st = check_scene(scene)) || (st = check_camera(cam))) return st;
  if (!ranges || !render_ws) return fail(GS_ERR_INVALID_ARGUMENT, "a required pointer is null");
  if (scene->n > 0 && !proj.tiles) return fail(GS_ERR_INVALID_ARGUMENT, "proj.tiles is null");
  RenderWs ws;
  if (!render_ws_layout(render_ws, render_ws_bytes, (int)n_tiles(*cam), scene->n, &ws))
    return fail(GS_ERR_INVALID_ARGUMENT, "render workspace too small or not 256-byte aligned");
  if ((st = check_render_capacity(*cam, scene->n, k, ws, render_ws_bytes))) return st;
  if (reinterpret_cast<uintptr_t>(ranges) & 7u) return fail(GS_ERR_INVALID_ARGUMENT, "ranges must be 8-byte aligned");
  const hipError_t e = launch_step_plan(make_cam(*cam), scene->n, proj.tiles, ranges, ws, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "gs_render_plan");
}

int gs_render_step(const gs_scene* scene, const gs_camera* cam, gs_proj proj, const uint32_t* vals,
                   const uint32_t* ranges, int64_t k, const float* bg, const float* target, float* image,
                   float* T_final, uint32_t* last_contrib, uint32_t* n_examined, uint64_t* blend_count,
                   float* loss, float* dL_dimage, float* grad2d, void* render_ws, size_t render_ws_bytes,
                   hipStream_t stream) {
  int st;
  if ((st = check_scene(scene)) || (st = check_camera(cam)) || (st = check_proj(proj, false, scene->n))) return st;
  if (!vals || !ranges || !bg || !target || !image || !T_final || !last_contrib || !loss || !dL_dimage ||
      !render_ws)
    return fail(GS_ERR_INVALID_ARGUMENT, "a required pointer is null");
  if (scene->n > 0 && !proj.tiles) return fail(GS_ERR_INVALID_ARGUMENT, "proj.tiles is null");
  RenderWs ws;
  if (!render_ws_layout(render_ws, render_ws_bytes, (int)n_tiles(*cam), scene->n, &ws))
    return fail(GS_ERR_INVALID_ARGUMENT, "render workspace too small or not 256-byte aligned");
  if ((st = check_render_capacity(*cam, scene->n, k, ws, render_ws_bytes))) return st;
  if (reinterpret_cast<uintptr_t>(ranges) & 7u) return fail(GS_ERR_INVALID_ARGUMENT, "ranges must be 8-byte aligned");
  if (!(finite(bg[0]) && finite(bg[1]) && finite(bg[2]))) return fail(GS_ERR_INVALID_ARGUMENT, "bg not finite");
  const hipError_t e = launch_blend_step(make_cam(*cam), scene->n, proj.splat, proj.tiles, vals, ranges, bg[0],
                                         bg[1], bg[2], target, image, T_final, last_contrib, n_examined,
                                         blend_count, loss, dL_dimage, grad2d, ws, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "gs_render_step");
}

int gs_render_init(void* render_ws, size_t render_ws_bytes, hipStream_t stream) {
  if (!render_ws) return fail(GS_ERR_INVALID_ARGUMENT, "render_ws is null");
  if (render_ws_bytes < 256 || (reinterpret_cast<uintptr_t>(render_ws) & 255u))
    return fail(GS_ERR_INVALID_ARGUMENT, "render workspace too small or not 256-byte aligned");
  const hipError_t e = launch_fill_u32(static_cast<uint32_t*>(render_ws), kHdrStatusWords, 0u, stream);
  return e == hipSuccess ? ok() : hip_fail(e, "gs_render_init");
}

int gs_render_status(void* render_ws, size_t render_ws_bytes, uint32_t* flags, int64_t* required,
                     hipStream_t stream) {
  if (flags) *flags = 0u;
  if (required) *required = 0;
  if (!render_ws) return fail(GS_ERR_INVALID_ARGUMENT, "render_ws is null");
  if (render_ws_bytes < 256 || (reinterpret_cast<uintptr_t>(render_ws) & 255u))
    return fail(GS_ERR_INVALID_ARGUMENT, "render workspace too small or not 256-byte aligned");
  uint32_t hdr[kHdrStatusWords];
  hipError_t e = hipMemcpyAsync(hdr, render_ws, sizeof(hdr), hipMemcpyDeviceToHost, stream);
  // read, then clear the status words (a fill kernel, ordered after the copy on the stream)
  if (e == hipSuccess) e = launch_fill_u32(static_cast<uint32_t*>(render_ws) + kHdrFlags, 2, 0u, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "gs_render_status");
  const uint32_t f = hdr[kHdrFlags];
  if (flags) *flags = f;
  if (required) *required = (int64_t)hdr[kHdrNeed];
  if (f & kFlagCapacity)
    return fail(GS_ERR_CAPACITY, "the lists need %u intersections, more than the render workspace holds: its "
                "results are not valid", hdr[kHdrNeed]);
  if (f & kFlagStall)
    return fail(GS_ERR_INCOMPLETE, "a bounded wait of the fused image pass gave up: some gradient sums are missing");
  return ok();
}

int gs_adam_step(int64_t count, float* params, const float* grads, const gs_adam* adam, hipStream_t stream) {
  int st;
  if (!adam) return fail(GS_ERR_INVALID_ARGUMENT, "adam is null");
  if ((st = check_adam(adam))) return st;
  if (count < 0) return fail(GS_ERR_INVALID_ARGUMENT, "count < 0");
  if (count > 0 && (!params || !grads)) return fail(GS_ERR_INVALID_ARGUMENT, "params / grads is null");
  const hipError_t e = launch_adam(count, params, grads, adam->m, adam->v, adam_coef(*adam), stream);
  return e == hipSuccess ? ok() : hip_fail(e, "gs_adam_step");
}

}  // extern "C"
