/*
 * gsmi.h -- C ABI of the MI355X (gfx950) 3D Gaussian Splatting training-step library
 * (libgsmi.so).
 *
 * One training step over one GPU's share of the Gaussians is, in order:
 *   gs_preprocess       EWA projection of every Gaussian to a 2D conic + SH colour
 *   gs_bin_and_sort     tile binning, stable (tile, depth) radix sort, per-tile ranges
 *   gs_render_forward   front-to-back alpha compositing per 16x16 tile
 *   gs_loss_l1          L1 image loss and its gradient
 *   gs_loss_l1_dssim    L1 + lambda-weighted D-SSIM image loss and its gradient
 *   gs_render_backward  reverse-order backward blend + preprocess backward
 *                       (optionally fused with the Adam update)
 *   gs_adam_step        Adam over all parameters (when not fused)
 * and, for batched steps (several views per optimizer step), gs_preprocess_backward_accumulate
 * with gs_adam_batch; adaptive density control with gs_densify_stats and gs_densify.
 *
 * The pages this follows name these stages but print no formulas:
 *   "Scaling 3D Gaussian Splatting with Distributed Compute: Why One GPU Is Never Enough"
 *     - Gaussian parameters: mean, covariance from scale and rotation, SH colour, opacity
 *       (its list of what a Gaussian is parameterised by);
 *     - projection to 2D means, depths, conics, radii and a visibility mask, with SH turned
 *       into RGB per camera first (walkthrough steps "Project locally" and "Evaluate
 *       spherical harmonics before communicating");
 *     - the ~12-scalar, ~48-byte projected record (step "Ship each camera's Gaussians");
 *     - per-tile sorted intersection lists and per-tile offsets into them (the memory
 *       accounting passage and the trace section on intersect_offset_kernel);
 *     - rasterization and an L1 (+ D-SSIM) loss with gradients flowing to mean, covariance,
 *       colour and opacity, then a local Adam step (steps "Rasterize locally", "Compute
 *       the loss locally", "Step the optimizer locally").
 *   "Toward Distributed 3D Gaussian Splatting for High-Resolution Isosurface
 *     Visualization", sections I and III: 3D-GS trained from synthetic orbit views.
 * Each formula is the standard 3D-GS / EWA-splatting reading of the stage.
 *
 * Conventions common to every call
 *   - All pointers to arrays are DEVICE pointers (hipMalloc'd or equivalent, coarse-grained)
 *     unless marked "host".  The caller owns every buffer; the library never allocates or
 *     frees device memory.  Host structs are read during the call only.
 *   - Every call enqueues work on `stream` and returns without waiting, except
 *     gs_bin_and_sort (with a non-null k_out), gs_bin_and_sort_count and gs_densify, which copy
 *     a count to the host and synchronise
 *     `stream` once, and gs_render_status, which reads the render workspace's status words
 *     (see there).
 *   - Outputs must not alias inputs, except where a call says it updates in place.
 *   - Every call returns a gs_status.  Arguments are checked before any HIP call; on an
 *     error nothing is enqueued and gs_last_error() describes it.  No exception or abort
 *     crosses the ABI.  Non-finite Gaussians are culled, not reported.
 *   - Floating point is IEEE float32 throughout.
 */
#ifndef GSMI_H
#define GSMI_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GSMI_VERSION 9
#define GS_TILE 16 /* tiles are GS_TILE x GS_TILE pixels */

typedef enum gs_status {
  GS_OK = 0,
  GS_ERR_INVALID_ARGUMENT = -1, /* null pointer, bad size, non-finite camera, ...      */
  GS_ERR_CAPACITY = -2,         /* intersection buffers too small; *k_out = required K */
  GS_ERR_HIP = -3,              /* a HIP runtime call failed (message in gs_last_error) */
  GS_ERR_UNSUPPORTED = -4,      /* a valid but unsupported variant                    */
  GS_ERR_INCOMPLETE = -5        /* a bounded device-side wait gave up (gs_render_status) */
} gs_status;

/* Pinhole camera.  viewmat is the row-major 3x4 world->camera transform [R | t] with
 * camera axes x right, y down, z forward; a world point p maps to R p + t.  Pixel (px, py)
 * has its centre at (px + 0.5, py + 0.5); u = fx x/z + cx, v = fy y/z + cy.  Gaussians
 * with z <= near_plane are culled.  Requires width, height in [1, 32768] and finite,
 * positive fx, fy, near_plane. */
typedef struct gs_camera {
  float viewmat[12];
  float fx, fy, cx, cy;
  int32_t width, height;
  float near_plane;
} gs_camera;

/* Gaussian set.  Parameters are planar float32 rows of stride ld (>= n) elements:
 *   rows 0-2 mean, 3-5 log-scale (scale = exp), 6-9 rotation quaternion (w, x, y, z; need
 *   not be unit), 10 opacity logit (opacity = sigmoid), 11 + 3k + c SH coefficient k of
 *   colour channel c for k < (sh_degree+1)^2.
 * R = 11 + 3 (sh_degree+1)^2 rows (14 at degree 0, 59 at degree 3).  n in [0, 2^31 - 1],
 * sh_degree in [0, 3]. */
typedef struct gs_scene {
  int64_t n;
  int64_t ld;
  int32_t sh_degree;
} gs_scene;

/* The projected record of one Gaussian for one camera (48 bytes, 16-byte aligned): the
 * pages' dozen scalars -- two radii, two mean coordinates, depth, three conic entries,
 * opacity and three colour channels -- laid out so that the blend's alpha test reads the
 * first 32 bytes.  A culled Gaussian has every field 0. */
typedef struct gs_splat {
  float u, v;                 /* 2D mean, pixels                                           */
  int32_t radius_x, radius_y; /* per-axis 3-sigma extents ceil(3 sqrt(S2_ii)), pixels      */
  float conic_a, conic_b;     /* inverse of the 2D covariance S2: [[a, b], [b, c]]         */
  float conic_c, opacity;     /* opacity = sigmoid(logit)                                  */
  float r, g, b;              /* max(0.5 + sum_k Y_k(view dir) f_k, 0) per channel        */
  float depth;                /* view-space z                                              */
} gs_splat;

/* Output of gs_preprocess, input of the later calls.  Each array has >= ld entries (rect:
 * >= 2 ld words, 8-byte aligned).
 *   tiles[i]     number of tiles the Gaussian's 3-sigma box touches (0 = culled)
 *   depth_key[i] the float32 bits of depth for a visible Gaussian, 0xFFFFFFFF if culled
 *   rect[2i], rect[2i+1]  that box's tile rect [x0, x1) x [y0, y1), packed x0 | y0 << 16 and
 *                x1 | y1 << 16 (both 0 if culled): the binning reads it in depth order */
typedef struct gs_proj {
  gs_splat* splat;
  uint32_t* tiles;
  uint32_t* depth_key;
  uint32_t* rect;
} gs_proj;

/* Adam state and hyper-parameters (Kingma & Ba, bias-corrected, dense over every float).
 * m and v are planar like params (R rows of stride ld) or, for gs_adam_step, flat arrays of
 * `count` floats.  step is the 1-based step number t.  The hyper-parameters are double so
 * that 1 - beta and the bias corrections 1 - beta^t are formed exactly before rounding to the
 * float32 the kernels use (1 - 0.999f alone is off by 1.3e-5). */
typedef struct gs_adam {
  float* m;
  float* v;
  int32_t step;
  double lr, beta1, beta2, eps;
} gs_adam;

/* ---------------------------------------------------------------------------------- */

/* Per-Gaussian preprocess ("Scaling 3D Gaussian Splatting with Distributed Compute", walkthrough
 * steps "Project locally" -- 2D means, depths, conics, radii and visibility per camera -- and
 * "Evaluate spherical harmonics before communicating" -- SH to RGB once per camera; the Gaussian's
 * parameters are the page's list: mean, covariance from scale and rotation, SH colour, opacity).
 * For each Gaussian i < n: scale = exp(log-scale), opacity = sigmoid(logit), rotation from the
 * normalised quaternion, Sigma = R S S^T R^T, view-space mean p = W mu + t (culled if z <=
 * near_plane or not finite), the EWA Jacobian J at p (x/z, y/z clamped to 1.3x the half field of
 * view), S2 = J W Sigma W^T J^T + 0.3 I (culled if det <= 0), conic = S2^-1, per-axis 3-sigma radii
 * ceil(3 sqrt(S2_ii)), the tile rect of the box (u +- radius_x, v +- radius_y) (culled if empty),
 * and rgb = max(0.5 + sum_k Y_k(dir) f_k, 0) with dir the unit vector from the camera centre to mu
 * and Y_k the real SH basis with the Condon-Shortley phase (l = 0..sh_degree, m = -l..l).
 *   params[R][ld]  device, read only
 *   out            device arrays of >= ld entries (rect: 2 ld words); writes out.splat[0..n),
 *                  out.tiles[0..n), out.depth_key[0..n), out.rect[0..2n); a culled Gaussian gets an
 *                  all-zero record, tiles 0, depth key 0xFFFFFFFF and rect (0, 0)
 * GS_ERR_INVALID_ARGUMENT for a bad scene or camera, a null params (n > 0) or a null / misaligned
 * proj array.  One thread per Gaussian; HBM-bound. */
int gs_preprocess(const gs_scene* scene, const float* params, const gs_camera* cam, gs_proj out,
                  hipStream_t stream);

/* Bytes of device workspace gs_bin_and_sort needs for n Gaussians, up to k_capacity
 * intersections and a width x height image (host-only query, no HIP call). */
int gs_bin_and_sort_workspace(int64_t n, int64_t k_capacity, int32_t width, int32_t height,
                              size_t* bytes);

/* Tile binning and sorting ("Scaling 3D Gaussian Splatting with Distributed Compute": the per-tile
 * sorted intersection lists of the memory-accounting passage, and the trace section's
 * intersection-offset kernel, one thread per intersection; the ties by Gaussian index are this
 * library's rule, which makes the order unique).  For every visible Gaussian i and every tile
 * (tx, ty) of its 3-sigma box, one intersection with key (ty*TX + tx) << 32 | depth_key[i] and value i;
 * the intersections are sorted ascending by key, ties in Gaussian index order (stable),
 * which gives per-tile lists in front-to-back depth order.
 *   vals[k_capacity]   out: sorted Gaussian indices
 *   ranges[2*T]        out: ranges[2t], ranges[2t+1] = [start, end) of tile t in vals;
 *                           (0, 0) for an empty tile.  T = ceil(W/16) * ceil(H/16).
 *   keys[k_capacity]   out, nullable: the sorted 64-bit keys
 *   workspace          device scratch of >= gs_bin_and_sort_workspace() bytes
 *   k_out              HOST out, nullable: the number of intersections K
 * The count, the depth-key range and K stay on the device: every kernel of the sort reads them
 * there, so the whole sort is enqueued without waiting.  With k_out non-null the call then copies
 * K to the host and waits for `stream` once, at the end; if K > k_capacity it sets *k_out = K and
 * returns GS_ERR_CAPACITY, and vals, ranges and keys are left unwritten (the caller grows its
 * buffers and calls again).  With k_out null the call returns without waiting; if K > k_capacity
 * then, vals and keys are left unwritten and every tile's range is set empty (nothing renders,
 * nothing is partial), and gs_bin_and_sort_count reports the overflow. */
int gs_bin_and_sort(const gs_scene* scene, const gs_camera* cam, gs_proj proj, void* workspace,
                    size_t workspace_bytes, int64_t k_capacity, uint32_t* vals, uint32_t* ranges,
                    uint64_t* keys, int64_t* k_out, hipStream_t stream);

/* K of the last gs_bin_and_sort on `workspace` (after the work enqueued on `stream` so far):
 * copies it to *k_out (HOST) and waits for `stream`.  GS_ERR_CAPACITY (with *k_out = K) if that
 * call's lists overflowed its k_capacity; GS_ERR_INVALID_ARGUMENT for a null or misaligned
 * workspace.  For callers that sort with k_out null and check the count later, e.g. once per
 * batch of steps instead of once per step. */
int gs_bin_and_sort_count(const void* workspace, size_t workspace_bytes, int64_t* k_out, hipStream_t stream);

/* Bytes of the render workspace that gs_render_forward fills and gs_render_backward uses, for
 * a width x height image, n Gaussians and lists of up to k_capacity intersections (host-only
 * query).  It holds, for every tile list longer than one segment (512 entries), each pixel's
 * transmittance and colour at every segment boundary and at the end of its walk, plus the
 * backward's work list: the backward walks the segments of a long list in parallel from these
 * states.  For every 64 entries of a tile list and pixel of the tile it holds the 64-bit mask
 * of the entries the forward composited at that pixel (8 bytes per pixel per 64 entries), so
 * the backward revisits exactly those.  It also holds the backward's per-intersection gradient
 * sums (36 bytes each), which are summed per Gaussian into grad2d instead of accumulating
 * grad2d with atomics. */
int gs_render_workspace(int32_t width, int32_t height, int64_t n, int64_t k_capacity, size_t* bytes);

/* The largest intersection count a render workspace of `bytes` serves for this image and n
 * (host-only query; the inverse of gs_render_workspace, rounded to whole 512-entry segments).
 * GS_ERR_INVALID_ARGUMENT if `bytes` is below the size for k_capacity 0. */
int gs_render_workspace_capacity(int32_t width, int32_t height, int64_t n, size_t bytes,
                                 int64_t* k_capacity);

/* Forward blend ("Scaling 3D Gaussian Splatting with Distributed Compute", walkthrough step
 * "Rasterize locally": alpha compositing of each camera's Gaussians over screen tiles, front to
 * back, with early termination).  For each pixel, walks its tile's list front to back: power =
 * -(a dx^2 + c dy^2)/2 - b dx dy with (dx, dy) = pixel centre - (u, v); skips power > 0;
 * alpha = min(0.99, opacity e^power); skips alpha < 1/255; stops before blending an entry
 * that would take the transmittance T below 1e-4; else C += rgb alpha T, T *= 1 - alpha.
 *   image[H][W][3]      out: C + T bg
 *   T_final[H][W]       out: final transmittance
 *   last_contrib[H][W]  out: 1-based list position of the last blended entry (0 = none)
 *   n_examined[H][W]    out, nullable: entries examined (list length, or the position of
 *                       the entry that stopped the pixel)
 *   k                   the number of intersections in vals (gs_bin_and_sort's K)
 *   blend_count         out, nullable: device uint64[4] to which four image sums are
 *                       ADDED (the caller zeroes them): [0] n_examined, [1] last_contrib
 *                       (the entries the backward pass walks), [2] the (pixel, entry)
 *                       pairs composited, [3] the (pixel, entry) pairs whose alpha the
 *                       kernel evaluates (the rest of the examined pairs are rejected by a
 *                       conservative per-record pixel box without evaluating alpha)
 *   render_ws           out: device workspace (256-byte aligned) of render_ws_bytes >= the
 *                       size gs_render_workspace gives for this image, n and a k_capacity
 *                       >= k; GS_ERR_INVALID_ARGUMENT if it is smaller than the size for
 *                       k_capacity 0, GS_ERR_CAPACITY (nothing enqueued; the message gives the
 *                       size needed) if it holds fewer than k intersections.  Should the lists
 *                       themselves need more than it holds (k understated), the kernels stay
 *                       inside the workspace, the results are not valid and gs_render_status
 *                       reports GS_ERR_CAPACITY.  A new workspace is cleared once with
 *                       gs_render_init.
 * bg is a HOST array of 3 floats.  A few persistent 256-thread workgroups per CU take the
 * tiles, longest lists first. */
int gs_render_forward(const gs_camera* cam, int64_t n, const gs_splat* splat, const uint32_t* vals,
                      const uint32_t* ranges, int64_t k, const float* bg, float* image, float* T_final,
                      uint32_t* last_contrib, uint32_t* n_examined, uint64_t* blend_count,
                      void* render_ws, size_t render_ws_bytes, hipStream_t stream);

/* Bytes of device workspace gs_loss_l1 needs for `count` elements (host-only query). */
int gs_loss_l1_workspace(int64_t count, size_t* bytes);

/* L1 loss over `count` = 3HW elements: *loss = mean |image - target| (device float),
 * dL_dimage = sign(image - target) / count with sign(0) = 0.  The page's loss is L1 plus a
 * lambda-weighted D-SSIM term; this call is the L1 term. */
int gs_loss_l1(int64_t count, const float* image, const float* target, float* loss,
               float* dL_dimage, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The L1 loss without allocation, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): gs_loss_l1 with its
 * per-workgroup partial sums in a static device array of the library (256 KiB on each GPU it runs
 * on, held until the process ends) instead of a workspace argument.  Same results as gs_loss_l1,
 * bit for bit.  count <= 268,435,456 (2^28) elements, else GS_ERR_CAPACITY; GS_ERR_INVALID_ARGUMENT
 * for count < 0 or a null pointer.  Calls that overlap on one GPU (two streams, two host threads)
 * share that array and race: serialise them.  Asynchronous. */
int gs_loss_l1_noalloc(int64_t count, const float* image, const float* target, float* loss,
                       float* dL_dimage, hipStream_t stream);

/* Bytes of device workspace gs_loss_l1_dssim needs for a width x height image (host-only
 * query): 36 bytes per SSIM window position plus per-workgroup sums, about 36 W H.
 * GS_ERR_INVALID_ARGUMENT if width or height is below 11 or bytes is null. */
int gs_loss_l1_dssim_workspace(int32_t width, int32_t height, size_t* bytes);

/* L1 + D-SSIM loss ("Scaling 3D Gaussian Splatting with Distributed Compute", the loss passage:
 * an L1 term and a D-SSIM term weighted by lambda; step "Compute the loss locally": L1 and a
 * fused SSIM).  The pages give no window or constants; this call takes SSIM with an 11x11
 * Gaussian window of standard deviation 1.5 (normalised to sum 1), C1 = 0.01^2, C2 = 0.03^2
 * (images in [0, 1]), per colour channel over the (W - 10)(H - 10) window positions wholly
 * inside the image, and
 *     L = (1 - lambda) mean |image - target| + lambda (1 - mean SSIM).
 *   image, target[H][W][3]  device, float32, interleaved RGB rows (as gs_render_forward writes)
 *   lambda                  in [0, 1] (0.2 is the usual weight)
 *   loss                    out: device float[3] = (L, mean |image - target|, mean SSIM)
 *   dL_dimage[H][W][3]      out: dL/dimage, the exact derivative of L (sign(0) = 0 in the L1
 *                           term); may be passed to gs_render_backward
 *   workspace               device, >= gs_loss_l1_dssim_workspace bytes; its contents on entry
 *                           are ignored and it must not be shared by calls in flight together
 * Sums run per workgroup in float32 and across workgroups in double, in a fixed order: the
 * result is deterministic.  GS_ERR_INVALID_ARGUMENT for width or height below 11, lambda
 * outside [0, 1] or not finite, a null pointer or a short workspace. */
int gs_loss_l1_dssim(int32_t width, int32_t height, const float* image, const float* target, float lambda,
                     float* loss, float* dL_dimage, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* Backward of the step from dL/dimage ("Scaling 3D Gaussian Splatting with Distributed Compute",
 * the loss passage -- gradients flow back through the rasterizer to the mean, covariance, colour
 * and opacity -- and walkthrough step "Backward pass"): the exact derivative of the branch the
 * forward took at every pixel, in reverse list order from last_contrib (alpha clamped at 0.99
 * passes no gradient to opacity or power; skipped entries contribute nothing), then the chain
 * rule back through the preprocess to every parameter row.
 *   k              the number of intersections in vals; capacity errors as gs_render_forward
 *   grad2d[ld][9]  out, nullable: per-Gaussian dL/d(u, v, conic_a, conic_b, conic_c, opacity,
 *                  r, g, b) from the reverse-order backward blend, the nine values of Gaussian i
 *                  at grad2d + 9 i, for i < n (rows n..ld-1 are not written).  Each
 *                  intersection's sums are staged in render_ws and each Gaussian's are added
 *                  in the order of its tile rect; within an intersection the pixel-block sums
 *                  meet in LDS atomics, so the summation order is not fixed.  Null: the sums
 *                  stay staged in render_ws, and the preprocess backward (here, with grads or
 *                  adam, or gs_preprocess_backward_staged later) adds each Gaussian's in the
 *                  same order itself, giving the same values without the grad2d round trip.
 *   grads[R][ld]   out, nullable: dL/dparams by the chain rule through the preprocess
 *   adam           nullable: when given, the preprocess backward also applies the Adam
 *                  update to params, adam->m and adam->v in place (params is then written)
 * With grads and adam both null only the backward blend runs (grad2d is the only output and
 * params may be null); gs_preprocess_backward then finishes the step.
 * T_final, last_contrib and render_ws are the forward's outputs for the same lists, camera and
 * bg (render_ws unmodified since, same size); proj.tiles is the preprocess output the lists
 * were built from.  The backward leaves the forward's part of render_ws intact, so it may be
 * run more than once per forward.  bg is a HOST array of 3 floats.  Culled
 * Gaussians receive zero gradients. */
int gs_render_backward(const gs_scene* scene, float* params, const gs_camera* cam, gs_proj proj,
                       const uint32_t* vals, const uint32_t* ranges, int64_t k, const float* bg,
                       const float* T_final, const uint32_t* last_contrib, const float* dL_dimage,
                       float* grad2d, float* grads, const gs_adam* adam, void* render_ws,
                       size_t render_ws_bytes, hipStream_t stream);

/* Prepares render_ws for gs_render_step over these lists (ranges from gs_bin_and_sort, proj.tiles
 * from gs_preprocess, the same camera): the segment plan and tile order of the forward, an empty
 * list of backward work items, and each Gaussian's cleared staging rows for the gradient sums.
 * k is the number of intersections in the lists.  Kept apart from gs_render_step so that the fused
 * kernel can be timed alone.  Errors as gs_render_forward. */
int gs_render_plan(const gs_scene* scene, const gs_camera* cam, gs_proj proj, const uint32_t* ranges, int64_t k,
                   void* render_ws, size_t render_ws_bytes, hipStream_t stream);

/* The image pass of one training step, fused: the forward blend (as gs_render_forward), the L1
 * loss against target (as gs_loss_l1) and the backward blend (as gs_render_backward with
 * grad2d, grads and adam null) in one persistent kernel.  Workgroups that finish a tile's
 * forward hand its backward segments to the others at once, so the backward runs beside the
 * forward's long tile walks instead of after them ("Scaling 3D Gaussian Splatting with
 * Distributed Compute", walkthrough steps "Rasterize locally" and "Backward pass").
 *   target[H][W][3]     the ground-truth image
 *   image, T_final, last_contrib, n_examined, blend_count   as gs_render_forward
 *   loss                out: device float, mean |image - target| over the 3HW values
 *   dL_dimage[H][W][3]  out: sign(image - target) / (3HW), sign(0) = 0
 *   grad2d[ld][9]       out, nullable: as gs_render_backward's grad2d (the staged sums added
 *                       per Gaussian in the order of its tile rect)
 *   render_ws           as left by gs_render_plan for the same lists, camera and proj (call it
 *                       first, once per step); on return it holds the forward's state and each
 *                       intersection's nine gradient sums, staged for
 *                       gs_preprocess_backward_staged (same camera, proj and render_ws), which
 *                       finishes the step.  gs_render_backward may also be run on it.
 * proj.splat and proj.tiles are the preprocess outputs the lists were built from; bg is a HOST
 * array of 3 floats; k as gs_render_forward.  A wait of one workgroup for another is bounded
 * (about a second); should one ever give up, that work item's gradient sums are missing and
 * gs_render_status reports GS_ERR_INCOMPLETE.  Errors as gs_render_forward. */
int gs_render_step(const gs_scene* scene, const gs_camera* cam, gs_proj proj, const uint32_t* vals,
                   const uint32_t* ranges, int64_t k, const float* bg, const float* target, float* image,
                   float* T_final, uint32_t* last_contrib, uint32_t* n_examined, uint64_t* blend_count,
                   float* loss, float* dL_dimage, float* grad2d, void* render_ws, size_t render_ws_bytes,
                   hipStream_t stream);

/* Clears the status words of a render workspace (its first 64 bytes) before its first use, so that
 * gs_render_status reports only what the calls on it flag.  Asynchronous (a fill kernel on
 * `stream`).  GS_ERR_INVALID_ARGUMENT for a null, short or misaligned workspace. */
int gs_render_init(void* render_ws, size_t render_ws_bytes, hipStream_t stream);

/* Status of the device-side checks the render calls on render_ws made since gs_render_init or the
 * last gs_render_status on it: the kernels set status bits and never clear them, so one call after
 * many steps covers them all.  Copies the status words to the host, clears them (a fill kernel)
 * and SYNCHRONISES `stream`.
 *   flags     host out, nullable: bit 0 a bounded wait of gs_render_step gave up, bit 1 some lists
 *             needed more intersections than the workspace holds
 *   required  host out, nullable: the most intersections those lists needed (their largest end,
 *             or the staged entries when larger); 0 when bit 1 is clear
 * Returns GS_ERR_CAPACITY when bit 1 is set (the image and gradients of those calls are not
 * valid), else GS_ERR_INCOMPLETE when bit 0 is set (some gradient sums are missing), else GS_OK. */
int gs_render_status(void* render_ws, size_t render_ws_bytes, uint32_t* flags, int64_t* required,
                     hipStream_t stream);

/* Preprocess backward alone: grads (and optionally the fused Adam update) from a given
 * grad2d[ld][9].  Same semantics as the second half of gs_render_backward. */
int gs_preprocess_backward(const gs_scene* scene, float* params, const gs_camera* cam,
                           const float* grad2d, float* grads, const gs_adam* adam,
                           hipStream_t stream);

/* Preprocess backward alone, reading each Gaussian's nine dL/d(2D) values as the sum of its
 * intersections' sums that gs_render_backward (called with grad2d = NULL on the same render_ws,
 * camera and proj) left staged in render_ws, added in the order of the Gaussian's tile rect:
 * the values gs_render_backward would have written into grad2d.  gs_render_step leaves the
 * same staged sums.  proj.tiles is the
 * preprocess output the lists were built from.  Otherwise as gs_preprocess_backward. */
int gs_preprocess_backward_staged(const gs_scene* scene, float* params, const gs_camera* cam, gs_proj proj,
                                  const void* render_ws, size_t render_ws_bytes, float* grads,
                                  const gs_adam* adam, hipStream_t stream);

/* gs_preprocess_backward_staged, then gs_preprocess of the next view on the parameters it leaves,
 * in one pass over the Gaussians: the training iteration of "Scaling 3D Gaussian Splatting with
 * Distributed Compute" (its trace section: the optimizer step, then the next iteration's
 * preprocess of the updated Gaussians) with the parameter rows read once instead of twice.  Each
 * Gaussian's thread finishes its rows (with the Adam update when adam is set, else the rows keep
 * their values) and projects the new values with next_cam into next: the records, tile counts,
 * depth keys and rects gs_preprocess(next_cam) writes for the parameters this call leaves, bit
 * for bit.  Those parameters, moments and grads are gs_preprocess_backward_staged's up to the
 * rounding of the fused multiply-adds the compiler forms differently in the two kernels (below
 * 1e-6 of each row's largest value where measured).
 *   next_cam  the next view's camera (any camera, the same one included)
 *   next      out: as gs_preprocess's out.  It may be proj itself (each Gaussian reads its own
 *             proj entries before it writes them); the lists and render_ws of this view must not
 *             be used with it afterwards.
 * GS_ERR_INVALID_ARGUMENT as gs_preprocess_backward_staged and as gs_preprocess for next_cam and
 * next. */
int gs_preprocess_backward_staged_next(const gs_scene* scene, float* params, const gs_camera* cam, gs_proj proj,
                                       const void* render_ws, size_t render_ws_bytes, float* grads,
                                       const gs_adam* adam, const gs_camera* next_cam, gs_proj next,
                                       hipStream_t stream);

/* Batched steps ("Scaling 3D Gaussian Splatting with Distributed Compute", the batch-size
 * passage: several camera views per optimizer step; the batch's loss is the mean of its views'
 * losses, so its gradient is the mean of theirs).  The preprocess backward of one view of the
 * batch, from the sums staged in render_ws (as gs_preprocess_backward_staged):
 *   grads_acc[R][ld]  the gradient accumulated over the batch's earlier views
 *   first             1 for the batch's first view (grads_acc is not read), else 0
 *   scale             this view's weight, normally 1 / BS
 *   adam              NULL for every view but the last: grads_acc <- (first ? 0 : grads_acc)
 *                     + scale * g.  For the last view: the total (first ? 0 : grads_acc) +
 *                     scale * g goes through the Adam update of params, m and v (with the
 *                     batch's hyper-parameters, gs_adam_batch) and grads_acc is not written; it
 *                     may then be NULL when first is 1 (a batch of one).
 * Rows n..ld-1 are not touched.  GS_ERR_INVALID_ARGUMENT as gs_preprocess_backward_staged, and
 * for first outside {0, 1}, a non-finite scale or a missing grads_acc. */
int gs_preprocess_backward_accumulate(const gs_scene* scene, float* params, const gs_camera* cam, gs_proj proj,
                                      const void* render_ws, size_t render_ws_bytes, float* grads_acc,
                                      int32_t first, float scale, const gs_adam* adam, hipStream_t stream);

/* Adam's hyper-parameters for `batch` views per optimizer step (host only; the same page's
 * batch-size passage): lr * sqrt(batch), eps / sqrt(batch), and each momentum coefficient
 * decayed linearly, beta <- 1 - batch (1 - beta), so beta1 = 0.9 reaches 0 at batch 10.  m, v
 * and step are copied.  GS_ERR_INVALID_ARGUMENT for batch < 1, a null pointer, or a batch that
 * takes a coefficient below zero (batch > 10 at beta1 = 0.9). */
int gs_adam_batch(const gs_adam* adam, int32_t batch, gs_adam* out);

/* Adaptive density control ("Scaling 3D Gaussian Splatting with Distributed Compute": pruning
 * and densifying, which grow N and drive memory; the page gives no rules, so these follow
 * 3D-GS).  Options (double, formed into float32 thresholds once):
 *   grad_threshold  averaged 2D-gradient statistic at or above which a Gaussian densifies
 *                   (3D-GS: 2e-4)
 *   percent_dense, extent   clone when the largest scale is <= percent_dense * extent, else
 *                   split (3D-GS: 0.01 x the scene's extent)
 *   min_opacity     prune below this opacity (3D-GS: 0.005)
 *   split_factor    a split child's scales are the parent's / split_factor (3D-GS: 1.6) */
typedef struct gs_densify_opts {
  double grad_threshold, percent_dense, extent, min_opacity, split_factor;
} gs_densify_opts;

/* Densification statistics of one view, after its backward blend (gs_render_step, or
 * gs_render_backward with grad2d = NULL) on the same render_ws, camera and proj: every
 * Gaussian with radius_x > 0 adds |(dL/du W/2, dL/dv H/2)| -- its 2D mean's gradient in
 * normalised device units, from the staged sums in the order gs_preprocess_backward_staged
 * adds them -- to grad_acc[i] and 1 to count[i] (both device float[n], accumulated over views;
 * the caller zeroes them after each densification).  Asynchronous. */
int gs_densify_stats(const gs_scene* scene, const gs_camera* cam, gs_proj proj, const void* render_ws,
                     size_t render_ws_bytes, float* grad_acc, float* count, hipStream_t stream);

/* Bytes of device workspace gs_densify needs for n Gaussians (host-only query). */
int gs_densify_workspace(int64_t n, size_t* bytes);

/* One clone / split / prune pass over the scene's n Gaussians.
 *   params, m, v[R][ld]   in: parameters and Adam moments
 *   grad_acc, count[n]    in: the statistics from gs_densify_stats
 *   z[2][3][ld]           in: standard normal draws, z[k][j][i] for split child k of Gaussian i
 *   params_out, m_out, v_out[R][ld_out]  out (must not alias the inputs)
 *   n_out                 host out: the Gaussian count after the pass
 *   codes[n]              out, nullable: 0 kept, 1 cloned, 2 split, 3 pruned
 * Gaussian i is pruned when its opacity logit is below logit(min_opacity); otherwise, when
 * grad_acc[i] / count[i] (0 when count is 0) reaches grad_threshold, it is cloned when its
 * largest log-scale is at most log(percent_dense * extent) and split otherwise.  Output order:
 * the kept Gaussians (neither pruned nor split, clones' originals included) in index order with
 * their moments; one copy of each cloned Gaussian in index order; the first child of each split
 * Gaussian in index order; then the second children.  Child k: mean mu + R(q) (exp(l) * z[k]),
 * log-scale l - log(split_factor), rotation, opacity and colour copied.  New Gaussians start
 * with zero moments.  The call counts first, copies the three totals to the host and
 * synchronises `stream`; when n_out > ld_out it returns GS_ERR_CAPACITY with *n_out set and
 * writes nothing.  Every comparison with NaN is false: a NaN statistic never densifies, a NaN
 * logit never prunes, three NaN log-scales neither clone nor split (a NaN among them is
 * skipped).  GS_ERR_INVALID_ARGUMENT for null pointers, aliasing outputs, a short
 * workspace or options out of range. */
int gs_densify(const gs_scene* scene, const float* params, const float* m, const float* v, const float* grad_acc,
               const float* count, const float* z, const gs_densify_opts* opts, float* params_out, float* m_out,
               float* v_out, int64_t ld_out, int64_t* n_out, int32_t* codes, void* workspace,
               size_t workspace_bytes, hipStream_t stream);

/* Adam ("Scaling 3D Gaussian Splatting with Distributed Compute", walkthrough step "Step the
 * optimizer locally", over the parameters and the two moment buffers the memory-accounting
 * passage counts per Gaussian; Kingma & Ba's bias-corrected update) over `count` floats, in place:
 * m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2; params -= lr (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps).
 *   params, grads  device float[count]; grads is read only
 *   adam           HOST struct: adam->m, adam->v device float[count] (in place), step t >= 1,
 *                  lr, beta1, beta2 in [0, 1), eps
 * Every float is updated, a zero gradient included (dense).  GS_ERR_INVALID_ARGUMENT for a null
 * adam, count < 0, null arrays or hyper-parameters out of range.  Asynchronous. */
int gs_adam_step(int64_t count, float* params, const float* grads, const gs_adam* adam,
                 hipStream_t stream);

/* Message for the last error on the calling thread; valid until the next call on it. */
const char* gs_last_error(void);

int gs_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GSMI_H */
