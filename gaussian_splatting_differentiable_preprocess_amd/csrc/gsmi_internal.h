// Internal declarations shared by the HIP translation units of libgsmi.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gsmi.h"

namespace gsmi {

constexpr int kTile = GS_TILE;
constexpr int kBlock = 256;  // threads per workgroup (4 wave64)

// Camera as the kernels use it (float32, passed by value as a kernel argument).
struct CamK {
  float R[9];        // world->camera rotation, row-major
  float t[3];
  float fx, fy, cx, cy;
  float near_plane;
  float limx, limy;  // guard band for x/z, y/z inside the EWA Jacobian: 1.3 x half-extent / f
  float pos[3];      // camera centre in world space, -R^T t
  int W, H, TX, TY;
};

CamK make_cam(const gs_camera& c);

inline int rows_for_degree(int d) { return 11 + 3 * (d + 1) * (d + 1); }

// Tile rect [x0,x1) x [y0,y1) of the box (u +- rx, v +- ry): x0 = clamp(floor((u-rx)/16), 0,
// TX), x1 = clamp(floor((u+rx)/16) + 1, 0, TX), the same in y.  u +- rx is a single float32
// add and the scale by 1/16 is exact, so every caller that passes the same stored (u, v, rx,
// ry) gets the same rect.  Contraction is off so no caller can fuse these adds.
__device__ __forceinline__ int clamp_tile(float f, int hi) {
  return !(f > 0.0f) ? 0 : (f > (float)hi ? hi : (int)f);
}
__device__ __forceinline__ void tile_rect(float u, float v, int rx, int ry, int TX, int TY,
                                          int& x0, int& y0, int& x1, int& y1) {
#pragma clang fp contract(off)
  const float frx = (float)rx, fry = (float)ry;
  const float ulo = u - frx, uhi = u + frx, vlo = v - fry, vhi = v + fry;
  x0 = clamp_tile(floorf(ulo * 0.0625f), TX);
  x1 = clamp_tile(floorf(uhi * 0.0625f) + 1.0f, TX);
  y0 = clamp_tile(floorf(vlo * 0.0625f), TY);
  y1 = clamp_tile(floorf(vhi * 0.0625f) + 1.0f, TY);
}

// ---- launchers (each returns the launch status) --------------------------------------
hipError_t launch_preprocess(const gs_scene& sc, const float* params, const CamK& cam,
                             gs_proj out, hipStream_t s);

struct PrebwdArgs {
  int64_t n, ld;
  int deg;
  float* params;
  const float* grad2d;  // null: each Gaussian's nine values are the sum of its staged rows
  // the backward blend's staged per-intersection sums (used when grad2d is null): Gaussian i's
  // rows are staging[9 (goff_blk[i / kGoffBlock] + goff[i] + j)], j < tiles[i]
  const float* staging;
  const uint32_t* goff;
  const uint32_t* goff_blk;
  const uint32_t* tiles;
  uint64_t staging_cap;
  // Batched steps: the row's gradient is gscale * (this view's) + gacc[row] when gacc is
  // non-null (gacc may be grads: each element is read before it is written, by one thread)
  const float* gacc;
  float gscale;
  float* grads;      // nullable when adam
  float* m;          // nullable: no Adam
  float* v;
  float lr, b1, omb1, b2, omb2, eps, inv_bc1, inv_bc2;
};

// Adam coefficients rounded to float32 from double: b1, 1 - b1, b2, 1 - b2, lr, eps,
// 1/(1 - b1^t), 1/(1 - b2^t).
struct AdamCoef {
  float lr, b1, omb1, b2, omb2, eps, inv_bc1, inv_bc2;
};
// Outputs of the next view's preprocess when it is fused into the preprocess backward (the
// arrays of gs_proj, typed).
struct NextOut {
  float4* splat;
  uint32_t* tiles;
  uint32_t* dkey;
  uint2* rect;
};
hipError_t launch_preprocess_backward(const PrebwdArgs& a, const CamK& cam, hipStream_t s,
                                      const CamK* next_cam = nullptr, const NextOut* next = nullptr);

// binning / sorting
struct BinLayout {
  size_t info, partials, dkA, dvA, dkB, dvB, counts, totals, rect, bsum, tkA, tvA, tkB, tvB;
  size_t total;
  int64_t nblk_n, nblk_k, nblk_rect;
};
BinLayout bin_layout(int64_t n, int64_t kcap, int32_t W, int32_t H);
// What the count leaves at the start of the sort workspace; every later sort kernel reads it.
struct BinInfo {
  unsigned long long K;     // intersections
  unsigned long long kcap;  // the capacity of the call
  uint32_t dmin, dmax;      // depth-key range of the visible Gaussians
  uint32_t over;            // K > kcap: nothing is sorted
  uint32_t pad;
};
// The whole binning and sort, enqueued without waiting: K and the depth range stay on the device.
// On overflow (K > kcap) vals and keys are not written, and ranges are cleared to empty unless
// keep_ranges_on_overflow.
hipError_t launch_bin_sort(int64_t n, int64_t kcap, const CamK& cam, gs_proj proj, char* ws, const BinLayout& L,
                           uint32_t* vals, uint32_t* ranges, uint64_t* keys, bool keep_ranges_on_overflow,
                           hipStream_t s);

// blending
//
// Render workspace.  The forward leaves in it what the backward needs to walk long tile lists
// back in parallel segments: a tile list longer than one segment (512 entries, or a larger
// power of two when the workspace is short) gets one state slot per segment boundary plus one
// for its final state; a slot holds (T, C_r, C_g, C_b) for the tile's 256 pixels.  The
// backward gathers each list entry's nine gradient sums in `staging`, grouped by Gaussian
// (Gaussian i's entries at goff(i) .. goff(i) + tiles_i, in the row-major order of its tile
// rect), and then sums each Gaussian's entries into grad2d: no float atomics in memory.
//   hdr[64]         header words (kHdr* below)
//   bnd_off[T + 1]  first slot of each tile
//   item_off[T + 1] first work item of each tile
//   order[T]        the forward's tile order: list-length classes (log2), longest first
//   plan_part[], plan_off[]  the segment plan's per-block partial sums and offsets
//   goff[n]         exclusive scan of tiles within blocks of kGoffBlock Gaussians; goff(i) =
//                   goff_blk[i / kGoffBlock] + goff[i]
//   goff_blk[]      exclusive scan of the block totals
//   items[]         (tile, segment) work items of the backward: tile-major after the forward; in
//                   the fused step, in the order the tiles' forwards completed
//   slots[][256]    float4 states
//   masks[][256]    per 64-entry chunk of a tile list and pixel of the tile: the chunk's
//                   entries the forward composited at that pixel (64-bit, as uint2 lo, hi);
//                   tile t's chunk j is at (ranges[t].x / 64 + t + j)
//   loss_part[T]    the fused step's per-tile sums of |image - target|
//   staging[][9]    per-entry gradient sums
// The forward of the longest lists (at least 2^(shift + kSplitLog) entries) is split: their
// first 2^(shift + kPhase1Log) entries are walked as any other list, and the pixels still going
// there walk the rest in forward segments of F = 2^fshift entries in parallel, each from T = 1,
// combined in list order per pixel:
//   fbase[T]        a split tile's first forward segment (low 27 bits) and fshift (high 5 bits),
//                   kNoSplit for the other tiles
//   split_tile[]    the split tiles (longest list classes first)
//   split_cnt[][4]  per split tile: first part walked, forward segments walked, combine done
//   fitems[]        (split tile index, segment) of every forward segment
//   fsum[][256]     per forward segment and pixel: (P, C_r, C_g, C_b) of the walk from T = 1
//   fstat[][256]    per forward segment and pixel: first and last composited position, composited
//                   count (bit 31: the walk stopped), evaluated count
//   fin[][256]      per forward segment and pixel: (T, C) in front of the segment
//   pstate[][256]   per split tile and pixel: (stop segment or a marker, last, composited,
//                   evaluated in front)
constexpr int kSegShiftMin = 9;  // 512 list entries per segment
constexpr int kFsegLog = 2;      // the shortest forward segment is 2^kFsegLog backward segments
constexpr int kSplitLog = 7;     // lists of at least 2^(shift + kSplitLog) entries are split
constexpr int kPhase1Log = 4;    // ... after a first part of 2^(shift + kPhase1Log) entries walked whole
constexpr uint32_t kMaxSplit = 1024;  // split tiles at most (one workgroup plans them)
constexpr uint32_t kNoSplit = 0xFFFFFFFFu;
constexpr uint32_t kFbaseMask = (1u << 27) - 1u;
// header words of the render workspace
constexpr int kHdrShift = 0;    // log2 segment length
constexpr int kHdrItems = 1;    // backward work items
constexpr int kHdrSlots = 2;    // state slots used
constexpr int kHdrBwdNext = 3;  // next backward work item (counter)
constexpr int kHdrEntries = 4;  // staged entries (sum of tiles)
constexpr int kHdrFwdNext = 5;  // next tile of the forward (counter)
constexpr int kHdrReady = 6;    // fused step: work items published so far
constexpr int kHdrRole = 7;     // fused step: workgroups started so far
constexpr int kHdrFlags = 8;    // status bits (kFlag* below): set by the kernels, kept until read
constexpr int kHdrNeed = 9;     // the most intersections lists needed (largest list end, or staged entries)
constexpr int kHdrSplit = 10;   // split tiles
constexpr int kHdrFsegs = 11;   // their forward segments
constexpr int kHdrLongNext = 12;  // next work item of the split tiles' forward (counter)
constexpr int kHdrStatusWords = 16;  // header words gs_render_init clears
constexpr uint32_t kFlagStall = 1u;     // fused step: a workgroup gave up waiting for a work item
constexpr uint32_t kFlagCapacity = 2u;  // the lists need more intersections than the workspace holds
constexpr int kGoffBlock = 4096;
struct RenderWs {
  uint32_t* hdr;
  uint32_t* bnd_off;
  uint32_t* item_off;
  uint32_t* order;
  uint32_t* plan_part;  // the segment plan's per-block sums and offsets (blocks of 1024 tiles)
  uint32_t* plan_off;
  uint32_t* goff;
  uint32_t* goff_blk;
  uint2* items;
  float4* slots;
  uint2* masks;
  float* loss_part;
  float* staging;
  uint32_t* fbase;
  uint32_t* split_tile;
  uint32_t* split_cnt;
  uint2* fitems;
  float4* fsum;
  uint4* fstat;
  float4* fin;
  uint4* pstate;
  uint32_t slots_cap;
  uint64_t mask_cap;     // chunks
  uint64_t staging_cap;  // entries
  uint32_t fseg_cap;     // forward segments
  uint32_t split_cap;    // split tiles
};
size_t render_ws_bytes(int T, int64_t n, int64_t k_capacity);
// Carves ws (bytes long) into the regions above; only the alignment of ws is read, so a
// placeholder address serves for capacity queries.
bool render_ws_layout(void* ws, size_t bytes, int T, int64_t n, RenderWs* out);

hipError_t launch_blend_forward(const CamK& cam, int64_t n, const gs_splat* splat, const uint32_t* vals,
                                const uint32_t* ranges, float bg0, float bg1, float bg2,
                                float* image, float* T_final, uint32_t* last_contrib,
                                uint32_t* n_examined, uint64_t* blend_count, const RenderWs& ws,
                                hipStream_t s);
hipError_t launch_blend_backward(const CamK& cam, int64_t n, const gs_splat* splat, const uint32_t* tiles,
                                 const uint32_t* vals, const uint32_t* ranges, float bg0,
                                 float bg1, float bg2, const float* T_final,
                                 const uint32_t* last_contrib, const float* dLdI, float* grad2d,
                                 const RenderWs& ws, hipStream_t s);

// elementwise
hipError_t launch_fill_u32(uint32_t* p, int64_t count, uint32_t value, hipStream_t s);
hipError_t launch_fill_f32(float* p, int64_t count, float value, hipStream_t s);
size_t loss_workspace_bytes(int64_t count);
// The fused step's preparation: segment plan, tile order, empty item list, staging offsets and
// cleared staging rows.
hipError_t launch_step_plan(const CamK& cam, int64_t n, const uint32_t* tiles, const uint32_t* ranges,
                            const RenderWs& ws, hipStream_t s);
// Fused forward, L1 loss and backward blend of one training step (after launch_step_plan);
// leaves the per-intersection gradient sums staged in ws for the preprocess backward.
hipError_t launch_blend_step(const CamK& cam, int64_t n, const gs_splat* splat, const uint32_t* tiles,
                             const uint32_t* vals, const uint32_t* ranges, float bg0, float bg1, float bg2,
                             const float* target, float* image, float* T_final, uint32_t* last_contrib,
                             uint32_t* n_examined, uint64_t* blend_count, float* loss, float* dLdI,
                             float* grad2d, const RenderWs& ws, hipStream_t s);
// *loss = inv_n * sum of part[0 .. count)
hipError_t launch_loss_sum(int64_t count, const float* part, double inv_n, float* loss, hipStream_t s);
hipError_t launch_loss_l1(int64_t count, const float* image, const float* target, float* loss,
                          float* dLdI, void* ws, hipStream_t s);
// L1 + D-SSIM loss (ssim.hip): workspace bytes for a W x H image (W, H >= 11), and the launch
// writing loss[0..2] = (L, mean L1, mean SSIM) and dL/dimage.
size_t ssim_workspace_bytes(int W, int H);
hipError_t launch_loss_l1_dssim(int W, int H, const float* image, const float* target, float lambda,
                                float* loss, float* dLdI, void* ws, hipStream_t s);
// Adaptive density control (densify.hip).
hipError_t launch_densify_stats(int64_t n, const gs_splat* splat, const uint32_t* tiles, const RenderWs& ws,
                                float half_w, float half_h, float* grad_acc, float* count, hipStream_t s);
struct DensifyLaunch {
  int64_t n, ld, ld_out;
  int R;
  const float* params;
  const float* m;
  const float* v;
  const float* grad_acc;
  const float* count;
  const float* z;
  float t_grad, t_lscale, t_logit, log_split;  // float32 thresholds formed in double
  float* params_out;
  float* m_out;
  float* v_out;
  int32_t* codes;
  void* ws;
};
size_t densify_workspace_bytes(int64_t n);
// Classifies and counts (then synchronises s to read the three totals into totals_host); writes
// the output only when it fits ld_out.
hipError_t launch_densify(const DensifyLaunch& d, uint32_t totals_host[3], hipStream_t s);
hipError_t launch_adam(int64_t count, float* params, const float* grads, float* m, float* v,
                       const AdamCoef& c, hipStream_t s);

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The C ABI's error reporting (capi.hip): sets the calling thread's message and returns `code`;
// ok_status() clears it and returns GS_OK; hip_status() reports a failed HIP call.
int fail_status(int code, const char* fmt, ...);
int ok_status();
int hip_status(hipError_t e, const char* where);

}  // namespace gsmi
