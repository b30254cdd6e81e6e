// Forward and backward alpha blending over 16x16 tiles, for gfx950.
//
// What is computed ("Scaling 3D Gaussian Splatting with Distributed Compute", walkthrough step
// "Rasterize locally" and the trace section's 8x8-tile rasterizer; tile size 16 here): for
// each pixel, its tile's depth-sorted list front to back,
//   power = -(A dx^2 + C dy^2)/2 - B dx dy,  skip if power > 0,
//   alpha = min(0.99, o e^power),            skip if alpha < 1/255,
//   stop (without blending) when T (1 - alpha) < 1e-4, else C += c alpha T, T *= 1 - alpha;
// and the exact derivative of that branch in reverse order (gradients to the 2D mean, conic,
// opacity and colour, "Gradients flow back ... to mu, Sigma, c and alpha").
//
// Work decomposition.  Each 8x8 quadrant of a tile is one wave64 (one pixel per lane); the
// four quadrant waves of a tile share a workgroup.  A tile's list is consumed in chunks of 64
// records.  For every record the conservative pixel box of its alpha >= 1/255 ellipse is
// formed, and sixteen ballots (one per quadrant column and row) give every lane a 64-bit mask
// of the chunk's records whose box holds its pixel.  Each lane then walks only its own records,
// in list order, so lanes evaluate different records at the same time: a record costs VALU
// work only on the pixels it can reach, and the per-pixel results are those of the plain walk
// (a skipped record has alpha < 1/255 at that pixel).  The forward's quadrant waves are
// independent (no workgroup barrier).  The forward also leaves, per pixel and chunk, the 64-bit
// mask of the chunk's entries it composited; the backward walks exactly those entries (per
// 4x4 pixel block of 16 lanes, whose sums are formed with DPP), so no record is tested twice.
// The backward's waves share per-entry gradient sums in LDS.
// Workgroup b renders tile b: the hardware deals consecutive workgroups to the 8 XCDs in turn,
// which spreads the (very uneven) per-tile work evenly over them.  Bound: VALU /
// transcendental and LDS, not HBM.
#include <algorithm>

#include "gsmi_internal.h"

namespace gsmi {

namespace {

constexpr float kAlphaMin = 1.0f / 255.0f;
constexpr float kAlphaMax = 0.99f;
constexpr float kTMin = 1e-4f;

// power = nA dx^2 + nC dy^2 + nB dx dy with (nA, nB, nC) = (-A/2, -B, -C/2); the rounding
// steps are spelled out so the forward and backward kernels evaluate bit-identical values.
__device__ __forceinline__ float eval_power(float nA, float nB, float nC, float dx, float dy) {
  const float dx2 = __fmul_rn(dx, dx), dy2 = __fmul_rn(dy, dy), dxy = __fmul_rn(dx, dy);
  return __fmaf_rn(nA, dx2, __fmaf_rn(nC, dy2, __fmul_rn(nB, dxy)));
}

__device__ __forceinline__ float eval_oG(float o, float power) { return __fmul_rn(o, __expf(power)); }

// One DPP step x op= permute(x) within each row of 16 lanes (every source lane is active, so
// the move folds into the DPP form of the add / or).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_or(uint32_t x) {
  return x | (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// OR of a 64-bit value over each row of 16 lanes: over each quad (quad_perm [1,0,3,2], then
// [2,3,0,1]), then each quad with its mirror in the row's half (row_half_mirror) and each half
// with the other (row_mirror).  Every lane must be active; every lane gets its row's OR.
__device__ __forceinline__ unsigned long long row_or(unsigned long long m) {
  uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
  lo = dpp_or<0xB1>(lo);
  hi = dpp_or<0xB1>(hi);
  lo = dpp_or<0x4E>(lo);
  hi = dpp_or<0x4E>(hi);
  lo = dpp_or<0x141>(lo);
  hi = dpp_or<0x141>(hi);
  lo = dpp_or<0x140>(lo);
  hi = dpp_or<0x140>(hi);
  return ((unsigned long long)hi << 32) | lo;
}

// Sums of nine values over each row of 16 lanes, spread over the row (a reduce-scatter): lane r
// of the row ends with the row's sum of v[4 b3 + 2 b2 + b1] (b the bits of r) and *s8 with the
// row's sum of v[8].  Four exchanges, each pairing lane r with r ^ 15 (row_mirror), r ^ 7
// (row_half_mirror), r ^ 2 and r ^ 1 (quad_perm): partners differ in bit 3, then bit 2, 1, 0,
// and agree on the bits already used.  At the first three each lane keeps the half of its values
// that its bit selects and adds its partner's copy of that half, so the partner's copy of the
// other half is added there; v[8] and the last step are summed whole.  27 VALU operations
// against 36 for summing all nine whole.  Every lane must be active.
__device__ __forceinline__ float row_scatter9(const float* v, int lane, float* s8) {
  const bool b3 = (lane & 8) != 0, b2 = (lane & 4) != 0, b1 = (lane & 2) != 0;
  float r[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = (b3 ? v[k + 4] : v[k]) + dpp_mov<0x140>(b3 ? v[k] : v[k + 4]);
  float r8 = dpp_add<0x140>(v[8]);
  float s[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) s[k] = (b2 ? r[k + 2] : r[k]) + dpp_mov<0x141>(b2 ? r[k] : r[k + 2]);
  r8 = dpp_add<0x141>(r8);
  const float t = (b1 ? s[1] : s[0]) + dpp_mov<0x4E>(b1 ? s[0] : s[1]);
  r8 = dpp_add<0x4E>(r8);
  *s8 = dpp_add<0xB1>(r8);
  return dpp_add<0xB1>(t);
}

constexpr int kChunk = 64;  // records staged per chunk (one per lane)
constexpr int kWin = kBlock;  // list entries whose gradient sums a workgroup gathers before adding them to grad2d

// Conservative pixel-index box [x0,x1] x [y0,y1] (relative to the quadrant origin, clamped to
// 0..7) of the pixels whose centres can satisfy o e^power >= 1/255.  That region is the ellipse
// d^T Q d <= tau, tau = 2 ln(255 o), with half-widths sqrt(tau C/det), sqrt(tau A/det); tau and
// the box are widened so float32 rounding of the per-pixel test can never fall outside.  Empty
// (x0 > x1) when o < 1/255 or the box misses the quadrant.
struct Box {
  int x0, x1, y0, y1;
};

__device__ __forceinline__ Box alpha_box(float u, float v, float A, float B, float C, float o, int xq,
                                         int yq) {
  Box b{1, 0, 1, 0};
  if (!(o >= kAlphaMin)) return b;
  const float det = A * C - B * B;
  float hx = 1e30f, hy = 1e30f;
  if (det > 0.0f && __builtin_isfinite(det)) {
    // the hardware log2, reciprocal and square root (errors of a few ulp, far inside the
    // widening); 255 o >= 1 here, and a huge or infinite half-width only widens the box
    const float tau = 1.38629436f * __builtin_amdgcn_logf(255.0f * o) * 1.001f + 1e-3f;  // 2 ln(255 o)
    const float rdet = __builtin_amdgcn_rcpf(det);
    hx = __builtin_amdgcn_sqrtf(tau * C * rdet) * 1.001f + 0.01f;
    hy = __builtin_amdgcn_sqrtf(tau * A * rdet) * 1.001f + 0.01f;
  }
  // pixel index p has its centre at p + 0.5: p in [u - hx - 0.5, u + hx - 0.5]
  const float fx0 = ceilf(u - hx - 0.5f - (float)xq), fx1 = floorf(u + hx - 0.5f - (float)xq);
  const float fy0 = ceilf(v - hy - 0.5f - (float)yq), fy1 = floorf(v + hy - 0.5f - (float)yq);
  if (!(fx0 <= 7.0f && fx1 >= 0.0f && fy0 <= 7.0f && fy1 >= 0.0f)) return b;  // also NaN
  b.x0 = fx0 < 0.0f ? 0 : (int)fx0;
  b.x1 = fx1 > 7.0f ? 7 : (int)fx1;
  b.y0 = fy0 < 0.0f ? 0 : (int)fy0;
  b.y1 = fy1 > 7.0f ? 7 : (int)fy1;
  return b;
}

// Per-lane masks: bit e set iff record e's box contains the lane's pixel (lx, ly).  Lane e
// holds record e's box as 16 coverage bits (columns x0..x1 in bits 0..7, rows y0..y1 in bits
// 8..15); ballot k over the records is column k's (k < 8) or row k - 8's mask.  The sixteen
// ballots are kept in lanes 0..15 of two registers (low and high halves), from which each lane
// fetches its column's and its row's mask (ds_bpermute, no LDS memory).
__device__ __forceinline__ unsigned long long lane_mask(const Box& b, int lane, int lx, int ly) {
  const uint32_t cov = b.x0 <= b.x1 ? ((2u << b.x1) - (1u << b.x0)) | (((2u << b.y1) - (1u << b.y0)) << 8) : 0u;
  int lo = 0, hi = 0;
  int ln = lane;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    // (an opaque copy of the lane index: the sixteen lane == k tests are formed here instead
    // of being held in 32 scalar registers across the walk, which spills)
    asm volatile("" : "+v"(ln));
    const unsigned long long m = __builtin_amdgcn_ballot_w64(((cov >> k) & 1u) != 0u);
    lo = ln == k ? (int)(uint32_t)m : lo;
    hi = ln == k ? (int)(uint32_t)(m >> 32) : hi;
  }
  const int ac = lx << 2, ar = (8 + ly) << 2;  // byte addresses of lanes lx and 8 + ly
  const uint32_t clo = (uint32_t)__builtin_amdgcn_ds_bpermute(ac, lo), chi = (uint32_t)__builtin_amdgcn_ds_bpermute(ac, hi);
  const uint32_t rlo = (uint32_t)__builtin_amdgcn_ds_bpermute(ar, lo), rhi = (uint32_t)__builtin_amdgcn_ds_bpermute(ar, hi);
  return ((unsigned long long)(chi & rhi) << 32) | (clo & rlo);
}

// One chunk of records in LDS, indexed by slot (read per lane).
struct Chunk {
  float4 geo[kChunk];   // u, v, -A/2, -B
  float4 col[kChunk];   // -C/2, o, r, g
  float b[kChunk];
};

// The fields of a record that the blend uses (zeros past the end of a list).  Only these are
// loaded: a loaded-but-unused register gets reused while its load is in flight, which forces
// a wait for every outstanding load.
struct Raw {
  float2 uv;
  float4 abco;  // conic A, B, C, opacity
  float3 rgb;
  uint32_t gid;
};

// Loads are unconditional (the index is clamped into the list and the result masked), so every
// pass of a chunk loop issues the same memory operations and the compiler can wait for exactly
// the load it needs instead of for all outstanding ones.
//   vals[j] for j < end, else 0xFFFFFFFF; `safe` is any index inside the list
__device__ __forceinline__ uint32_t load_gid(const uint32_t* __restrict__ vals, uint32_t j, uint32_t end,
                                             uint32_t safe) {
  const uint32_t v = vals[j < end ? j : safe];
  return j < end ? v : 0xFFFFFFFFu;
}

// The record of Gaussian gid, or of Gaussian 0 for gid >= n (past the end of a list); callers
// give such a record opacity 0 (an empty box) where they use it.  The loaded registers are left
// untouched here: overwriting a load's destination before it lands would force a wait for
// every outstanding load.  Requires n >= 1.
__device__ __forceinline__ Raw load_raw(const float4* __restrict__ splat, uint32_t gid, int64_t n) {
  const float* rec = reinterpret_cast<const float*>(splat + 3 * ((int64_t)gid < n ? (int64_t)gid : 0));
  Raw r;
  r.gid = gid;
  r.uv = *reinterpret_cast<const float2*>(rec);
  r.abco = *reinterpret_cast<const float4*>(rec + 4);
  r.rgb = *reinterpret_cast<const float3*>(rec + 8);
  return r;
}

// opacity of a loaded record as the blend sees it (0 past the end of a list)
__device__ __forceinline__ float opacity_of(const Raw& r, int64_t n) {
  return (int64_t)r.gid < n ? r.abco.w : 0.f;
}

// Makes the compiler wait here for the loads of r (an empty asm statement that reads them), so a
// chunk loop entered with r still in flight does not carry that wait into every pass.
__device__ __forceinline__ void settle(const Raw& r) {
  asm volatile("" ::"v"(r.uv.x), "v"(r.uv.y), "v"(r.abco.x), "v"(r.abco.y), "v"(r.abco.z), "v"(r.abco.w),
               "v"(r.rgb.x), "v"(r.rgb.y), "v"(r.rgb.z));
}

__device__ __forceinline__ void put(Chunk& S, int e, const Raw& r) {
  S.geo[e] = make_float4(r.uv.x, r.uv.y, -0.5f * r.abco.x, -r.abco.y);
  S.col[e] = make_float4(-0.5f * r.abco.z, r.abco.w, r.rgb.x, r.rgb.y);
  S.b[e] = r.rgb.z;
}

// Makes a wave's LDS writes visible to its own later reads.
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int lowest_bit(unsigned long long m) { return __builtin_ctzll(m); }
__device__ __forceinline__ int highest_bit(unsigned long long m) { return 63 - __builtin_clzll(m); }

// Inside the fused step (k_blend_step) one workgroup hands data to another: a tile's per-pixel
// state, its composited masks and its work items.  Those accesses are relaxed atomics at device
// scope, which bypass the per-XCD L2s (they are not coherent with one another), so no cache-wide
// write-back or invalidate is needed.  Everywhere else (kDev false) they are plain accesses.
template <bool kDev>
__device__ __forceinline__ void put_u2(uint2* p, uint2 v) {
  if constexpr (kDev)
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), (uint64_t)v.x | ((uint64_t)v.y << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}
template <bool kDev>
__device__ __forceinline__ uint2 get_u2(const uint2* p) {
  if constexpr (kDev) {
    const uint64_t x = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_uint2((uint32_t)x, (uint32_t)(x >> 32));
  } else {
    return *p;
  }
}
template <bool kDev>
__device__ __forceinline__ void put_f4(float4* p, float4 v) {
  uint2* q = reinterpret_cast<uint2*>(p);
  put_u2<kDev>(q, make_uint2(__float_as_uint(v.x), __float_as_uint(v.y)));
  put_u2<kDev>(q + 1, make_uint2(__float_as_uint(v.z), __float_as_uint(v.w)));
}
template <bool kDev>
__device__ __forceinline__ float4 get_f4(const float4* p) {
  if constexpr (kDev) {
    const uint2* q = reinterpret_cast<const uint2*>(p);
    const uint2 a = get_u2<true>(q), b = get_u2<true>(q + 1);
    return make_float4(__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(b.x), __uint_as_float(b.y));
  } else {
    return *p;
  }
}
template <bool kDev>
__device__ __forceinline__ void put_u4(uint4* p, uint4 v) {
  uint2* q = reinterpret_cast<uint2*>(p);
  put_u2<kDev>(q, make_uint2(v.x, v.y));
  put_u2<kDev>(q + 1, make_uint2(v.z, v.w));
}
template <bool kDev>
__device__ __forceinline__ uint4 get_u4(const uint4* p) {
  const uint2* q = reinterpret_cast<const uint2*>(p);
  const uint2 a = get_u2<kDev>(q), b = get_u2<kDev>(q + 1);
  return make_uint4(a.x, a.y, b.x, b.y);
}
template <bool kDev, typename T>
__device__ __forceinline__ void put_32(T* p, T v) {
  if constexpr (kDev)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}
template <bool kDev, typename T>
__device__ __forceinline__ T get_32(const T* p) {
  if constexpr (kDev)
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}
// Waits until every memory access this wave has issued has completed: its device-scope stores
// are then visible to every XCD.
__device__ __forceinline__ void drain_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------------------------------------
// Segment plan.  For every tile, its list length len decides
//   items(t) = ceil(len / SEG) backward work items (0 for an empty tile),
//   slots(t) = ceil(len / SEG) state slots if len > SEG (one per boundary + the final state),
// SEG = 2^shift is the smallest power of two >= 2^kSegShiftMin whose slots fit the workspace.
// The forward's tile order groups the tiles by list-length class (1 + floor(log2 len), 0 for
// an empty list), longest first.  Three kernels over blocks of 1024 tiles: per-block sums for
// every candidate shift and class counts; one workgroup picks the shift and turns the sums
// into per-block offsets; then every tile writes bnd_off (exclusive scan of slots), item_off
// and its place in the order.
// ---------------------------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;
// list-length classes: 0 for an empty list, else 1 + floor(log2 len)
constexpr int kLenClasses = 33;
__device__ __forceinline__ int len_class(uint32_t len) { return len ? 32 - __clz((int)len) : 0; }
constexpr int kShifts = 32 - kSegShiftMin;  // candidate shifts kSegShiftMin .. 31
// per-block partial sums: slots(shift), long tiles(shift), non-empty tiles, class counts, and the
// largest list end (a maximum, not a sum)
constexpr int kPartSlots = 0, kPartLong = kShifts, kPartNonEmpty = 2 * kShifts, kPartClass = 2 * kShifts + 1;
constexpr int kPartMaxEnd = kPartClass + kLenClasses;
constexpr int kPartVals = kPartMaxEnd + 1;
// per-block offsets: slots, items, then each class's first position in the order
constexpr int kOffVals = 2 + kLenClasses;

// exclusive scan over the 1024 threads
__device__ uint32_t block_exscan_1024(uint32_t x, uint32_t* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t inc = x;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) red[w] = inc;
  __syncthreads();
  uint32_t base = 0;
  for (int k = 0; k < w; ++k) base += red[k];
  __syncthreads();
  return base + inc - x;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__global__ __launch_bounds__(kPlanThreads) void k_plan_count(const uint2* __restrict__ ranges, int T,
                                                             uint32_t* __restrict__ part) {
  __shared__ uint32_t red[kPlanThreads / 64][2 * kShifts + 1];
  __shared__ uint32_t cls[kLenClasses];
  __shared__ uint32_t emax[kPlanThreads / 64];
  const int t = (int)(blockIdx.x * kPlanThreads + threadIdx.x), w = threadIdx.x >> 6;
  uint32_t len = 0, end = 0;
  if (t < T) {
    const uint2 rg = ranges[t];
    len = rg.y - rg.x;
    end = rg.y;
  }
  for (int o = 32; o > 0; o >>= 1) end = max(end, (uint32_t)__shfl_xor(end, o, 64));
  if ((threadIdx.x & 63) == 0) emax[w] = end;
  if (threadIdx.x < kLenClasses) cls[threadIdx.x] = 0u;
  __syncthreads();
  if (t < T) atomicAdd(&cls[len_class(len)], 1u);
  uint32_t mlen = len;  // the wave's longest list: no list is longer than 2^shift past it
  for (int o = 32; o > 0; o >>= 1) mlen = max(mlen, (uint32_t)__shfl_xor(mlen, o, 64));
  for (int q = 0; q < kShifts; ++q) {
    const int sh = kSegShiftMin + q;
    uint32_t sl = 0, nl = 0;
    if (mlen > (1u << sh)) {  // (wave-uniform)
      const bool lg = len > (1u << sh);
      sl = wave_sum(lg ? ((len - 1u) >> sh) + 1u : 0u);
      nl = wave_sum(lg ? 1u : 0u);
    }
    if ((threadIdx.x & 63) == 0) {
      red[w][kPartSlots + q] = sl;
      red[w][kPartLong + q] = nl;
    }
  }
  const uint32_t ne = wave_sum(len > 0u ? 1u : 0u);
  if ((threadIdx.x & 63) == 0) red[w][kPartNonEmpty] = ne;
  __syncthreads();
  uint32_t* out = part + (size_t)blockIdx.x * kPartVals;
  if (threadIdx.x < 2 * kShifts + 1) {
    uint32_t v = 0;
    for (int k = 0; k < kPlanThreads / 64; ++k) v += red[k][threadIdx.x];
    out[threadIdx.x] = v;
  } else if (threadIdx.x < kPartMaxEnd) {
    out[threadIdx.x] = cls[threadIdx.x - kPartClass];
  } else if (threadIdx.x == kPartMaxEnd) {
    uint32_t v = 0;
    for (int k = 0; k < kPlanThreads / 64; ++k) v = max(v, emax[k]);
    out[threadIdx.x] = v;
  }
}

// One workgroup: the shift, the header, bnd_off[T] / item_off[T] and the per-block offsets.
// The lists need room for their largest end: a workspace that holds fewer intersections sets the
// capacity flag (the kernels then stay inside the workspace and the results are not valid).  The
// status words are not cleared here: they gather the flags of every call until read.
__global__ __launch_bounds__(kPlanThreads) void k_plan_scan(const uint32_t* __restrict__ part, int nb, int T,
                                                            uint32_t slots_cap, uint64_t entries_cap,
                                                            uint32_t* __restrict__ off,
                                                            uint32_t* __restrict__ hdr,
                                                            uint32_t* __restrict__ bnd_off,
                                                            uint32_t* __restrict__ item_off) {
  __shared__ uint32_t tot[kPartVals];
  __shared__ uint32_t cbase[kLenClasses];
  __shared__ int s_q;
  if (threadIdx.x < kPartMaxEnd) {
    uint32_t v = 0;
    for (int b = 0; b < nb; ++b) v += part[(size_t)b * kPartVals + threadIdx.x];
    tot[threadIdx.x] = v;
  } else if (threadIdx.x == kPartMaxEnd) {
    uint32_t v = 0;
    for (int b = 0; b < nb; ++b) v = max(v, part[(size_t)b * kPartVals + threadIdx.x]);
    tot[threadIdx.x] = v;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int q = 0;  // the first shift whose slots fit (the last one if none does)
    while (q < kShifts - 1 && tot[kPartSlots + q] > slots_cap) ++q;
    s_q = q;
    uint32_t run = 0;  // classes longest first
    for (int c = kLenClasses - 1; c >= 0; --c) {
      cbase[c] = run;
      run += tot[kPartClass + c];
    }
    const uint32_t slots = tot[kPartSlots + q];
    const uint32_t items = slots + tot[kPartNonEmpty] - tot[kPartLong + q];
    bnd_off[T] = slots;
    item_off[T] = items;
    hdr[kHdrShift] = (uint32_t)(kSegShiftMin + q);
    hdr[kHdrItems] = items;
    hdr[kHdrSlots] = slots;
    hdr[kHdrBwdNext] = 0u;
    hdr[kHdrFwdNext] = 0u;
    hdr[kHdrReady] = 0u;
    hdr[kHdrRole] = 0u;
    if ((uint64_t)tot[kPartMaxEnd] > entries_cap) {
      hdr[kHdrFlags] |= kFlagCapacity;
      hdr[kHdrNeed] = max(hdr[kHdrNeed], tot[kPartMaxEnd]);
    }
  }
  __syncthreads();
  const int q = s_q;
  if (threadIdx.x == 0) {  // slot and item offsets of the blocks
    uint32_t rs = 0, ri = 0;
    for (int b = 0; b < nb; ++b) {
      const uint32_t* pb = part + (size_t)b * kPartVals;
      off[(size_t)b * kOffVals + 0] = rs;
      off[(size_t)b * kOffVals + 1] = ri;
      rs += pb[kPartSlots + q];
      ri += pb[kPartSlots + q] + pb[kPartNonEmpty] - pb[kPartLong + q];
    }
  } else if (threadIdx.x <= kLenClasses) {  // each class's offsets of the blocks
    const int c = threadIdx.x - 1;
    uint32_t r = cbase[c];
    for (int b = 0; b < nb; ++b) {
      off[(size_t)b * kOffVals + 2 + c] = r;
      r += part[(size_t)b * kPartVals + kPartClass + c];
    }
  }
}

__global__ __launch_bounds__(kPlanThreads) void k_plan_write(const uint2* __restrict__ ranges, int T,
                                                             const uint32_t* __restrict__ off,
                                                             const uint32_t* __restrict__ hdr,
                                                             uint32_t* __restrict__ bnd_off,
                                                             uint32_t* __restrict__ item_off,
                                                             uint32_t* __restrict__ order,
                                                             uint32_t* __restrict__ fbase) {
  __shared__ uint32_t red32[kPlanThreads / 64];
  __shared__ uint32_t cur[kLenClasses];
  const int t = (int)(blockIdx.x * kPlanThreads + threadIdx.x);
  const uint32_t* ob = off + (size_t)blockIdx.x * kOffVals;
  if (threadIdx.x < kLenClasses) cur[threadIdx.x] = ob[2 + threadIdx.x];
  uint32_t len = 0;
  if (t < T) {
    const uint2 rg = ranges[t];
    len = rg.y - rg.x;
  }
  const uint32_t shift = hdr[kHdrShift];
  const uint32_t k = len ? ((len - 1u) >> shift) + 1u : 0u;
  const uint32_t sl = len > (1u << shift) ? k : 0u;
  const uint32_t pre_s = block_exscan_1024(sl, red32);  // (its barriers also publish cur)
  const uint32_t pre_i = block_exscan_1024(k, red32);
  if (t < T) {
    bnd_off[t] = ob[0] + pre_s;
    item_off[t] = ob[1] + pre_i;
    order[atomicAdd(&cur[len_class(len)], 1u)] = (uint32_t)t;
    fbase[t] = kNoSplit;  // k_split_plan marks the split tiles
  }
}

// One workgroup: the split tiles and their forward segments.  A tile is split when its list
// holds at least 2^(shift + kSplitLog) entries; its forward segments are F = 2^fshift entries,
// fshift = max(shift + kFsegLog, round(log2 sqrt(48 len))).  Such tiles lead the order
// (list-length classes, longest first); whole classes are split or not, so the choice does not
// depend on the order inside a class: a class is split only if it lies wholly in the first
// split_cap places of the order and every class up to it fits fseg_cap segments.
// A split tile's place in the order carries kOrderSplit, so the forward kernels know it from the
// word they read anyway.
constexpr uint32_t kOrderSplit = 0x80000000u;
__device__ void split_plan(const uint2* __restrict__ ranges, int T, uint32_t* __restrict__ order,
                           uint32_t* __restrict__ hdr, uint32_t* __restrict__ fbase, uint32_t* __restrict__ split_tile,
                           uint32_t* __restrict__ split_cnt, uint2* __restrict__ fitems, uint32_t fseg_cap,
                           uint32_t split_cap) {
  __shared__ uint32_t red[kPlanThreads / 64];
  __shared__ uint32_t cls[kPlanThreads];
  __shared__ uint32_t first_seg[kPlanThreads];
  __shared__ uint32_t cend[kLenClasses];  // segments of the classes up to and including c
  __shared__ uint32_t s_cut, s_nf;
  const int i = threadIdx.x;
  const uint32_t shift = hdr[kHdrShift];
  const uint64_t min_len = (uint64_t)1 << (shift + kSplitLog);
  const uint32_t window = min((uint32_t)T, min(split_cap, (uint32_t)kPlanThreads));
  uint32_t tile = 0, c = 0, nseg = 0, fshift = 0;
  if ((uint32_t)i < window) {
    tile = order[i];
    const uint2 rg = ranges[tile];
    const uint32_t len = rg.y - rg.x;
    if (len >= min_len) {
      c = (uint32_t)len_class(len);
      fshift = max(shift + (uint32_t)kFsegLog, (c - 1u + 7u) >> 1);  // c - 1 = floor(log2 len)
      nseg = ((len - 1u) >> fshift) + 1u;
    }
  }
  cls[i] = c;
  if (i < kLenClasses) cend[i] = 0xFFFFFFFFu;
  if (i == 0) {  // the class that continues past the window is not split
    uint32_t cut = 0;
    if (window < (uint32_t)T) {
      const uint2 rg = ranges[order[window]];
      if (rg.y - rg.x >= min_len) cut = (uint32_t)len_class(rg.y - rg.x);
    }
    s_cut = cut;
    s_nf = 0;
  }
  const uint32_t excl = block_exscan_1024(nseg, red);  // (its barriers publish cls, cend, s_cut)
  if (c != 0u && (i + 1 == kPlanThreads || cls[i + 1] != c)) cend[c] = excl + nseg;
  __syncthreads();
  const bool take = c != 0u && c > s_cut && cend[c] <= fseg_cap;  // a prefix of the order
  const uint32_t ns = (uint32_t)__syncthreads_count(take);
  if (take) {
    fbase[tile] = excl | (fshift << 27);
    order[i] = tile | kOrderSplit;
    split_tile[i] = tile;
#pragma unroll
    for (int q = 0; q < 4; ++q) split_cnt[4 * i + q] = 0u;
    first_seg[i] = excl;
    atomicMax(&s_nf, excl + nseg);
  }
  __syncthreads();
  const uint32_t nf = s_nf;
  // fitems[j] = (split tile, segment): the split tile is the last one whose first segment <= j
  for (uint32_t j = (uint32_t)i; j < nf; j += kPlanThreads) {
    uint32_t lo = 0, hi = ns - 1u;
    while (lo < hi) {
      const uint32_t mid = (lo + hi + 1u) >> 1;
      if (first_seg[mid] <= j) lo = mid; else hi = mid - 1u;
    }
    fitems[j] = make_uint2(lo, j - first_seg[lo]);
  }
  if (i == 0) {
    hdr[kHdrSplit] = ns;
    hdr[kHdrFsegs] = nf;
    hdr[kHdrLongNext] = 0u;
  }
}

// The item list: one wave per tile writes the tile's items (tile, 0), (tile, 1), ...; for the
// fused step (empty), the marker of a not yet published item instead.  Block 0 first plans the
// split tiles (split_plan).
constexpr uint32_t kNoTile = 0xFFFFFFFFu;
struct SplitPlanArgs {
  const uint2* ranges;
  uint32_t* order;
  uint32_t* hdr;
  uint32_t* fbase;
  uint32_t* split_tile;
  uint32_t* split_cnt;
  uint2* fitems;
  uint32_t fseg_cap, split_cap;
};
__global__ __launch_bounds__(kPlanThreads) void k_seg_items(int T, const uint32_t* __restrict__ item_off,
                                                            uint2* __restrict__ items, bool empty, SplitPlanArgs sp) {
  if (blockIdx.x == 0)
    split_plan(sp.ranges, T, sp.order, sp.hdr, sp.fbase, sp.split_tile, sp.split_cnt, sp.fitems, sp.fseg_cap,
               sp.split_cap);
  const int t = (int)(blockIdx.x * (kPlanThreads / 64) + (threadIdx.x >> 6));
  if (t >= T) return;
  const uint32_t o = item_off[t], k = item_off[t + 1] - o;
  for (uint32_t j = threadIdx.x & 63; j < k; j += 64) items[o + j] = make_uint2(empty ? kNoTile : (uint32_t)t, j);
}

// pixel index inside its tile of lane (lx, ly) of quadrant wave w
__device__ __forceinline__ int tile_pixel(int w, int lx, int ly) {
  return (((w >> 1) << 3) + ly) * kTile + ((w & 1) << 3) + lx;
}

// ---------------------------------------------------------------------------------------------
// Forward.  Besides the image, a tile whose list is longer than one segment leaves each pixel's
// (T, C) at every segment boundary it reaches and its final (T, C) in the render workspace.
// ---------------------------------------------------------------------------------------------
struct FwdArgs {
  int W, H, TX, T;
  int64_t n;
  const float4* splat;
  const uint32_t* vals;
  const uint2* ranges;
  float bg0, bg1, bg2;
  float* image;
  float* T_final;
  uint32_t* last_contrib;
  uint32_t* n_examined;             // optional
  unsigned long long* blend_count;  // optional
  const uint32_t* bnd_off;
  float4* slots;
  uint2* masks;
  uint64_t mask_cap;
  const uint32_t* order;
  const uint32_t* fbase;  // kNoSplit, or the split tile's first forward segment
  // the fused step only: the L1 loss against the target image, per pixel
  const float* target;
  float* dLdI;
  float* loss_part;  // per tile: sum over its pixels of |image - target|
  float inv_n;       // 1 / (3 W H)
};

// A pixel's state along its walk.  Positions are 1-based and relative to the tile's list.
struct WalkState {
  float Tr, c0, c1, c2;
  uint32_t first;     // first composited position (recorded only when asked for)
  uint32_t last;      // last composited position, 0 if none
  uint32_t examined;  // the stop's position; unchanged if the walk does not stop
  uint32_t blended, evaluated;
  bool done;          // takes no part in the walk
};

// A quadrant wave's walk over the entries [rs, re) of tile list [start, start + len) (rs a
// multiple of 64) for the lane's pixel, from the state in s, stopping a pixel when T would fall
// below 1e-4.  kWrite: each walked chunk's composited mask is stored (at chunk cbase + rel / 64)
// and, with long_list, the state at every segment boundary rel in [rs, re), rel > 0 (at st +
// (rel / SEG - 1) slots).  kFirst: records the first composited position.
template <bool kDev, bool kWrite, bool kFirst>
__device__ __forceinline__ void walk_entries(const FwdArgs& a, uint32_t shift, uint32_t start, uint32_t rs,
                                             uint32_t re, bool long_list, float4* st, uint64_t cbase, int pix,
                                             int xq, int yq, float pxc, float pyc, Chunk& S, WalkState& s) {
  const int64_t n = a.n;
  const float4* __restrict__ splat = a.splat;
  const uint32_t* __restrict__ vals = a.vals;
  uint2* __restrict__ masks = a.masks;
  const uint64_t mask_cap = a.mask_cap;
  const int lane = threadIdx.x & 63;
  const int lx = lane & 7, ly = lane >> 3;
  const uint32_t end = start + re;
  const uint32_t seg_mask = (1u << shift) - 1u;
  float Tr = s.Tr, c0 = s.c0, c1 = s.c1, c2 = s.c2;
  uint32_t first = s.first, last = s.last, examined = s.examined, blended = s.blended, evaluated = s.evaluated;
  bool done = s.done;

  uint32_t gnext = load_gid(vals, start + rs + lane, end, start);
  Raw cur = load_raw(splat, gnext, n);
  gnext = load_gid(vals, start + rs + kChunk + lane, end, start);
  // The first chunk has landed before the loop starts; each pass waits for the next chunk's
  // loads only at its end.  A chunk's composited mask is stored at the start of the next
  // pass, so that pass's work covers the store's latency.
  settle(cur);
  unsigned long long pend = 0ull;
  uint64_t pend_mc = ~0ull;
  for (uint32_t b0 = start + rs; b0 < end; b0 += kChunk) {
    if (__ballot(!done) == 0ull) break;
    if constexpr (kWrite) {
      if (pend_mc < mask_cap)
        put_u2<kDev>(masks + pend_mc * (kTile * kTile) + pix, make_uint2((uint32_t)pend, (uint32_t)(pend >> 32)));
    }
    const Raw nxt = load_raw(splat, gnext, n);  // next chunk in flight
    gnext = load_gid(vals, b0 + 2 * kChunk + lane, end, start);
    const uint32_t rel = b0 - start;
    if constexpr (kWrite) {
      if (long_list && rel != 0u && (rel & seg_mask) == 0u)  // state at segment boundary rel
        put_f4<kDev>(st + (size_t)((rel >> shift) - 1u) * (kTile * kTile), make_float4(Tr, c0, c1, c2));
    }
    put(S, lane, cur);
    const Box bx = alpha_box(cur.uv.x, cur.uv.y, cur.abco.x, cur.abco.y, cur.abco.z, opacity_of(cur, n), xq, yq);
    // every lane takes part in the ballots: lane e holds record e's box
    unsigned long long m = lane_mask(bx, lane, lx, ly);
    if (done) m = 0ull;
    evaluated += (uint32_t)__popcll(m);
    wave_sync_lds();
    const uint32_t base = rel + 1u;  // 1-based position of slot 0
    unsigned long long cm = 0ull;    // the chunk's entries composited at this pixel
    while (m) {  // this lane's records, in list order
      const int e = lowest_bit(m);
      m &= m - 1ull;
      const float4 g = S.geo[e];
      const float4 cl = S.col[e];
      const float bb = S.b[e];
      const float dx = pxc - g.x, dy = pyc - g.y;
      const float power = eval_power(g.z, g.w, cl.x, dx, dy);
      const float alpha = fminf(kAlphaMax, eval_oG(cl.y, power));
      if (power <= 0.0f && alpha >= kAlphaMin) {
        const float Tn = Tr * (1.0f - alpha);
        const uint32_t pos = base + (uint32_t)e;
        if (Tn < kTMin) {
          done = true;
          examined = pos;
          evaluated -= (uint32_t)__popcll(m);  // the entries behind the stop are not evaluated
          m = 0ull;
        } else {
          const float wt = alpha * Tr;
          c0 += cl.z * wt;
          c1 += cl.w * wt;
          c2 += bb * wt;
          Tr = Tn;
          if constexpr (kFirst) first = first ? first : pos;
          last = pos;
          ++blended;
          cm |= 1ull << e;
        }
      }
    }
    pend = cm;
    pend_mc = cbase + rel / kChunk;
    wave_sync_lds();  // this chunk's reads finish before the next chunk is staged
    cur = nxt;
  }
  if constexpr (kWrite) {
    if (pend_mc < mask_cap)
      put_u2<kDev>(masks + pend_mc * (kTile * kTile) + pix, make_uint2((uint32_t)pend, (uint32_t)(pend >> 32)));
  }
  s.Tr = Tr;
  s.c0 = c0;
  s.c1 = c1;
  s.c2 = c2;
  s.first = first;
  s.last = last;
  s.examined = examined;
  s.blended = blended;
  s.evaluated = evaluated;
  s.done = done;
}

// The forward's outputs at pixel p (inside the image); returns the pixel's colour.
template <bool kDev>
__device__ __forceinline__ float3 store_pixel(const FwdArgs& a, int64_t p, const WalkState& s) {
  const float i0 = s.c0 + s.Tr * a.bg0, i1 = s.c1 + s.Tr * a.bg1, i2 = s.c2 + s.Tr * a.bg2;
  a.image[3 * p + 0] = i0;
  a.image[3 * p + 1] = i1;
  a.image[3 * p + 2] = i2;
  put_32<kDev>(a.T_final + p, s.Tr);
  put_32<kDev>(a.last_contrib + p, s.last);
  if (a.n_examined) a.n_examined[p] = s.examined;
  return make_float3(i0, i1, i2);
}

// Adds the workgroup's per-pixel counts (examined, walked = last, composited, evaluated) to
// blend_count; every thread of the workgroup calls it.
__device__ void add_blend_stats(unsigned long long* bc, uint32_t examined, uint32_t last, uint32_t blended,
                                uint32_t evaluated) {
  if (!bc) return;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  unsigned long long ex = examined, lc = last, bl = blended, ev = evaluated;
  for (int o = 32; o > 0; o >>= 1) {
    ex += __shfl_xor(ex, o, 64);
    lc += __shfl_xor(lc, o, 64);
    bl += __shfl_xor(bl, o, 64);
    ev += __shfl_xor(ev, o, 64);
  }
  // one atomic per counter and workgroup: same-address atomics from every wave of the image
  // serialise and would cost more than the blending of a light view
  __shared__ unsigned long long part[4][4];
  if (lane == 0) {
    part[0][w] = ex;
    part[1][w] = lc;
    part[2][w] = bl;
    part[3][w] = ev;
  }
  __syncthreads();
  if (tid < 4) {
    const unsigned long long x = (part[tid][0] + part[tid][1]) + (part[tid][2] + part[tid][3]);
    if (x != 0ull) atomicAdd(bc + tid, x);
  }
  __syncthreads();  // part is read before a later call overwrites it
}

// L1 loss at pixel p of image colour i: dL/dI = sign(I - target) / (3 W H), sign(0) = 0;
// returns |I - target| summed over the channels.
__device__ __forceinline__ float l1_pixel(const FwdArgs& a, int64_t p, float3 i) {
  const float d0 = i.x - a.target[3 * p + 0], d1 = i.y - a.target[3 * p + 1], d2 = i.z - a.target[3 * p + 2];
  const float q = a.inv_n;
  put_32<true>(a.dLdI + 3 * p + 0, d0 > 0.f ? q : (d0 < 0.f ? -q : 0.f));
  put_32<true>(a.dLdI + 3 * p + 1, d1 > 0.f ? q : (d1 < 0.f ? -q : 0.f));
  put_32<true>(a.dLdI + 3 * p + 2, d2 > 0.f ? q : (d2 < 0.f ? -q : 0.f));
  return (fabsf(d0) + fabsf(d1)) + fabsf(d2);
}

// the tile's loss_part from each thread's pixel sum; every thread calls it
__device__ void store_loss_part(const FwdArgs& a, int tile, float l1) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  for (int o = 32; o > 0; o >>= 1) l1 += __shfl_xor(l1, o, 64);
  __shared__ float lpart[4];
  if (lane == 0) lpart[w] = l1;
  __syncthreads();
  if (tid == 0) a.loss_part[tile] = (lpart[0] + lpart[1]) + (lpart[2] + lpart[3]);
}

// One tile by the workgroup's four quadrant waves (kStep: the fused step, which also takes the
// pixel's L1 loss and gradient and hands its state to other workgroups at device scope).  A
// split tile's forward ran before (k_long_forward): the fused step takes only its loss.
template <bool kStep>
__device__ void forward_tile(const FwdArgs& a, uint32_t shift, int tile, bool split, Chunk* stg) {
  const int W = a.W, H = a.H, TX = a.TX;
  const int tx = tile % TX, ty = tile / TX;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int lx = lane & 7, ly = lane >> 3;
  const int xq = tx * kTile + (w & 1) * 8, yq = ty * kTile + (w >> 1) * 8;  // quadrant origin
  const int px = xq + lx, py = yq + ly;
  const bool inside = px < W && py < H;
  const uint2 rg = a.ranges[tile];
  const uint32_t start = rg.x, len = rg.y - rg.x;
  const bool long_list = len > (1u << shift);
  const int pix = tile_pixel(w, lx, ly);
  float4* const st = a.slots + (size_t)(long_list ? a.bnd_off[tile] : 0u) * (kTile * kTile) + pix;
  const uint64_t cbase = (uint64_t)(start / kChunk) + (uint64_t)tile;  // the tile's first mask chunk

  WalkState s{1.0f, 0.f, 0.f, 0.f, 0u, 0u, len, 0u, 0u, !inside};
  if (len > 0 && !split) {
    walk_entries<kStep, true, false>(a, shift, start, 0u, len, long_list, st, cbase, pix, xq, yq, (float)px + 0.5f,
                                     (float)py + 0.5f, stg[w], s);
    if (long_list)  // final state
      put_f4<kStep>(st + (size_t)((len - 1u) >> shift) * (kTile * kTile), make_float4(s.Tr, s.c0, s.c1, s.c2));
  }

  float l1 = 0.f;  // the pixel's sum of |image - target| (fused step)
  if (inside) {
    const int64_t p = (int64_t)py * W + px;
    const float3 i = split ? make_float3(a.image[3 * p + 0], a.image[3 * p + 1], a.image[3 * p + 2])
                           : store_pixel<kStep>(a, p, s);
    if constexpr (kStep) l1 = l1_pixel(a, p, i);
  }
  if constexpr (kStep) store_loss_part(a, tile, l1);
  add_blend_stats(a.blend_count, inside && !split ? s.examined : 0u, s.last, s.blended, s.evaluated);
}

// ---------------------------------------------------------------------------------------------
// Forward of the split tiles: the longest lists, whose one sequential walk per pixel would
// outlast the rest of the image while only a few of their pixels are still going after the first
// thousands of entries.  Four kinds of work items run in one persistent kernel before the other
// tiles' forward:
//   first (tile)     the first 2^(shift + kPhase1Log) entries, walked as any list is: a pixel that
//                    stops there is finished; the others (the survivors) go on in segments.
//   walk (tile, f)   the survivors walk forward segment f from T = 1, C = 0: their composited
//                    entries in f do not depend on the T they enter with, so the walk gives the
//                    segment's product P of (1 - alpha), its colour sum C, and the composited
//                    masks.  A pixel whose T falls below 1e-4 inside the walk certainly stops
//                    there or earlier, so the walk stops it (bit 31 of the composited count).
//   combine (tile)   per survivor, in segment order: (T, C) in front of segment f is (T_in,
//                    C_in); the pixel stops in f when the walk stopped or T_in P < 1e-4; else
//                    C_in += T_in C, T_in *= P.  A survivor that never stops is finished here.
//   redo (tile, f)   the survivors that stop in f walk it again from (T_in, C_in), exactly as
//                    the sequential walk does, which places the stop.
// A tile's segments are F = 2^fshift entries, F about sqrt(48 len): a walk costs about F / 64
// chunk steps and the combine about len / (4 F) dependent loads, so this balances the two.
// Each item waits only for items of its tile that come before it in the one counter's order
// (first, walks, combines, redos), i.e. for items that running workgroups already hold and that
// wait for nothing later.  The waits are bounded all the same (the stall flag).
// The walks' boundary states are relative to their segment's start: the backward converts
// them with fin, (T, C) = (T_in T_b, C_in + T_in C_b).  The composited masks past a pixel's
// stop are not cleared: the backward masks each pixel's bits by its last_contrib.
// ---------------------------------------------------------------------------------------------
struct LongArgs {
  const uint32_t* split_tile;
  uint32_t* split_cnt;
  const uint2* fitems;
  float4* fsum;
  uint4* fstat;
  float4* fin;
  uint4* pstate;
};

constexpr uint32_t kSpinLimit = 1u << 20;  // about a second of polling
constexpr uint32_t kPixDone = 0xFFFFFFFFu;   // pstate: finished in the first part
constexpr uint32_t kPixAlive = 0xFFFFFFFEu;  // pstate: a survivor (until the combine places its stop)

// Waits (thread 0) until *p >= v; gives up after kSpinLimit polls and flags the stall.
__device__ void wait_for(const uint32_t* p, uint32_t v, uint32_t* hdr) {
  for (uint32_t spin = 0;; ++spin) {
    if (get_32<true>(p) >= v) return;
    if (spin == kSpinLimit) {
      atomicOr(hdr + kHdrFlags, kFlagStall);
      return;
    }
    __builtin_amdgcn_s_sleep(4);
  }
}

// A split tile's geometry and its quadrant wave's pixel.
struct SplitTile {
  int tile, xq, yq, px, py, pix;
  bool inside;
  uint32_t start, len, fb, fshift, nseg, f0;
};

__device__ __forceinline__ SplitTile split_tile_of(const FwdArgs& a, const LongArgs& L, uint32_t shift, uint32_t c) {
  SplitTile t;
  t.tile = (int)L.split_tile[c];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lx = lane & 7, ly = lane >> 3;
  t.xq = (t.tile % a.TX) * kTile + (w & 1) * 8;
  t.yq = (t.tile / a.TX) * kTile + (w >> 1) * 8;
  t.px = t.xq + lx;
  t.py = t.yq + ly;
  t.pix = tile_pixel(w, lx, ly);
  t.inside = t.px < a.W && t.py < a.H;
  const uint2 rg = a.ranges[t.tile];
  t.start = rg.x;
  t.len = rg.y - rg.x;
  const uint32_t fbv = a.fbase[t.tile];
  t.fb = fbv & kFbaseMask;
  t.fshift = fbv >> 27;
  t.nseg = ((t.len - 1u) >> t.fshift) + 1u;
  t.f0 = (((1u << (shift + kPhase1Log)) - 1u) >> t.fshift) + 1u;  // segments in the first part
  return t;
}

// the forward outputs and the final state slot of a finished pixel of a split tile
__device__ __forceinline__ void finish_split_pixel(const FwdArgs& a, uint32_t shift, const SplitTile& t,
                                                   const WalkState& s) {
  store_pixel<false>(a, (int64_t)t.py * a.W + t.px, s);
  put_f4<false>(a.slots + ((size_t)a.bnd_off[t.tile] + ((t.len - 1u) >> shift)) * (kTile * kTile) + t.pix,
                make_float4(s.Tr, s.c0, s.c1, s.c2));
}

__device__ void long_first(const FwdArgs& a, const LongArgs& L, uint32_t shift, uint32_t c, Chunk* stg) {
  const SplitTile t = split_tile_of(a, L, shift, c);
  float4* const st = a.slots + (size_t)a.bnd_off[t.tile] * (kTile * kTile) + t.pix;
  const uint64_t cbase = (uint64_t)(t.start / kChunk) + (uint64_t)t.tile;
  WalkState s{1.0f, 0.f, 0.f, 0.f, 0u, 0u, 0u, 0u, 0u, !t.inside};
  walk_entries<false, true, false>(a, shift, t.start, 0u, t.f0 << t.fshift, true, st, cbase, t.pix, t.xq, t.yq,
                                   (float)t.px + 0.5f, (float)t.py + 0.5f, stg[threadIdx.x >> 6], s);
  const bool done = t.inside && s.examined != 0u;
  if (done) finish_split_pixel(a, shift, t, s);
  if (t.inside) {
    put_u4<true>(L.pstate + (size_t)c * (kTile * kTile) + t.pix,
                 make_uint4(done ? kPixDone : kPixAlive, s.last, s.blended, s.evaluated));
    if (!done) put_f4<true>(L.fin + ((size_t)t.fb + t.f0) * (kTile * kTile) + t.pix, make_float4(s.Tr, s.c0, s.c1, s.c2));
  }
  add_blend_stats(a.blend_count, done ? s.examined : 0u, done ? s.last : 0u, done ? s.blended : 0u,
                  done ? s.evaluated : 0u);
  drain_memory();
  __syncthreads();
  if (threadIdx.x == 0) put_32<true>(L.split_cnt + 4 * c, 1u);
  // A barrier between this thread-0 region and the next item's: with the two adjacent, the
  // compiler merges them into a loop that only thread 0 can leave, and the other lanes take
  // the same item again for ever.
  __syncthreads();
}

__device__ void long_walk(const FwdArgs& a, const LongArgs& L, uint32_t shift, uint2 it, Chunk* stg, uint32_t* hdr) {
  const uint32_t c = it.x, f = it.y;
  const SplitTile t = split_tile_of(a, L, shift, c);
  if (f < t.f0) return;  // (workgroup-uniform) the first part's segments
  if (threadIdx.x == 0) wait_for(L.split_cnt + 4 * c, 1u, hdr);
  __syncthreads();
  const bool alive = t.inside && get_32<true>(&L.pstate[(size_t)c * (kTile * kTile) + t.pix].x) == kPixAlive;
  if (__ballot(alive) != 0ull) {  // (wave-uniform) a wave without survivors has nothing to walk
    float4* const st = a.slots + (size_t)a.bnd_off[t.tile] * (kTile * kTile) + t.pix;
    const uint64_t cbase = (uint64_t)(t.start / kChunk) + (uint64_t)t.tile;
    const uint32_t fs = f << t.fshift, fe = min(t.len, fs + (1u << t.fshift));
    WalkState s{1.0f, 0.f, 0.f, 0.f, 0u, 0u, 0u, 0u, 0u, !alive};
    walk_entries<false, true, true>(a, shift, t.start, fs, fe, true, st, cbase, t.pix, t.xq, t.yq,
                                    (float)t.px + 0.5f, (float)t.py + 0.5f, stg[threadIdx.x >> 6], s);
    const size_t o = ((size_t)t.fb + f) * (kTile * kTile) + t.pix;
    put_f4<true>(L.fsum + o, make_float4(s.Tr, s.c0, s.c1, s.c2));
    put_u4<true>(L.fstat + o, make_uint4(s.first, s.last, s.blended | (s.examined ? 0x80000000u : 0u), s.evaluated));
  }
  drain_memory();
  __syncthreads();
  if (threadIdx.x == 0) atomicAdd(L.split_cnt + 4 * c + 1, 1u);
  __syncthreads();  // (as at the end of long_first)
}

constexpr uint32_t kCombineBatch = 4;  // forward segments whose sums one pass loads at once

__device__ void long_combine(const FwdArgs& a, const LongArgs& L, uint32_t shift, uint32_t c, uint32_t* hdr) {
  const SplitTile t = split_tile_of(a, L, shift, c);
  if (threadIdx.x == 0) wait_for(L.split_cnt + 4 * c + 1, t.nseg - t.f0, hdr);  // the walks past the first part
  __syncthreads();
  const uint4 ps = t.inside ? get_u4<true>(L.pstate + (size_t)c * (kTile * kTile) + t.pix) : make_uint4(kPixDone, 0u, 0u, 0u);
  const bool alive = ps.x == kPixAlive;
  float4 fi = make_float4(1.f, 0.f, 0.f, 0.f);
  if (alive) fi = get_f4<true>(L.fin + ((size_t)t.fb + t.f0) * (kTile * kTile) + t.pix);
  WalkState s{fi.x, fi.y, fi.z, fi.w, 0u, ps.y, t.len, ps.z, ps.w, !alive};
  uint32_t stop = t.nseg;
  for (uint32_t f0 = t.f0; __ballot(!s.done) != 0ull; f0 += kCombineBatch) {
    float4 P[kCombineBatch];
    uint4 Q[kCombineBatch];
#pragma unroll
    for (uint32_t j = 0; j < kCombineBatch; ++j) {  // loads clamped into the list, all in flight at once
      const size_t o = ((size_t)t.fb + min(f0 + j, t.nseg - 1u)) * (kTile * kTile) + t.pix;
      P[j] = get_f4<true>(L.fsum + o);
      Q[j] = get_u4<true>(L.fstat + o);
    }
#pragma unroll
    for (uint32_t j = 0; j < kCombineBatch; ++j) {
      const uint32_t f = f0 + j;
      if (!s.done && f >= t.nseg) s.done = true;  // walked the whole list
      if (s.done) continue;
      put_f4<true>(L.fin + ((size_t)t.fb + f) * (kTile * kTile) + t.pix, make_float4(s.Tr, s.c0, s.c1, s.c2));
      if ((Q[j].z >> 31) || s.Tr * P[j].x < kTMin) {  // the stop lies in segment f
        stop = f;
        s.done = true;
        continue;
      }
      s.c0 += s.Tr * P[j].y;
      s.c1 += s.Tr * P[j].z;
      s.c2 += s.Tr * P[j].w;
      s.Tr *= P[j].x;
      s.last = Q[j].y ? Q[j].y : s.last;
      s.blended += Q[j].z;
      s.evaluated += Q[j].w;
    }
  }
  const bool finished = alive && stop == t.nseg;  // never stops: its outputs are complete
  if (alive) {
    put_u4<true>(L.pstate + (size_t)c * (kTile * kTile) + t.pix, make_uint4(stop, s.last, s.blended, s.evaluated));
    if (finished) finish_split_pixel(a, shift, t, s);
  }
  add_blend_stats(a.blend_count, finished ? s.examined : 0u, finished ? s.last : 0u, finished ? s.blended : 0u,
                  finished ? s.evaluated : 0u);
  drain_memory();
  __syncthreads();
  if (threadIdx.x == 0) put_32<true>(L.split_cnt + 4 * c + 2, 1u);
  __syncthreads();  // (as at the end of long_first)
}

__device__ void long_redo(const FwdArgs& a, const LongArgs& L, uint32_t shift, uint2 it, Chunk* stg,
                          uint32_t* hdr) {
  const uint32_t c = it.x, f = it.y;
  const SplitTile t = split_tile_of(a, L, shift, c);
  if (f < t.f0) return;  // (workgroup-uniform) the first part's stops are exact already
  if (threadIdx.x == 0) wait_for(L.split_cnt + 4 * c + 2, 1u, hdr);
  __syncthreads();
  const bool mine = t.inside && get_32<true>(&L.pstate[(size_t)c * (kTile * kTile) + t.pix].x) == f;  // stops in f
  if (!__syncthreads_or(mine)) return;
  const float4 fi = mine ? get_f4<true>(L.fin + ((size_t)t.fb + f) * (kTile * kTile) + t.pix) : make_float4(1.f, 0.f, 0.f, 0.f);
  WalkState s{fi.x, fi.y, fi.z, fi.w, 0u, 0u, 0u, 0u, 0u, !mine};
  const uint32_t fs = f << t.fshift, fe = min(t.len, fs + (1u << t.fshift));
  walk_entries<false, false, false>(a, shift, t.start, fs, fe, true, nullptr, 0, t.pix, t.xq, t.yq,
                                    (float)t.px + 0.5f, (float)t.py + 0.5f, stg[threadIdx.x >> 6], s);
  if (mine) {
    const uint4 ps = get_u4<true>(L.pstate + (size_t)c * (kTile * kTile) + t.pix);  // (reloaded: fewer registers)
    if (s.examined == 0u) {
      // No stop inside the segment: the combine's product fell below 1e-4 only by rounding,
      // and T is now within rounding of 1e-4, so the next composited entry (alpha >= 1/255)
      // stops the pixel -- the first composited position of a later segment, else none.
      s.examined = t.len;
      for (uint32_t g = f + 1u; g < t.nseg; ++g) {
        const uint32_t q = get_u4<true>(L.fstat + ((size_t)t.fb + g) * (kTile * kTile) + t.pix).x;
        if (q) {
          s.examined = q;
          break;
        }
      }
    }
    s.last = s.last ? s.last : ps.y;
    s.blended += ps.z;
    s.evaluated += ps.w;
    finish_split_pixel(a, shift, t, s);
  }
  add_blend_stats(a.blend_count, mine ? s.examined : 0u, mine ? s.last : 0u, mine ? s.blended : 0u,
                  mine ? s.evaluated : 0u);
}

// Persistent: with S split tiles and F forward segments, items 0 .. S-1 walk the first parts,
// S .. S+F-1 the segments (in fitems' order), S+F .. 2S+F-1 combine, 2S+F .. 2S+2F-1 redo.
// (Capped at six waves per SIMD, as the other forward kernels are, it spills; it runs at four.)
__global__ __launch_bounds__(kBlock) void k_long_forward(FwdArgs a, LongArgs L, uint32_t* __restrict__ hdr) {
  __shared__ Chunk stg[4];
  __shared__ uint32_t s_q;
  const uint32_t shift = hdr[kHdrShift], ns = hdr[kHdrSplit], nf = hdr[kHdrFsegs];
  if (ns == 0u) return;
  for (;;) {
    if (threadIdx.x == 0) s_q = atomicAdd(hdr + kHdrLongNext, 1u);
    __syncthreads();
    const uint32_t q = s_q;
    __syncthreads();  // every wave has read s_q before it is overwritten
    if (q < ns)
      long_first(a, L, shift, q, stg);
    else if (q < ns + nf)
      long_walk(a, L, shift, L.fitems[q - ns], stg, hdr);
    else if (q < 2 * ns + nf)
      long_combine(a, L, shift, q - ns - nf, hdr);
    else if (q < 2 * ns + 2 * nf)
      long_redo(a, L, shift, L.fitems[q - 2 * ns - nf], stg, hdr);
    else
      break;
  }
}

// ---------------------------------------------------------------------------------------------
// Backward.  Work item = (tile, segment k): list positions [k SEG, (k+1) SEG), walked back to
// front by each quadrant wave over its pixels.  A pixel whose last blended entry lies beyond
// the segment starts from the forward's state at the segment's end: T there, and the colour
// behind it, (C_final - C_boundary) / T_boundary; otherwise from T_final with nothing behind.
// The segments of one tile are independent, so a long list is spread over many CUs.
// Persistent workgroups take items from a counter in the workspace until none are left.
// Each 4x4 pixel block walks the entries its pixels composited (the forward's masks), back to
// front; the block's nine gradient sums per entry go into the workgroup's LDS sums over a window
// of 256 entries, whose sums then go to the staging area, one row per (entry, tile).
// ---------------------------------------------------------------------------------------------
struct BwdArgs {
  int W, H, TX, TY;
  int64_t n;
  const float4* splat;
  const uint32_t* vals;
  const uint2* ranges;
  float bg0, bg1, bg2;
  const float* T_final;
  const uint32_t* last_contrib;
  const float* dLdI;
  const uint32_t* bnd_off;
  const float4* slots;
  const uint2* masks;
  uint64_t mask_cap;
  const uint32_t* goff;
  const uint32_t* goff_blk;
  float* staging;
  uint64_t staging_cap;
  const uint32_t* fbase;  // split tiles: their first forward segment (else kNoSplit)
  const float4* fin;      // split tiles: (T, C) in front of each forward segment, per pixel
};

// LDS of a blending workgroup
struct BlendShared {
  Chunk stg[4];        // per quadrant wave: its current chunk
  float acc[9][kWin];  // the backward's gradient sums over a window of entries
  uint32_t mx[4];
};

// One work item (tile, segment k) by the workgroup's four quadrant waves (kStep: inside the
// fused step, which reads the tile's state from other workgroups at device scope).
template <bool kStep>
__device__ void backward_item(const BwdArgs& a, uint32_t shift, uint2 it, BlendShared& sh) {
  const int W = a.W, H = a.H, TX = a.TX, TY = a.TY;
  const int64_t n = a.n;
  const float4* __restrict__ splat = a.splat;
  const uint32_t* __restrict__ vals = a.vals;
  const uint2* __restrict__ masks = a.masks;
  const uint64_t mask_cap = a.mask_cap;
  const uint32_t* __restrict__ goff = a.goff;
  const uint32_t* __restrict__ goff_blk = a.goff_blk;
  float* __restrict__ staging = a.staging;
  const uint64_t staging_cap = a.staging_cap;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  Chunk& S = sh.stg[w];
  float(*acc)[kWin] = sh.acc;
  uint32_t* s_mx = sh.mx;
  // the 16 lanes of DPP row q (lanes 16 q .. 16 q + 15) are the 4x4 pixel block q of the
  // quadrant (blocks row-major): each block reduces over one row
  const int lx = ((lane >> 4) & 1) * 4 + ((lane >> 2) & 1) * 2 + (lane & 1);
  const int ly = (lane >> 5) * 4 + ((lane >> 3) & 1) * 2 + ((lane >> 1) & 1);
  const int pix = tile_pixel(w, lx, ly);
  // the block's sum this lane adds to the window's sums (row_scatter9): lanes 0, 2, .., 14 of
  // the row hold sums 0..7, lane 1 sum 8
  const int rl = lane & 15;
  const bool own = (rl & 1) == 0 || rl == 1;
  float* const acc_own = acc[rl == 1 ? 8 : ((rl >> 3) & 1) * 4 + ((rl >> 2) & 1) * 2 + ((rl >> 1) & 1)];
  const int tile = (int)it.x;
  const uint32_t k = it.y;
  const int tx = tile % TX, ty = tile / TX;
  const int xq = tx * kTile + (w & 1) * 8, yq = ty * kTile + (w >> 1) * 8;
  const int px = xq + lx, py = yq + ly;
  const bool inside = px < W && py < H;
  const float pxc = (float)px + 0.5f, pyc = (float)py + 0.5f;
  const uint2 rg = a.ranges[tile];
  const uint32_t start = rg.x, end = rg.y, len = rg.y - rg.x;
  const uint64_t cbase = (uint64_t)(start / kChunk) + (uint64_t)tile;  // the tile's first mask chunk
  const uint32_t fbv = a.fbase[tile];
  const bool split = fbv != kNoSplit;  // (a split tile's masks go on past each pixel's stop)

  // Tr: the transmittance behind the current entry; Sg: the colour behind it (normalised by
  // Tr) dotted with dL/dI -- the gradient needs that colour only through this product
  float Tr = 0.f, Sg = 0.f, g0 = 0.f, g1 = 0.f, g2 = 0.f, bgT = 0.f;
  uint32_t last = 0;
  if (inside) {
    const int64_t p = (int64_t)py * W + px;
    Tr = get_32<kStep>(a.T_final + p);
    last = get_32<kStep>(a.last_contrib + p);
    g0 = get_32<kStep>(a.dLdI + 3 * p);
    g1 = get_32<kStep>(a.dLdI + 3 * p + 1);
    g2 = get_32<kStep>(a.dLdI + 3 * p + 2);
    bgT = Tr * (a.bg0 * g0 + a.bg1 * g1 + a.bg2 * g2);
  }
  uint32_t mx = last;  // the wave's largest last_contrib
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor(mx, o, 64));
  if (lane == 0) s_mx[w] = mx;
  __syncthreads();
  const uint32_t mxb = max(max(s_mx[0], s_mx[1]), max(s_mx[2], s_mx[3]));
  const uint32_t seg_lo = k << shift;
  const uint32_t seg_end = seg_lo + (1u << shift);
  const uint32_t hi_w = min(seg_end, min(mx, len));   // this wave walks [seg_lo, hi_w)
  const uint32_t hi_b = min(seg_end, min(mxb, len));  // the workgroup walks [seg_lo, hi_b)
  if (seg_lo >= hi_b) return;  // workgroup-uniform: the segment lies behind every pixel's walk
  if (last > seg_end) {  // the pixel's walk starts behind this segment
    const float4* st = a.slots + (size_t)a.bnd_off[tile] * (kTile * kTile) + pix;
    float4 sb = get_f4<kStep>(st + (size_t)k * (kTile * kTile));
    // a split tile's boundary state past its first part is relative to its forward segment
    const uint32_t fsh = fbv >> 27;
    if (split && (seg_end >> fsh) > (((1u << (shift + kPhase1Log)) - 1u) >> fsh)) {
      const float4 fi = a.fin[((size_t)(fbv & kFbaseMask) + (seg_end >> fsh)) * (kTile * kTile) + pix];
      sb = make_float4(fi.x * sb.x, fi.y + fi.x * sb.y, fi.z + fi.x * sb.z, fi.w + fi.x * sb.w);
    }
    const float4 sf = get_f4<kStep>(st + (size_t)((len - 1u) >> shift) * (kTile * kTile));
    Tr = sb.x;  // T >= 1e-4 at every boundary
    Sg = ((sf.y - sb.y) * g0 + (sf.z - sb.z) * g1 + (sf.w - sb.w) * g2) / sb.x;
  }

  // windows of kWin entries, top down; the waves walk a window independently, then the
  // workgroup adds the window's sums to grad2d
  for (uint32_t wtop = hi_b; wtop > seg_lo;) {
    const uint32_t wlo = seg_lo + ((wtop - 1u - seg_lo) & ~(uint32_t)(kWin - 1));
#pragma unroll
    for (int q = 0; q < 9; ++q) acc[q][tid] = 0.f;
    __syncthreads();
    const uint32_t whi = min(wtop, hi_w);
    if (whi > wlo) {  // wave-uniform
      // the window's chunks j (tile-relative entries [64 j, 64 j + 64)), top down
      const uint32_t jlo = wlo / kChunk, jtop = (whi - 1u) / kChunk, nchunks = jtop - jlo + 1u;
      // list entry of lane `lane` in chunk c (c >= nchunks: past the end of the list)
      auto gid_of = [&](uint32_t c) -> uint32_t {
        return load_gid(vals, c < nchunks ? start + (jtop - c) * kChunk + lane : end, end, start);
      };
      auto mask_of = [&](uint32_t c) -> uint2 {
        const uint64_t mc = cbase + (c < nchunks ? jtop - c : jtop);
        return get_u2<kStep>(masks + (mc < mask_cap ? mc : 0) * (kTile * kTile) + pix);
      };
      uint32_t gnext = gid_of(0);
      Raw cur = load_raw(splat, gnext, n);
      uint2 mcur = mask_of(0);
      gnext = gid_of(1);
      for (uint32_t c = 0; c < nchunks; ++c) {
        const uint32_t j = jtop - c;
        const Raw nxt = load_raw(splat, gnext, n);  // next chunk in flight
        const uint2 mnxt = mask_of(c + 1);
        gnext = gid_of(c + 2);
        put(S, lane, cur);
        wave_sync_lds();
        // The entries this pixel composited in the chunk (the forward's mask): exactly those
        // with power <= 0, alpha >= 1/255 in front of the pixel's stop.  Each 4x4 pixel block
        // of the quadrant (16 lanes) takes the entries any of its pixels composited, back to
        // front, its lanes on the same entry; the block's nine sums are formed in registers,
        // spread over nine of its lanes, and each of those lanes adds its sum to the window's.
        unsigned long long mine = cbase + j < mask_cap ? ((unsigned long long)mcur.y << 32) | mcur.x : 0ull;
        if (split) {  // only entries up to the pixel's last composited one
          const uint32_t jlo0 = j * kChunk;
          if (last < jlo0 + kChunk) mine &= last > jlo0 ? (1ull << (last - jlo0)) - 1ull : 0ull;
        }
        unsigned long long rem = row_or(mine);
        const uint32_t wbase = j * kChunk - wlo;  // window position of slot 0
        for (;;) {
          const bool has = rem != 0ull;
          if (__ballot(has) == 0ull) break;
          const int e = has ? highest_bit(rem) : 0;
          rem &= ~(1ull << e);
          const float4 g = S.geo[e];  // one address per block: a broadcast within the block
          const float4 cl = S.col[e];
          const float cb = S.b[e];
          const float dx = pxc - g.x, dy = pyc - g.y;
          const float power = eval_power(g.z, g.w, cl.x, dx, dy);
          const float G = __expf(power);
          const float oG = __fmul_rn(cl.y, G);  // the same operations as eval_oG
          const float alpha = fminf(kAlphaMax, oG);
          const bool act = has && ((mine >> e) & 1ull);
          const float om = 1.0f - alpha;
          const float rom = __builtin_amdgcn_rcpf(om);  // om >= 0.01
          const float Tk = Tr * rom;                    // transmittance in front of this entry
          const float wt = alpha * Tk;
          const float cdg = cl.z * g0 + cl.w * g1 + cb * g2;  // c . dL/dI
          const float dL_dalpha = Tk * (cdg - Sg) - bgT * rom;
          const bool unclamped = act && oG <= kAlphaMax;  // alpha = o G depends on o and power
          const float dpow = unclamped ? oG * dL_dalpha : 0.0f;
          // moments of dL/dpower over the pixels; the conic gradients are linear in them
          float v[9];
          v[0] = dx * dpow;
          v[1] = dy * dpow;
          v[2] = dx * v[0];
          v[3] = dy * v[0];
          v[4] = dy * v[1];
          v[5] = unclamped ? G * dL_dalpha : 0.0f;
          v[6] = act ? wt * g0 : 0.0f;
          v[7] = act ? wt * g1 : 0.0f;
          v[8] = act ? wt * g2 : 0.0f;
          if (act) {
            Sg = alpha * cdg + om * Sg;
            Tr = Tk;
          }
          float s8;
          const float sq = row_scatter9(v, lane, &s8);
          if (own && has)  // the raw moments: the conic enters once per entry
            atomicAdd(acc_own + wbase + (uint32_t)e, rl == 1 ? s8 : sq);
        }
        wave_sync_lds();  // this chunk's reads finish before the next chunk is staged
        cur = nxt;
        mcur = mnxt;
      }
    }
    __syncthreads();
    // one thread per entry of the window: the entry's sums go to its Gaussian's staging
    // slot, the entry's place in the row-major order of the Gaussian's tile rect
    if (wlo + (uint32_t)tid < wtop) {
      float x[9];
      bool any = false;
#pragma unroll
      for (int q = 0; q < 9; ++q) {
        x[q] = acc[q][tid];
        any = any || x[q] != 0.f;
      }
      if (any) {
        const uint32_t gid = vals[start + wlo + tid];
        const float4 q0 = splat[3 * (int64_t)gid];      // u, v, radius_x, radius_y
        const float4 q1 = splat[3 * (int64_t)gid + 1];  // conic A, B, C, opacity
        // from the moments m of dL/dpower (power = -(A dx^2 + C dy^2)/2 - B dx dy):
        // dL/du = A m_x + B m_y, dL/dv = B m_x + C m_y, dL/dA = -m_xx/2, dL/dB = -m_xy, dL/dC = -m_yy/2
        const float mx_ = x[0], my_ = x[1];
        x[0] = q1.x * mx_ + q1.y * my_;
        x[1] = q1.y * mx_ + q1.z * my_;
        x[2] = -0.5f * x[2];
        x[3] = -x[3];
        x[4] = -0.5f * x[4];
        int x0, y0, x1, y1;
        tile_rect(q0.x, q0.y, __float_as_int(q0.z), __float_as_int(q0.w), TX, TY, x0, y0, x1, y1);
        const uint64_t slot = (uint64_t)goff_blk[gid / kGoffBlock] + goff[gid] +
                              (uint32_t)((ty - y0) * (x1 - x0) + (tx - x0));
        if (slot < staging_cap) {
          float* o = staging + 9 * slot;
#pragma unroll
          for (int q = 0; q < 9; ++q) o[q] = x[q];
        }
      }
    }
    __syncthreads();  // the window's sums are read before the next window clears them
    wtop = wlo;
  }
}

__global__ __launch_bounds__(kBlock) void k_blend_backward(BwdArgs a, uint32_t* __restrict__ ws_hdr,
                                                           const uint2* __restrict__ items) {
  __shared__ BlendShared sh;
  __shared__ uint32_t s_item;
  const uint32_t shift = ws_hdr[kHdrShift], n_items = ws_hdr[kHdrItems];
  for (;;) {
    if (threadIdx.x == 0) s_item = atomicAdd(ws_hdr + kHdrBwdNext, 1u);
    __syncthreads();
    const uint32_t item = s_item;
    __syncthreads();  // every wave has read s_item before it is overwritten
    if (item >= n_items) break;
    backward_item<false>(a, shift, items[item], sh);
  }
}

// Persistent forward: the workgroups take tiles in the plan's order (list-length classes,
// longest first) from a counter.  Longest first, a tile's waves walk its list alone, so the
// longest walks start at once and the short tiles fill in around them.  A few workgroups per CU
// suffice: fewer waves share each SIMD with the long walks, which then finish sooner.
// Six waves per SIMD (80 registers, no spills) measured faster than the compiler's default of five;
// seven and eight spill and are slower.
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(6))) void k_blend_forward(FwdArgs a,
                                                                                               uint32_t* __restrict__ hdr) {
  __shared__ Chunk stg[4];
  __shared__ uint32_t s_next;
  const uint32_t shift = hdr[kHdrShift];
  for (;;) {
    if (threadIdx.x == 0) s_next = atomicAdd(hdr + kHdrFwdNext, 1u);
    __syncthreads();
    const uint32_t i = s_next;
    __syncthreads();  // every wave has read s_next before it is overwritten
    if (i >= (uint32_t)a.T) break;
    const uint32_t ot = a.order[i];
    if (!(ot & kOrderSplit)) forward_tile<false>(a, shift, (int)ot, false, stg);  // else done by k_long_forward
  }
}

// ---------------------------------------------------------------------------------------------
// The fused step: forward, L1 loss and backward blend in one persistent kernel, so that the
// backward's work fills the CUs the forward's long tile walks leave idle.
//   - The first fwd_workers workgroups to start take tiles, longest first, and run the forward
//     at raised wave priority.  When a tile is done (every wave's stores complete), its
//     backward items are appended to the item list.
//   - Every workgroup (the forward workers once the tiles run out) takes item slots in list
//     order and waits until its slot has been published.
// No workgroup waits for anything but a tile that a running workgroup has already taken, and
// the forward never waits, so every wait ends; a wait is still bounded, and one that gives up
// flags the stall word of the header and leaves its item undone.
// ---------------------------------------------------------------------------------------------
// Six waves per SIMD, as for the forward: 1.56 instead of 1.61 ms on the 4M-Gaussian 2048x2048 step.
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(6))) void k_blend_step(
    FwdArgs fa, BwdArgs ba, uint32_t* __restrict__ hdr, uint2* __restrict__ items,
    const uint32_t* __restrict__ item_off, uint32_t fwd_workers) {
  __shared__ BlendShared sh;
  __shared__ uint32_t s_next, s_pos;
  __shared__ uint2 s_it;
  const int tid = threadIdx.x;
  const uint32_t shift = hdr[kHdrShift], n_items = hdr[kHdrItems];
  if (tid == 0) s_next = atomicAdd(hdr + kHdrRole, 1u);
  __syncthreads();
  const bool forward_worker = s_next < fwd_workers;
  __syncthreads();
  if (forward_worker) {
    __builtin_amdgcn_s_setprio(2);
    for (;;) {
      if (tid == 0) s_next = atomicAdd(hdr + kHdrFwdNext, 1u);
      __syncthreads();
      const uint32_t i = s_next;
      __syncthreads();
      if (i >= (uint32_t)fa.T) break;
      const uint32_t ot = fa.order[i];
      const int tile = (int)(ot & ~kOrderSplit);
      forward_tile<true>(fa, shift, tile, (ot & kOrderSplit) != 0u, sh.stg);
      drain_memory();
      __syncthreads();  // the tile's state is visible to every XCD
      const uint32_t o = item_off[tile], k = item_off[tile + 1] - o;
      if (k != 0u) {  // workgroup-uniform
        if (tid == 0) s_pos = atomicAdd(hdr + kHdrReady, k);
        __syncthreads();
        const uint32_t pos = s_pos;
        for (uint32_t j = tid; j < k; j += kBlock) put_u2<true>(items + pos + j, make_uint2((uint32_t)tile, j));
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }
  for (;;) {
    if (tid == 0) {
      const uint32_t b = atomicAdd(hdr + kHdrBwdNext, 1u);
      uint2 it = make_uint2(kNoTile, 0u);
      if (b < n_items) {
        for (uint32_t spin = 0;; ++spin) {
          it = get_u2<true>(items + b);
          if (it.x != kNoTile) break;
          if (spin == kSpinLimit) {
            atomicOr(hdr + kHdrFlags, kFlagStall);
            break;
          }
          __builtin_amdgcn_s_sleep(4);
        }
      }
      s_it = it;
    }
    __syncthreads();
    const uint2 it = s_it;
    __syncthreads();
    if (it.x == kNoTile) break;
    backward_item<true>(ba, shift, it, sh);
  }
}

// ---------------------------------------------------------------------------------------------
// Per-Gaussian staging offsets: exclusive scan of tiles_i in Gaussian order, two levels.
// ---------------------------------------------------------------------------------------------
constexpr int kGoffItems = kGoffBlock / kBlock;  // 16 Gaussians per thread

__global__ __launch_bounds__(kBlock) void k_goff_local(int64_t n, const uint32_t* __restrict__ tiles,
                                                       uint32_t* __restrict__ goff, uint32_t* __restrict__ blk) {
  __shared__ uint32_t wsum[kBlock / 64];
  // item j of thread t is base + j kBlock + t: the block scans its kGoffBlock Gaussians in
  // kGoffItems rounds of kBlock consecutive ones, every load and store coalesced
  const int64_t base = (int64_t)blockIdx.x * kGoffBlock + threadIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t t[kGoffItems];
#pragma unroll
  for (int j = 0; j < kGoffItems; ++j) {
    const int64_t i = base + (int64_t)j * kBlock;
    t[j] = i < n ? tiles[i] : 0u;
  }
  uint32_t run = 0;  // the block's earlier rounds
#pragma unroll
  for (int j = 0; j < kGoffItems; ++j) {
    uint32_t inc = t[j];
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    uint32_t pre = inc - t[j], tot = 0;
#pragma unroll
    for (int k = 0; k < kBlock / 64; ++k) {
      pre += k < w ? wsum[k] : 0u;
      tot += wsum[k];
    }
    __syncthreads();
    const int64_t i = base + (int64_t)j * kBlock;
    if (i < n) goff[i] = run + pre;
    run += tot;
  }
  if (threadIdx.x == 0) blk[blockIdx.x] = run;  // the block's total
}

// exclusive scan of the nblk block totals in place (one workgroup); total entries -> header, and
// the capacity flag when the staging area holds fewer
__global__ __launch_bounds__(kPlanThreads) void k_goff_blocks(int64_t nblk, uint32_t* __restrict__ blk,
                                                              uint32_t* __restrict__ hdr, uint64_t entries_cap) {
  __shared__ uint32_t red32[kPlanThreads / 64];
  const int64_t per = (nblk + kPlanThreads - 1) / kPlanThreads;
  const int64_t lo = std::min<int64_t>(nblk, (int64_t)threadIdx.x * per), hi = std::min<int64_t>(nblk, lo + per);
  uint32_t s = 0;
  for (int64_t b = lo; b < hi; ++b) s += blk[b];
  uint32_t run = block_exscan_1024(s, red32);
  for (int64_t b = lo; b < hi; ++b) {
    const uint32_t x = blk[b];
    blk[b] = run;
    run += x;
  }
  if (threadIdx.x == kPlanThreads - 1) {  // the last thread's end is the total
    hdr[kHdrEntries] = run;
    if ((uint64_t)run > entries_cap) {
      hdr[kHdrFlags] |= kFlagCapacity;
      hdr[kHdrNeed] = max(hdr[kHdrNeed], run);
    }
  }
}

// staging[0 .. 9 * entries) = 0; entries from the header, capped at the workspace's capacity
__global__ __launch_bounds__(kBlock) void k_clear_staging(const uint32_t* __restrict__ hdr, float4* __restrict__ st,
                                                          uint64_t cap) {
  const uint64_t e = std::min<uint64_t>((uint64_t)hdr[kHdrEntries], cap);
  const uint64_t n4 = (9 * e + 3) / 4;  // the staging region is padded to whole float4s
  for (uint64_t j = (uint64_t)blockIdx.x * kBlock + threadIdx.x; j < n4; j += (uint64_t)gridDim.x * kBlock)
    st[j] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// grad2d[i] = sum of Gaussian i's staged entries, in the order of its tile rect
__global__ __launch_bounds__(kBlock) void k_gather_grad2d(int64_t n, const uint32_t* __restrict__ tiles,
                                                          const uint32_t* __restrict__ goff,
                                                          const uint32_t* __restrict__ goff_blk,
                                                          const float* __restrict__ staging, uint64_t cap,
                                                          float* __restrict__ grad2d) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= n) return;
  const uint32_t t = tiles[i];
  const uint64_t base = (uint64_t)goff_blk[i / kGoffBlock] + goff[i];
  float x[9] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (uint32_t j = 0; j < t; ++j) {
    if (base + j >= cap) break;
    const float* e = staging + 9 * (base + j);
#pragma unroll
    for (int q = 0; q < 9; ++q) x[q] += e[q];
  }
  float* o = grad2d + 9 * i;
#pragma unroll
  for (int q = 0; q < 9; ++q) o[q] = x[q];
}

int cu_count() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] <= 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cached[dev] = v;
  }
  return cached[dev];
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }
constexpr size_t kSlotBytes = sizeof(float4) * kTile * kTile;
constexpr size_t kMaskChunkBytes = sizeof(uint2) * kTile * kTile;  // one 64-bit mask per pixel
constexpr uint64_t kSegEntries = 1u << kSegShiftMin;

size_t n_goff_blocks(int64_t n) { return (size_t)((n + kGoffBlock - 1) / kGoffBlock); }
size_t plan_blocks(int T) { return (size_t)((T + kPlanThreads - 1) / kPlanThreads); }
size_t plan_bytes(int T) { return round256(4 * plan_blocks(T) * kPartVals) + round256(4 * plan_blocks(T) * kOffVals); }

// Split tiles and forward segments for k entries: a split list holds len >= kSplitMinLen
// entries and ceil(len / F) <= len / F + len / kSplitMinLen segments of F >= kFsegMin entries
// (at the smallest shift; a larger shift only lengthens both).
constexpr uint64_t kFsegMin = kSegEntries << kFsegLog;
constexpr uint64_t kSplitMinLen = kSegEntries << kSplitLog;
size_t split_cap_for(uint64_t k) { return (size_t)std::min<uint64_t>(kMaxSplit, k / kSplitMinLen + 1); }
size_t fseg_cap_for(uint64_t k) { return (size_t)(k / kFsegMin + k / kSplitMinLen + 2); }
size_t split_bytes(int T, uint64_t k) {
  const size_t sc = split_cap_for(k), fc = fseg_cap_for(k);
  return round256(4 * (size_t)T) + round256(4 * sc) + round256(16 * sc) + round256(8 * fc) + 3 * kSlotBytes * fc +
         round256(16 * (size_t)(kTile * kTile) * sc);
}

// bytes of the layout for T tiles, n Gaussians and k staged entries (k a multiple of 256)
// (tile t's 64-entry chunks start at ranges[t].x / 64 + t, so K entries need at most
// K / 64 + T mask chunks)
size_t layout_bytes(int T, int64_t n, uint64_t k) {
  const size_t slots = (size_t)T + (size_t)(k / kSegEntries);
  const size_t chunks = (size_t)T + (size_t)(k / kChunk);
  return 256 + 2 * round256(4 * (size_t)(T + 1)) + 2 * round256(4 * (size_t)T) + plan_bytes(T) + round256(4 * (size_t)n) +
         round256(4 * (n_goff_blocks(n) + 1)) +
         round256(8 * ((size_t)T + slots)) + round256(kSlotBytes * slots) + kMaskChunkBytes * chunks +
         split_bytes(T, k) + round256(36 * (size_t)k + 16);
}
// per segment (512 entries) of capacity, at least (the split tiles' arrays grow in larger steps)
constexpr size_t kBytesPerSeg = kSlotBytes + 8 + (kSegEntries / kChunk) * kMaskChunkBytes + 36 * kSegEntries;

}  // namespace

size_t render_ws_bytes(int T, int64_t n, int64_t k_capacity) {
  const uint64_t kc = k_capacity > 0 ? (uint64_t)k_capacity : 0;
  return layout_bytes(T, n, (kc + kSegEntries - 1) / kSegEntries * kSegEntries);
}

bool render_ws_layout(void* ws, size_t bytes, int T, int64_t n, RenderWs* out) {
  const size_t base = layout_bytes(T, n, 0);
  if (!ws || bytes < base || (reinterpret_cast<uintptr_t>(ws) & 255u)) return false;
  // a segment more of capacity costs at least kBytesPerSeg - 8 bytes (the item array may not
  // grow by a whole 256-byte step), so hi is an upper bound; bisect for the largest fit (the
  // layout grows with k)
  uint64_t lo = 0, hi = (bytes - base) / (kBytesPerSeg - 8);  // in units of segments
  while (lo < hi) {
    const uint64_t mid = lo + (hi - lo + 1) / 2;
    if (layout_bytes(T, n, mid * kSegEntries) <= bytes) lo = mid; else hi = mid - 1;
  }
  const uint64_t k = lo * kSegEntries;
  const size_t slots = (size_t)T + (size_t)(k / kSegEntries);
  if (slots > 0x7FFFFFFFull) return false;
  char* b = static_cast<char*>(ws);
  out->hdr = reinterpret_cast<uint32_t*>(b);
  b += 256;
  out->bnd_off = reinterpret_cast<uint32_t*>(b);
  b += round256(4 * (size_t)(T + 1));
  out->item_off = reinterpret_cast<uint32_t*>(b);
  b += round256(4 * (size_t)(T + 1));
  out->order = reinterpret_cast<uint32_t*>(b);
  b += round256(4 * (size_t)T);
  out->loss_part = reinterpret_cast<float*>(b);
  b += round256(4 * (size_t)T);
  out->plan_part = reinterpret_cast<uint32_t*>(b);
  b += round256(4 * plan_blocks(T) * kPartVals);
  out->plan_off = reinterpret_cast<uint32_t*>(b);
  b += round256(4 * plan_blocks(T) * kOffVals);
  out->goff = reinterpret_cast<uint32_t*>(b);
  b += round256(4 * (size_t)n);
  out->goff_blk = reinterpret_cast<uint32_t*>(b);
  b += round256(4 * (n_goff_blocks(n) + 1));
  out->items = reinterpret_cast<uint2*>(b);  // T + slots items at most
  b += round256(8 * ((size_t)T + slots));
  out->slots = reinterpret_cast<float4*>(b);
  b += round256(kSlotBytes * slots);
  const size_t chunks = (size_t)T + (size_t)(k / kChunk);
  out->masks = reinterpret_cast<uint2*>(b);
  b += kMaskChunkBytes * chunks;
  const size_t sc = split_cap_for(k), fc = fseg_cap_for(k);
  out->fbase = reinterpret_cast<uint32_t*>(b);
  b += round256(4 * (size_t)T);
  out->split_tile = reinterpret_cast<uint32_t*>(b);
  b += round256(4 * sc);
  out->split_cnt = reinterpret_cast<uint32_t*>(b);
  b += round256(16 * sc);
  out->fitems = reinterpret_cast<uint2*>(b);
  b += round256(8 * fc);
  out->fsum = reinterpret_cast<float4*>(b);
  b += kSlotBytes * fc;
  out->fstat = reinterpret_cast<uint4*>(b);
  b += kSlotBytes * fc;
  out->fin = reinterpret_cast<float4*>(b);
  b += kSlotBytes * fc;
  out->pstate = reinterpret_cast<uint4*>(b);
  b += round256(16 * (size_t)(kTile * kTile) * sc);
  out->staging = reinterpret_cast<float*>(b);
  out->slots_cap = (uint32_t)slots;
  out->mask_cap = chunks;
  out->staging_cap = k;
  out->fseg_cap = (uint32_t)fc;
  out->split_cap = (uint32_t)sc;
  return true;
}

namespace {

constexpr int kFwdPerCu = 3;      // workgroups per CU of the forward alone
constexpr int kStepFwdPerCu = 2;  // the fused step's forward workers per CU (measured best)

// workgroups of `kernel` that fit on one CU at once
int resident_per_cu(const void* kernel, int* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  if (cache[dev] <= 0) {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kernel, kBlock, 0) != hipSuccess || v <= 0) v = 1;
    cache[dev] = v;
  }
  return cache[dev];
}

// the segment plan, the tile order and the item list (empty markers for the fused step)
void launch_plan(int T, const uint2* rg, const RenderWs& ws, bool empty_items, hipStream_t s) {
  const int nb = (int)ceil_div(T, kPlanThreads);
  hipLaunchKernelGGL(k_plan_count, dim3((unsigned)nb), dim3(kPlanThreads), 0, s, rg, T, ws.plan_part);
  hipLaunchKernelGGL(k_plan_scan, dim3(1), dim3(kPlanThreads), 0, s, (const uint32_t*)ws.plan_part, nb, T,
                     ws.slots_cap, (uint64_t)ws.staging_cap, ws.plan_off, ws.hdr, ws.bnd_off, ws.item_off);
  hipLaunchKernelGGL(k_plan_write, dim3((unsigned)nb), dim3(kPlanThreads), 0, s, rg, T,
                     (const uint32_t*)ws.plan_off, (const uint32_t*)ws.hdr, ws.bnd_off, ws.item_off, ws.order,
                     ws.fbase);
  const SplitPlanArgs sp{rg, ws.order, ws.hdr, ws.fbase, ws.split_tile, ws.split_cnt, ws.fitems, ws.fseg_cap,
                         ws.split_cap};
  hipLaunchKernelGGL(k_seg_items, dim3((unsigned)std::max(1, (int)ceil_div(T, kPlanThreads / 64))), dim3(kPlanThreads),
                     0, s, T, (const uint32_t*)ws.item_off, ws.items, empty_items, sp);
}

// the per-Gaussian staging offsets and the cleared staging rows
void launch_staging(int64_t n, const uint32_t* tiles, const RenderWs& ws, hipStream_t s) {
  const size_t nblk = n_goff_blocks(n);
  hipLaunchKernelGGL(k_goff_local, dim3((unsigned)nblk), dim3(kBlock), 0, s, n, tiles, ws.goff, ws.goff_blk);
  hipLaunchKernelGGL(k_goff_blocks, dim3(1), dim3(kPlanThreads), 0, s, (int64_t)nblk, ws.goff_blk, ws.hdr,
                     (uint64_t)ws.staging_cap);
  const unsigned fill_grid = (unsigned)std::max(1, cu_count() * 8);
  hipLaunchKernelGGL(k_clear_staging, dim3(fill_grid), dim3(kBlock), 0, s, (const uint32_t*)ws.hdr,
                     reinterpret_cast<float4*>(ws.staging), ws.staging_cap);
}

FwdArgs fwd_args(const CamK& cam, int64_t n, const gs_splat* splat, const uint32_t* vals, const uint32_t* ranges,
                 float bg0, float bg1, float bg2, float* image, float* T_final, uint32_t* last_contrib,
                 uint32_t* n_examined, uint64_t* blend_count, const RenderWs& ws) {
  FwdArgs a{};
  a.W = cam.W;
  a.H = cam.H;
  a.TX = cam.TX;
  a.T = cam.TX * cam.TY;
  a.n = n;
  a.splat = reinterpret_cast<const float4*>(splat);
  a.vals = vals;
  a.ranges = reinterpret_cast<const uint2*>(ranges);
  a.bg0 = bg0;
  a.bg1 = bg1;
  a.bg2 = bg2;
  a.image = image;
  a.T_final = T_final;
  a.last_contrib = last_contrib;
  a.n_examined = n_examined;
  a.blend_count = reinterpret_cast<unsigned long long*>(blend_count);
  a.bnd_off = ws.bnd_off;
  a.slots = ws.slots;
  a.masks = ws.masks;
  a.mask_cap = ws.mask_cap;
  a.order = ws.order;
  a.fbase = ws.fbase;
  return a;
}

LongArgs long_args(const RenderWs& ws) {
  return LongArgs{ws.split_tile, ws.split_cnt, ws.fitems, ws.fsum, ws.fstat, ws.fin, ws.pstate};
}

constexpr int kLongPerCu = 4;  // workgroups per CU of the split tiles' forward

// the split tiles' forward (its workgroups return at once when no tile is split)
void launch_long_forward(const FwdArgs& a, const RenderWs& ws, hipStream_t s) {
  const unsigned grid = (unsigned)std::max(1, cu_count() * kLongPerCu);
  hipLaunchKernelGGL(k_long_forward, dim3(grid), dim3(kBlock), 0, s, a, long_args(ws), ws.hdr);
}

BwdArgs bwd_args(const CamK& cam, int64_t n, const gs_splat* splat, const uint32_t* vals, const uint32_t* ranges,
                 float bg0, float bg1, float bg2, const float* T_final, const uint32_t* last_contrib,
                 const float* dLdI, const RenderWs& ws) {
  BwdArgs a{};
  a.W = cam.W;
  a.H = cam.H;
  a.TX = cam.TX;
  a.TY = cam.TY;
  a.n = n;
  a.splat = reinterpret_cast<const float4*>(splat);
  a.vals = vals;
  a.ranges = reinterpret_cast<const uint2*>(ranges);
  a.bg0 = bg0;
  a.bg1 = bg1;
  a.bg2 = bg2;
  a.T_final = T_final;
  a.last_contrib = last_contrib;
  a.dLdI = dLdI;
  a.bnd_off = ws.bnd_off;
  a.slots = ws.slots;
  a.masks = ws.masks;
  a.mask_cap = ws.mask_cap;
  a.goff = ws.goff;
  a.goff_blk = ws.goff_blk;
  a.staging = ws.staging;
  a.staging_cap = ws.staging_cap;
  a.fbase = ws.fbase;
  a.fin = ws.fin;
  return a;
}

}  // namespace

hipError_t launch_blend_forward(const CamK& cam, int64_t n, const gs_splat* splat, const uint32_t* vals,
                                const uint32_t* ranges, float bg0, float bg1, float bg2,
                                float* image, float* T_final, uint32_t* last_contrib,
                                uint32_t* n_examined, uint64_t* blend_count, const RenderWs& ws,
                                hipStream_t s) {
  const int T = cam.TX * cam.TY;
  launch_plan(T, reinterpret_cast<const uint2*>(ranges), ws, false, s);
  const FwdArgs a = fwd_args(cam, n, splat, vals, ranges, bg0, bg1, bg2, image, T_final, last_contrib, n_examined,
                             blend_count, ws);
  launch_long_forward(a, ws, s);
  const unsigned grid = (unsigned)std::max(1, std::min(T, cu_count() * kFwdPerCu));
  hipLaunchKernelGGL(k_blend_forward, dim3(grid), dim3(kBlock), 0, s, a, ws.hdr);
  return hipGetLastError();
}

hipError_t launch_blend_backward(const CamK& cam, int64_t n, const gs_splat* splat, const uint32_t* tiles,
                                 const uint32_t* vals, const uint32_t* ranges, float bg0,
                                 float bg1, float bg2, const float* T_final,
                                 const uint32_t* last_contrib, const float* dLdI, float* grad2d,
                                 const RenderWs& ws, hipStream_t s) {
  const int T = cam.TX * cam.TY;
  if (n <= 0) return hipSuccess;
  launch_staging(n, tiles, ws, s);
  hipError_t e = launch_fill_u32(ws.hdr + kHdrBwdNext, 1, 0u, s);  // work-item counter
  if (e != hipSuccess) return e;
  // enough persistent workgroups to fill every CU; never more than the items can be
  const int64_t most = (int64_t)T + ws.slots_cap;
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(most, (int64_t)cu_count() * 8));
  const BwdArgs a = bwd_args(cam, n, splat, vals, ranges, bg0, bg1, bg2, T_final, last_contrib, dLdI, ws);
  hipLaunchKernelGGL(k_blend_backward, dim3(grid), dim3(kBlock), 0, s, a, ws.hdr, (const uint2*)ws.items);
  if (grad2d)  // else the sums stay staged for the preprocess backward
    hipLaunchKernelGGL(k_gather_grad2d, dim3((unsigned)ceil_div(n, (int64_t)kBlock)), dim3(kBlock), 0, s, n,
                       tiles, (const uint32_t*)ws.goff, (const uint32_t*)ws.goff_blk, (const float*)ws.staging,
                       ws.staging_cap, grad2d);
  return hipGetLastError();
}

hipError_t launch_step_plan(const CamK& cam, int64_t n, const uint32_t* tiles, const uint32_t* ranges,
                            const RenderWs& ws, hipStream_t s) {
  launch_plan(cam.TX * cam.TY, reinterpret_cast<const uint2*>(ranges), ws, true, s);
  if (n > 0) launch_staging(n, tiles, ws, s);
  return hipGetLastError();
}

hipError_t launch_blend_step(const CamK& cam, int64_t n, const gs_splat* splat, const uint32_t* tiles,
                             const uint32_t* vals, const uint32_t* ranges, float bg0, float bg1, float bg2,
                             const float* target, float* image, float* T_final, uint32_t* last_contrib,
                             uint32_t* n_examined, uint64_t* blend_count, float* loss, float* dLdI,
                             float* grad2d, const RenderWs& ws, hipStream_t s) {
  const int T = cam.TX * cam.TY;
  FwdArgs fa = fwd_args(cam, n, splat, vals, ranges, bg0, bg1, bg2, image, T_final, last_contrib, n_examined,
                        blend_count, ws);
  const int64_t count = 3 * (int64_t)cam.W * cam.H;
  fa.target = target;
  fa.dLdI = dLdI;
  fa.loss_part = ws.loss_part;
  fa.inv_n = (float)(1.0 / (double)count);
  const BwdArgs ba = bwd_args(cam, n, splat, vals, ranges, bg0, bg1, bg2, T_final, last_contrib, dLdI, ws);
  // every workgroup resident at once: the backward wants all the occupancy it can get
  static int resident[64];
  const int per_cu = resident_per_cu(reinterpret_cast<const void*>(k_blend_step), resident);
  const unsigned grid = (unsigned)std::max(1, cu_count() * per_cu);
  const uint32_t fwd_workers = (uint32_t)std::max(1, std::min(per_cu, kStepFwdPerCu) * cu_count());
  launch_long_forward(fa, ws, s);
  hipLaunchKernelGGL(k_blend_step, dim3(grid), dim3(kBlock), 0, s, fa, ba, ws.hdr, ws.items,
                     (const uint32_t*)ws.item_off, fwd_workers);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (grad2d && n > 0)
    hipLaunchKernelGGL(k_gather_grad2d, dim3((unsigned)ceil_div(n, (int64_t)kBlock)), dim3(kBlock), 0, s, n,
                       tiles, (const uint32_t*)ws.goff, (const uint32_t*)ws.goff_blk, (const float*)ws.staging,
                       ws.staging_cap, grad2d);
  return launch_loss_sum(T, ws.loss_part, 1.0 / (double)count, loss, s);
}

}  // namespace gsmi
