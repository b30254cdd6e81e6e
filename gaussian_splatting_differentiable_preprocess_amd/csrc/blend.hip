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
// independent (no workgroup barrier); the backward's share per-chunk gradient sums in LDS.
// Workgroup b renders tile b: the hardware deals consecutive workgroups to the 8 XCDs in turn,
// which spreads the (very uneven) per-tile work evenly over them.  Bound: VALU /
// transcendental and LDS, not HBM.
#include "gsmi_internal.h"

namespace gsmi {

namespace {

constexpr int kBatch = kBlock;
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

// One DPP step x += permute(x) (old value 0 = identity of the add, so the move folds into
// v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sums each of N values over the 16 lanes of every row (all lanes of a row get the row
// sum).  The steps are interleaved across the N values so consecutive DPP reads never
// depend on the instruction just before them.
template <int N>
__device__ __forceinline__ void row_sum16(float* v) {
#pragma unroll
  for (int q = 0; q < N; ++q) v[q] = dpp_add<0xB1>(v[q]);   // quad_perm [1,0,3,2]: xor 1
#pragma unroll
  for (int q = 0; q < N; ++q) v[q] = dpp_add<0x4E>(v[q]);   // quad_perm [2,3,0,1]: xor 2
#pragma unroll
  for (int q = 0; q < N; ++q) v[q] = dpp_add<0x141>(v[q]);  // row_half_mirror
#pragma unroll
  for (int q = 0; q < N; ++q) v[q] = dpp_add<0x140>(v[q]);  // row_mirror
}

constexpr int kChunk = 64;  // records staged per chunk (one per lane)

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
    const float tau = 2.0f * __logf(255.0f * o) * 1.001f + 1e-3f;
    hx = sqrtf(tau * C / det) * 1.001f + 0.01f;
    hy = sqrtf(tau * A / det) * 1.001f + 0.01f;
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
// holds record e's box; COL[x] / ROW[y] are ballots over the records.
__device__ __forceinline__ unsigned long long lane_mask(const Box& b, int lx, int ly) {
  unsigned long long col = 0ull, row = 0ull;
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const unsigned long long c = __ballot(b.x0 <= x && x <= b.x1);
    col = (lx == x) ? c : col;
  }
#pragma unroll
  for (int y = 0; y < 8; ++y) {
    const unsigned long long r = __ballot(b.y0 <= y && y <= b.y1);
    row = (ly == y) ? r : row;
  }
  return col & row;
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

__device__ __forceinline__ uint32_t load_gid(const uint32_t* __restrict__ vals, uint32_t j, uint32_t end) {
  return j < end ? vals[j] : 0xFFFFFFFFu;
}

__device__ __forceinline__ Raw load_raw(const float4* __restrict__ splat, uint32_t gid, int64_t n) {
  Raw r;
  r.gid = gid;
  if ((int64_t)gid < n) {  // lists from gs_bin_and_sort are in range; 0xFFFFFFFF past the end
    const float* rec = reinterpret_cast<const float*>(splat + 3 * (int64_t)gid);
    r.uv = *reinterpret_cast<const float2*>(rec);
    r.abco = *reinterpret_cast<const float4*>(rec + 4);
    r.rgb = *reinterpret_cast<const float3*>(rec + 8);
  } else {
    r.uv = make_float2(0.f, 0.f);
    r.abco = make_float4(0.f, 0.f, 0.f, 0.f);  // opacity 0: empty box
    r.rgb = make_float3(0.f, 0.f, 0.f);
  }
  return r;
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

__global__ __launch_bounds__(kBlock) void k_blend_forward(
    int W, int H, int TX, int T, int64_t n, const float4* __restrict__ splat,
    const uint32_t* __restrict__ vals, const uint2* __restrict__ ranges, float bg0, float bg1,
    float bg2, float* __restrict__ image, float* __restrict__ T_final, uint32_t* __restrict__ last_contrib,
    uint32_t* __restrict__ n_examined, unsigned long long* __restrict__ blend_count) {
  __shared__ Chunk stg[4];
  const int tile = blockIdx.x;  // consecutive tiles land on different XCDs: balances the load
  const int tx = tile % TX, ty = tile / TX;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  Chunk& S = stg[w];
  const int lx = lane & 7, ly = lane >> 3;
  const int xq = tx * kTile + (w & 1) * 8, yq = ty * kTile + (w >> 1) * 8;  // quadrant origin
  const int px = xq + lx, py = yq + ly;
  const bool inside = px < W && py < H;
  const float pxc = (float)px + 0.5f, pyc = (float)py + 0.5f;
  const uint2 rg = ranges[tile];
  const uint32_t start = rg.x, end = rg.y;

  float Tr = 1.0f, c0 = 0.f, c1 = 0.f, c2 = 0.f;
  uint32_t last = 0, examined = end - start, blended = 0;
  bool done = !inside;

  uint32_t gnext = load_gid(vals, start + lane, end);
  Raw cur = load_raw(splat, gnext, n);
  gnext = load_gid(vals, start + kChunk + lane, end);
  for (uint32_t b0 = start; b0 < end; b0 += kChunk) {
    if (__ballot(!done) == 0ull) break;
    const Raw nxt = load_raw(splat, gnext, n);  // next chunk in flight
    gnext = load_gid(vals, b0 + 2 * kChunk + lane, end);
    put(S, lane, cur);
    const Box bx = alpha_box(cur.uv.x, cur.uv.y, cur.abco.x, cur.abco.y, cur.abco.z, cur.abco.w, xq, yq);
    // every lane takes part in the ballots: lane e holds record e's box
    unsigned long long m = lane_mask(bx, lx, ly);
    if (done) m = 0ull;
    wave_sync_lds();
    const uint32_t base = b0 - start + 1u;  // 1-based position of slot 0
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
          m = 0ull;
        } else {
          const float wt = alpha * Tr;
          c0 += cl.z * wt;
          c1 += cl.w * wt;
          c2 += bb * wt;
          Tr = Tn;
          last = pos;
          ++blended;
        }
      }
    }
    wave_sync_lds();  // this chunk's reads finish before the next chunk is staged
    cur = nxt;
  }

  if (inside) {
    const int64_t p = (int64_t)py * W + px;
    image[3 * p + 0] = c0 + Tr * bg0;
    image[3 * p + 1] = c1 + Tr * bg1;
    image[3 * p + 2] = c2 + Tr * bg2;
    T_final[p] = Tr;
    last_contrib[p] = last;
    if (n_examined) n_examined[p] = examined;
  }
  if (blend_count) {
    unsigned long long ex = inside ? examined : 0u, lc = last, bl = blended;
    for (int o = 32; o > 0; o >>= 1) {
      ex += __shfl_xor(ex, o, 64);
      lc += __shfl_xor(lc, o, 64);
      bl += __shfl_xor(bl, o, 64);
    }
    // one atomic per counter and non-empty tile: same-address atomics from every wave of
    // the image serialise and would cost more than the blending of a light view
    __shared__ unsigned long long part[3][4];
    if (lane == 0) {
      part[0][w] = ex;
      part[1][w] = lc;
      part[2][w] = bl;
    }
    __syncthreads();
    if (tid < 3) {
      const unsigned long long x = (part[tid][0] + part[tid][1]) + (part[tid][2] + part[tid][3]);
      if (x != 0ull) atomicAdd(blend_count + tid, x);
    }
  }
}

__global__ __launch_bounds__(kBlock) void k_blend_backward(
    int W, int H, int TX, int T, int64_t n, int64_t ld, const float4* __restrict__ splat,
    const uint32_t* __restrict__ vals, const uint2* __restrict__ ranges, float bg0, float bg1,
    float bg2, const float* __restrict__ T_final, const uint32_t* __restrict__ last_contrib,
    const float* __restrict__ dLdI, float* __restrict__ grad2d) {
  __shared__ Chunk stg[4];                // per quadrant wave: its current chunk
  __shared__ float accs[4][9][kChunk];    // per quadrant wave: gradient sums of the chunk's records
  const int tile = blockIdx.x;  // consecutive tiles land on different XCDs: balances the load
  const int tx = tile % TX, ty = tile / TX;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  Chunk& S = stg[w];
  float(&acc)[9][kChunk] = accs[w];
  const int lx = lane & 7, ly = lane >> 3;
  const int xq = tx * kTile + (w & 1) * 8, yq = ty * kTile + (w >> 1) * 8;
  const int px = xq + lx, py = yq + ly;
  const bool inside = px < W && py < H;
  const float pxc = (float)px + 0.5f, pyc = (float)py + 0.5f;
  const uint2 rg = ranges[tile];
  const uint32_t start = rg.x;

  float Tr = 0.f, g0 = 0.f, g1 = 0.f, g2 = 0.f, bgT = 0.f;
  uint32_t last = 0;
  if (inside) {
    const int64_t p = (int64_t)py * W + px;
    Tr = T_final[p];
    last = last_contrib[p];
    g0 = dLdI[3 * p];
    g1 = dLdI[3 * p + 1];
    g2 = dLdI[3 * p + 2];
    bgT = Tr * (bg0 * g0 + bg1 * g1 + bg2 * g2);
  }
  float S0 = 0.f, S1 = 0.f, S2 = 0.f;  // colour accumulated behind the current entry, / T_{k+1}

  // this wave walks [start, start + its largest last_contrib), back to front
  uint32_t mx = last;
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor(mx, o, 64));
  const uint32_t end_eff = start + min(mx, rg.y - start);
  const uint32_t nchunks = (end_eff - start + kChunk - 1) / kChunk;
  // chunk c covers [lo_c, hi_c) with hi_c = end_eff - 64 c
  auto lo_of = [&](uint32_t c) -> uint32_t {
    const uint32_t hi = end_eff - c * kChunk;
    return hi - start > (uint32_t)kChunk ? hi - kChunk : start;
  };

  uint32_t gnext = nchunks > 0 ? load_gid(vals, lo_of(0) + lane, end_eff) : 0xFFFFFFFFu;
  Raw cur = load_raw(splat, gnext, n);
  gnext = nchunks > 1 ? load_gid(vals, lo_of(1) + lane, end_eff - kChunk) : 0xFFFFFFFFu;
  for (uint32_t c = 0; c < nchunks; ++c) {
    const uint32_t lo = lo_of(c);
    const Raw nxt = load_raw(splat, gnext, n);  // next chunk in flight
    gnext = c + 2 < nchunks ? load_gid(vals, lo_of(c + 2) + lane, end_eff - (c + 2) * kChunk) : 0xFFFFFFFFu;
    put(S, lane, cur);
#pragma unroll
    for (int k = 0; k < 9; ++k) acc[k][lane] = 0.f;
    const Box bx = alpha_box(cur.uv.x, cur.uv.y, cur.abco.x, cur.abco.y, cur.abco.z, cur.abco.w, xq, yq);
    unsigned long long m = lane_mask(bx, lx, ly);  // all lanes take part in the ballots
    const unsigned long long touched = __ballot(bx.x0 <= bx.x1 && bx.y0 <= bx.y1);
    wave_sync_lds();
    const uint32_t base = lo - start;  // 0-based position of slot 0
    while (m) {  // this lane's records, back to front
      const int e = highest_bit(m);
      m &= ~(1ull << e);
      const uint32_t pos = base + (uint32_t)e;
      if (pos >= last) continue;  // behind the pixel's last blended entry
      const float4 g = S.geo[e];
      const float4 cl = S.col[e];
      const float cb = S.b[e];
      const float dx = pxc - g.x, dy = pyc - g.y;
      const float power = eval_power(g.z, g.w, cl.x, dx, dy);
      const float G = __expf(power);
      const float oG = __fmul_rn(cl.y, G);  // the same operations as eval_oG
      const float alpha = fminf(kAlphaMax, oG);
      if (!(power <= 0.0f && alpha >= kAlphaMin)) continue;
      const float om = 1.0f - alpha;
      const float rom = __builtin_amdgcn_rcpf(om);  // om >= 0.01
      const float Tk = Tr * rom;                    // transmittance in front of this entry
      const float wt = alpha * Tk;
      const float cr = cl.z, cg = cl.w;
      const float dL_dalpha = Tk * ((cr - S0) * g0 + (cg - S1) * g1 + (cb - S2) * g2) - bgT * rom;
      S0 = alpha * cr + om * S0;
      S1 = alpha * cg + om * S1;
      S2 = alpha * cb + om * S2;
      Tr = Tk;
      atomicAdd(&acc[6][e], wt * g0);
      atomicAdd(&acc[7][e], wt * g1);
      atomicAdd(&acc[8][e], wt * g2);
      if (oG <= kAlphaMax) {  // unclamped: alpha = o G depends on o and power
        const float dpow = oG * dL_dalpha;
        atomicAdd(&acc[0][e], -(2.0f * g.z * dx + g.w * dy) * dpow);  // A = -2 nA, B = -nB
        atomicAdd(&acc[1][e], -(g.w * dx + 2.0f * cl.x * dy) * dpow);  // C = -2 nC
        atomicAdd(&acc[2][e], -0.5f * dx * dx * dpow);
        atomicAdd(&acc[3][e], -dx * dy * dpow);
        atomicAdd(&acc[4][e], -0.5f * dy * dy * dpow);
        atomicAdd(&acc[5][e], G * dL_dalpha);
      }
    }
    wave_sync_lds();
    if (((touched >> lane) & 1ull) && (int64_t)cur.gid < n) {
#pragma unroll
      for (int k = 0; k < 9; ++k) {
        const float x = acc[k][lane];
        if (x != 0.f) unsafeAtomicAdd(grad2d + (int64_t)k * ld + cur.gid, x);
      }
    }
    wave_sync_lds();  // the flush has read acc before the next chunk clears it
    cur = nxt;
  }
}

}  // namespace

hipError_t launch_blend_forward(const CamK& cam, int64_t n, const gs_splat* splat, const uint32_t* vals,
                                const uint32_t* ranges, float bg0, float bg1, float bg2,
                                float* image, float* T_final, uint32_t* last_contrib,
                                uint32_t* n_examined, uint64_t* blend_count, hipStream_t s) {
  const int T = cam.TX * cam.TY;
  hipLaunchKernelGGL(k_blend_forward, dim3(T), dim3(kBlock), 0, s, cam.W, cam.H, cam.TX, T, n,
                     reinterpret_cast<const float4*>(splat), vals, reinterpret_cast<const uint2*>(ranges),
                     bg0, bg1, bg2, image, T_final, last_contrib, n_examined,
                     reinterpret_cast<unsigned long long*>(blend_count));
  return hipGetLastError();
}

hipError_t launch_blend_backward(const CamK& cam, int64_t n, int64_t ld, const gs_splat* splat,
                                 const uint32_t* vals, const uint32_t* ranges, float bg0,
                                 float bg1, float bg2, const float* T_final,
                                 const uint32_t* last_contrib, const float* dLdI, float* grad2d,
                                 hipStream_t s) {
  const int T = cam.TX * cam.TY;
  hipLaunchKernelGGL(k_blend_backward, dim3(T), dim3(kBlock), 0, s, cam.W, cam.H, cam.TX, T, n, ld,
                     reinterpret_cast<const float4*>(splat), vals, reinterpret_cast<const uint2*>(ranges),
                     bg0, bg1, bg2, T_final, last_contrib, dLdI, grad2d);
  return hipGetLastError();
}

}  // namespace gsmi
