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
// Work decomposition.  One 256-thread workgroup per tile; wave w owns the 8x8 quadrant
// (w & 1, w >> 1).  The list is consumed in batches of 256 records staged in LDS (one gather
// per (tile, Gaussian)).  Each record gets a 4-bit mask of the quadrants its alpha >= 1/255
// ellipse can reach (a conservative bound), and each wave walks only the records of its bit
// with a scalar bit-scan loop, so a wave spends no VALU work on Gaussians that cannot touch
// its pixels -- the per-pixel results are those of the plain walk.  Workgroups are mapped to
// tiles so that each of the 8 XCDs (each with its own L2) renders a contiguous band of tiles.
// Bound: VALU / transcendental (one exp per evaluated pair), not HBM.
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

// Quadrants (bit q = qx + 2 qy, 8x8 each) of the tile at (x_t, y_t) whose pixel centres can
// satisfy o e^power >= 1/255.  That region is the ellipse d^T Q d <= tau, tau = 2 ln(255 o),
// whose bounding box has half-widths sqrt(tau C/det), sqrt(tau A/det); tau and the box are
// widened so float32 rounding of the per-pixel test can never fall outside.
__device__ __forceinline__ uint32_t quadrant_mask(float u, float v, float A, float B, float C, float o,
                                                  int x_t, int y_t) {
  if (!(o >= kAlphaMin)) return 0u;
  const float tau = 2.0f * __logf(255.0f * o) * 1.001f + 1e-3f;
  const float det = A * C - B * B;
  if (!(det > 0.0f) || !__builtin_isfinite(det) || !__builtin_isfinite(u) || !__builtin_isfinite(v))
    return 0xFu;
  const float hx = sqrtf(tau * C / det) * 1.001f + 0.01f;
  const float hy = sqrtf(tau * A / det) * 1.001f + 0.01f;
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float xlo = (float)(x_t + (q & 1) * 8) + 0.5f, xhi = xlo + 7.0f;
    const float ylo = (float)(y_t + (q >> 1) * 8) + 0.5f, yhi = ylo + 7.0f;
    if (u + hx >= xlo && u - hx <= xhi && v + hy >= ylo && v - hy <= yhi) m |= 1u << q;
  }
  return m;
}

// Workgroup -> tile: consecutive workgroups go round-robin to the 8 XCDs, so XCD x receives
// workgroups x, x+8, ...; give it the contiguous tile band [prefix(x), prefix(x+1)).
__device__ __forceinline__ int xcd_tile(int b, int T) {
  const int x = b & 7, k = b >> 3;
  int pre = 0;
  for (int y = 0; y < x; ++y) pre += (T - y + 7) >> 3;
  return pre + k;
}

// DPP sum over the 16 lanes of a row; every lane of the row gets the row sum.
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));  // xor 1
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));  // xor 2
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false)); // half-row mirror
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false)); // row mirror
  return x;
}

struct Staged {
  float4 geo[kBatch];   // u, v, -A/2, -B
  float4 col[kBatch];   // -C/2, o, r, g
  float b[kBatch];
  uint32_t mask[kBatch];
  uint32_t gid[kBatch];
};

__device__ __forceinline__ void stage_entry(Staged& S, int e, const float4* __restrict__ splat,
                                            uint32_t i, int64_t n, int x_t, int y_t) {
  if ((int64_t)i >= n) {  // never for lists from gs_bin_and_sort; keeps reads in bounds
    S.mask[e] = 0u;
    S.gid[e] = 0u;
    return;
  }
  const float4 q0 = splat[3 * (int64_t)i];
  const float4 q1 = splat[3 * (int64_t)i + 1];
  const float4 q2 = splat[3 * (int64_t)i + 2];
  S.geo[e] = make_float4(q0.x, q0.y, -0.5f * q1.x, -q1.y);
  S.col[e] = make_float4(-0.5f * q1.z, q1.w, q2.x, q2.y);
  S.b[e] = q2.z;
  S.mask[e] = quadrant_mask(q0.x, q0.y, q1.x, q1.y, q1.z, q1.w, x_t, y_t);
  S.gid[e] = i;
}

__global__ __launch_bounds__(kBlock) void k_blend_forward(
    int W, int H, int TX, int T, int64_t n, const float4* __restrict__ splat,
    const uint32_t* __restrict__ vals, const uint2* __restrict__ ranges, float bg0, float bg1,
    float bg2, float* __restrict__ image,
    float* __restrict__ T_final, uint32_t* __restrict__ last_contrib,
    uint32_t* __restrict__ n_examined, unsigned long long* __restrict__ blend_count) {
  __shared__ Staged S;
  __shared__ unsigned long long s_ex[4];
  const int tile = xcd_tile(blockIdx.x, T);
  const int tx = tile % TX, ty = tile / TX;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int px = tx * kTile + (w & 1) * 8 + (lane & 7);
  const int py = ty * kTile + (w >> 1) * 8 + (lane >> 3);
  const bool inside = px < W && py < H;
  const float pxc = (float)px + 0.5f, pyc = (float)py + 0.5f;
  const uint2 rg = ranges[tile];
  const uint32_t start = rg.x, end = rg.y;

  float Tr = 1.0f, c0 = 0.f, c1 = 0.f, c2 = 0.f;
  uint32_t last = 0, examined = end - start;
  bool done = !inside;
  const uint32_t wbit = 1u << w;

  for (uint32_t b0 = start; b0 < end; b0 += kBatch) {
    if (__syncthreads_count(!done) == 0) break;
    const uint32_t j = b0 + tid;
    if (j < end) stage_entry(S, tid, splat, vals[j], n, tx * kTile, ty * kTile);
    else S.mask[tid] = 0u;
    __syncthreads();
    const int cnt = (int)min((uint32_t)kBatch, end - b0);
    if (__ballot(!done) != 0ull) {
      for (int c = 0; c * 64 < cnt; ++c) {
        unsigned long long M = __ballot((S.mask[c * 64 + lane] & wbit) != 0u);
        while (M) {
          const int e = c * 64 + __builtin_ctzll(M);
          M &= M - 1ull;
          const float4 g = S.geo[e];
          const float4 cl = S.col[e];
          const float bb = S.b[e];
          if (!done) {
            const float dx = pxc - g.x, dy = pyc - g.y;
            const float power = eval_power(g.z, g.w, cl.x, dx, dy);
            if (power <= 0.0f) {
              const float alpha = fminf(kAlphaMax, eval_oG(cl.y, power));
              if (alpha >= kAlphaMin) {
                const float Tn = Tr * (1.0f - alpha);
                const uint32_t pos = b0 + (uint32_t)e - start + 1u;
                if (Tn < kTMin) {
                  done = true;
                  examined = pos;
                } else {
                  const float wt = alpha * Tr;
                  c0 += cl.z * wt;
                  c1 += cl.w * wt;
                  c2 += bb * wt;
                  Tr = Tn;
                  last = pos;
                }
              }
            }
          }
          if (__ballot(!done) == 0ull) { M = 0ull; c = 4; }
        }
      }
    }
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
    unsigned long long ex = inside ? examined : 0u;
    for (int o = 32; o > 0; o >>= 1) ex += __shfl_xor(ex, o, 64);
    if (lane == 0) s_ex[w] = ex;
    __syncthreads();
    if (tid == 0) atomicAdd(blend_count, s_ex[0] + s_ex[1] + s_ex[2] + s_ex[3]);
  }
}

__global__ __launch_bounds__(kBlock) void k_blend_backward(
    int W, int H, int TX, int T, int64_t n, int64_t ld, const float4* __restrict__ splat,
    const uint32_t* __restrict__ vals, const uint2* __restrict__ ranges, float bg0, float bg1,
    float bg2, const float* __restrict__ T_final, const uint32_t* __restrict__ last_contrib,
    const float* __restrict__ dLdI, float* __restrict__ grad2d) {
  __shared__ Staged S;
  __shared__ float s_grad[9][kBatch];
  __shared__ uint32_t s_max;
  const int tile = xcd_tile(blockIdx.x, T);
  const int tx = tile % TX, ty = tile / TX;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int px = tx * kTile + (w & 1) * 8 + (lane & 7);
  const int py = ty * kTile + (w >> 1) * 8 + (lane >> 3);
  const bool inside = px < W && py < H;
  const float pxc = (float)px + 0.5f, pyc = (float)py + 0.5f;
  const uint2 rg = ranges[tile];
  const uint32_t start = rg.x;

  float Tr = 0.f, Tfin = 0.f, g0 = 0.f, g1 = 0.f, g2 = 0.f;
  uint32_t last = 0;
  if (inside) {
    const int64_t p = (int64_t)py * W + px;
    Tfin = Tr = T_final[p];
    last = last_contrib[p];
    g0 = dLdI[3 * p];
    g1 = dLdI[3 * p + 1];
    g2 = dLdI[3 * p + 2];
  }
  const float bgdot = bg0 * g0 + bg1 * g1 + bg2 * g2;
  float S0 = 0.f, S1 = 0.f, S2 = 0.f;  // colour accumulated behind the current entry, / T_{k+1}

  if (tid == 0) s_max = 0u;
#pragma unroll
  for (int r = 0; r < 9; ++r) s_grad[r][tid] = 0.f;
  __syncthreads();
  {
    uint32_t m = last;
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor(m, o, 64));
    if (lane == 0) atomicMax(&s_max, m);
  }
  __syncthreads();
  const uint32_t end_eff = start + min(s_max, rg.y - start);
  const uint32_t wbit = 1u << w;

  for (uint32_t b1 = end_eff; b1 > start;) {
    const uint32_t b0 = b1 - start > (uint32_t)kBatch ? b1 - kBatch : start;
    const int cnt = (int)(b1 - b0);
    __syncthreads();  // the previous batch's flush has read the staged entries
    if (tid < cnt) stage_entry(S, tid, splat, vals[b0 + tid], n, tx * kTile, ty * kTile);
    else S.mask[tid] = 0u;
    __syncthreads();
    for (int c = (cnt - 1) >> 6; c >= 0; --c) {
      unsigned long long M = __ballot((S.mask[c * 64 + lane] & wbit) != 0u);
      while (M) {
        const int hb = 63 - __builtin_clzll(M);
        M &= ~(1ull << hb);
        const int e = c * 64 + hb;
        const uint32_t pos = b0 + (uint32_t)e - start;  // 0-based list position
        const float4 g = S.geo[e];
        const float4 cl = S.col[e];
        const float bb = S.b[e];
        float v_u = 0.f, v_v = 0.f, v_a = 0.f, v_b = 0.f, v_c = 0.f, v_o = 0.f, v_r = 0.f,
              v_g = 0.f, v_bl = 0.f;
        bool contrib = false;
        if (pos < last) {
          const float dx = pxc - g.x, dy = pyc - g.y;
          const float power = eval_power(g.z, g.w, cl.x, dx, dy);
          if (power <= 0.0f) {
            const float G = __expf(power);
            const float oG = __fmul_rn(cl.y, G);  // the same operations as eval_oG
            const float alpha = fminf(kAlphaMax, oG);
            if (alpha >= kAlphaMin) {
              contrib = true;
              const float om = 1.0f - alpha;
              const float Tk = Tr / om;  // transmittance in front of this entry
              const float wt = alpha * Tk;
              v_r = wt * g0;
              v_g = wt * g1;
              v_bl = wt * g2;
              const float dL_dalpha =
                  Tk * ((cl.z - S0) * g0 + (cl.w - S1) * g1 + (bb - S2) * g2) - Tfin * bgdot / om;
              S0 = alpha * cl.z + om * S0;
              S1 = alpha * cl.w + om * S1;
              S2 = alpha * bb + om * S2;
              Tr = Tk;
              if (oG <= kAlphaMax) {  // unclamped: alpha = o G
                const float dpow = oG * dL_dalpha;
                v_o = G * dL_dalpha;
                // A = -2 nA, B = -nB, C = -2 nC
                v_a = -0.5f * dx * dx * dpow;
                v_b = -dx * dy * dpow;
                v_c = -0.5f * dy * dy * dpow;
                v_u = -(2.0f * g.z * dx + g.w * dy) * dpow;
                v_v = -(g.w * dx + 2.0f * cl.x * dy) * dpow;
              }
            }
          }
        }
        const unsigned long long act = __ballot(contrib);
        if (act) {
          const float vals9[9] = {v_u, v_v, v_a, v_b, v_c, v_o, v_r, v_g, v_bl};
          const bool leader = (lane & 15) == 0 && ((act >> (lane & 48)) & 0xFFFFull) != 0ull;
#pragma unroll
          for (int r = 0; r < 9; ++r) {
            const float s = row_sum16(vals9[r]);
            if (leader) atomicAdd(&s_grad[r][e], s);
          }
        }
      }
    }
    __syncthreads();
    if (tid < cnt) {
      const uint32_t i = S.gid[tid];
#pragma unroll
      for (int r = 0; r < 9; ++r) {
        const float v = s_grad[r][tid];
        if (v != 0.f && (int64_t)i < n) unsafeAtomicAdd(grad2d + (int64_t)r * ld + i, v);
        s_grad[r][tid] = 0.f;
      }
    }
    b1 = b0;
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
