// Per-Gaussian preprocess (EWA projection + SH colour) and its backward, for gfx950.
//
// Follows "Scaling 3D Gaussian Splatting with Distributed Compute" (the Gaussian parameter
// list; walkthrough steps "Project locally" and "Evaluate spherical harmonics before
// communicating") with the standard 3D-GS / EWA-splatting formulas for each stage:
//   scale = exp(log-scale), opacity = sigmoid(logit), rotation from the normalised quaternion,
//   Sigma = R S S^T R^T, p = Rc mu + t, (u, v) = (fx x/z + cx, fy y/z + cy),
//   S2 = J Rc Sigma Rc^T J^T + 0.3 I (J at the guard-band clamped x/z, y/z),
//   conic = S2^-1, radii = ceil(3 sqrt(S2_ii)), colour = max(0.5 + sum_k Y_k(dir) f_k, 0).
//
// Layout: params are planar rows of stride ld (coalesced: lane i reads element i of each
// row).  One thread per Gaussian, 256-thread workgroups; the 48-byte records are staged in
// LDS so each workgroup writes its 12 KB of records with fully coalesced 16-byte stores.
// The kernels are HBM-bound: forward reads 4R B and writes 56 B per Gaussian; the backward
// reads 4R + 36 B and writes 4R B (with fused Adam: reads 12R + 36 B, writes 12R B).
#include "gsmi_internal.h"

namespace gsmi {

namespace {

// Real spherical harmonics with the Condon-Shortley phase, l = 0..3, m = -l..l, for a unit
// vector.  Constants from their closed forms:
//   C0 = 1/(2 sqrt(pi)); C1 = sqrt(3/(4 pi));
//   C2 = {sqrt(15/pi)/2, sqrt(15/pi)/2, sqrt(5/pi)/4, sqrt(15/pi)/2, sqrt(15/pi)/4};
//   C3 = {sqrt(35/(2pi))/4, sqrt(105/pi)/2, sqrt(21/(2pi))/4, sqrt(7/pi)/4,
//         sqrt(21/(2pi))/4, sqrt(105/pi)/4, sqrt(35/(2pi))/4}.
constexpr float kC0 = 0.28209479177387814f;
constexpr float kC1 = 0.4886025119029199f;
constexpr float kC2a = 1.0925484305920792f;  // sqrt(15/pi)/2
constexpr float kC2b = 0.31539156525252005f; // sqrt(5/pi)/4
constexpr float kC2c = 0.5462742152960396f;  // sqrt(15/pi)/4
constexpr float kC3a = 0.5900435899266435f;  // sqrt(35/(2pi))/4
constexpr float kC3b = 2.890611442640554f;   // sqrt(105/pi)/2
constexpr float kC3c = 0.4570457994644658f;  // sqrt(21/(2pi))/4
constexpr float kC3d = 0.3731763325901154f;  // sqrt(7/pi)/4
constexpr float kC3e = 1.445305721320277f;   // sqrt(105/pi)/4

__device__ __forceinline__ void sh_eval(int deg, float x, float y, float z, float* Y) {
  Y[0] = kC0;
  if (deg < 1) return;
  Y[1] = -kC1 * y;
  Y[2] = kC1 * z;
  Y[3] = -kC1 * x;
  if (deg < 2) return;
  const float xx = x * x, yy = y * y, zz = z * z;
  Y[4] = kC2a * x * y;
  Y[5] = -kC2a * y * z;
  Y[6] = kC2b * (2.0f * zz - xx - yy);
  Y[7] = -kC2a * x * z;
  Y[8] = kC2c * (xx - yy);
  if (deg < 3) return;
  Y[9] = -kC3a * y * (3.0f * xx - yy);
  Y[10] = kC3b * x * y * z;
  Y[11] = -kC3c * y * (4.0f * zz - xx - yy);
  Y[12] = kC3d * z * (2.0f * zz - 3.0f * xx - 3.0f * yy);
  Y[13] = -kC3c * x * (4.0f * zz - xx - yy);
  Y[14] = kC3e * z * (xx - yy);
  Y[15] = -kC3a * x * (xx - 3.0f * yy);
}

// Adds w_k * grad Y_k(x, y, z) (gradient of the polynomial forms above) into g.
__device__ __forceinline__ void sh_grad_acc(int deg, float x, float y, float z, const float* w,
                                            float g[3]) {
  if (deg < 1) return;
  g[0] += -kC1 * w[3];
  g[1] += -kC1 * w[1];
  g[2] += kC1 * w[2];
  if (deg < 2) return;
  const float xx = x * x, yy = y * y, zz = z * z;
  // Y4 = C2a xy, Y5 = -C2a yz, Y6 = C2b(2z^2-x^2-y^2), Y7 = -C2a xz, Y8 = C2c(x^2-y^2)
  g[0] += kC2a * y * w[4] - 2.0f * kC2b * x * w[6] - kC2a * z * w[7] + 2.0f * kC2c * x * w[8];
  g[1] += kC2a * x * w[4] - kC2a * z * w[5] - 2.0f * kC2b * y * w[6] - 2.0f * kC2c * y * w[8];
  g[2] += -kC2a * y * w[5] + 4.0f * kC2b * z * w[6] - kC2a * x * w[7];
  if (deg < 3) return;
  // Y9 = -C3a(3x^2 y - y^3)
  g[0] += -kC3a * 6.0f * x * y * w[9];
  g[1] += -kC3a * 3.0f * (xx - yy) * w[9];
  // Y10 = C3b xyz
  g[0] += kC3b * y * z * w[10];
  g[1] += kC3b * x * z * w[10];
  g[2] += kC3b * x * y * w[10];
  // Y11 = -C3c(4yz^2 - x^2 y - y^3)
  g[0] += kC3c * 2.0f * x * y * w[11];
  g[1] += -kC3c * (4.0f * zz - xx - 3.0f * yy) * w[11];
  g[2] += -kC3c * 8.0f * y * z * w[11];
  // Y12 = C3d(2z^3 - 3x^2 z - 3y^2 z)
  g[0] += -kC3d * 6.0f * x * z * w[12];
  g[1] += -kC3d * 6.0f * y * z * w[12];
  g[2] += kC3d * (6.0f * zz - 3.0f * xx - 3.0f * yy) * w[12];
  // Y13 = -C3c(4xz^2 - x^3 - xy^2)
  g[0] += -kC3c * (4.0f * zz - 3.0f * xx - yy) * w[13];
  g[1] += kC3c * 2.0f * x * y * w[13];
  g[2] += -kC3c * 8.0f * x * z * w[13];
  // Y14 = C3e(x^2 z - y^2 z)
  g[0] += kC3e * 2.0f * x * z * w[14];
  g[1] += -kC3e * 2.0f * y * z * w[14];
  g[2] += kC3e * (xx - yy) * w[14];
  // Y15 = -C3a(x^3 - 3xy^2)
  g[0] += -kC3a * 3.0f * (xx - yy) * w[15];
  g[1] += kC3a * 6.0f * x * y * w[15];
}

__device__ __forceinline__ bool finitef(float x) { return __builtin_isfinite(x); }

// Forward quantities of one Gaussian that the backward also needs.
struct Proj {
  bool vis;
  float s[3], o, qn[4], inv_qlen;
  float Rq[9];       // rotation (row-major)
  float M[9];        // Rq diag(s)
  float Sg[6];       // Sigma: xx, xy, xz, yy, yz, zz
  float x, y, z, iz;
  float xr, yr;      // x/z, y/z after the guard-band clamp
  bool xcl, ycl;     // clamp active
  float T[6];        // J Rc, 2x3 row-major
  float Qa, Qb, Qc;  // conic
  float u, v;
  int rx, ry, tiles;
  uint32_t rect_lo, rect_hi;  // tile rect, packed x0 | y0 << 16, x1 | y1 << 16
};

// Geometry part of the forward (everything but colour).  mu, ls, q, a: the parameters.
__device__ __forceinline__ void project_geometry(const CamK& c, const float mu[3],
                                                 const float ls[3], const float q[4], float a,
                                                 Proj& P) {
  P.vis = false;
  P.tiles = 0;
  bool ok = true;
  for (int j = 0; j < 3; ++j) ok = ok && finitef(mu[j]) && finitef(ls[j]);
  for (int j = 0; j < 4; ++j) ok = ok && finitef(q[j]);
  ok = ok && finitef(a);
  if (!ok) return;
  for (int j = 0; j < 3; ++j) P.s[j] = __expf(ls[j]);
  P.o = 1.0f / (1.0f + __expf(-a));
  const float qq = q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3];
  if (!(qq > 0.0f) || !finitef(qq)) return;
  P.inv_qlen = 1.0f / sqrtf(qq);
  for (int j = 0; j < 4; ++j) P.qn[j] = q[j] * P.inv_qlen;
  const float w = P.qn[0], x = P.qn[1], y = P.qn[2], z = P.qn[3];
  P.Rq[0] = 1.f - 2.f * (y * y + z * z); P.Rq[1] = 2.f * (x * y - w * z); P.Rq[2] = 2.f * (x * z + w * y);
  P.Rq[3] = 2.f * (x * y + w * z); P.Rq[4] = 1.f - 2.f * (x * x + z * z); P.Rq[5] = 2.f * (y * z - w * x);
  P.Rq[6] = 2.f * (x * z - w * y); P.Rq[7] = 2.f * (y * z + w * x); P.Rq[8] = 1.f - 2.f * (x * x + y * y);
  for (int r = 0; r < 3; ++r)
    for (int k = 0; k < 3; ++k) P.M[3 * r + k] = P.Rq[3 * r + k] * P.s[k];
  // Sigma = M M^T
  const float* M = P.M;
  P.Sg[0] = M[0] * M[0] + M[1] * M[1] + M[2] * M[2];
  P.Sg[1] = M[0] * M[3] + M[1] * M[4] + M[2] * M[5];
  P.Sg[2] = M[0] * M[6] + M[1] * M[7] + M[2] * M[8];
  P.Sg[3] = M[3] * M[3] + M[4] * M[4] + M[5] * M[5];
  P.Sg[4] = M[3] * M[6] + M[4] * M[7] + M[5] * M[8];
  P.Sg[5] = M[6] * M[6] + M[7] * M[7] + M[8] * M[8];

  P.x = c.R[0] * mu[0] + c.R[1] * mu[1] + c.R[2] * mu[2] + c.t[0];
  P.y = c.R[3] * mu[0] + c.R[4] * mu[1] + c.R[5] * mu[2] + c.t[1];
  P.z = c.R[6] * mu[0] + c.R[7] * mu[1] + c.R[8] * mu[2] + c.t[2];
  if (!finitef(P.x) || !finitef(P.y) || !finitef(P.z)) return;
  if (!(P.z > c.near_plane)) return;
  P.iz = 1.0f / P.z;
  P.u = c.fx * P.x * P.iz + c.cx;
  P.v = c.fy * P.y * P.iz + c.cy;

  const float tx = P.x * P.iz, ty = P.y * P.iz;
  P.xcl = tx < -c.limx || tx > c.limx;
  P.ycl = ty < -c.limy || ty > c.limy;
  P.xr = fminf(fmaxf(tx, -c.limx), c.limx);
  P.yr = fminf(fmaxf(ty, -c.limy), c.limy);
  // J = [[fx/z, 0, -fx xr/z], [0, fy/z, -fy yr/z]];  T = J Rc
  const float j00 = c.fx * P.iz, j02 = -c.fx * P.xr * P.iz;
  const float j11 = c.fy * P.iz, j12 = -c.fy * P.yr * P.iz;
  for (int k = 0; k < 3; ++k) {
    P.T[k] = j00 * c.R[k] + j02 * c.R[6 + k];
    P.T[3 + k] = j11 * c.R[3 + k] + j12 * c.R[6 + k];
  }
  // S2 = T Sigma T^T + 0.3 I
  const float* S = P.Sg;
  const float* T = P.T;
  float TS0[3], TS1[3];
  TS0[0] = T[0] * S[0] + T[1] * S[1] + T[2] * S[2];
  TS0[1] = T[0] * S[1] + T[1] * S[3] + T[2] * S[4];
  TS0[2] = T[0] * S[2] + T[1] * S[4] + T[2] * S[5];
  TS1[0] = T[3] * S[0] + T[4] * S[1] + T[5] * S[2];
  TS1[1] = T[3] * S[1] + T[4] * S[3] + T[5] * S[4];
  TS1[2] = T[3] * S[2] + T[4] * S[4] + T[5] * S[5];
  const float s00 = TS0[0] * T[0] + TS0[1] * T[1] + TS0[2] * T[2] + 0.3f;
  const float s01 = TS0[0] * T[3] + TS0[1] * T[4] + TS0[2] * T[5];
  const float s11 = TS1[0] * T[3] + TS1[1] * T[4] + TS1[2] * T[5] + 0.3f;
  const float det = s00 * s11 - s01 * s01;
  if (!(det > 0.0f) || !finitef(det)) return;
  const float idet = 1.0f / det;
  P.Qa = s11 * idet;
  P.Qb = -s01 * idet;
  P.Qc = s00 * idet;
  P.rx = (int)ceilf(3.0f * sqrtf(s00));
  P.ry = (int)ceilf(3.0f * sqrtf(s11));
  int x0, y0, x1, y1;
  tile_rect(P.u, P.v, P.rx, P.ry, c.TX, c.TY, x0, y0, x1, y1);
  const int tiles = (x1 > x0 && y1 > y0) ? (x1 - x0) * (y1 - y0) : 0;
  if (tiles == 0) return;
  P.tiles = tiles;
  P.rect_lo = (uint32_t)x0 | ((uint32_t)y0 << 16);
  P.rect_hi = (uint32_t)x1 | ((uint32_t)y1 << 16);
  P.vis = true;
}

template <int DEG>
__global__ __launch_bounds__(kBlock) void k_preprocess(int64_t n, int64_t ld,
                                                        const float* __restrict__ params, CamK c,
                                                        float4* __restrict__ splat,
                                                        uint32_t* __restrict__ tiles,
                                                        uint32_t* __restrict__ dkey,
                                                        uint2* __restrict__ rect) {
  constexpr int NB = (DEG + 1) * (DEG + 1);
  __shared__ float4 stage[kBlock * 3];
  const int64_t i0 = (int64_t)blockIdx.x * kBlock;
  const int64_t i = i0 + threadIdx.x;
  float4 r0 = make_float4(0.f, 0.f, 0.f, 0.f), r1 = r0, r2 = r0;
  uint32_t nt = 0, key = 0xFFFFFFFFu;
  uint2 rc = make_uint2(0u, 0u);
  if (i < n) {
    float mu[3], ls[3], q[4];
#pragma unroll
    // the parameters stream through once: non-temporal loads keep them from evicting what
    // the binning reads next
    for (int j = 0; j < 3; ++j) mu[j] = __builtin_nontemporal_load(params + j * ld + i);
#pragma unroll
    for (int j = 0; j < 3; ++j) ls[j] = __builtin_nontemporal_load(params + (3 + j) * ld + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) q[j] = __builtin_nontemporal_load(params + (6 + j) * ld + i);
    const float a = __builtin_nontemporal_load(params + 10 * ld + i);
    // all 59 rows are requested before any arithmetic: more loads in flight per wave (measured
    // 0.26 -> 0.20 ms), at no cost in bytes, as culled Gaussians are rare
    float f[NB][3];
#pragma unroll
    for (int k = 0; k < NB; ++k)
#pragma unroll
      for (int ch = 0; ch < 3; ++ch) f[k][ch] = __builtin_nontemporal_load(params + (11 + 3 * k + ch) * ld + i);
    Proj P;
    project_geometry(c, mu, ls, q, a, P);
    if (P.vis) {
      // SH colour along the direction from the camera centre to the mean
      float d0 = mu[0] - c.pos[0], d1 = mu[1] - c.pos[1], d2 = mu[2] - c.pos[2];
      const float il = 1.0f / sqrtf(d0 * d0 + d1 * d1 + d2 * d2);
      d0 *= il; d1 *= il; d2 *= il;
      float Y[16];
      sh_eval(DEG, d0, d1, d2, Y);
      float rgb[3] = {0.5f, 0.5f, 0.5f};
#pragma unroll
      for (int k = 0; k < NB; ++k)
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) rgb[ch] += Y[k] * f[k][ch];
      r0 = make_float4(P.u, P.v, __int_as_float(P.rx), __int_as_float(P.ry));
      r1 = make_float4(P.Qa, P.Qb, P.Qc, P.o);
      r2 = make_float4(fmaxf(rgb[0], 0.f), fmaxf(rgb[1], 0.f), fmaxf(rgb[2], 0.f), P.z);
      nt = (uint32_t)P.tiles;
      key = __float_as_uint(P.z);
      rc = make_uint2(P.rect_lo, P.rect_hi);
    }
    tiles[i] = nt;
    dkey[i] = key;
    rect[i] = rc;
  }
  stage[3 * threadIdx.x + 0] = r0;
  stage[3 * threadIdx.x + 1] = r1;
  stage[3 * threadIdx.x + 2] = r2;
  __syncthreads();
  const int64_t cnt = (n - i0 < kBlock ? n - i0 : kBlock) * 3;
  float4* dst = splat + i0 * 3;
  for (int e = threadIdx.x; e < cnt; e += kBlock) dst[e] = stage[e];
}

// Backward through the per-Gaussian forward, optionally followed by the Adam update of every
// parameter row of this Gaussian (m, v non-null).  For batched steps each row's gradient is
// scaled (the batch mean) and added to the gradient accumulated over the batch's earlier views.
//
// NEXT: the same pass then preprocesses the next view (camera cn) from the rows' new values, as
// k_preprocess would from the updated parameters, and writes its outputs (nx).
template <int DEG, bool NEXT>
__device__ __forceinline__ void prebwd_gaussian(const PrebwdArgs& A, const CamK& c, const CamK& cn,
                                                const NextOut& nx, int64_t i, float4& r0, float4& r1,
                                                float4& r2);
template <int DEG, bool NEXT>
__global__ __launch_bounds__(kBlock) void k_preprocess_backward(PrebwdArgs A, CamK c, CamK cn, NextOut nx) {
  constexpr int NB = (DEG + 1) * (DEG + 1);
  const int64_t i0 = (int64_t)blockIdx.x * kBlock;
  const int64_t i = i0 + threadIdx.x;
  if constexpr (NEXT) {
    // the records are staged per workgroup and written out whole, as k_preprocess does
    __shared__ float4 stage[kBlock * 3];
    float4 r0 = make_float4(0.f, 0.f, 0.f, 0.f), r1 = r0, r2 = r0;
    if (i < A.n) prebwd_gaussian<DEG, true>(A, c, cn, nx, i, r0, r1, r2);
    stage[3 * threadIdx.x + 0] = r0;
    stage[3 * threadIdx.x + 1] = r1;
    stage[3 * threadIdx.x + 2] = r2;
    __syncthreads();
    const int64_t cnt = (A.n - i0 < kBlock ? A.n - i0 : kBlock) * 3;
    float4* dst = nx.splat + i0 * 3;
    for (int e = threadIdx.x; e < cnt; e += kBlock) dst[e] = stage[e];
  } else {
    if (i >= A.n) return;
    float4 r0, r1, r2;
    prebwd_gaussian<DEG, false>(A, c, cn, nx, i, r0, r1, r2);
  }
}

// One Gaussian of k_preprocess_backward; with NEXT, r0..r2 receive its next-view record.
template <int DEG, bool NEXT>
__device__ __forceinline__ void prebwd_gaussian(const PrebwdArgs& A, const CamK& c, const CamK& cn,
                                                const NextOut& nx, int64_t i, float4& r0, float4& r1,
                                                float4& r2) {
  constexpr int NB = (DEG + 1) * (DEG + 1);
  const int64_t ld = A.ld;
  float* __restrict__ prm = A.params;
  const bool adam = A.m != nullptr;
  // Row r's gradient goes to grads and/or through Adam as soon as it is known.  Parameters,
  // moments and the updated parameters stream through once: non-temporal loads and stores
  // (measured 8% faster than cached ones).  A row's inputs (its moments, and the running sum in
  // accumulate mode) are loaded by row_in ahead of finish_row, several rows at a time: the
  // stores of one row would otherwise keep the next row's loads from issuing before them.
  // (finish_row returns the row's new value: the parameter itself when there is no Adam update)
  struct RowIn {
    float m, v, ga;
  };
  auto row_in = [&](int r) -> RowIn {
    const int64_t e = (int64_t)r * ld + i;
    RowIn o{0.f, 0.f, 0.f};
    if (A.gacc) o.ga = A.gacc[e];
    if (adam) {
      o.m = __builtin_nontemporal_load(A.m + e);
      o.v = __builtin_nontemporal_load(A.v + e);
    }
    return o;
  };
  auto finish_row = [&](int r, float gv, float th, const RowIn& in) -> float {
    const int64_t e = (int64_t)r * ld + i;
    float gr_ = A.gscale * gv;
    if (A.gacc) gr_ += in.ga;
    if (A.grads) A.grads[e] = gr_;
    if (adam) {
      const float m = A.b1 * in.m + A.omb1 * gr_;
      const float v = A.b2 * in.v + A.omb2 * gr_ * gr_;
      __builtin_nontemporal_store(m, A.m + e);
      __builtin_nontemporal_store(v, A.v + e);
      const float nth = th - A.lr * (m * A.inv_bc1) / (sqrtf(v * A.inv_bc2) + A.eps);
      __builtin_nontemporal_store(nth, prm + e);
      return nth;
    }
    return th;
  };

  float mu[3], ls[3], q[4];
  float na = 0.f;  // the new logit
  for (int j = 0; j < 3; ++j) mu[j] = __builtin_nontemporal_load(prm + j * ld + i);
  for (int j = 0; j < 3; ++j) ls[j] = __builtin_nontemporal_load(prm + (3 + j) * ld + i);
  for (int j = 0; j < 4; ++j) q[j] = __builtin_nontemporal_load(prm + (6 + j) * ld + i);
  const float a = __builtin_nontemporal_load(prm + 10 * ld + i);
  float g[11];  // dL/d(mu, log-scale, q, logit)
  for (int j = 0; j < 11; ++j) g[j] = 0.f;
  float gr[3] = {0.f, 0.f, 0.f};  // dL/drgb
  bool vis;
  // Two phases, so that the projection's state and the 48 SH coefficients are never live at
  // once: first the geometry (projection, conic, covariance, opacity), whose rows other than
  // the mean are finished at once; then the colour, which adds the view-direction term to the
  // mean's gradient and finishes the mean and SH rows.
  {
    Proj P;
    project_geometry(c, mu, ls, q, a, P);
    vis = P.vis;
    if (vis) {
      float g2[9];  // this Gaussian's nine values: grad2d, or the sum of its staged rows
      if (A.grad2d) {
#pragma unroll
        for (int k = 0; k < 9; ++k) g2[k] = A.grad2d[9 * i + k];
      } else {
        // the same rows in the same order as the gather into grad2d, so the values are identical
#pragma unroll
        for (int k = 0; k < 9; ++k) g2[k] = 0.f;
        const uint32_t t = A.tiles[i];
        const uint64_t base = (uint64_t)A.goff_blk[i / kGoffBlock] + A.goff[i];
        for (uint32_t j = 0; j < t; ++j) {
          if (base + j >= A.staging_cap) break;
          const float* e = A.staging + 9 * (base + j);
#pragma unroll
          for (int k = 0; k < 9; ++k) g2[k] += e[k];
        }
      }
      const float gu = g2[0], gv = g2[1];
      const float gA = g2[2], gB = g2[3], gC = g2[4];
      const float go = g2[5];
      gr[0] = g2[6];
      gr[1] = g2[7];
      gr[2] = g2[8];

      // ---- opacity ----------------------------------------------------------------------
      g[10] = P.o * (1.f - P.o) * go;

      // ---- conic = S2^-1:  dL/dS2 = -Q G Q with G = [[gA, gB/2], [gB/2, gC]] -------------
      const float hb = 0.5f * gB;
      const float q00 = P.Qa * gA + P.Qb * hb, q01 = P.Qa * hb + P.Qb * gC;
      const float q10 = P.Qb * gA + P.Qc * hb, q11 = P.Qb * hb + P.Qc * gC;
      const float G00 = -(q00 * P.Qa + q01 * P.Qb);
      const float G01 = -(q00 * P.Qb + q01 * P.Qc);
      const float G11 = -(q10 * P.Qb + q11 * P.Qc);

      // ---- S2 = T Sigma T^T (+0.3 I): dL/dSigma = T^T G T, dL/dT = 2 G T Sigma ---------
      const float* T = P.T;
      const float* S = P.Sg;
      // GT = G T (2x3)
      float GT0[3], GT1[3];
      for (int k = 0; k < 3; ++k) {
        GT0[k] = G00 * T[k] + G01 * T[3 + k];
        GT1[k] = G01 * T[k] + G11 * T[3 + k];
      }
      // dL/dSigma (symmetric, xx xy xz yy yz zz) = T^T (G T)
      float gS[6];
      gS[0] = T[0] * GT0[0] + T[3] * GT1[0];
      gS[1] = T[0] * GT0[1] + T[3] * GT1[1];
      gS[2] = T[0] * GT0[2] + T[3] * GT1[2];
      gS[3] = T[1] * GT0[1] + T[4] * GT1[1];
      gS[4] = T[1] * GT0[2] + T[4] * GT1[2];
      gS[5] = T[2] * GT0[2] + T[5] * GT1[2];
      // dL/dT = 2 (G T) Sigma
      float gT[6];
      gT[0] = 2.f * (GT0[0] * S[0] + GT0[1] * S[1] + GT0[2] * S[2]);
      gT[1] = 2.f * (GT0[0] * S[1] + GT0[1] * S[3] + GT0[2] * S[4]);
      gT[2] = 2.f * (GT0[0] * S[2] + GT0[1] * S[4] + GT0[2] * S[5]);
      gT[3] = 2.f * (GT1[0] * S[0] + GT1[1] * S[1] + GT1[2] * S[2]);
      gT[4] = 2.f * (GT1[0] * S[1] + GT1[1] * S[3] + GT1[2] * S[4]);
      gT[5] = 2.f * (GT1[0] * S[2] + GT1[1] * S[4] + GT1[2] * S[5]);
      // T = J Rc: dL/dJ = dL/dT Rc^T (only J00, J02, J11, J12 vary)
      const float gJ00 = gT[0] * c.R[0] + gT[1] * c.R[1] + gT[2] * c.R[2];
      const float gJ02 = gT[0] * c.R[6] + gT[1] * c.R[7] + gT[2] * c.R[8];
      const float gJ11 = gT[3] * c.R[3] + gT[4] * c.R[4] + gT[5] * c.R[5];
      const float gJ12 = gT[3] * c.R[6] + gT[4] * c.R[7] + gT[5] * c.R[8];

      // ---- camera-space position ----------------------------------------------------------
      const float iz = P.iz, iz2 = iz * iz;
      float gx = gu * c.fx * iz;
      float gy = gv * c.fy * iz;
      float gz = -(gu * c.fx * P.x + gv * c.fy * P.y) * iz2;
      gz += -(gJ00 * c.fx + gJ11 * c.fy) * iz2;
      // J02 = -fx xr / z: xr = x/z when unclamped, a constant when clamped
      if (!P.xcl) {
        gx += -gJ02 * c.fx * iz2;
        gz += 2.f * gJ02 * c.fx * P.x * iz2 * iz;
      } else {
        gz += gJ02 * c.fx * P.xr * iz2;  // d(-fx xr / z)/dz with xr constant
      }
      if (!P.ycl) {
        gy += -gJ12 * c.fy * iz2;
        gz += 2.f * gJ12 * c.fy * P.y * iz2 * iz;
      } else {
        gz += gJ12 * c.fy * P.yr * iz2;
      }
      // p = Rc mu + t
      g[0] += c.R[0] * gx + c.R[3] * gy + c.R[6] * gz;
      g[1] += c.R[1] * gx + c.R[4] * gy + c.R[7] * gz;
      g[2] += c.R[2] * gx + c.R[5] * gy + c.R[8] * gz;

      // ---- Sigma = M M^T: dL/dM = 2 dL/dSigma M ------------------------------------------
      const float* M = P.M;
      float gM[9];
      const float Sfull[9] = {gS[0], gS[1], gS[2], gS[1], gS[3], gS[4], gS[2], gS[4], gS[5]};
      for (int r = 0; r < 3; ++r)
        for (int k = 0; k < 3; ++k)
          gM[3 * r + k] = 2.f * (Sfull[3 * r + 0] * M[k] + Sfull[3 * r + 1] * M[3 + k] +
                                 Sfull[3 * r + 2] * M[6 + k]);
      // M = Rq diag(s): dL/ds_k = sum_r gM_rk Rq_rk; dL/dRq_rk = gM_rk s_k; s = exp(l)
      float gR[9];
      for (int k = 0; k < 3; ++k) {
        const float gs = gM[k] * P.Rq[k] + gM[3 + k] * P.Rq[3 + k] + gM[6 + k] * P.Rq[6 + k];
        g[3 + k] = gs * P.s[k];
        gR[k] = gM[k] * P.s[k];
        gR[3 + k] = gM[3 + k] * P.s[k];
        gR[6 + k] = gM[6 + k] * P.s[k];
      }
      // rotation entries -> unit quaternion (w, x, y, z)
      const float w = P.qn[0], x = P.qn[1], y = P.qn[2], z = P.qn[3];
      const float s01 = gR[1] + gR[3], s02 = gR[2] + gR[6], s12 = gR[5] + gR[7];
      const float a10 = gR[3] - gR[1], a02 = gR[2] - gR[6], a21 = gR[7] - gR[5];
      float gq[4];
      gq[0] = 2.f * (z * a10 + y * a02 + x * a21);
      gq[1] = 2.f * (y * s01 + z * s02 + w * a21) - 4.f * x * (gR[4] + gR[8]);
      gq[2] = 2.f * (x * s01 + w * a02 + z * s12) - 4.f * y * (gR[0] + gR[8]);
      gq[3] = 2.f * (w * a10 + x * s02 + y * s12) - 4.f * z * (gR[0] + gR[4]);
      // q_hat = q / |q|
      const float qd = w * gq[0] + x * gq[1] + y * gq[2] + z * gq[3];
      for (int j = 0; j < 4; ++j) g[6 + j] = (gq[j] - P.qn[j] * qd) * P.inv_qlen;
    }
    RowIn gin[8];  // rows 3..10
#pragma unroll
    for (int r = 3; r < 11; ++r) gin[r - 3] = row_in(r);
#pragma unroll
    for (int r = 3; r < 11; ++r) {
      const float nv = finish_row(r, g[r], r < 6 ? ls[r - 3] : (r < 10 ? q[r - 6] : a), gin[r - 3]);
      if constexpr (NEXT) {  // (the old values are not needed past this point)
        if (r < 6) ls[r - 3] = nv;
        else if (r < 10) q[r - 6] = nv;
      }
      if (r == 10) na = nv;
    }
  }

  float f[NB][3];  // SH coefficients
#pragma unroll
  for (int k = 0; k < NB; ++k)
#pragma unroll
    for (int ch = 0; ch < 3; ++ch) f[k][ch] = __builtin_nontemporal_load(prm + (11 + 3 * k + ch) * ld + i);
  float gc[3] = {0.f, 0.f, 0.f};  // dL/drgb gated by the clamp
  float Y[16];
  if (vis) {
    // ---- colour: raw = 0.5 + sum_k Y_k f_k, rgb = max(raw, 0) -------------------------
    const float dv0 = mu[0] - c.pos[0], dv1 = mu[1] - c.pos[1], dv2 = mu[2] - c.pos[2];
    const float idist = 1.0f / sqrtf(dv0 * dv0 + dv1 * dv1 + dv2 * dv2);
    const float d0 = dv0 * idist, d1 = dv1 * idist, d2 = dv2 * idist;
    sh_eval(DEG, d0, d1, d2, Y);
    float raw[3] = {0.5f, 0.5f, 0.5f};
#pragma unroll
    for (int k = 0; k < NB; ++k)
#pragma unroll
      for (int ch = 0; ch < 3; ++ch) raw[ch] += Y[k] * f[k][ch];
#pragma unroll
    for (int ch = 0; ch < 3; ++ch) gc[ch] = raw[ch] > 0.f ? gr[ch] : 0.f;
    // dL/ddir = sum_k (sum_ch gc_ch f_k,ch) grad Y_k
    float wk[16];
#pragma unroll
    for (int k = 0; k < NB; ++k) wk[k] = gc[0] * f[k][0] + gc[1] * f[k][1] + gc[2] * f[k][2];
    float gdir[3] = {0.f, 0.f, 0.f};
    sh_grad_acc(DEG, d0, d1, d2, wk, gdir);
    // direction = (mu - pos)/|mu - pos|: project out the radial part
    const float dd = d0 * gdir[0] + d1 * gdir[1] + d2 * gdir[2];
    g[0] += (gdir[0] - d0 * dd) * idist;
    g[1] += (gdir[1] - d1 * dd) * idist;
    g[2] += (gdir[2] - d2 * dd) * idist;
  }
  // the SH rows' inputs, kShGroup coefficients (3 kShGroup rows) at a time
  constexpr int kShGroup = 2;
  auto sh_in = [&](int k0, RowIn (&in)[kShGroup][3]) {
#pragma unroll
    for (int kk = 0; kk < kShGroup; ++kk)
      if (k0 + kk < NB)
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) in[kk][ch] = row_in(11 + 3 * (k0 + kk) + ch);
  };
  RowIn min_in[3];  // the mean rows
#pragma unroll
  for (int r = 0; r < 3; ++r) min_in[r] = row_in(r);
  if constexpr (!NEXT) {
#pragma unroll
    for (int r = 0; r < 3; ++r) finish_row(r, g[r], mu[r], min_in[r]);
#pragma unroll
    for (int k0 = 0; k0 < NB; k0 += kShGroup) {
      RowIn in[kShGroup][3];
      sh_in(k0, in);
#pragma unroll
      for (int kk = 0; kk < kShGroup; ++kk)
        if (k0 + kk < NB)
#pragma unroll
          for (int ch = 0; ch < 3; ++ch) {
            const int k = k0 + kk;
            finish_row(11 + 3 * k + ch, vis ? Y[k] * gc[ch] : 0.f, f[k][ch], in[kk][ch]);
          }
    }
  } else {
    float nmu[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) nmu[r] = finish_row(r, g[r], mu[r], min_in[r]);
    // the next view's preprocess of the new values: the operations of k_preprocess
    Proj Pn;
    project_geometry(cn, nmu, ls, q, na, Pn);
    float Yn[16];
    if (Pn.vis) {
      float d0 = nmu[0] - cn.pos[0], d1 = nmu[1] - cn.pos[1], d2 = nmu[2] - cn.pos[2];
      const float il = 1.0f / sqrtf(d0 * d0 + d1 * d1 + d2 * d2);
      d0 *= il; d1 *= il; d2 *= il;
      sh_eval(DEG, d0, d1, d2, Yn);
    }
    float rgb[3] = {0.5f, 0.5f, 0.5f};
#pragma unroll
    for (int k0 = 0; k0 < NB; k0 += kShGroup) {
      RowIn in[kShGroup][3];
      sh_in(k0, in);
#pragma unroll
      for (int kk = 0; kk < kShGroup; ++kk)
        if (k0 + kk < NB)
#pragma unroll
          for (int ch = 0; ch < 3; ++ch) {
            const int k = k0 + kk;
            const float nf = finish_row(11 + 3 * k + ch, vis ? Y[k] * gc[ch] : 0.f, f[k][ch], in[kk][ch]);
            if (Pn.vis) rgb[ch] += Yn[k] * nf;
          }
    }
    uint32_t nt = 0, key = 0xFFFFFFFFu;
    uint2 rc = make_uint2(0u, 0u);
    r0 = r1 = r2 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (Pn.vis) {
      r0 = make_float4(Pn.u, Pn.v, __int_as_float(Pn.rx), __int_as_float(Pn.ry));
      r1 = make_float4(Pn.Qa, Pn.Qb, Pn.Qc, Pn.o);
      r2 = make_float4(fmaxf(rgb[0], 0.f), fmaxf(rgb[1], 0.f), fmaxf(rgb[2], 0.f), Pn.z);
      nt = (uint32_t)Pn.tiles;
      key = __float_as_uint(Pn.z);
      rc = make_uint2(Pn.rect_lo, Pn.rect_hi);
    }
    nx.tiles[i] = nt;
    nx.dkey[i] = key;
    nx.rect[i] = rc;
  }
}

}  // namespace

hipError_t launch_preprocess(const gs_scene& sc, const float* params, const CamK& cam,
                             gs_proj out, hipStream_t s) {
  if (sc.n == 0) return hipSuccess;
  const unsigned grid = (unsigned)ceil_div(sc.n, kBlock);
  float4* sp = reinterpret_cast<float4*>(out.splat);
  uint2* rc = reinterpret_cast<uint2*>(out.rect);
  switch (sc.sh_degree) {
    case 0: hipLaunchKernelGGL(k_preprocess<0>, dim3(grid), dim3(kBlock), 0, s, sc.n, sc.ld, params, cam, sp, out.tiles, out.depth_key, rc); break;
    case 1: hipLaunchKernelGGL(k_preprocess<1>, dim3(grid), dim3(kBlock), 0, s, sc.n, sc.ld, params, cam, sp, out.tiles, out.depth_key, rc); break;
    case 2: hipLaunchKernelGGL(k_preprocess<2>, dim3(grid), dim3(kBlock), 0, s, sc.n, sc.ld, params, cam, sp, out.tiles, out.depth_key, rc); break;
    default: hipLaunchKernelGGL(k_preprocess<3>, dim3(grid), dim3(kBlock), 0, s, sc.n, sc.ld, params, cam, sp, out.tiles, out.depth_key, rc); break;
  }
  return hipGetLastError();
}

hipError_t launch_preprocess_backward(const PrebwdArgs& a, const CamK& cam, hipStream_t s, const CamK* next_cam,
                                      const NextOut* next) {
  if (a.n == 0) return hipSuccess;
  const unsigned grid = (unsigned)ceil_div(a.n, kBlock);
  const CamK cn = next_cam ? *next_cam : cam;
  const NextOut nx = next ? *next : NextOut{};
#define GSMI_PREBWD(D)                                                                                  \
  if (next_cam)                                                                                         \
    hipLaunchKernelGGL((k_preprocess_backward<D, true>), dim3(grid), dim3(kBlock), 0, s, a, cam, cn, nx); \
  else                                                                                                  \
    hipLaunchKernelGGL((k_preprocess_backward<D, false>), dim3(grid), dim3(kBlock), 0, s, a, cam, cn, nx);
  switch (a.deg) {
    case 0: GSMI_PREBWD(0); break;
    case 1: GSMI_PREBWD(1); break;
    case 2: GSMI_PREBWD(2); break;
    default: GSMI_PREBWD(3); break;
  }
#undef GSMI_PREBWD
  return hipGetLastError();
}

}  // namespace gsmi
