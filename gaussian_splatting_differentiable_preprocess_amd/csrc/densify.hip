// Adaptive density control: the densification statistics and one clone / split / prune pass
// (gfx950).
//
// "Scaling 3D Gaussian Splatting with Distributed Compute" names adaptive density control
// (densifying and pruning, which grows N and drives memory) without its rules; these kernels
// follow 3D-GS:
//   statistics  per view, every Gaussian the view sees (radius > 0) adds the norm of its 2D
//               mean's gradient in normalised device units, |(dL/du W/2, dL/dv H/2)|, and 1;
//   decision    prune when the opacity logit is below logit(min_opacity); otherwise, when the
//               averaged statistic (one float32 division) reaches the threshold, clone when the
//               largest log-scale is at most log(percent_dense x extent), else split;
//   output      kept Gaussians (neither pruned nor split) in index order, then one copy of each
//               cloned one, then the first children of the split ones, then the second
//               children; child k: mean mu + R(q) (exp(log-scale) * z_k), log-scale minus
//               log(split_factor), rotation, opacity and colour copied; new Gaussians start
//               with zero Adam moments.
// Every decision compares float32 values against float32 thresholds formed on the host in
// double, so it is exact and order-independent.  The output order comes from exclusive scans
// of the three categories: per workgroup of 256 Gaussians, then over workgroups.
#include "gsmi_internal.h"

namespace gsmi {

namespace {

constexpr int kDensBlock = 256;
enum : uint32_t { kKeep = 0, kClone = 1, kSplit = 2, kPrune = 3 };

__global__ __launch_bounds__(kBlock) void k_densify_stats(int64_t n, const gs_splat* __restrict__ splat,
                                                          const uint32_t* __restrict__ tiles,
                                                          const uint32_t* __restrict__ goff,
                                                          const uint32_t* __restrict__ goff_blk,
                                                          const float* __restrict__ staging,
                                                          uint64_t staging_cap, float half_w, float half_h,
                                                          float* __restrict__ grad_acc, float* __restrict__ count) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= n || splat[i].radius_x <= 0) return;
  // the same staged rows in the same order as the preprocess backward reads them
  float gu = 0.f, gv = 0.f;
  const uint32_t t = tiles[i];
  const uint64_t base = (uint64_t)goff_blk[i / kGoffBlock] + goff[i];
  for (uint32_t j = 0; j < t; ++j) {
    if (base + j >= staging_cap) break;
    const float* e = staging + 9 * (base + j);
    gu += e[0];
    gv += e[1];
  }
  const float x = gu * half_w, y = gv * half_h;
  grad_acc[i] += sqrtf(x * x + y * y);
  count[i] += 1.f;
}

struct DensArgs {
  int64_t n, ld, ld_out;
  int R;
  const float* params;
  const float* m;
  const float* v;
  const float* grad_acc;
  const float* count;
  const float* z;  // [2][3][ld]
  float t_grad, t_lscale, t_logit, log_split;
  float* params_out;
  float* m_out;
  float* v_out;
  int32_t* codes;        // nullable
  uint32_t* blk;         // [nblk][3] per-workgroup counts, scanned in place
  uint32_t* totals;      // [3]
};

__device__ __forceinline__ uint32_t dens_code(const DensArgs& a, int64_t i) {
  const float* p = a.params;
  if (p[10 * a.ld + i] < a.t_logit) return kPrune;
  const float c = a.count[i];
  const float g = c > 0.f ? a.grad_acc[i] / c : 0.f;
  if (!(g >= a.t_grad)) return kKeep;
  // fmaxf skips a NaN operand; with all three NaN the Gaussian is kept as it is
  const float l = fmaxf(fmaxf(p[3 * a.ld + i], p[4 * a.ld + i]), p[5 * a.ld + i]);
  return l > a.t_lscale ? kSplit : (l <= a.t_lscale ? kClone : kKeep);
}

// Exclusive scan of (kept, clone, split) flags over the workgroup's 256 Gaussians.
__device__ __forceinline__ uint3 block_scan3(uint3 x, uint3* tmp, uint3* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint3 inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t a = __shfl_up(inc.x, o, 64), b = __shfl_up(inc.y, o, 64), c = __shfl_up(inc.z, o, 64);
    if (lane >= o) {
      inc.x += a;
      inc.y += b;
      inc.z += c;
    }
  }
  if (lane == 63) tmp[w] = inc;
  __syncthreads();
  uint3 pre = make_uint3(0, 0, 0), tot = make_uint3(0, 0, 0);
#pragma unroll
  for (int k = 0; k < kDensBlock / 64; ++k) {
    const uint3 t = tmp[k];
    if (k < w) {
      pre.x += t.x;
      pre.y += t.y;
      pre.z += t.z;
    }
    tot.x += t.x;
    tot.y += t.y;
    tot.z += t.z;
  }
  *total = tot;
  return make_uint3(pre.x + inc.x - x.x, pre.y + inc.y - x.y, pre.z + inc.z - x.z);
}

__device__ __forceinline__ uint3 flags_of(uint32_t code) {
  return make_uint3(code == kKeep || code == kClone ? 1u : 0u, code == kClone ? 1u : 0u, code == kSplit ? 1u : 0u);
}

__global__ __launch_bounds__(kDensBlock) void k_densify_count(DensArgs a) {
  __shared__ uint3 tmp[kDensBlock / 64];
  const int64_t i = (int64_t)blockIdx.x * kDensBlock + threadIdx.x;
  const uint32_t code = i < a.n ? dens_code(a, i) : kPrune;
  if (i < a.n && a.codes) a.codes[i] = (int32_t)code;
  uint3 tot;
  block_scan3(flags_of(code), tmp, &tot);
  if (threadIdx.x == 0) {
    a.blk[3 * blockIdx.x + 0] = tot.x;
    a.blk[3 * blockIdx.x + 1] = tot.y;
    a.blk[3 * blockIdx.x + 2] = tot.z;
  }
}

// One workgroup: exclusive scan of the per-workgroup counts in place, totals out.
__global__ __launch_bounds__(1024) void k_densify_scan(int64_t nblk, uint32_t* __restrict__ blk,
                                                       uint32_t* __restrict__ totals) {
  __shared__ uint32_t s[3][1024];
  uint32_t carry[3] = {0, 0, 0};
  for (int64_t b0 = 0; b0 < nblk; b0 += 1024) {
    const int64_t b = b0 + threadIdx.x;
    for (int c = 0; c < 3; ++c) s[c][threadIdx.x] = b < nblk ? blk[3 * b + c] : 0u;
    __syncthreads();
    // Hillis-Steele inclusive scan of each column
    for (int o = 1; o < 1024; o <<= 1) {
      uint32_t add[3];
      for (int c = 0; c < 3; ++c) add[c] = threadIdx.x >= (unsigned)o ? s[c][threadIdx.x - o] : 0u;
      __syncthreads();
      for (int c = 0; c < 3; ++c) s[c][threadIdx.x] += add[c];
      __syncthreads();
    }
    for (int c = 0; c < 3; ++c) {
      const uint32_t incl = s[c][threadIdx.x];
      const uint32_t mine = b < nblk ? blk[3 * b + c] : 0u;
      if (b < nblk) blk[3 * b + c] = carry[c] + incl - mine;
    }
    for (int c = 0; c < 3; ++c) carry[c] += s[c][1023];
    __syncthreads();
  }
  if (threadIdx.x == 0)
    for (int c = 0; c < 3; ++c) totals[c] = carry[c];
}

__global__ __launch_bounds__(kDensBlock) void k_densify_write(DensArgs a, uint32_t n_kept, uint32_t n_clone,
                                                              uint32_t n_split) {
  __shared__ uint3 tmp[kDensBlock / 64];
  const int64_t i = (int64_t)blockIdx.x * kDensBlock + threadIdx.x;
  const uint32_t code = i < a.n ? dens_code(a, i) : kPrune;
  uint3 tot;
  const uint3 off = block_scan3(flags_of(code), tmp, &tot);
  if (i >= a.n || code == kPrune) return;
  const uint32_t bk = a.blk[3 * blockIdx.x], bc = a.blk[3 * blockIdx.x + 1], bs = a.blk[3 * blockIdx.x + 2];
  const int64_t ld = a.ld, lo = a.ld_out;
  if (code == kKeep || code == kClone) {
    const int64_t o = bk + off.x;
    for (int r = 0; r < a.R; ++r) {
      a.params_out[r * lo + o] = a.params[r * ld + i];
      a.m_out[r * lo + o] = a.m[r * ld + i];
      a.v_out[r * lo + o] = a.v[r * ld + i];
    }
  }
  if (code == kClone) {
    const int64_t o = (int64_t)n_kept + bc + off.y;
    for (int r = 0; r < a.R; ++r) {
      a.params_out[r * lo + o] = a.params[r * ld + i];
      a.m_out[r * lo + o] = 0.f;
      a.v_out[r * lo + o] = 0.f;
    }
  }
  if (code == kSplit) {
    float q[4];
    for (int j = 0; j < 4; ++j) q[j] = a.params[(6 + j) * ld + i];
    const float qn = 1.f / sqrtf(q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3]);
    const float w = q[0] * qn, x = q[1] * qn, y = q[2] * qn, zq = q[3] * qn;
    const float Rm[3][3] = {{1.f - 2.f * (y * y + zq * zq), 2.f * (x * y - w * zq), 2.f * (x * zq + w * y)},
                            {2.f * (x * y + w * zq), 1.f - 2.f * (x * x + zq * zq), 2.f * (y * zq - w * x)},
                            {2.f * (x * zq - w * y), 2.f * (y * zq + w * x), 1.f - 2.f * (x * x + y * y)}};
    float s[3];
    for (int j = 0; j < 3; ++j) s[j] = expf(a.params[(3 + j) * ld + i]);
    for (int k = 0; k < 2; ++k) {
      const int64_t o = (int64_t)n_kept + n_clone + (int64_t)k * n_split + bs + off.z;
      float d[3];
      for (int j = 0; j < 3; ++j) d[j] = s[j] * a.z[((int64_t)k * 3 + j) * ld + i];
      for (int r = 0; r < 3; ++r)
        a.params_out[r * lo + o] = a.params[r * ld + i] + (Rm[r][0] * d[0] + Rm[r][1] * d[1] + Rm[r][2] * d[2]);
      for (int r = 3; r < 6; ++r) a.params_out[r * lo + o] = a.params[r * ld + i] - a.log_split;
      for (int r = 6; r < a.R; ++r) a.params_out[r * lo + o] = a.params[r * ld + i];
      for (int r = 0; r < a.R; ++r) {
        a.m_out[r * lo + o] = 0.f;
        a.v_out[r * lo + o] = 0.f;
      }
    }
  }
}

}  // namespace

hipError_t launch_densify_stats(int64_t n, const gs_splat* splat, const uint32_t* tiles, const RenderWs& ws,
                                float half_w, float half_h, float* grad_acc, float* count, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_densify_stats, dim3((unsigned)ceil_div(n, kBlock)), dim3(kBlock), 0, s, n, splat, tiles,
                     ws.goff, ws.goff_blk, ws.staging, ws.staging_cap, half_w, half_h, grad_acc, count);
  return hipGetLastError();
}

size_t densify_workspace_bytes(int64_t n) {
  const int64_t nblk = ceil_div(n > 0 ? n : 1, kDensBlock);
  return (size_t)(3 * nblk + 64) * sizeof(uint32_t);
}

hipError_t launch_densify(const DensifyLaunch& d, uint32_t totals_host[3], hipStream_t s) {
  DensArgs a{};
  a.n = d.n;
  a.ld = d.ld;
  a.ld_out = d.ld_out;
  a.R = d.R;
  a.params = d.params;
  a.m = d.m;
  a.v = d.v;
  a.grad_acc = d.grad_acc;
  a.count = d.count;
  a.z = d.z;
  a.t_grad = d.t_grad;
  a.t_lscale = d.t_lscale;
  a.t_logit = d.t_logit;
  a.log_split = d.log_split;
  a.params_out = d.params_out;
  a.m_out = d.m_out;
  a.v_out = d.v_out;
  a.codes = d.codes;
  const int64_t nblk = ceil_div(d.n, kDensBlock);
  a.blk = static_cast<uint32_t*>(d.ws);
  a.totals = a.blk + 3 * nblk;
  hipLaunchKernelGGL(k_densify_count, dim3((unsigned)nblk), dim3(kDensBlock), 0, s, a);
  hipLaunchKernelGGL(k_densify_scan, dim3(1), dim3(1024), 0, s, nblk, a.blk, a.totals);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipMemcpyAsync(totals_host, a.totals, 3 * sizeof(uint32_t), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e;
  const int64_t n_out = (int64_t)totals_host[0] + totals_host[1] + 2 * (int64_t)totals_host[2];
  if (n_out > d.ld_out) return hipSuccess;  // the caller reports the capacity error
  hipLaunchKernelGGL(k_densify_write, dim3((unsigned)nblk), dim3(kDensBlock), 0, s, a, totals_host[0],
                     totals_host[1], totals_host[2]);
  return hipGetLastError();
}

}  // namespace gsmi
