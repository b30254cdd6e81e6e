// Elementwise kernels: fills, the L1 image loss and the standalone Adam step (gfx950).
//
// L1 ("Scaling 3D Gaussian Splatting with Distributed Compute", the loss passage: an L1 term
// between rendered and ground-truth images, mean over the pixel count): dL/dI = sign(I - I*) / N
// with N = 3HW elements, loss = mean |I - I*| from per-workgroup partial sums reduced in double
// by one final workgroup (deterministic).
// Adam (the same page, step "Step the optimizer locally"): bias-corrected Kingma-Ba update,
// dense over every float.
// All HBM-bound; 16-byte vector loads where the buffers allow.
#include "gsmi_internal.h"

namespace gsmi {

namespace {

constexpr int kLossItems = 16;  // floats per thread in the loss kernel

__global__ __launch_bounds__(kBlock) void k_fill_u32(uint32_t* __restrict__ p, int64_t count, uint32_t v) {
  for (int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x; j < count; j += (int64_t)gridDim.x * kBlock)
    p[j] = v;
}

__global__ __launch_bounds__(kBlock) void k_fill_f32(float* __restrict__ p, int64_t count, float v) {
  for (int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x; j < count; j += (int64_t)gridDim.x * kBlock)
    p[j] = v;
}

__global__ __launch_bounds__(kBlock) void k_loss_l1(int64_t count, const float* __restrict__ img,
                                                     const float* __restrict__ tgt, float inv_n,
                                                     float* __restrict__ dLdI, float* __restrict__ part) {
  __shared__ float s[4];
  const int64_t base = (int64_t)blockIdx.x * kBlock * kLossItems;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < kLossItems; ++j) {
    const int64_t e = base + (int64_t)j * kBlock + threadIdx.x;
    if (e < count) {
      const float d = img[e] - tgt[e];
      acc += fabsf(d);
      dLdI[e] = d > 0.f ? inv_n : (d < 0.f ? -inv_n : 0.f);
    }
  }
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = (s[0] + s[1]) + (s[2] + s[3]);
}

__global__ __launch_bounds__(1024) void k_loss_final(int64_t nblk, const float* __restrict__ part,
                                                     double inv_n, float* __restrict__ loss) {
  __shared__ double s[16];
  constexpr int kBatch = 16;  // a batch's loads in flight together; the adds keep the order b, b + 1024, ...
  double acc = 0.0;
  for (int64_t b0 = threadIdx.x; b0 < nblk; b0 += 1024 * kBatch) {
    float x[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) x[q] = part[std::min<int64_t>(b0 + 1024 * q, nblk - 1)];
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      if (b0 + 1024 * q < nblk) acc += (double)x[q];
  }
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int k = 0; k < 16; ++k) t += s[k];
    *loss = (float)(t * inv_n);
  }
}

__device__ __forceinline__ void adam1(float& th, float g, float& m, float& v, const AdamCoef& c) {
  m = c.b1 * m + c.omb1 * g;
  v = c.b2 * v + c.omb2 * g * g;
  th -= c.lr * (m * c.inv_bc1) / (sqrtf(v * c.inv_bc2) + c.eps);
}

__global__ __launch_bounds__(kBlock) void k_adam4(int64_t n4, float4* __restrict__ th,
                                                   const float4* __restrict__ gr, float4* __restrict__ m,
                                                   float4* __restrict__ v, AdamCoef c) {
  for (int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x; j < n4; j += (int64_t)gridDim.x * kBlock) {
    float4 t = th[j], g = gr[j], mm = m[j], vv = v[j];
    adam1(t.x, g.x, mm.x, vv.x, c);
    adam1(t.y, g.y, mm.y, vv.y, c);
    adam1(t.z, g.z, mm.z, vv.z, c);
    adam1(t.w, g.w, mm.w, vv.w, c);
    th[j] = t;
    m[j] = mm;
    v[j] = vv;
  }
}

__global__ __launch_bounds__(kBlock) void k_adam1(int64_t start, int64_t n, float* __restrict__ th,
                                                   const float* __restrict__ gr, float* __restrict__ m,
                                                   float* __restrict__ v, AdamCoef c) {
  const int64_t j = start + (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (j >= n) return;
  float t = th[j], mm = m[j], vv = v[j];
  adam1(t, gr[j], mm, vv, c);
  th[j] = t;
  m[j] = mm;
  v[j] = vv;
}

unsigned grid_for(int64_t work) {
  const int64_t g = ceil_div(work > 0 ? work : 1, kBlock);
  return (unsigned)(g < 65536 ? g : 65536);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

hipError_t launch_fill_u32(uint32_t* p, int64_t count, uint32_t value, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(count)), dim3(kBlock), 0, s, p, count, value);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t count, float value, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_f32, dim3(grid_for(count)), dim3(kBlock), 0, s, p, count, value);
  return hipGetLastError();
}

size_t loss_workspace_bytes(int64_t count) {
  const int64_t nblk = ceil_div(count > 0 ? count : 1, (int64_t)kBlock * kLossItems);
  return (size_t)nblk * sizeof(float);
}

hipError_t launch_loss_l1(int64_t count, const float* image, const float* target, float* loss,
                          float* dLdI, void* ws, hipStream_t s) {
  const int64_t nblk = count > 0 ? ceil_div(count, (int64_t)kBlock * kLossItems) : 0;
  float* part = static_cast<float*>(ws);
  if (nblk > 0)
    hipLaunchKernelGGL(k_loss_l1, dim3((unsigned)nblk), dim3(kBlock), 0, s, count, image, target,
                       (float)(1.0 / (double)count), dLdI, part);
  hipLaunchKernelGGL(k_loss_final, dim3(1), dim3(1024), 0, s, nblk, part,
                     count > 0 ? 1.0 / (double)count : 0.0, loss);
  return hipGetLastError();
}

hipError_t launch_loss_sum(int64_t count, const float* part, double inv_n, float* loss, hipStream_t s) {
  hipLaunchKernelGGL(k_loss_final, dim3(1), dim3(1024), 0, s, count, part, count > 0 ? inv_n : 0.0, loss);
  return hipGetLastError();
}

hipError_t launch_adam(int64_t count, float* params, const float* grads, float* m, float* v,
                       const AdamCoef& c, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  int64_t done = 0;
  if (aligned16(params) && aligned16(grads) && aligned16(m) && aligned16(v)) {
    const int64_t n4 = count / 4;
    if (n4 > 0)
      hipLaunchKernelGGL(k_adam4, dim3(grid_for(n4)), dim3(kBlock), 0, s, n4,
                         reinterpret_cast<float4*>(params), reinterpret_cast<const float4*>(grads),
                         reinterpret_cast<float4*>(m), reinterpret_cast<float4*>(v), c);
    done = n4 * 4;
  }
  if (done < count)
    hipLaunchKernelGGL(k_adam1, dim3((unsigned)ceil_div(count - done, kBlock)), dim3(kBlock), 0, s,
                       done, count, params, grads, m, v, c);
  return hipGetLastError();
}

}  // namespace gsmi
