// L1 + D-SSIM image loss and its gradient (gfx950).
//
// "Scaling 3D Gaussian Splatting with Distributed Compute", the loss passage (a lambda-weighted
// combination of an L1 term and a D-SSIM term) and step "Compute the loss locally" (L1 and a
// fused SSIM).  The pages fix no window or constants; these kernels compute SSIM with an 11x11
// Gaussian window (sigma 1.5, weights g[a] g[b] normalised to sum 1), C1 = 0.01^2 and
// C2 = 0.03^2, over the window positions wholly inside the image, per colour channel, and
//     L = (1 - lambda) mean |I - I*| + lambda (1 - mean SSIM).
// With mu_x = sum_w x, var_x = sum_w x^2 - mu_x^2, cov = sum_w xy - mu_x mu_y and
// S = A B / (C D), A = 2 mu_x mu_y + C1, B = 2 cov + C2, C = mu_x^2 + mu_y^2 + C1,
// D = var_x + var_y + C2, the gradient with respect to the rendered image reaches each pixel
// through the three window sums that contain it:
//     dS/d(sum_w x) = S (2 mu_y / A - 2 mu_y / B - 2 mu_x / C + 2 mu_x / D),
//     dS/d(sum_w x^2) = -S / D,   dS/d(sum_w xy) = 2 S / B,
//     dL/dx(q) = (1 - lambda) sign(x - y) / (3HW)
//                - lambda / M  sum_{p : q in window(p)} w(q - p) (dS_mu(p) + 2 x dS_xx(p) + y dS_xy(p))
// with M = 3 (H - 10)(W - 10) positions.
//
// Two passes, both separable sliding windows with an 11-row register ring per thread:
//   k_ssim_stats   one thread per (channel, window position) column of a 256-column strip: per
//                  input row the block stages the row's pixels in LDS (one coalesced read of
//                  the interleaved [W][3] row), each thread forms the five horizontal window
//                  sums of its column, and once 11 rows are in the ring it forms the vertical
//                  sums, S and the three partials, written planar to the workspace.
//   k_ssim_grad    the same shape over the partials: horizontal then vertical window sums of
//                  the three partial maps (zero outside the positions), combined with x and y
//                  into dL/dx, plus the L1 sum.
// Both fetch each row two steps before they stage it in LDS, so the loads of the next rows
// overlap the window sums of the current one (one barrier per row, two LDS buffers).
// A final one-workgroup kernel sums the per-workgroup partial sums in double.
#include "gsmi_internal.h"

namespace gsmi {

namespace {

constexpr int kWin = 11;
constexpr int kHalf = kWin - 1;          // 10: window extent beyond its first row / column
constexpr int kCols = 256;               // window positions (or pixels) per workgroup row
constexpr int kSsimThreads = 3 * kCols;  // one thread per (channel, column)
constexpr int kRows = 64;                // output rows per workgroup
constexpr int kSpan = kCols + kHalf;     // 266 staged columns per row
constexpr int kSpanPad = 272;

struct SsimCoef {
  float g[kWin];  // 1D window weights (float32 of the double-precision normalised weights)
  float c1, c2;
  float l1_scale;  // (1 - lambda) / (3 H W)
  float s_scale;   // lambda / M
};

__global__ __launch_bounds__(kSsimThreads) void k_ssim_stats(int W, int H, const float* __restrict__ img,
                                                            const float* __restrict__ tgt, SsimCoef k,
                                                            float* __restrict__ dmap, float* __restrict__ part) {
  __shared__ float sx[2][3][kSpanPad];
  __shared__ float sy[2][3][kSpanPad];
  __shared__ float red[kSsimThreads / 64];
  const int Wv = W - kHalf, Hv = H - kHalf;
  const int64_t nv = (int64_t)Wv * Hv;
  const int c0 = blockIdx.x * kCols, r0 = blockIdx.y * kRows;
  const int ch = threadIdx.x / kCols, j = threadIdx.x % kCols;
  const int col = c0 + j;                                 // window position column
  const int nrows = min(kRows + kHalf, H - r0);           // input rows this workgroup reads
  const int span = min(kSpan, W - c0);                    // staged pixel columns
  // Each thread stages the same two of a row's 3 x 266 interleaved values at every row:
  // element e -> pixel column e / 3, channel e % 3 (zero past the image's right edge).
  const int e0 = threadIdx.x, e1 = threadIdx.x + kSsimThreads;
  const int pc0 = e0 / 3, pch0 = e0 - 3 * pc0, pc1 = e1 / 3, pch1 = e1 - 3 * pc1;
  const bool ok0 = pc0 < span, ok1 = pc1 < span, has1 = e1 < 3 * kSpan;
  const float* __restrict__ img_b = img + (int64_t)c0 * 3;
  const float* __restrict__ tgt_b = tgt + (int64_t)c0 * 3;
  // rows are fetched two steps ahead of their use, so the loads overlap the window sums
  auto fetch = [&](int i, float4& f) {
    f = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < nrows) {
      const int64_t off = (int64_t)(r0 + i) * W * 3;
      if (ok0) {
        f.x = img_b[off + e0];
        f.y = tgt_b[off + e0];
      }
      if (ok1) {
        f.z = img_b[off + e1];
        f.w = tgt_b[off + e1];
      }
    }
  };
  auto stage = [&](int buf, const float4& f) {
    sx[buf][pch0][pc0] = f.x;
    sy[buf][pch0][pc0] = f.y;
    if (has1) {
      sx[buf][pch1][pc1] = f.z;
      sy[buf][pch1][pc1] = f.w;
    }
  };
  float ring[kWin][5];
#pragma unroll
  for (int a = 0; a < kWin; ++a)
#pragma unroll
    for (int q = 0; q < 5; ++q) ring[a][q] = 0.f;
  float acc = 0.f;
  float4 fa, fb;  // rows i + 1 and i + 2
  fetch(0, fa);
  stage(0, fa);
  fetch(1, fa);
  fetch(2, fb);
  __syncthreads();

  for (int base = 0; base < nrows; base += kWin) {
#pragma unroll
    for (int s = 0; s < kWin; ++s) {
      const int i = base + s;
      if (i < nrows) {  // uniform over the workgroup
        const int buf = i & 1;
        float h0 = 0.f, h1 = 0.f, h2 = 0.f, h3 = 0.f, h4 = 0.f;
#pragma unroll
        for (int b = 0; b < kWin; ++b) {
          const float x = sx[buf][ch][j + b], y = sy[buf][ch][j + b], w = k.g[b];
          const float wx = w * x, wy = w * y;
          h0 += wx;
          h1 += wy;
          h2 += wx * x;
          h3 += wy * y;
          h4 += wx * y;
        }
        ring[s][0] = h0;
        ring[s][1] = h1;
        ring[s][2] = h2;
        ring[s][3] = h3;
        ring[s][4] = h4;
        if (i >= kHalf) {
          // window position row p = r0 + i - 10 covers input rows i - 10 .. i of this workgroup
          float mx = 0.f, my = 0.f, exx = 0.f, eyy = 0.f, exy = 0.f;
#pragma unroll
          for (int a = 0; a < kWin; ++a) {
            const int sl = (s + 1 + a) % kWin;  // ring slot of input row i - 10 + a
            const float w = k.g[a];
            mx += w * ring[sl][0];
            my += w * ring[sl][1];
            exx += w * ring[sl][2];
            eyy += w * ring[sl][3];
            exy += w * ring[sl][4];
          }
          const int p = r0 + i - kHalf;
          if (col < Wv) {
            const float vx = exx - mx * mx, vy = eyy - my * my, cxy = exy - mx * my;
            const float A = 2.f * mx * my + k.c1, B = 2.f * cxy + k.c2;
            const float C = mx * mx + my * my + k.c1, D = vx + vy + k.c2;
            // four hardware reciprocals (1 ulp) instead of seven IEEE divisions: the kernel is
            // bound by VALU issue, and each division expands to about ten instructions
            const float rA = __builtin_amdgcn_rcpf(A), rB = __builtin_amdgcn_rcpf(B);
            const float rC = __builtin_amdgcn_rcpf(C), rD = __builtin_amdgcn_rcpf(D);
            const float S = (A * B) * (rC * rD);
            acc += S;
            const int64_t o = (int64_t)ch * nv + (int64_t)p * Wv + col;
            dmap[o] = 2.f * S * (my * (rA - rB) + mx * (rD - rC));
            dmap[3 * nv + o] = -S * rD;
            dmap[6 * nv + o] = 2.f * S * rB;
          }
        }
        // row i + 1 into the other buffer (last read at step i - 1, before that step's barrier)
        stage(buf ^ 1, fa);
        fa = fb;
        fetch(i + 3, fb);
        __syncthreads();
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < kSsimThreads / 64; ++w) t += red[w];
    part[blockIdx.y * gridDim.x + blockIdx.x] = t;
  }
}

__global__ __launch_bounds__(kSsimThreads) void k_ssim_grad(int W, int H, const float* __restrict__ img,
                                                           const float* __restrict__ tgt, SsimCoef k,
                                                           const float* __restrict__ dmap,
                                                           float* __restrict__ dLdI, float* __restrict__ part) {
  __shared__ float sd[2][9][kSpanPad];  // [map * 3 + channel][position column - (c0 - 10)]
  __shared__ float red[kSsimThreads / 64];
  const int Wv = W - kHalf, Hv = H - kHalf;
  const int64_t nv = (int64_t)Wv * Hv;
  const int c0 = blockIdx.x * kCols, r0 = blockIdx.y * kRows;
  const int ch = threadIdx.x / kCols, j = threadIdx.x % kCols;
  const int qc = c0 + j;                           // pixel column
  const int nrows = min(kRows, H - r0) + kHalf;    // partial-map rows r0 - 10 .. r0 + rows - 1
  // Each thread stages the same four of a row's 9 x 266 partials at every row: element
  // e -> map row e / 266 (map * 3 + channel), staged column e % 266 = position column
  // c0 - 10 + e % 266 (zero outside the positions).
  int64_t moff[4];
  int mrow[4], mcol[4];
  bool mok[4], mhas[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = threadIdx.x + q * kSsimThreads;
    mhas[q] = e < 9 * kSpan;
    mrow[q] = e / kSpan;
    mcol[q] = e - mrow[q] * kSpan;
    const int pc = c0 - kHalf + mcol[q];
    mok[q] = mhas[q] && pc >= 0 && pc < Wv;
    const int m = mrow[q] / 3, c = mrow[q] - 3 * m;
    moff[q] = mok[q] ? (int64_t)m * 3 * nv + (int64_t)c * nv + pc : 0;
  }
  // step i stages position row r0 - 10 + i and outputs pixel row r0 + i - 10 (i >= 10); both
  // are fetched two steps ahead of their use, so the loads overlap the window sums
  struct Pf {
    float v[4];
    float x, y;
  };
  auto fetch = [&](int i, Pf& f) {
#pragma unroll
    for (int q = 0; q < 4; ++q) f.v[q] = 0.f;
    f.x = f.y = 0.f;
    if (i < nrows) {
      const int pr = r0 - kHalf + i;
      if (pr >= 0 && pr < Hv) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (mok[q]) f.v[q] = dmap[moff[q] + (int64_t)pr * Wv];
      }
      if (i >= kHalf && qc < W) {
        const int64_t e = ((int64_t)(r0 + i - kHalf) * W + qc) * 3 + ch;
        f.x = img[e];
        f.y = tgt[e];
      }
    }
  };
  auto stage = [&](int buf, const Pf& f) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (mhas[q]) sd[buf][mrow[q]][mcol[q]] = f.v[q];
  };
  float ring[kWin][3];
#pragma unroll
  for (int a = 0; a < kWin; ++a)
#pragma unroll
    for (int q = 0; q < 3; ++q) ring[a][q] = 0.f;
  float acc = 0.f;
  Pf fa, fb;  // steps i + 1 and i + 2
  fetch(0, fa);
  stage(0, fa);
  float xc = fa.x, yc = fa.y;  // step i's pixel
  fetch(1, fa);
  fetch(2, fb);
  __syncthreads();

  for (int base = 0; base < nrows; base += kWin) {
#pragma unroll
    for (int s = 0; s < kWin; ++s) {
      const int i = base + s;
      if (i < nrows) {  // uniform over the workgroup
        const int buf = i & 1;
        float h0 = 0.f, h1 = 0.f, h2 = 0.f;
#pragma unroll
        for (int b = 0; b < kWin; ++b) {
          // position column qc - b sits at staged column j + 10 - b
          const float w = k.g[b];
          h0 += w * sd[buf][ch][j + kHalf - b];
          h1 += w * sd[buf][3 + ch][j + kHalf - b];
          h2 += w * sd[buf][6 + ch][j + kHalf - b];
        }
        ring[s][0] = h0;
        ring[s][1] = h1;
        ring[s][2] = h2;
        if (i >= kHalf) {
          // pixel row qr = r0 + i - 10 gathers position rows qr - a, a = 0..10 (steps i - a)
          float gm = 0.f, gxx = 0.f, gxy = 0.f;
#pragma unroll
          for (int a = 0; a < kWin; ++a) {
            const int sl = (s - a + kWin) % kWin;
            const float w = k.g[a];
            gm += w * ring[sl][0];
            gxx += w * ring[sl][1];
            gxy += w * ring[sl][2];
          }
          const int qr = r0 + i - kHalf;
          if (qc < W) {
            const int64_t e = ((int64_t)qr * W + qc) * 3 + ch;
            const float d = xc - yc;
            acc += fabsf(d);
            const float dS = gm + 2.f * xc * gxx + yc * gxy;
            const float sg = d > 0.f ? k.l1_scale : (d < 0.f ? -k.l1_scale : 0.f);
            dLdI[e] = sg - k.s_scale * dS;
          }
        }
        // step i + 1's row into the other buffer (last read at step i - 1, before its barrier)
        stage(buf ^ 1, fa);
        xc = fa.x;
        yc = fa.y;
        fa = fb;
        fetch(i + 3, fb);
        __syncthreads();
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < kSsimThreads / 64; ++w) t += red[w];
    part[blockIdx.y * gridDim.x + blockIdx.x] = t;
  }
}

// loss[0] = L, loss[1] = mean |I - I*|, loss[2] = mean SSIM, from the per-workgroup sums.
__global__ __launch_bounds__(1024) void k_ssim_final(int64_t n_ssim, const float* __restrict__ part_ssim,
                                                     int64_t n_l1, const float* __restrict__ part_l1,
                                                     double inv_m, double inv_p, double lambda,
                                                     float* __restrict__ loss) {
  __shared__ double s1[16], s2[16];
  double a = 0.0, b = 0.0;
  for (int64_t q = threadIdx.x; q < n_ssim; q += 1024) a += (double)part_ssim[q];
  for (int64_t q = threadIdx.x; q < n_l1; q += 1024) b += (double)part_l1[q];
  for (int o = 32; o > 0; o >>= 1) {
    a += __shfl_xor(a, o, 64);
    b += __shfl_xor(b, o, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    s1[threadIdx.x >> 6] = a;
    s2[threadIdx.x >> 6] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double ts = 0.0, tl = 0.0;
    for (int w = 0; w < 16; ++w) {
      ts += s1[w];
      tl += s2[w];
    }
    const double ssim = ts * inv_m, l1 = tl * inv_p;
    loss[0] = (float)((1.0 - lambda) * l1 + lambda * (1.0 - ssim));
    loss[1] = (float)l1;
    loss[2] = (float)ssim;
  }
}

struct SsimLayout {
  size_t dmap, part_ssim, part_l1, total;
  dim3 g_stats, g_grad;
};

SsimLayout ssim_layout(int W, int H) {
  SsimLayout L{};
  const int64_t Wv = W - kHalf, Hv = H - kHalf;
  L.g_stats = dim3((unsigned)ceil_div(Wv, kCols), (unsigned)ceil_div(Hv, kRows));
  L.g_grad = dim3((unsigned)ceil_div(W, kCols), (unsigned)ceil_div(H, kRows));
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  L.dmap = 0;
  L.part_ssim = up((size_t)9 * Wv * Hv * sizeof(float));
  L.part_l1 = L.part_ssim + up((size_t)L.g_stats.x * L.g_stats.y * sizeof(float));
  L.total = L.part_l1 + up((size_t)L.g_grad.x * L.g_grad.y * sizeof(float));
  return L;
}

}  // namespace

size_t ssim_workspace_bytes(int W, int H) { return ssim_layout(W, H).total; }

hipError_t launch_loss_l1_dssim(int W, int H, const float* image, const float* target, float lambda,
                                float* loss, float* dLdI, void* ws, hipStream_t s) {
  const SsimLayout L = ssim_layout(W, H);
  SsimCoef k{};
  double g[kWin], gs = 0.0;
  for (int a = 0; a < kWin; ++a) {
    const double d = (double)(a - kWin / 2);
    g[a] = exp(-d * d / (2.0 * 1.5 * 1.5));
    gs += g[a];
  }
  for (int a = 0; a < kWin; ++a) k.g[a] = (float)(g[a] / gs);
  k.c1 = (float)(0.01 * 0.01);
  k.c2 = (float)(0.03 * 0.03);
  const double npx3 = 3.0 * (double)W * (double)H;
  const double m = 3.0 * (double)(W - kHalf) * (double)(H - kHalf);
  k.l1_scale = (float)((1.0 - (double)lambda) / npx3);
  k.s_scale = (float)((double)lambda / m);
  char* base = static_cast<char*>(ws);
  float* dmap = reinterpret_cast<float*>(base + L.dmap);
  float* ps = reinterpret_cast<float*>(base + L.part_ssim);
  float* pl = reinterpret_cast<float*>(base + L.part_l1);
  hipLaunchKernelGGL(k_ssim_stats, L.g_stats, dim3(kSsimThreads), 0, s, W, H, image, target, k, dmap, ps);
  hipLaunchKernelGGL(k_ssim_grad, L.g_grad, dim3(kSsimThreads), 0, s, W, H, image, target, k, dmap, dLdI, pl);
  hipLaunchKernelGGL(k_ssim_final, dim3(1), dim3(1024), 0, s, (int64_t)L.g_stats.x * L.g_stats.y, ps,
                     (int64_t)L.g_grad.x * L.g_grad.y, pl, 1.0 / m, 1.0 / npx3, (double)lambda, loss);
  return hipGetLastError();
}

}  // namespace gsmi
