// Row-wise kernels: rotary/timestep tables, embedding gather (+ timestep
// embedding) fused with the first RMSNorm, plain RMSNorm, and the MoE combine
// fused with the residual add and the next RMSNorm.  All are HBM/latency bound
// row sweeps: one 256-thread workgroup per token row, coalesced along d.
#include "dg_common.h"
#include "dg_internal.h"

namespace dg {

// rope_tab[m][i] = (cos, sin)(pos(m) * theta^(-2i/hd)), computed in fp64 so that
// positions in the tens of thousands keep full fp32 accuracy.
// temb[j] = sin(1000 t f_j) (j < d/2), cos(1000 t f_{j-d/2}) (j >= d/2), f_j = 10000^(-j/(d/2)).
__global__ void prep_kernel(PassGeom g, int hd, float theta, float2* rope_tab, int d, float t,
                            float* temb) {
  const int half = hd / 2;
  const int M = g.batch * g.n;
  const long total = (long)M * half + (temb ? d : 0);
  for (long idx = blockIdx.x * (long)blockDim.x + threadIdx.x; idx < total;
       idx += (long)gridDim.x * blockDim.x) {
    if (idx < (long)M * half) {
      const int m = (int)(idx / half), i = (int)(idx - (long)m * half);
      const int b = m / g.n;
      const double pos = (double)(g.len[b] + (m - b * g.n));
      const double ang = pos * pow((double)theta, -2.0 * i / hd);
      rope_tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
    } else {
      const int j = (int)(idx - (long)M * half);
      const int hh = d / 2;
      const int jj = j < hh ? j : j - hh;
      const double a = 1000.0 * (double)t * pow(10000.0, -(double)jj / hh);
      temb[j] = (float)(j < hh ? sin(a) : cos(a));
    }
  }
}

void launch_prep(const PassGeom& g, int hd, float theta, float2* rope_tab, int d, float t,
                 float* temb, hipStream_t s) {
  const long total = (long)g.batch * g.n * (hd / 2) + (temb ? d : 0);
  const int blocks = (int)std::min<long>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(prep_kernel, dim3(blocks), dim3(256), 0, s, g, hd, theta, rope_tab, d, t, temb);
}

__device__ __forceinline__ void norm_row(const float* xr, const float* gain, float eps, uint16_t* hr,
                                         int d, float ss, float* red) {
  const float tot = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
  for (int c = threadIdx.x; c < d; c += blockDim.x) hr[c] = f2bf(xr[c] * inv * gain[c]);
}

__global__ __launch_bounds__(256) void embed_norm_kernel(const int32_t* tokens, const uint16_t* embed,
                                                         const float* temb, const float* gain,
                                                         float eps, float* x, uint16_t* h, int d,
                                                         int vocab) {
  __shared__ float red[16];
  const int m = blockIdx.x;
  // ids outside [0, V] (V = [MASK]) are clamped so a bad id can never read past the table
  const int tok = min(max(tokens[m], 0), vocab);
  const uint16_t* er = embed + (size_t)tok * d;
  float* xr = x + (size_t)m * d;
  float ss = 0.f;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float v = bf2f(er[c]);
    if (temb) v += temb[c];
    xr[c] = v;
    ss += v * v;
  }
  norm_row(xr, gain, eps, h + (size_t)m * d, d, ss, red);
}

void launch_embed_norm(const int32_t* tokens, const uint16_t* embed, const float* temb,
                       const float* gain, float eps, float* x, uint16_t* h, int M, int d, int vocab,
                       hipStream_t s) {
  hipLaunchKernelGGL(embed_norm_kernel, dim3(M), dim3(256), 0, s, tokens, embed, temb, gain, eps, x,
                     h, d, vocab);
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* x, const float* gain, float eps,
                                                      uint16_t* h, int d) {
  __shared__ float red[16];
  const int m = blockIdx.x;
  const float* xr = x + (size_t)m * d;
  float ss = 0.f;
  for (int c = threadIdx.x; c < d; c += blockDim.x) ss += xr[c] * xr[c];
  norm_row(xr, gain, eps, h + (size_t)m * d, d, ss, red);
}

void launch_rmsnorm(const float* x, const float* gain, float eps, uint16_t* h, int M, int d,
                    hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(M), dim3(256), 0, s, x, gain, eps, h, d);
}

// x[m] += sum_j w[m][j] * Y[inv[m*k + j]]  (j ascending), then h[m] = norm(x[m]) * next_gain.
__global__ __launch_bounds__(256) void combine_kernel(float* x, const float* Y, const float* wts,
                                                      const int32_t* inv, int k, int d,
                                                      const float* next_gain, float eps,
                                                      uint16_t* h) {
  __shared__ float red[16];
  __shared__ int slot[16];
  __shared__ float wt[16];
  const int m = blockIdx.x;
  if (threadIdx.x < k) {
    slot[threadIdx.x] = inv[(size_t)m * k + threadIdx.x];
    wt[threadIdx.x] = wts[(size_t)m * k + threadIdx.x];
  }
  __syncthreads();
  float* xr = x + (size_t)m * d;
  float ss = 0.f;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float y = 0.f;
    for (int j = 0; j < k; ++j) y += wt[j] * Y[(size_t)slot[j] * d + c];
    const float v = xr[c] + y;
    xr[c] = v;
    ss += v * v;
  }
  if (next_gain) norm_row(xr, next_gain, eps, h + (size_t)m * d, d, ss, red);
}

void launch_combine(float* x, const float* Y, const float* wts, const int32_t* inv, int M, int k,
                    int d, const float* next_gain, float eps, uint16_t* h, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3(M), dim3(256), 0, s, x, Y, wts, inv, k, d, next_gain, eps,
                     h);
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

void launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t s) {
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(blocks), dim3(256), 0, s, p, v, n);
}

}  // namespace dg
