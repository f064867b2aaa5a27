// Row-wise kernels: rotary/timestep tables, embedding gather (+ timestep
// embedding) fused with the first RMSNorm, plain RMSNorm, and the MoE combine
// fused with the residual add and the next RMSNorm.  One workgroup per token row
// with one thread per 8 consecutive features (16 B of bf16), rounded up to whole
// waves (row_threads), so each thread makes a single pass over its features.
// The residual stream x is fp32 row-major; the normed output h is written in
// fragment-major layout for the GEMMs that consume it.
#include "dg_common.h"
#include "dg_internal.h"

namespace dg {

// rope_tab[m][i] = (cos, sin)(pos(m) * theta^(-2i/hd)), computed in fp64 so that
// positions in the tens of thousands keep full fp32 accuracy.
// temb[b][j] = sin(1000 t_b f_j) (j < d/2), cos(1000 t_b f_{j-d/2}) (j >= d/2), f_j =
// 10000^(-j/(d/2)), t_b sequence b's denoising time.
// Workgroup 0 also clears the pass's counters zero[0 .. nzero).
__global__ void prep_kernel(PassGeom g, int hd, float theta, float2* rope_tab, int d,
                            float* temb, int32_t* zero, int nzero) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nzero; i += blockDim.x) zero[i] = 0;
  const int half = hd / 2;
  const int M = g.batch * g.n;
  const long total = (long)M * half + (temb ? (long)g.batch * d : 0);
  for (long idx = blockIdx.x * (long)blockDim.x + threadIdx.x; idx < total;
       idx += (long)gridDim.x * blockDim.x) {
    if (idx < (long)M * half) {
      const int m = (int)(idx / half), i = (int)(idx - (long)m * half);
      const int b = m / g.n;
      const double pos = (double)(g.len[b] + (m - b * g.n));
      const double ang = pos * pow((double)theta, -2.0 * i / hd);
      rope_tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
    } else {
      const long e = idx - (long)M * half;
      const int b = (int)(e / d), j = (int)(e - (long)b * d);
      const int hh = d / 2;
      const int jj = j < hh ? j : j - hh;
      const double a = 1000.0 * (double)g.t[b] * pow(10000.0, -(double)jj / hh);
      temb[e] = (float)(j < hh ? sin(a) : cos(a));
    }
  }
}

void launch_prep(const PassGeom& g, int hd, float theta, float2* rope_tab, int d,
                 float* temb, int32_t* zero, int nzero, hipStream_t s) {
  const long total = (long)g.batch * g.n * (hd / 2) + (temb ? (long)g.batch * d : 0);
  const int blocks = (int)std::min<long>((total + 255) / 256, 4096);
  launch_kernel(prep_kernel, dim3(std::max(blocks, 1)), dim3(256), 0, s, nullptr, g, hd, theta, rope_tab, d,
                temb, zero, nzero);
}

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
}

__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// h[m] (fragment-major, K = d) = x[m] / sqrt(mean(x^2) + eps) * gain, given ss = this
// thread's share of sum(x^2); also row-major into h_rm when given.
__device__ __forceinline__ void norm_row(const float* xr, const float* gain, float eps, uint16_t* h,
                                         int m, int d, float ss, float* red,
                                         uint16_t* h_rm = nullptr) {
  const float tot = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
  for (int c = 8 * threadIdx.x; c < d; c += 8 * blockDim.x) {
    float v[8], gg[8];
    load8(xr + c, v);
    load8(gain + c, gg);
    u32x4 o;
    o.x = pack_bf2(v[0] * inv * gg[0], v[1] * inv * gg[1]);
    o.y = pack_bf2(v[2] * inv * gg[2], v[3] * inv * gg[3]);
    o.z = pack_bf2(v[4] * inv * gg[4], v[5] * inv * gg[5]);
    o.w = pack_bf2(v[6] * inv * gg[6], v[7] * inv * gg[7]);
    *reinterpret_cast<u32x4*>(h + fm_index(m, c, d)) = o;
    if (h_rm) *reinterpret_cast<u32x4*>(h_rm + (size_t)m * d + c) = o;
  }
}

// x[m] = E[token] (+ temb of its sequence) (+ z[m], the self-conditioning signal) -- the
// two added only on the rows of denoising sequences -- then the first RMSNorm.
__global__ __launch_bounds__(1024) void embed_norm_kernel(const int32_t* tokens, const uint16_t* embed,
                                                         const float* temb, const float* z, int n, uint64_t enc,
                                                         const float* gain, float eps, float* x, uint16_t* h,
                                                         int d, int vocab) {
  __shared__ float red[16];
  const int m = blockIdx.x;
  const int b = m / n;
  if ((enc >> b) & 1) {                // a row of an encoding sequence: the token alone
    temb = nullptr;
    z = nullptr;
  }
  if (temb) temb += (size_t)b * d;
  // ids outside [0, V] (V = [MASK]) are clamped so a bad id can never read past the table
  const int tok = min(max(tokens[m], 0), vocab);
  float* xr = x + (size_t)m * d;
  float ss = 0.f;
  for (int c = 8 * threadIdx.x; c < d; c += 8 * blockDim.x) {
    const u32x4 e = ld16(embed + fm_index(tok, c, d));
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(e[j] << 16);
      v[2 * j + 1] = __uint_as_float(e[j] & 0xffff0000u);
    }
    if (temb) {
      float tt[8];
      load8(temb + c, tt);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] += tt[j];
    }
    if (z) {
      float zz[8];
      load8(z + (size_t)m * d + c, zz);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] += zz[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += v[j] * v[j];
    store8(xr + c, v);
  }
  norm_row(xr, gain, eps, h, m, d, ss, red);
}

// threads of a row workgroup: one per 8 features, whole waves, at most 1024
static int row_threads(int d) { return std::min(1024, std::max(64, (d / 8 + 63) / 64 * 64)); }

void launch_embed_norm(const int32_t* tokens, const uint16_t* embed, const float* temb, const float* z,
                       int n, uint64_t enc, const float* gain, float eps, float* x, uint16_t* h, int M, int d,
                       int vocab, hipStream_t s) {
  launch_kernel(embed_norm_kernel, dim3(M), dim3(row_threads(d)), 0, s, nullptr, tokens, embed, temb, z, n, enc,
                gain, eps, x, h, d, vocab);
}

__global__ __launch_bounds__(1024) void rmsnorm_kernel(const float* x, const float* gain, float eps,
                                                      uint16_t* h, uint16_t* h_rm, int d) {
  __shared__ float red[16];
  const int m = blockIdx.x;
  const float* xr = x + (size_t)m * d;
  float ss = 0.f;
  for (int c = 8 * threadIdx.x; c < d; c += 8 * blockDim.x) {
    float v[8];
    load8(xr + c, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += v[j] * v[j];
  }
  norm_row(xr, gain, eps, h, m, d, ss, red, h_rm);
}

void launch_rmsnorm(const float* x, const float* gain, float eps, uint16_t* h, uint16_t* h_rm, int M,
                    int d, hipStream_t s, hipEvent_t done) {
  // `done`, when given, is signalled by the kernel's own completion (no separate
  // marker on the stream)
  launch_kernel(rmsnorm_kernel, dim3(M), dim3(row_threads(d)), 0, s, done, x, gain, eps, h, h_rm, d);
}

// x[m] += ys[m] (the shared expert), then += sum_j w[m][j] * Y[inv[m*k + j]]
// (j ascending), then h[m] = norm(x[m]) * next_gain.  With rows_out given (the
// last layer of a pass whose head needs only some rows: those of the denoising
// sequences -- skip has the bits of the others -- and, with canvas given, only their
// [MASK] rows), only those rows are normed, each into the next free h row i taken
// from *count (zero on entry; it ends as the number of rows kept), with
// rows_out[i] = m - row_base (the head's output row).
// The order of the compacted rows varies from run to run; every logits row the
// head computes from them does not depend on it.
__global__ __launch_bounds__(1024) void combine_kernel(float* x, const float* ys, const float* Y,
                                                      const float* wts,
                                                      const int32_t* inv, int k, int d,
                                                      const float* next_gain, float eps,
                                                      uint16_t* h, const int32_t* canvas, int mask_id,
                                                      uint64_t skip, int n, int32_t* rows_out, int32_t* count,
                                                      int row_base) {
  __shared__ float red[16];
  __shared__ int out_row;
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
  for (int c = 8 * threadIdx.x; c < d; c += 8 * blockDim.x) {
    float v[8], u[8];
    load8(xr + c, v);
    load8(ys + (size_t)m * d + c, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = u[e] + v[e];
    for (int j = 0; j < k; ++j) {
      float y[8];
      load8(Y + (size_t)slot[j] * d + c, y);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += wt[j] * y[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
    store8(xr + c, v);
  }
  if (!next_gain) return;
  if (rows_out) {
    if ((skip >> (m / n)) & 1) return;                 // uniform per workgroup
    if (canvas && canvas[m] != mask_id) return;
    if (threadIdx.x == 0) {
      const int i = atomicAdd(count, 1);
      rows_out[i] = m - row_base;
      out_row = i;
    }
    __syncthreads();
    norm_row(xr, next_gain, eps, h, out_row, d, ss, red);
  } else {
    norm_row(xr, next_gain, eps, h, m, d, ss, red);
  }
}

void launch_combine(float* x, const float* ys, const float* Y, const float* wts, const int32_t* inv,
                    int M, int k, int d, const float* next_gain, float eps, uint16_t* h,
                    const int32_t* canvas, int mask_id, uint64_t skip, int n, int32_t* rows_out, int32_t* count,
                    int row_base, hipStream_t s) {
  launch_kernel(combine_kernel, dim3(M), dim3(row_threads(d)), 0, s, nullptr, x, ys, Y, wts, inv, k, d, next_gain, eps, h,
                canvas, mask_id, skip, n, rows_out, count, row_base);
}

// End of a serving pass: every sequence whose bit in enc is set has just appended its
// finished canvas; its canvas row is copied to out + off.v[b] (when out is given) and
// refilled with [MASK] for its next block.
__global__ void serve_finish_kernel(int32_t* canvas, int C, int32_t mask_id, uint64_t enc, int32_t* out,
                                    SeqOffsets off) {
  const int b = blockIdx.y;
  if (!((enc >> b) & 1)) return;   // uniform per workgroup
  int32_t* row = canvas + (size_t)b * C;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < C; i += gridDim.x * 256) {
    if (out) out[off.v[b] + i] = row[i];
    row[i] = mask_id;
  }
}

void launch_serve_finish(int32_t* canvas, int batch, int C, int32_t mask_id, uint64_t enc, int32_t* out,
                         const SeqOffsets& off, hipStream_t s) {
  launch_kernel(serve_finish_kernel, dim3((C + 255) / 256, batch), dim3(256), 0, s, nullptr, canvas, C, mask_id,
                enc, out, off);
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ __launch_bounds__(256) void copy16_kernel(const u32x4* __restrict__ src,
                                                     u32x4* __restrict__ dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

void launch_copy16(const void* src, void* dst, size_t n_bytes, hipStream_t s) {
  const size_t n = n_bytes / 16;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 8192);
  launch_kernel(copy16_kernel, dim3(blocks), dim3(256), 0, s, nullptr, reinterpret_cast<const u32x4*>(src),
                reinterpret_cast<u32x4*>(dst), n);
}

// Achievable bf16 MFMA rate: each wave runs iters rounds over kRateChains independent
// accumulators, each round one dependent pair of v_mfma_f32_16x16x32_bf16 per
// accumulator (the order in which this core issues MFMAs at full rate, as the GEMMs
// do), on register operands (all ones: every element gains 32 per MFMA), with no
// memory traffic; then each lane writes the sum of its accumulators --
// kRateChains * 4 * 64 * iters exactly while that stays below 2^24 -- so the work
// cannot be dropped and its count can be checked.
constexpr int kRateChains = 4;
__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, float* __restrict__ out) {
  const uint32_t one2 = 0x3f803f80u;   // two bf16 ones
  const u32x4 a = {one2, one2, one2, one2};
  f32x4 acc[kRateChains];
#pragma unroll
  for (int c = 0; c < kRateChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kRateChains; ++c) acc[c] = mfma16x2(a, a, a, a, acc[c]);
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < kRateChains; ++c) sum += (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

void launch_mfma_rate(int blocks, int iters, float* out, hipStream_t s) {
  launch_kernel(mfma_rate_kernel, dim3(blocks), dim3(256), 0, s, nullptr, iters, out);
}

// Achievable HBM read rate: thread t of the grid XORs the 16-byte words t, t + S,
// t + 2S, ... (S = the grid's thread count) of src, four loads in flight per step, and
// writes the first 32-bit lane of its XOR to out[t] (a checkable result: src filled
// with one repeated word w gives w where the thread read an odd number of words).
__global__ __launch_bounds__(256) void read_rate_kernel(const u32x4* __restrict__ src, size_t n,
                                                        uint32_t* __restrict__ out) {
  const size_t S = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t t = i;
  u32x4 x = {0u, 0u, 0u, 0u};
  for (; i + 3 * S < n; i += 4 * S) {
    const u32x4 a = src[i], b = src[i + S], c = src[i + 2 * S], d = src[i + 3 * S];
    x ^= a ^ b ^ c ^ d;
  }
  for (; i < n; i += S) x ^= src[i];
  out[t] = x.x;
}

void launch_read_rate(const void* src, size_t n_bytes, int blocks, uint32_t* out, hipStream_t s) {
  launch_kernel(read_rate_kernel, dim3(blocks), dim3(256), 0, s, nullptr, reinterpret_cast<const u32x4*>(src),
                n_bytes / 16, out);
}

void launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t s) {
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 1024);
  launch_kernel(fill_i32_kernel, dim3(blocks), dim3(256), 0, s, nullptr, p, v, n);
}

}  // namespace dg
