// Entropy-bounded sampler (DiffusionGemma Technical Report §3.3): per masked
// canvas row, entropy and argmax of softmax(logits); then the masked positions
// are accepted in order of increasing entropy while the running entropy sum
// stays within the budget gamma (at least one per step).
//
// Pass 1 streams the bf16 logits once (HBM-bound: 512 KiB per 262144-wide
// row): one 256-thread workgroup per (row, 8192-logit chunk) computes the
// chunk max m_c, its lowest argmax, s_c = sum exp(x - m_c) and
// t_c = sum exp(x - m_c) (m_c - x).  Rows that are not [MASK] are skipped.
// Pass 2 (one workgroup per sequence) merges the chunks of each row in index
// order, H = log S + T / S, ranks the masked rows by (H, position), takes the
// running fp64 sum in rank order, and commits the argmax of the first k* rows.
#include <math.h>

#include "dg_common.h"
#include "dg_internal.h"

namespace dg {

__global__ __launch_bounds__(256) void sample_partials_kernel(const uint16_t* __restrict__ logits,
                                                              const int32_t* __restrict__ canvas,
                                                              int vocab, int nchunks,
                                                              float4* __restrict__ part,
                                                              int* __restrict__ part_arg) {
  __shared__ float rv[4];
  __shared__ int ri[4];
  __shared__ float red[16];
  const int row = blockIdx.y, ch = blockIdx.x;
  if (canvas[row] != vocab) return;
  const int tid = threadIdx.x;
  const int c0 = ch * kSampleChunk;
  const uint16_t* lp = logits + (size_t)row * vocab;

  float x[32];
  float bv = -INFINITY;
  int bi = INT_MAX;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e0 = c0 + (i * 256 + tid) * 8;
    if (e0 < vocab && e0 < c0 + kSampleChunk) {
      const u32x4 v = ld16(lp + e0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * i + 2 * j] = __uint_as_float(v[j] << 16);
        x[8 * i + 2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (x[8 * i + j] > bv) {
          bv = x[8 * i + j];
          bi = e0 + j;
        }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[8 * i + j] = -INFINITY;
    }
  }
  // (max, lowest index) over the workgroup
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if ((tid & 63) == 0) {
    rv[tid >> 6] = bv;
    ri[tid >> 6] = bi;
  }
  __syncthreads();
  float m = rv[0];
  int am = ri[0];
  for (int w = 1; w < 4; ++w)
    if (rv[w] > m || (rv[w] == m && ri[w] < am)) {
      m = rv[w];
      am = ri[w];
    }
  float s = 0.f, t = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    // padding lanes (past the end of the vocabulary) hold -inf and contribute nothing
    if (x[j] != -INFINITY) {
      const float dlt = m - x[j];
      const float e = __expf(-dlt);
      s += e;
      t += e * dlt;
    }
  }
  s = block_sum(s, red);
  t = block_sum(t, red);
  if (tid == 0) {
    part[(size_t)row * nchunks + ch] = make_float4(m, s, t, 0.f);
    part_arg[(size_t)row * nchunks + ch] = am;
  }
}

void launch_sample_partials(const uint16_t* logits, const int32_t* canvas, int rows, int vocab,
                            float4* part, int* part_arg, hipStream_t s) {
  const int nchunks = (vocab + kSampleChunk - 1) / kSampleChunk;
  hipLaunchKernelGGL(sample_partials_kernel, dim3(nchunks, rows), dim3(256), 0, s, logits, canvas,
                     vocab, nchunks, part, part_arg);
}

__global__ __launch_bounds__(1024) void eb_select_kernel(const float4* __restrict__ part,
                                                         const int* __restrict__ part_arg,
                                                         int nchunks, const float* __restrict__ H_in,
                                                         const int32_t* __restrict__ amax_in,
                                                         int32_t* __restrict__ canvas, int C,
                                                         int vocab, float gamma, int commit_all,
                                                         float* __restrict__ H_out,
                                                         int32_t* __restrict__ amax_out,
                                                         int32_t* __restrict__ n_masked) {
  __shared__ float Hs[1024];
  __shared__ int msk[1024];
  __shared__ int order[1024];
  __shared__ int nm_s, kstar_s;
  const int b = blockIdx.x, c = threadIdx.x;
  const size_t idx = (size_t)b * C + c;
  const bool masked = c < C && canvas[idx] == vocab;
  float H = INFINITY;
  int a = 0;
  if (masked) {
    if (part) {
      const float4* pr = part + idx * nchunks;
      const int* pa = part_arg + idx * nchunks;
      float M = -INFINITY;
      for (int k = 0; k < nchunks; ++k) M = fmaxf(M, pr[k].x);
      a = INT_MAX;
      float S = 0.f, T = 0.f;
      for (int k = 0; k < nchunks; ++k) {
        const float4 p = pr[k];
        if (p.x == M && a == INT_MAX) a = pa[k];
        const float sc = expf(p.x - M);
        S += p.y * sc;
        T += sc * (p.z + (M - p.x) * p.y);
      }
      H = logf(S) + T / S;
    } else {
      H = H_in[idx];
      a = amax_in[idx];
    }
    if (a < 0 || a >= vocab) a = min(max(a, 0), vocab - 1);
  }
  const float key = (masked && !(H != H)) ? H : INFINITY;
  if (c < C) {
    Hs[c] = key;
    msk[c] = masked ? 1 : 0;
  }
  __syncthreads();
  int rank = 0, nm = 0;
  if (masked) {
    for (int j = 0; j < C; ++j) {
      if (!msk[j]) continue;
      nm += 1;
      const float hj = Hs[j];
      if (hj < key || (hj == key && j < c)) rank += 1;
    }
    order[rank] = c;
  }
  if (c == 0) {
    int cntm = 0;
    for (int j = 0; j < C; ++j) cntm += msk[j];
    nm_s = cntm;
  }
  __syncthreads();
  if (c == 0) {
    const int n = nm_s;
    int ks;
    if (commit_all || n == 0) {
      ks = n;
    } else {
      double S = 0.0;
      int k = 0;
      for (int j = 0; j < n; ++j) {
        S += (double)Hs[order[j]];
        if (S <= (double)gamma)
          k = j + 1;
        else
          break;
      }
      ks = k < 1 ? 1 : k;
    }
    kstar_s = ks;
    n_masked[b] = n - ks;
  }
  __syncthreads();
  if (c < C) {
    if (H_out) H_out[idx] = masked ? H : __int_as_float(0x7fc00000);
    if (amax_out) amax_out[idx] = masked ? a : -1;
    if (masked && rank < kstar_s) canvas[idx] = a;
  }
  (void)nm;
}

void launch_eb_select(const float4* part, const int* part_arg, int nchunks, const float* H_in,
                      const int32_t* amax_in, int32_t* canvas, int batch, int C, int vocab,
                      float gamma, int commit_all, float* H_out, int32_t* amax_out,
                      int32_t* n_masked, hipStream_t s) {
  const int threads = ((C + 63) / 64) * 64;
  hipLaunchKernelGGL(eb_select_kernel, dim3(batch), dim3(threads), 0, s, part, part_arg, nchunks,
                     H_in, amax_in, canvas, C, vocab, gamma, commit_all, H_out, amax_out, n_masked);
}

}  // namespace dg
