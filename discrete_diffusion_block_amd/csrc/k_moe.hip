// Mixture-of-experts block: router top-k, deterministic token->expert
// permutation, and the two grouped expert GEMMs.
//
// At a 256-token canvas with 128 experts and top-8 routing, 2048 assignments
// spread over (nearly) every expert, ~16 tokens each: the expert GEMMs stream
// ~1.5 GB of weights per layer at an arithmetic intensity of ~16 flop/B, so
// they are HBM-bound weight streamers.  Each wave owns 16 output features of
// one expert and all of that expert's tokens: weight rows go to the MFMA A
// side and are read from HBM exactly once; the expert's gathered token rows
// (B side, a few KB) come from L2.  No token ever moves: rows are gathered
// through the permutation at load time.
#include <limits.h>
#include <math.h>

#include "dg_common.h"
#include "dg_internal.h"

namespace dg {

// ---------------------------------------------------------------- top-k

// One wave per token.  Experts are ranked by (logit desc, id asc); NaN logits
// rank below every number.  Weights: softmax over the k selected logits.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ r, int M, int E, int k,
                                                   int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    float x = e < E ? r[(size_t)m * E + e] : -INFINITY;
    if (x != x) x = -INFINITY;
    v[i] = e < E ? x : -INFINITY;
  }
  unsigned taken = 0;
  float sel[16];
  for (int t = 0; t < k; ++t) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    sel[t] = bv;
    if (lane == 0) ids[(size_t)m * k + t] = bi;
  }
  if (lane == 0) {
    float z = 0.f;
    float ex[16];
    for (int t = 0; t < k; ++t) {
      ex[t] = (sel[t] == -INFINITY) ? 0.f : expf(sel[t] - sel[0]);
      z += ex[t];
    }
    for (int t = 0; t < k; ++t) w[(size_t)m * k + t] = ex[t] / z;
  }
}

void launch_topk(const float* r, int M, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3((M + 3) / 4), dim3(256), 0, s, r, M, E, k, ids, w);
}

// ---------------------------------------------------------------- permutation

// Stable counting sort of the M*k assignments (a = m*k + j) by expert, in one
// 1024-thread workgroup: per-expert counts, exclusive offsets, then slots in
// assignment order within each expert.  perm[slot] = token, inv[a] = slot.
__global__ __launch_bounds__(1024) void route_kernel(const int32_t* __restrict__ ids, int A, int k,
                                                     int E, int32_t* __restrict__ cnt,
                                                     int32_t* __restrict__ offs,
                                                     int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ inv) {
  __shared__ int hist[256];
  __shared__ int base[256];
  __shared__ int wcnt[16][256];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int e = tid; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  for (int a = tid; a < A; a += blockDim.x) atomicAdd(&hist[ids[a]], 1);
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      base[e] = run;
      offs[e] = run;
      cnt[e] = hist[e];
      run += hist[e];
    }
    offs[E] = run;
  }
  __syncthreads();
  for (int start = 0; start < A; start += blockDim.x) {
    for (int i = tid; i < 16 * E; i += blockDim.x) wcnt[i / E][i % E] = 0;
    __syncthreads();
    const int a = start + tid;
    const int e = a < A ? ids[a] : -1;
    int rank = 0, tot = 0;
    for (int j = 0; j < 64; ++j) {
      const int ej = __shfl(e, j, 64);
      if (ej == e) {
        tot += 1;
        if (j < lane) rank += 1;
      }
    }
    if (e >= 0 && rank == tot - 1) wcnt[wv][e] = tot;
    __syncthreads();
    if (e >= 0) {
      int before = 0;
      for (int w2 = 0; w2 < wv; ++w2) before += wcnt[w2][e];
      const int slot = base[e] + before + rank;
      perm[slot] = a / k;
      inv[a] = slot;
    }
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += blockDim.x) {
      int s = 0;
      for (int w2 = 0; w2 < 16; ++w2) s += wcnt[w2][e2];
      base[e2] += s;
    }
    __syncthreads();
  }
}

void launch_route(const int32_t* ids, int M, int k, int E, int32_t* cnt, int32_t* offs,
                  int32_t* perm, int32_t* inv, hipStream_t s) {
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(1024), 0, s, ids, M * k, k, E, cnt, offs, perm, inv);
}

// ---------------------------------------------------------------- grouped GEMMs

__device__ __forceinline__ float silu_f(float v) { return v / (1.0f + __expf(-v)); }

// A[slot][f] = silu(x W_g[e][f]^T) * (x W_u[e][f]^T) for every slot of expert e,
// x = h[perm[slot]].  Wave = (expert, 16 features); TT token tiles per pass.
template <int TT>
__global__ __launch_bounds__(256) void moe_gate_up_kernel(const uint16_t* __restrict__ h,
                                                          const uint16_t* __restrict__ wgu,
                                                          const int32_t* __restrict__ cnt,
                                                          const int32_t* __restrict__ offs,
                                                          const int32_t* __restrict__ perm, int E,
                                                          int F, int d, uint16_t* __restrict__ A) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int nfb = F >> 4;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int e = wid / nfb, fb = wid - e * nfb;
  if (e >= E) return;
  const int ne = cnt[e];
  if (ne == 0) return;
  const int off = offs[e];
  const uint16_t* wg = wgu + ((size_t)e * 2 * F + fb * 16 + r) * d + 16 * g;
  const uint16_t* wu = wg + (size_t)F * d;
  const int nk = d >> 6;

  for (int t0 = 0; t0 < ne; t0 += 16 * TT) {
    const int nt = min(TT, (ne - t0 + 15) >> 4);
    const uint16_t* xp[TT];
#pragma unroll
    for (int j = 0; j < TT; ++j) {
      const int t = min(t0 + 16 * j + r, ne - 1);
      xp[j] = h + (size_t)perm[off + t] * d + 16 * g;
    }
    f32x4 ag[TT], au[TT];
#pragma unroll
    for (int j = 0; j < TT; ++j) ag[j] = au[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 G0[2], U0[2], X0[TT][2], G1[2], U1[2], X1[TT][2];
    auto load = [&](u32x4 (&G)[2], u32x4 (&U)[2], u32x4 (&X)[TT][2], int it) {
      const int k = it * 64;
      G[0] = ld16(wg + k);
      G[1] = ld16(wg + k + 8);
      U[0] = ld16(wu + k);
      U[1] = ld16(wu + k + 8);
#pragma unroll
      for (int j = 0; j < TT; ++j)
        if (j < nt) {
          X[j][0] = ld16(xp[j] + k);
          X[j][1] = ld16(xp[j] + k + 8);
        }
    };
    auto mma = [&](u32x4 (&G)[2], u32x4 (&U)[2], u32x4 (&X)[TT][2]) {
#pragma unroll
      for (int j = 0; j < TT; ++j)
        if (j < nt) {
          ag[j] = mfma16(G[0], X[j][0], ag[j]);
          ag[j] = mfma16(G[1], X[j][1], ag[j]);
          au[j] = mfma16(U[0], X[j][0], au[j]);
          au[j] = mfma16(U[1], X[j][1], au[j]);
        }
    };
    load(G0, U0, X0, 0);
    for (int it = 0; it < nk; it += 2) {
      if (it + 1 < nk) load(G1, U1, X1, it + 1);
      mma(G0, U0, X0);
      if (it + 1 >= nk) break;
      if (it + 2 < nk) load(G0, U0, X0, it + 2);
      mma(G1, U1, X1);
    }
#pragma unroll
    for (int j = 0; j < TT; ++j) {
      const int t = t0 + 16 * j + r;
      if (j < nt && t < ne) {
        u32x2 o;
        o.x = pack_bf2(silu_f(ag[j][0]) * au[j][0], silu_f(ag[j][1]) * au[j][1]);
        o.y = pack_bf2(silu_f(ag[j][2]) * au[j][2], silu_f(ag[j][3]) * au[j][3]);
        *reinterpret_cast<u32x2*>(A + (size_t)(off + t) * F + fb * 16 + 4 * g) = o;
      }
    }
  }
}

// Y[slot][n] = A[slot] . W_d[e][n]^T.  Wave = (expert, 16*WN output rows).
template <int TT, int WN>
__global__ __launch_bounds__(256) void moe_down_kernel(const uint16_t* __restrict__ A,
                                                       const uint16_t* __restrict__ wd,
                                                       const int32_t* __restrict__ cnt,
                                                       const int32_t* __restrict__ offs, int E,
                                                       int F, int d, float* __restrict__ Y) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int nnb = d / (16 * WN);
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int e = wid / nnb, nb = wid - e * nnb;
  if (e >= E) return;
  const int ne = cnt[e];
  if (ne == 0) return;
  const int off = offs[e];
  const uint16_t* wp[WN];
#pragma unroll
  for (int i = 0; i < WN; ++i) wp[i] = wd + ((size_t)e * d + nb * 16 * WN + 16 * i + r) * F + 16 * g;
  const int nk = F >> 6;

  for (int t0 = 0; t0 < ne; t0 += 16 * TT) {
    const int nt = min(TT, (ne - t0 + 15) >> 4);
    const uint16_t* xp[TT];
#pragma unroll
    for (int j = 0; j < TT; ++j) xp[j] = A + (size_t)(off + min(t0 + 16 * j + r, ne - 1)) * F + 16 * g;
    f32x4 acc[WN][TT];
#pragma unroll
    for (int i = 0; i < WN; ++i)
#pragma unroll
      for (int j = 0; j < TT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 W0[WN][2], X0[TT][2], W1[WN][2], X1[TT][2];
    auto load = [&](u32x4 (&W)[WN][2], u32x4 (&X)[TT][2], int it) {
      const int k = it * 64;
#pragma unroll
      for (int i = 0; i < WN; ++i) {
        W[i][0] = ld16(wp[i] + k);
        W[i][1] = ld16(wp[i] + k + 8);
      }
#pragma unroll
      for (int j = 0; j < TT; ++j)
        if (j < nt) {
          X[j][0] = ld16(xp[j] + k);
          X[j][1] = ld16(xp[j] + k + 8);
        }
    };
    auto mma = [&](u32x4 (&W)[WN][2], u32x4 (&X)[TT][2]) {
#pragma unroll
      for (int j = 0; j < TT; ++j)
        if (j < nt) {
#pragma unroll
          for (int i = 0; i < WN; ++i) {
            acc[i][j] = mfma16(W[i][0], X[j][0], acc[i][j]);
            acc[i][j] = mfma16(W[i][1], X[j][1], acc[i][j]);
          }
        }
    };
    load(W0, X0, 0);
    for (int it = 0; it < nk; it += 2) {
      if (it + 1 < nk) load(W1, X1, it + 1);
      mma(W0, X0);
      if (it + 1 >= nk) break;
      if (it + 2 < nk) load(W0, X0, it + 2);
      mma(W1, X1);
    }
#pragma unroll
    for (int j = 0; j < TT; ++j) {
      const int t = t0 + 16 * j + r;
      if (j < nt && t < ne) {
#pragma unroll
        for (int i = 0; i < WN; ++i)
          *reinterpret_cast<f32x4*>(Y + (size_t)(off + t) * d + nb * 16 * WN + 16 * i + 4 * g) = acc[i][j];
      }
    }
  }
}

void launch_moe_gate_up(const uint16_t* h, const uint16_t* w_gate_up, const int32_t* cnt,
                        const int32_t* offs, const int32_t* perm, int E, int F, int d,
                        uint16_t* a, hipStream_t s) {
  const int waves = E * (F / 16);
  hipLaunchKernelGGL(moe_gate_up_kernel<2>, dim3((waves + 3) / 4), dim3(256), 0, s, h, w_gate_up, cnt,
                     offs, perm, E, F, d, a);
}

void launch_moe_down(const uint16_t* a, const uint16_t* w_down, const int32_t* cnt,
                     const int32_t* offs, int E, int F, int d, float* Y, hipStream_t s) {
  constexpr int WN = 2;
  const int waves = E * (d / (16 * WN));
  hipLaunchKernelGGL((moe_down_kernel<2, WN>), dim3((waves + 3) / 4), dim3(256), 0, s, a, w_down, cnt,
                     offs, E, F, d, Y);
}

}  // namespace dg
