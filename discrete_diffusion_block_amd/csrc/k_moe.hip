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
// 1024-thread workgroup.  Expert e owns the padded slot range
// [poff[e], poff[e] + cnt[e]) with poff 16-aligned, so each expert's gathered
// rows start on a fragment-tile boundary; slots keep assignment order within an
// expert.  perm[slot] = token (-1 on padding), inv[a] = slot; items lists the
// (expert, first slot) of every 32-token group.  Offsets come from one-wave
// prefix scans; slot ranks from per-wave match counts.
__global__ __launch_bounds__(1024) void route_kernel(const int32_t* __restrict__ ids, int A, int k,
                                                     int E, int P, int32_t* __restrict__ cnt,
                                                     int32_t* __restrict__ poff,
                                                     int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ inv,
                                                     int2* __restrict__ items,
                                                     int32_t* __restrict__ n_items,
                                                     int32_t* __restrict__ cnt_log) {
  __shared__ int hist[256];
  __shared__ int base[256];
  __shared__ int ibase[256];
  __shared__ int wcnt[16][256];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int e = tid; e < E; e += blockDim.x) hist[e] = 0;
  for (int i = tid; i < P; i += blockDim.x) perm[i] = -1;
  __syncthreads();
  for (int a = tid; a < A; a += blockDim.x) atomicAdd(&hist[ids[a]], 1);
  __syncthreads();
  if (wv == 0) {
    // lane owns experts [lane*epl, lane*epl + epl)
    const int epl = (E + 63) / 64;
    int ps = 0, is = 0;
    for (int i = 0; i < epl; ++i) {
      const int e = lane * epl + i;
      if (e < E) {
        ps += (hist[e] + 15) & ~15;
        is += (hist[e] + kMoeGroup - 1) / kMoeGroup;
      }
    }
    int incl_p = ps, incl_i = is;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int tp = __shfl_up(incl_p, o, 64), ti = __shfl_up(incl_i, o, 64);
      if (lane >= o) {
        incl_p += tp;
        incl_i += ti;
      }
    }
    int run_p = incl_p - ps, run_i = incl_i - is;
    for (int i = 0; i < epl; ++i) {
      const int e = lane * epl + i;
      if (e < E) {
        const int c = hist[e];
        base[e] = run_p;
        poff[e] = run_p;
        cnt[e] = c;
        if (cnt_log) cnt_log[e] = c;
        ibase[e] = run_i;
        run_p += (c + 15) & ~15;
        run_i += (c + kMoeGroup - 1) / kMoeGroup;
      }
    }
    if (lane == 63) {
      poff[E] = incl_p;
      *n_items = incl_i;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    int it = ibase[e];
    for (int t0 = 0; t0 < hist[e]; t0 += kMoeGroup) items[it++] = make_int2(e, t0);
  }
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
      int s2 = 0;
      for (int w2 = 0; w2 < 16; ++w2) s2 += wcnt[w2][e2];
      base[e2] += s2;
    }
    __syncthreads();
  }
}

void launch_route(const int32_t* ids, int M, int k, int E, int32_t* cnt, int32_t* poff,
                  int32_t* perm, int32_t* inv, int2* items, int32_t* n_items, int32_t* cnt_log,
                  hipStream_t s) {
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(1024), 0, s, ids, M * k, k, E, moe_max_slots(M, k, E),
                     cnt, poff, perm, inv, items, n_items, cnt_log);
}

// Xg[slot] = h[perm[slot]] (zeros on padding), both fragment-major with K = d.
// One wave per padded slot; a lane moves 16-byte chunks.
__global__ __launch_bounds__(256) void gather_kernel(const uint16_t* __restrict__ h,
                                                     const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ poff, int E, int P,
                                                     int d, uint16_t* __restrict__ xg) {
  const int lane = threadIdx.x & 63;
  const int slot = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (slot >= P || slot >= poff[E]) return;
  const int tok = perm[slot];
  for (int c = 8 * lane; c < d; c += 8 * 64) {
    const u32x4 v = tok >= 0 ? ld16(h + fm_index(tok, c, d)) : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(xg + fm_index(slot, c, d)) = v;
  }
}

void launch_gather(const uint16_t* h, const int32_t* perm, const int32_t* poff, int M, int k, int E,
                   int d, uint16_t* xg, hipStream_t s) {
  const int P = moe_max_slots(M, k, E);
  hipLaunchKernelGGL(gather_kernel, dim3((P + 3) / 4), dim3(256), 0, s, h, perm, poff, E, P, d, xg);
}

// ---------------------------------------------------------------- grouped GEMMs

__device__ __forceinline__ float silu_f(float v) { return v / (1.0f + __expf(-v)); }

// Grouped expert GEMMs.  A workgroup owns one work item (expert e, group of up
// to 32 of its tokens) and one tile of 16 output features; its 4 waves split
// the K loop (interleaved 64-wide steps) and reduce through LDS.  Splitting K
// keeps every wave's dependent chain short, so the kernel stays bandwidth-bound
// both when tokens spread over all experts (~16 each) and when a uniform canvas
// sends every token to the same few experts (many groups per expert, whose
// workgroups then share the expert's weight tiles through L2).
//
// Lane group g reads bytes [64q + 16g, +16) of each 128-byte step q, so the 4
// lanes of a row read 64 contiguous bytes per instruction.

// gate/up: ag = x W_g^T, au = x W_u^T over this wave's k steps.  Every operand
// pointer addresses a fragment tile (row block, k block 0) plus the lane slot;
// a 64-wide k step covers two consecutive 1 KiB tiles.
template <int NT>
__device__ __forceinline__ void gate_up_partial(const uint16_t* wg, const uint16_t* wu,
                                                const uint16_t* const (&xp)[NT], int nk, int w,
                                                f32x4 (&ag)[NT], f32x4 (&au)[NT]) {
  u32x4 Ga[2], Ua[2], Xa[NT][2], Gb[2], Ub[2], Xb[NT][2], Gc[2], Uc[2], Xc[NT][2];
  auto ld = [&](u32x4 (&G)[2], u32x4 (&U)[2], u32x4 (&X)[NT][2], int step) {
    const int k = (w + 4 * step) * 1024;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      G[q] = ld16_stream(wg + k + 512 * q);
      U[q] = ld16_stream(wu + k + 512 * q);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int q = 0; q < 2; ++q) X[j][q] = ld16(xp[j] + k + 512 * q);
  };
  auto mm = [&](u32x4 (&G)[2], u32x4 (&U)[2], u32x4 (&X)[NT][2]) {
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        ag[j] = mfma16(G[q], X[j][q], ag[j]);
        au[j] = mfma16(U[q], X[j][q], au[j]);
      }
  };
  const int n = w < nk ? (nk - w + 3) >> 2 : 0;
  pipeline3(n, [&](int t) { ld(Ga, Ua, Xa, t); }, [&](int t) { ld(Gb, Ub, Xb, t); },
            [&](int t) { ld(Gc, Uc, Xc, t); }, [&] { mm(Ga, Ua, Xa); }, [&] { mm(Gb, Ub, Xb); },
            [&] { mm(Gc, Uc, Xc); });
}

template <int NT>
__device__ __forceinline__ void gate_up_item(const uint16_t* wg, const uint16_t* wu,
                                             const uint16_t* xg, int slot0, int t0, int ne, int F,
                                             int fb, int d, int lane, int w, uint16_t* A,
                                             f32x4 (*red)[2][2][64]) {
  const int r = lane & 15, g = lane >> 4;
  const uint16_t* xp[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) xp[j] = xg + fm_tile((slot0 >> 4) + j, 0, d, lane);
  f32x4 ag[NT], au[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) ag[j] = au[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  gate_up_partial<NT>(wg, wu, xp, d >> 6, w, ag, au);
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    red[w][0][j][lane] = ag[j];
    red[w][1][j][lane] = au[j];
  }
  __syncthreads();
  if (w < NT) {
    const int j = w;
    const f32x4 G = red[0][0][j][lane] + red[1][0][j][lane] + red[2][0][j][lane] + red[3][0][j][lane];
    const f32x4 U = red[0][1][j][lane] + red[1][1][j][lane] + red[2][1][j][lane] + red[3][1][j][lane];
    const int t = t0 + 16 * j + r;
    if (t < ne) {
      u32x2 o;
      o.x = pack_bf2(silu_f(G[0]) * U[0], silu_f(G[1]) * U[1]);
      o.y = pack_bf2(silu_f(G[2]) * U[2], silu_f(G[3]) * U[3]);
      *reinterpret_cast<u32x2*>(A + fm_index(slot0 + 16 * j + r, fb * 16 + 4 * g, F)) = o;
    }
  }
}

// A[slot][f] = silu(x W_g[e][f]^T) * (x W_u[e][f]^T) for every slot of expert e,
// x = Xg[slot].  Workgroup = (work item, 16 features); items vary fastest.
// The packed expert weight holds gate block f and up block f as row blocks
// 2f and 2f + 1.
__global__ __launch_bounds__(256) void moe_gate_up_kernel(const uint16_t* __restrict__ xg,
                                                          const uint16_t* __restrict__ wgu,
                                                          const int32_t* __restrict__ cnt,
                                                          const int32_t* __restrict__ poff,
                                                          const int2* __restrict__ items,
                                                          const int32_t* __restrict__ n_items,
                                                          int max_items, int F, int d,
                                                          uint16_t* __restrict__ A) {
  __shared__ f32x4 red[4][2][2][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int item, fb;
  if (!xcd_item_schedule(*n_items, F >> 4, &item, &fb)) return;   // uniform over the workgroup
  const int2 it = items[item];
  const int e = it.x, t0 = it.y;
  const int ne = cnt[e], slot0 = poff[e] + t0;
  const size_t wmat = (size_t)e * 2 * F * d;
  const uint16_t* wg = wgu + wmat + fm_tile(2 * fb, 0, d, lane);
  const uint16_t* wu = wgu + wmat + fm_tile(2 * fb + 1, 0, d, lane);
  if (ne - t0 <= 16)
    gate_up_item<1>(wg, wu, xg, slot0, t0, ne, F, fb, d, lane, w, A, red);
  else
    gate_up_item<2>(wg, wu, xg, slot0, t0, ne, F, fb, d, lane, w, A, red);
}

// down: Y[slot][n] = A[slot] . W_d[e][n]^T for 16*WN output rows.
template <int NT, int WN>
__device__ __forceinline__ void down_item(const uint16_t* const (&wp)[WN], const uint16_t* A,
                                          int slot0, int t0, int ne, int F, int d, int n0, int lane,
                                          int w, float* Y, f32x4 (*red)[2][2][64]) {
  const int r = lane & 15, g = lane >> 4;
  const uint16_t* xp[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) xp[j] = A + fm_tile((slot0 >> 4) + j, 0, F, lane);
  f32x4 acc[WN][NT];
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 Wa[WN][2], Xa[NT][2], Wb[WN][2], Xb[NT][2], Wc[WN][2], Xc[NT][2];
  auto ld = [&](u32x4 (&W)[WN][2], u32x4 (&X)[NT][2], int step) {
    const int k = (w + 4 * step) * 1024;
#pragma unroll
    for (int i = 0; i < WN; ++i)
#pragma unroll
      for (int q = 0; q < 2; ++q) W[i][q] = ld16_stream(wp[i] + k + 512 * q);
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int q = 0; q < 2; ++q) X[j][q] = ld16(xp[j] + k + 512 * q);
  };
  auto mm = [&](u32x4 (&W)[WN][2], u32x4 (&X)[NT][2]) {
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int i = 0; i < WN; ++i)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[i][j] = mfma16(W[i][q], X[j][q], acc[i][j]);
  };
  const int nk = F >> 6;
  const int n = w < nk ? (nk - w + 3) >> 2 : 0;
  pipeline3(n, [&](int t) { ld(Wa, Xa, t); }, [&](int t) { ld(Wb, Xb, t); },
            [&](int t) { ld(Wc, Xc, t); }, [&] { mm(Wa, Xa); }, [&] { mm(Wb, Xb); },
            [&] { mm(Wc, Xc); });
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) red[w][i][j][lane] = acc[i][j];
  __syncthreads();
  // wave w finalises (row block i, token tile j) pairs w, w+4, ...
  for (int p = w; p < WN * NT; p += 4) {
    const int i = p / NT, j = p - i * NT;
    const int t = t0 + 16 * j + r;
    if (t < ne) {
      const f32x4 v = red[0][i][j][lane] + red[1][i][j][lane] + red[2][i][j][lane] + red[3][i][j][lane];
      *reinterpret_cast<f32x4*>(Y + (size_t)(slot0 + 16 * j + r) * d + n0 + 16 * i + 4 * g) = v;
    }
  }
}

template <int WN>
__global__ __launch_bounds__(256) void moe_down_kernel(const uint16_t* __restrict__ A,
                                                       const uint16_t* __restrict__ wd,
                                                       const int32_t* __restrict__ cnt,
                                                       const int32_t* __restrict__ poff,
                                                       const int2* __restrict__ items,
                                                       const int32_t* __restrict__ n_items,
                                                       int max_items, int F, int d,
                                                       float* __restrict__ Y) {
  static_assert(WN <= 2, "LDS tile holds at most 2 row blocks");
  __shared__ f32x4 red[4][2][2][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int item, nb;
  if (!xcd_item_schedule(*n_items, d / (16 * WN), &item, &nb)) return;
  const int2 it = items[item];
  const int e = it.x, t0 = it.y;
  const int ne = cnt[e], slot0 = poff[e] + t0;
  const int n0 = nb * 16 * WN;
  const uint16_t* wp[WN];
#pragma unroll
  for (int i = 0; i < WN; ++i) wp[i] = wd + (size_t)e * d * F + fm_tile((n0 >> 4) + i, 0, F, lane);
  if (ne - t0 <= 16)
    down_item<1, WN>(wp, A, slot0, t0, ne, F, d, n0, lane, w, Y, red);
  else
    down_item<2, WN>(wp, A, slot0, t0, ne, F, d, n0, lane, w, Y, red);
}

int moe_max_items(int M, int k, int E) { return (M * k + kMoeGroup - 1) / kMoeGroup + E; }
int moe_max_slots(int M, int k, int E) { return M * k + 15 * E; }

void launch_moe_gate_up(const uint16_t* xg, const uint16_t* w_gate_up, const int32_t* cnt,
                        const int32_t* poff, const int2* items, const int32_t* n_items, int max_items,
                        int F, int d, uint16_t* a, hipStream_t s) {
  const int blocks = kXcd * ((max_items + kXcd - 1) / kXcd) * (F / 16);
  hipLaunchKernelGGL(moe_gate_up_kernel, dim3(blocks), dim3(256), 0, s, xg, w_gate_up, cnt, poff, items,
                     n_items, max_items, F, d, a);
}

void launch_moe_down(const uint16_t* a, const uint16_t* w_down, const int32_t* cnt,
                     const int32_t* poff, const int2* items, const int32_t* n_items, int max_items,
                     int F, int d, float* Y, hipStream_t s) {
  constexpr int WN = 2;
  const int blocks = kXcd * ((max_items + kXcd - 1) / kXcd) * (d / (16 * WN));
  hipLaunchKernelGGL((moe_down_kernel<WN>), dim3(blocks), dim3(256), 0, s, a, w_down, cnt, poff, items,
                     n_items, max_items, F, d, Y);
}

}  // namespace dg
