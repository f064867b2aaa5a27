// Mixture-of-experts block: router top-k, deterministic token->expert
// permutation, and the two grouped expert GEMMs.
//
// With a trained router, a 256-token canvas spreads its 2048 assignments over
// most of the 128 experts (~16-24 tokens each): the expert GEMMs then stream
// ~1 GB of weights per layer at a low arithmetic intensity and are HBM-bound.
// When a uniform canvas sends every token to a few experts, the same kernels
// run many work items per expert and the weight tiles are shared through L2.
// Weight rows sit on the MFMA A side and are read from HBM once per work item;
// token rows never move: the gate/up GEMM gathers them through the permutation
// while copying its operand tiles into LDS.
#include <limits.h>
#include <math.h>

#include "dg_common.h"
#include "dg_internal.h"

namespace dg {

// ---------------------------------------------------------------- top-k

// One wave ranks one token's E router logits by (logit desc, id asc); NaN logits
// rank below every number.  ids/w get the k selected experts and the softmax of
// their logits.  Selected logits stay in registers (k <= 16).
__device__ __forceinline__ void topk_row(const float* __restrict__ rr, int E, int k, int lane,
                                         int32_t* __restrict__ ids, float* __restrict__ w) {
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    float x = e < E ? rr[e] : -INFINITY;
    if (x != x) x = -INFINITY;
    v[i] = x;
  }
  unsigned taken = 0;
  float sel[16];
  int sid[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    sel[t] = -INFINITY;
    sid[t] = 0;
    if (t < k) {
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
      sid[t] = bi;
    }
  }
  float z = 0.f, ex[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    ex[t] = (t < k && sel[t] != -INFINITY) ? expf(sel[t] - sel[0]) : 0.f;
    z += ex[t];
  }
  // lane t < k writes selection t
#pragma unroll
  for (int t = 0; t < 16; ++t)
    if (t < k && lane == t) {
      ids[t] = sid[t];
      w[t] = ex[t] / z;
    }
}

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ r, int M, int E, int k,
                                                   int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  topk_row(r + (size_t)m * E, E, k, lane, ids + (size_t)m * k, w + (size_t)m * k);
}

void launch_topk(const float* r, int M, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3((M + 3) / 4), dim3(256), 0, s, r, M, E, k, ids, w);
}

// ---------------------------------------------------------------- permutation

// Stable counting sort of the A = M*k assignments (a = m*k + j) by expert, by one
// workgroup of NW waves.  Expert e owns the padded slot range [poff[e],
// poff[e] + cnt[e]) with poff 16-aligned, so each expert's gathered rows start on
// a fragment-tile boundary; slots keep assignment order within an expert.
// perm[slot] = token (-1 on padding), inv[a] = slot; items lists the
// (expert, first token) of every kMoeGroup-token group.  Offsets come from
// one-wave prefix scans; the rank of an assignment among equal experts of its
// wave comes from ballots on the expert id's bits.
template <int NW>
struct RouteLds {
  int hist[256];
  int base[256];
  int ibase[256];
  int wcnt[NW][256];
};

template <int NW>
__device__ void route_block(const int32_t* __restrict__ ids, int A, int k, int E, int P,
                            int32_t* __restrict__ cnt, int32_t* __restrict__ poff,
                            int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                            int2* __restrict__ items, int32_t* __restrict__ n_items,
                            int32_t* __restrict__ cnt_log, RouteLds<NW>& L) {
  constexpr int NT = 64 * NW;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int e = tid; e < E; e += NT) L.hist[e] = 0;
  for (int i = tid; i < P; i += NT) perm[i] = -1;
  __syncthreads();
  for (int a = tid; a < A; a += NT) atomicAdd(&L.hist[ids[a]], 1);
  __syncthreads();
  if (wv == 0) {
    // lane owns experts [lane*epl, lane*epl + epl)
    const int epl = (E + 63) / 64;
    int ps = 0, is = 0;
    for (int i = 0; i < epl; ++i) {
      const int e = lane * epl + i;
      if (e < E) {
        ps += (L.hist[e] + 15) & ~15;
        is += (L.hist[e] + kMoeGroup - 1) / kMoeGroup;
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
        const int c = L.hist[e];
        L.base[e] = run_p;
        poff[e] = run_p;
        cnt[e] = c;
        if (cnt_log) cnt_log[e] = c;
        L.ibase[e] = run_i;
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
  for (int e = tid; e < E; e += NT) {
    int it = L.ibase[e];
    for (int t0 = 0; t0 < L.hist[e]; t0 += kMoeGroup) items[it++] = make_int2(e, t0);
  }
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int start = 0; start < A; start += NT) {
    for (int i = tid; i < NW * E; i += NT) L.wcnt[i / E][i % E] = 0;
    __syncthreads();
    const int a = start + tid;
    const int e = a < A ? ids[a] : -1;
    // lanes holding the same expert: agree on validity and on each of 8 id bits
    unsigned long long same = __ballot(e >= 0);
    if (e < 0) same = ~same;
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const unsigned long long b1 = __ballot(e >= 0 && ((e >> bit) & 1));
      same &= ((e >> bit) & 1) ? b1 : ~b1;
    }
    const int rank = __popcll(same & below), tot = __popcll(same);
    if (e >= 0 && rank == tot - 1) L.wcnt[wv][e] = tot;
    __syncthreads();
    if (e >= 0) {
      int before = 0;
      for (int w2 = 0; w2 < wv; ++w2) before += L.wcnt[w2][e];
      const int slot = L.base[e] + before + rank;
      perm[slot] = a / k;
      inv[a] = slot;
    }
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += NT) {
      int s2 = 0;
      for (int w2 = 0; w2 < NW; ++w2) s2 += L.wcnt[w2][e2];
      L.base[e2] += s2;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(1024) void route_kernel(const int32_t* __restrict__ ids, int A, int k,
                                                     int E, int P, int32_t* __restrict__ cnt,
                                                     int32_t* __restrict__ poff,
                                                     int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ inv,
                                                     int2* __restrict__ items,
                                                     int32_t* __restrict__ n_items,
                                                     int32_t* __restrict__ cnt_log) {
  __shared__ RouteLds<16> L;
  route_block<16>(ids, A, k, E, P, cnt, poff, perm, inv, items, n_items, cnt_log, L);
}

void launch_route(const int32_t* ids, int M, int k, int E, int32_t* cnt, int32_t* poff,
                  int32_t* perm, int32_t* inv, int2* items, int32_t* n_items, int32_t* cnt_log,
                  hipStream_t s) {
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(1024), 0, s, ids, M * k, k, E, moe_max_slots(M, k, E),
                     cnt, poff, perm, inv, items, n_items, cnt_log);
}

// ---------------------------------------------------------------- grouped GEMMs

__device__ __forceinline__ float silu_f(float v) { return v / (1.0f + __expf(-v)); }

// Grouped expert GEMMs.  A workgroup owns one work item (expert e, a group of up
// to kMoeGroup = 64 of its tokens) and a tile of output features.  The gate/up
// GEMM (K = d_model) stages weight and token fragment tiles through LDS rings by
// direct global->LDS copies and computes a 128-row x 64-token tile; the down GEMM
// (K = F, short) gives each wave 32 output rows over the whole K loop, with its
// weights in registers and the item's activation tiles shared through an LDS ring.
// Either way every operand byte is read once per workgroup, so the kernels hold up
// both when tokens spread over all experts (~16
// each: a weight-streaming, HBM-bound regime) and when a uniform canvas sends
// every token to a few experts (many work items per expert, whose workgroups
// share the expert's weight tiles through L2).
//
// Every operand pointer addresses a fragment tile (row block, k block 0) plus
// the lane's 16-byte slot; a 64-wide k step covers two consecutive 1 KiB tiles.

constexpr int kDownRows = 128; // output rows per down workgroup (32 per wave)

// STREAM (both GEMMs): the weight tiles are read by this workgroup only (the expert
// has a single work item), so they bypass cache retention; otherwise the expert's
// other items re-read them from L2.
//
// Gate/up, operands staged through LDS.  Workgroup tile: 128 packed weight rows
// (gate and up blocks of 4 feature blocks) x one work item (up to 64 tokens); the
// 4 waves form a 2 x 2 grid of 64-row x 32-token sub-tiles.  Per 64-wide k
// step the workgroup copies 8 weight and 4 token blocks (two 1 KiB fragment
// tiles each) straight into LDS: weights into a three-step ring (two steps
// ahead), token tiles -- L2 hits -- into a two-step ring (one step ahead).  The
// 64 KiB of rings let two workgroups share a CU, which hides more latency than
// deeper rings in one.  Every weight byte is read once per workgroup and shared
// by all its token tiles.
constexpr int kGuRB = 8, kGuTB = 4, kGuKT = 2;
constexpr int kGuWSlots = 3, kGuXSlots = 2;
constexpr int kGuWBytes = kGuRB * kGuKT * 1024, kGuXBytes = kGuTB * kGuKT * 1024;
constexpr int kGuLds = kGuWSlots * kGuWBytes + kGuXSlots * kGuXBytes;
constexpr int kGuCopies = kGuRB * kGuKT / 4;   // weight tile copies per wave per step

template <bool STREAM>
__device__ __forceinline__ void gate_up_tile_lds(const uint16_t* wgu_e, const uint16_t* h_rm,
                                                 const int32_t* perm, int slot0, int t0, int ne, int F,
                                                 int f0, int d, int lane, int wv, uint16_t* A,
                                                 char* ring) {
  constexpr int WI = kGuRB / 2, WJ = kGuTB / 2;
  const int ntb = min(kGuTB, (ne - t0 + 15) >> 4);   // token blocks of this item (>= 1)
  const int nk = d / (32 * kGuKT);
  constexpr int WB = kGuRB / 4, XB = kGuTB / 4;
  const uint16_t* wsrc[WB];
  const uint16_t* xsrc[XB];
#pragma unroll
  for (int u = 0; u < WB; ++u) wsrc[u] = wgu_e + fm_tile(2 * f0 + wv * WB + u, 0, d, lane);
  // The token tiles are gathered on the fly: lane (r, g) of a fragment tile copies
  // the 16 bytes of its slot's token row (row-major h) at k columns 8g .. 8g + 7 of
  // the tile.  Token blocks past the item's last one re-read that block, and
  // padding slots read row 0: their outputs are dropped.
#pragma unroll
  for (int u = 0; u < XB; ++u) {
    const int tok = perm[slot0 + 16 * min(wv * XB + u, ntb - 1) + (lane & 15)];
    xsrc[u] = h_rm + (size_t)max(tok, 0) * d + 8 * (lane >> 4);
  }
  char* const wring = ring;
  char* const xring = ring + kGuWSlots * kGuWBytes;
  auto issue_w = [&](int step) {
    char* dst = wring + (step % kGuWSlots) * kGuWBytes + wv * WB * kGuKT * 1024;
#pragma unroll
    for (int u = 0; u < WB; ++u)
#pragma unroll
      for (int t = 0; t < kGuKT; ++t)
        tile_to_lds<STREAM>(wsrc[u] + (step * kGuKT + t) * 512, dst + (u * kGuKT + t) * 1024);
  };
  auto issue_x = [&](int step) {
    char* dst = xring + (step % kGuXSlots) * kGuXBytes + wv * XB * kGuKT * 1024;
#pragma unroll
    for (int u = 0; u < XB; ++u)
#pragma unroll
      for (int t = 0; t < kGuKT; ++t)
        tile_to_lds<false>(xsrc[u] + (step * kGuKT + t) * 32, dst + (u * kGuKT + t) * 1024);
  };
  const int wr = wv & 1, wt = wv >> 1;
  f32x4 acc[WI][WJ];
#pragma unroll
  for (int i = 0; i < WI; ++i)
#pragma unroll
    for (int j = 0; j < WJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  lds_char* const lw = lds_launder(wring);
  lds_char* const lx = lds_launder(xring);
  // After step j's barrier the wave copies X(j + XS - 1) then W(j + WS - 1); the
  // prologue runs the same order for j = -(WS - 1) .. -1.  At the top of step s,
  // X(s) and everything issued before it (W(s) included) have landed once at most
  // the copies issued after X(s) are in flight.
  constexpr int WS = kGuWSlots, XS = kGuXSlots;
  static_assert(WS > XS && XS >= 2, "weights run further ahead than token tiles");
  constexpr int kAfterX = kGuCopies + (XS - 2) * 2 * kGuCopies;
  static_assert(kAfterX < 64, "vmcnt range");
#pragma unroll
  for (int j = -(WS - 1); j < 0; ++j) {
    if (j + XS - 1 >= 0 && j + XS - 1 < nk) issue_x(j + XS - 1);
    if (j + WS - 1 < nk) issue_w(j + WS - 1);
  }
  u32x4 Af[WI][kGuKT], Bf[WJ][kGuKT];
  for (int s = 0; s < nk; ++s) {
    if (s + WS - 2 < nk) vm_wait<kAfterX>();
    else vm_wait<0>();
    __builtin_amdgcn_s_barrier();
    if (s + XS - 1 < nk) issue_x(s + XS - 1);
    if (s + WS - 1 < nk) issue_w(s + WS - 1);
    const lds_char* sw = lw + (s % kGuWSlots) * kGuWBytes + lane * 16;
    const lds_char* sx = lx + (s % kGuXSlots) * kGuXBytes + lane * 16;
#pragma unroll
    for (int i = 0; i < WI; ++i)
#pragma unroll
      for (int t = 0; t < kGuKT; ++t) Af[i][t] = ld16_lds(sw + ((wr * WI + i) * kGuKT + t) * 1024);
#pragma unroll
    for (int j = 0; j < WJ; ++j)
#pragma unroll
      for (int t = 0; t < kGuKT; ++t) Bf[j][t] = ld16_lds(sx + ((wt * WJ + j) * kGuKT + t) * 1024);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < WJ; ++j)
#pragma unroll
      for (int i = 0; i < WI; ++i) acc[i][j] = mfma16x2(Af[i][0], Bf[j][0], Af[i][1], Bf[j][1], acc[i][j]);
  }
  // wave rows: row blocks 2 f0 + wr * WI + i; pairs (i, i + 1) are gate / up of
  // feature block f0 + wr * WI / 2 + i / 2
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < WJ; ++j) {
    const int tb = wt * WJ + j;
    const int t = t0 + 16 * tb + r;
    if (tb >= ntb || t >= ne) continue;
#pragma unroll
    for (int i = 0; i < WI; i += 2) {
      const f32x4 G = acc[i][j], U = acc[i + 1][j];
      u32x2 o;
      o.x = pack_bf2(silu_f(G[0]) * U[0], silu_f(G[1]) * U[1]);
      o.y = pack_bf2(silu_f(G[2]) * U[2], silu_f(G[3]) * U[3]);
      const int f = f0 + (wr * WI + i) / 2;
      *reinterpret_cast<u32x2*>(A + fm_index(slot0 + 16 * tb + r, f * 16 + 4 * g, F)) = o;
    }
  }
}

__global__ __launch_bounds__(256) void moe_gate_up_kernel(const uint16_t* __restrict__ h_rm,
                                                          const int32_t* __restrict__ perm,
                                                          const uint16_t* __restrict__ wgu,
                                                              const int32_t* __restrict__ cnt,
                                                              const int32_t* __restrict__ poff,
                                                              const int2* __restrict__ items,
                                                              const int32_t* __restrict__ n_items,
                                                              int F, int d, uint16_t* __restrict__ A) {
  extern __shared__ __attribute__((aligned(1024))) char ring[];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int item, fb;
  if (!xcd_item_schedule(*n_items, F / (16 * kGuRB / 2), &item, &fb)) return;
  const int2 it = items[item];
  const int e = it.x, t0 = it.y;
  const int ne = cnt[e], slot0 = poff[e] + t0;
  const uint16_t* wgu_e = wgu + (size_t)e * 2 * F * d;
  if (ne <= kMoeGroup)
    gate_up_tile_lds<true>(wgu_e, h_rm, perm, slot0, t0, ne, F, fb * (kGuRB / 2), d, lane, wv, A, ring);
  else
    gate_up_tile_lds<false>(wgu_e, h_rm, perm, slot0, t0, ne, F, fb * (kGuRB / 2), d, lane, wv, A, ring);
}

void launch_moe_gate_up(const uint16_t* h_rm, const int32_t* perm, const uint16_t* w_gate_up,
                        const int32_t* cnt, const int32_t* poff, const int2* items,
                        const int32_t* n_items, int max_items, int F, int d, uint16_t* a,
                        hipStream_t s) {
  static bool raised = false;
  if (!raised) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(&moe_gate_up_kernel),
                        hipFuncAttributeMaxDynamicSharedMemorySize, kGuLds);
    raised = true;
  }
  const int blocks = kXcd * ((max_items + kXcd - 1) / kXcd) * (F / (16 * kGuRB / 2));
  hipLaunchKernelGGL(moe_gate_up_kernel, dim3(blocks), dim3(256), kGuLds, s, h_rm, perm, w_gate_up,
                     cnt, poff, items, n_items, F, d, a);
}

// down: Y[slot][n] = A[slot] . W_d[e][n]^T over K = F.  Workgroup tile: 128 output
// rows x one work item.  Wave wv owns row blocks 2wv, 2wv + 1 and loads their weight
// fragments straight into registers two steps ahead (each weight byte is used by that
// wave alone); the item's activation tiles, shared by the four waves, are copied once
// per workgroup into a three-step LDS ring.
constexpr int kDnXS = 3;
constexpr int kDnXBytes = 4 * kGuKT * 1024;      // 64 tokens x 64 k
constexpr int kDnLds = kDnXS * kDnXBytes;

template <bool STREAM, int NT>
__device__ __forceinline__ void down_tile(const uint16_t* wd_e, const uint16_t* A, int slot0, int t0,
                                          int ne, int F, int d, int n0, int lane, int wv, float* Y,
                                          char* ring) {
  const int nblk = d >> 4;
  const int nk = F / (32 * kGuKT);                // >= 1 (F % 64 == 0)
  const int rb0 = (n0 >> 4) + 2 * wv;
  const uint16_t* w0 = wd_e + fm_tile(min(rb0, nblk - 1), 0, F, lane);
  const uint16_t* w1 = wd_e + fm_tile(min(rb0 + 1, nblk - 1), 0, F, lane);
  // wave wv copies token block wv (the item's last block again past its end; unread)
  const uint16_t* xsrc = A + fm_tile((slot0 >> 4) + min(wv, NT - 1), 0, F, lane);
  lds_char* const lx = lds_launder(ring);
  typedef u32x4 WSet[4];                           // rows rb0 k0, k1; rows rb0+1 k0, k1
  auto issue = [&](int step, WSet& w) {
    char* dst = ring + (step % kDnXS) * kDnXBytes + wv * kGuKT * 1024;
#pragma unroll
    for (int t = 0; t < kGuKT; ++t) tile_to_lds_untracked(xsrc + (step * kGuKT + t) * 512, dst + t * 1024);
    const int o = step * kGuKT * 512;
    if (STREAM) {
      w[0] = ld16_stream(w0 + o); w[1] = ld16_stream(w0 + o + 512);
      w[2] = ld16_stream(w1 + o); w[3] = ld16_stream(w1 + o + 512);
    } else {
      w[0] = ld16(w0 + o); w[1] = ld16(w0 + o + 512);
      w[2] = ld16(w1 + o); w[3] = ld16(w1 + o + 512);
    }
  };
  f32x4 acc[2][NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[0][j] = acc[1][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // step s: its copies and loads were issued two iterations earlier; the previous
  // iteration's (kGuKT copies + 4 loads) may still be in flight unless it issued none.
  // Refilling ring slot (s + 2) % 3 is safe after the barrier: every wave consumed
  // that slot's step s - 1 before arriving.
  auto body = [&](int s, WSet& wc, WSet& wn, bool more, bool last) {
    if (!last) vm_wait<kGuKT + 4>();
    else vm_wait<0>();
    __builtin_amdgcn_s_barrier();
    if (more) issue(s + 2, wn);
    const lds_char* sx = lx + (s % kDnXS) * kDnXBytes + lane * 16;
    u32x4 X[NT][kGuKT];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int t = 0; t < kGuKT; ++t) X[j][t] = ld16_lds(sx + (j * kGuKT + t) * 1024);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      acc[0][j] = mfma16x2(wc[0], X[j][0], wc[1], X[j][1], acc[0][j]);
      acc[1][j] = mfma16x2(wc[2], X[j][0], wc[3], X[j][1], acc[1][j]);
    }
  };
  WSet ws0, ws1, ws2;
  issue(0, ws0);
  if (nk > 1) issue(1, ws1);
  int s = 0;
  for (; s + 5 <= nk; s += 3) {     // steady state: every iteration issues step s + 2
    body(s, ws0, ws2, true, false);
    body(s + 1, ws1, ws0, true, false);
    body(s + 2, ws2, ws1, true, false);
  }
  const int r = nk - s;             // 1 .. 4 steps left
  if (r > 0) body(s, ws0, ws2, r > 2, r == 1);
  if (r > 1) body(s + 1, ws1, ws0, r > 3, r == 2);
  if (r > 2) body(s + 2, ws2, ws1, false, r == 3);
  if (r > 3) body(s + 3, ws0, ws2, false, true);
  const int rr = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int t = t0 + 16 * j + rr;
    if (t >= ne) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (rb0 + i < nblk)
        *reinterpret_cast<f32x4*>(Y + (size_t)(slot0 + 16 * j + rr) * d + (rb0 + i) * 16 + 4 * g) = acc[i][j];
  }
}

__global__ __launch_bounds__(256) void moe_down_kernel(const uint16_t* __restrict__ A,
                                                       const uint16_t* __restrict__ wd,
                                                       const int32_t* __restrict__ cnt,
                                                       const int32_t* __restrict__ poff,
                                                       const int2* __restrict__ items,
                                                       const int32_t* __restrict__ n_items,
                                                       int F, int d, float* __restrict__ Y) {
  extern __shared__ __attribute__((aligned(1024))) char ring[];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int item, nb;
  if (!xcd_item_schedule(*n_items, (d + kDownRows - 1) / kDownRows, &item, &nb)) return;
  const int2 it = items[item];
  const int e = it.x, t0 = it.y;
  const int ne = cnt[e], slot0 = poff[e] + t0;
  const int n0 = nb * kDownRows;
  const uint16_t* wd_e = wd + (size_t)e * d * F;
  const int nt = min(4, (ne - t0 + 15) >> 4);
  // an expert with a single work item streams its weights (read by no other item)
#define DOWN_TILE(NT)                                                                            \
  (ne <= kMoeGroup ? down_tile<true, NT>(wd_e, A, slot0, t0, ne, F, d, n0, lane, wv, Y, ring)   \
                   : down_tile<false, NT>(wd_e, A, slot0, t0, ne, F, d, n0, lane, wv, Y, ring))
  switch (nt) {
    case 1: DOWN_TILE(1); break;
    case 2: DOWN_TILE(2); break;
    case 3: DOWN_TILE(3); break;
    default: DOWN_TILE(4); break;
  }
#undef DOWN_TILE
}

int moe_max_items(int M, int k, int E) { return (M * k + kMoeGroup - 1) / kMoeGroup + E; }
int moe_max_slots(int M, int k, int E) { return M * k + 15 * E; }

void launch_moe_down(const uint16_t* a, const uint16_t* w_down, const int32_t* cnt,
                     const int32_t* poff, const int2* items, const int32_t* n_items, int max_items,
                     int F, int d, float* Y, hipStream_t s) {
  const int blocks = kXcd * ((max_items + kXcd - 1) / kXcd) * ((d + kDownRows - 1) / kDownRows);
  hipLaunchKernelGGL(moe_down_kernel, dim3(blocks), dim3(256), kDnLds, s, a, w_down, cnt, poff, items,
                     n_items, F, d, Y);
}

}  // namespace dg
