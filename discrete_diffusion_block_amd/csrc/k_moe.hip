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

// Selection key of logit x of expert e: larger key = larger logit, then lower id;
// NaN ranks as -inf and -0 as +0.  Keys are unique and nonzero.
__device__ __forceinline__ uint64_t sel_key(float x, int e) {
  if (x != x) x = -INFINITY;
  const uint32_t u = __float_as_uint(x + 0.0f);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (uint64_t)o << 32 | (uint32_t)(0xffffffffu - (uint32_t)e);
}
__device__ __forceinline__ float key_logit(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
// rotation by N lanes within each 16-lane DPP row
template <int N>
__device__ __forceinline__ uint32_t row_ror(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x120 + N, 0xf, 0xf, false);
}
template <int N>
__device__ __forceinline__ uint64_t row_max64(uint64_t v) {
  const uint64_t o = (uint64_t)row_ror<N>((uint32_t)(v >> 32)) << 32 | row_ror<N>((uint32_t)v);
  return o > v ? o : v;
}

constexpr int kTopkRows = 16;                // token rows per workgroup (16 lanes each)
constexpr int kTopkStride = 256 + 16;        // LDS row stride (floats): rows 16 banks apart

// The k largest of one token row's E logits, 16 lanes per row, lane l holding
// experts l + 16 i (i < EPL).  Round t takes on every lane the largest key below
// the previous round's winner, then the row maximum by DPP rotations within the
// 16 lanes; the winners come out in rank order.  The weights are the softmax of
// the k selected logits.
template <int EPL>
__device__ __forceinline__ void select_row(const float* rl, int row, int m, int M, int E, int k,
                                           int32_t* __restrict__ ids, float* __restrict__ w) {
  const int sl = threadIdx.x & 15;
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = sl + 16 * i;
    key[i] = e < E ? sel_key(rl[row * kTopkStride + e], e) : 0ull;
  }
  float sel[16];
  int sid[16];
  uint64_t prev = ~0ull;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    sel[t] = -INFINITY;
    sid[t] = 0;
    if (t < k) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) best = (key[i] < prev && key[i] > best) ? key[i] : best;
      best = row_max64<8>(best);
      best = row_max64<4>(best);
      best = row_max64<2>(best);
      best = row_max64<1>(best);
      prev = best;
      sel[t] = key_logit(best);
      sid[t] = (int)(0xffffffffu - (uint32_t)best);
    }
  }
  float z = 0.f, ex[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    ex[t] = (t < k && sel[t] != -INFINITY) ? expf(sel[t] - sel[0]) : 0.f;
    z += ex[t];
  }
  if (m < M)
#pragma unroll
    for (int t = 0; t < 16; ++t)
      if (t < k && sl == t) {
        ids[(size_t)m * k + t] = sid[t];
        w[(size_t)m * k + t] = ex[t] / z;
      }
}

// Workgroup = 16 token rows: the rows' logits are staged in LDS, then each wave
// selects for 4 rows at once.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ r, int M, int E, int k,
                                                   int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ float rl[kTopkRows * kTopkStride];
  const int tid = threadIdx.x, m0 = blockIdx.x * kTopkRows;
  // 16 rows x E logits as 16-byte pieces (E % 4 == 0), at most 4 per thread, all in flight
  const int q = E >> 2;
  f32x4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = tid + 256 * u, row = i / q;
    if (i < kTopkRows * q && m0 + row < M)
      v[u] = *reinterpret_cast<const f32x4*>(r + (size_t)(m0 + row) * E + 4 * (i - row * q));
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = tid + 256 * u, row = i / q;
    if (i < kTopkRows * q && m0 + row < M)
      *reinterpret_cast<f32x4*>(&rl[row * kTopkStride + 4 * (i - row * q)]) = v[u];
  }
  __syncthreads();
  const int row = tid >> 4, m = m0 + row;
  switch ((E + 15) >> 4) {
    case 1: select_row<1>(rl, row, m, M, E, k, ids, w); break;
    case 2: select_row<2>(rl, row, m, M, E, k, ids, w); break;
    case 3: case 4: select_row<4>(rl, row, m, M, E, k, ids, w); break;
    case 5: case 6: case 7: case 8: select_row<8>(rl, row, m, M, E, k, ids, w); break;
    default: select_row<16>(rl, row, m, M, E, k, ids, w); break;
  }
}

void launch_topk(const float* r, int M, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  launch_kernel(topk_kernel, dim3((M + kTopkRows - 1) / kTopkRows), dim3(256), 0, s, nullptr, r, M, E, k,
                ids, w);
}

// Routing with the experts given (a test tap): row m takes the k expert ids
// forced[m][0..k) in that order; its weights are the softmax of the router logits
// r[m][id] at those ids (taken against their largest, as in the top-k kernel).
// One thread per row.
__global__ __launch_bounds__(256) void forced_route_kernel(const float* __restrict__ r, int M, int E,
                                                           int k, const int32_t* __restrict__ forced,
                                                           int32_t* __restrict__ ids,
                                                           float* __restrict__ w) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= M) return;
  float x[16];
  float mx = -INFINITY;
  for (int j = 0; j < k; ++j) {
    const int e = min(max(forced[(size_t)m * k + j], 0), E - 1);
    ids[(size_t)m * k + j] = e;
    x[j] = r[(size_t)m * E + e];
    mx = fmaxf(mx, x[j]);
  }
  float z = 0.f;
  for (int j = 0; j < k; ++j) {
    x[j] = expf(x[j] - mx);
    z += x[j];
  }
  for (int j = 0; j < k; ++j) w[(size_t)m * k + j] = x[j] / z;
}

void launch_forced_route(const float* r, int M, int E, int k, const int32_t* forced, int32_t* ids, float* w,
                         hipStream_t s) {
  launch_kernel(forced_route_kernel, dim3((M + 255) / 256), dim3(256), 0, s, nullptr, r, M, E, k, forced, ids,
                w);
}

// ---------------------------------------------------------------- permutation

// Stable counting sort of the A = M*k assignments (a = m*k + j) by expert, by one
// workgroup of NW waves.  Expert e owns the padded slot range [poff[e],
// poff[e] + cnt[e]) with poff 16-aligned, so each expert's gathered rows start on
// a fragment-tile boundary; slots keep assignment order within an expert.
// perm[slot] = token (-1 on padding), inv[a] = slot; items lists the
// (expert, first token) of every kMoeGroup-token group.
//
// Wave w owns the contiguous assignment range [w*per, (w+1)*per).  A first walk
// counts every expert per wave (LDS atomic additions: counts do not depend on their
// order), a one-wave prefix scan turns the totals into offsets, a scan across the
// waves gives each (wave, expert) its first slot, and a second walk, 64 assignments
// at a time, writes slot = that slot + running rank, where the lanes holding one
// expert find each other by ballots on the id's bits, which gives each assignment
// its rank among them.  The ids are staged in LDS (sids) when at most CAP of them
// come (CAP > 0), else both walks read them from memory.
template <int NW, int CAP>
struct RouteLds {
  int base[256];
  int ibase[256];
  int ibase2[256];
  int tot[256];
  int wcnt[NW][256];
};

// Lanes of this wave holding the same expert id e (8 bits; e < 0: no assignment):
// the rank of this lane among them and their number.
__device__ __forceinline__ void same_expert(int e, int lane, int& rank, int& tot) {
  unsigned long long same = __ballot(e >= 0);
  if (e < 0) same = ~same;
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const unsigned long long b1 = __ballot(e >= 0 && ((e >> bit) & 1));
    same &= ((e >> bit) & 1) ? b1 : ~b1;
  }
  rank = __popcll(same & ((1ull << lane) - 1ull));
  tot = __popcll(same);
}

template <int NW, int CAP>
__device__ void route_block(const int32_t* __restrict__ ids, int A, int k, int E, int P,
                            int32_t* __restrict__ cnt, int32_t* __restrict__ poff,
                            int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                            int2* __restrict__ items, int32_t* __restrict__ n_items,
                            int2* __restrict__ items2, int32_t* __restrict__ n_items2,
                            int32_t* __restrict__ cnt_log, RouteLds<NW, CAP>& L, int* sids) {
  constexpr int NT = 64 * NW;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < NW * E; i += NT) L.wcnt[i / E][i % E] = 0;
  for (int i = tid; i < P; i += NT) perm[i] = -1;
  const bool staged = CAP > 0 && A <= CAP;
  if constexpr (CAP > 0) {
    if (staged) {
      constexpr int U = (CAP + NT - 1) / NT;   // every load in flight at once
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (tid + u * NT < A) v[u] = ids[tid + u * NT];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (tid + u * NT < A) sids[tid + u * NT] = v[u];
    }
  }
  __syncthreads();
  const int per = ((A + NW - 1) / NW + 63) & ~63;
  const int w0 = min(A, wv * per), w1 = min(A, w0 + per);
  auto id_at = [&](int a) { return a < w1 ? (staged ? sids[a] : ids[a]) : -1; };
  int* wc = L.wcnt[wv];
  // per-wave histogram (counts only: the order of the LDS additions does not matter)
  for (int c = w0; c < w1; c += 64) {
    const int e = id_at(c + lane);
    if (e >= 0) atomicAdd(&wc[e], 1);
  }
  __syncthreads();
  if (wv == 0) {
    // lane owns experts [lane*epl, lane*epl + epl)
    const int epl = (E + 63) / 64;
    int ps = 0, is = 0, is2 = 0;
    for (int i = 0; i < epl; ++i) {
      const int e = lane * epl + i;
      if (e < E) {
        int c = 0;
        for (int w2 = 0; w2 < NW; ++w2) c += L.wcnt[w2][e];
        L.tot[e] = c;
        ps += (c + 15) & ~15;
        is += (c + kMoeGroup - 1) / kMoeGroup;
        is2 += (c + kMoeGroup2 - 1) / kMoeGroup2;
      }
    }
    int incl_p = ps, incl_i = is, incl_i2 = is2;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int tp = __shfl_up(incl_p, o, 64), ti = __shfl_up(incl_i, o, 64), ti2 = __shfl_up(incl_i2, o, 64);
      if (lane >= o) {
        incl_p += tp;
        incl_i += ti;
        incl_i2 += ti2;
      }
    }
    int run_p = incl_p - ps, run_i = incl_i - is, run_i2 = incl_i2 - is2;
    for (int i = 0; i < epl; ++i) {
      const int e = lane * epl + i;
      if (e < E) {
        const int c = L.tot[e];
        L.base[e] = run_p;
        poff[e] = run_p;
        cnt[e] = c;
        if (cnt_log) cnt_log[e] = c;
        L.ibase[e] = run_i;
        L.ibase2[e] = run_i2;
        run_p += (c + 15) & ~15;
        run_i += (c + kMoeGroup - 1) / kMoeGroup;
        run_i2 += (c + kMoeGroup2 - 1) / kMoeGroup2;
      }
    }
    if (lane == 63) {
      poff[E] = incl_p;
      *n_items = incl_i;
      if (n_items2) *n_items2 = incl_i2;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += NT) {
    int it = L.ibase[e];
    for (int t0 = 0; t0 < L.tot[e]; t0 += kMoeGroup) items[it++] = make_int2(e, t0);
    if (items2) {
      // the expert's 16-token blocks dealt into its items as evenly as they go (at
      // most kMoeGroup2 tokens each); .y packs the item's token range [t0, t1)
      const int c = L.tot[e], ni = (c + kMoeGroup2 - 1) / kMoeGroup2, nb = (c + 15) >> 4;
      int it2 = L.ibase2[e];
      for (int i = 0; i < ni; ++i) {
        const int b0 = i * nb / ni, b1 = (i + 1) * nb / ni;
        items2[it2++] = make_int2(e, 16 * b0 | min(c, 16 * b1) << 16);
      }
    }
  }
  // per-wave running slot of expert e: its offset plus the earlier waves' counts, a
  // scan over NW consecutive lanes (one lane group per expert, one lane per wave)
  static_assert(NW <= 64 && (NW & (NW - 1)) == 0, "waves: a power of two");
  for (int i0 = 0; i0 < E * NW; i0 += NT) {
    const int i = i0 + tid, e = i / NW, w2 = i % NW;   // a lane group never straddles E * NW
    const int c = i < E * NW ? L.wcnt[w2][e] : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < NW; o <<= 1) {
      const int t = __shfl_up(incl, o, NW);
      if (w2 >= o) incl += t;
    }
    if (i < E * NW) L.wcnt[w2][e] = L.base[e] + incl - c;
  }
  __syncthreads();
  for (int c = w0; c < w1; c += 64) {
    const int a = c + lane, e = id_at(a);
    int rank, tot;
    same_expert(e, lane, rank, tot);
    if (e >= 0) {
      const int slot = wc[e] + rank;
      perm[slot] = a / k;
      inv[a] = slot;
    }
    if (e >= 0 && rank == tot - 1) wc[e] += tot;
  }
}

// Up to kRouteIdsSmall ids (a batch-1 canvas: 2048; a fused two-sequence pass: 4096)
// are staged in a static LDS array; more are read from memory (L2) in both walks.
// Larger passes run beside the side stream's wide-tile shared-expert GEMM, which
// holds 128 KiB of LDS on its CUs: a sort workgroup that also staged its 16384 ids
// (84 KiB in all) could start only on a CU with that much free and waited for one
// (~47 us per launch at batch 8); at 20 KiB it starts at once.
constexpr int kRouteIdsSmall = 4096;

// CAP > 0: up to CAP ids staged in LDS; CAP == 0: ids read from memory
template <int CAP>
__global__ __launch_bounds__(1024) void route_kernel(const int32_t* __restrict__ ids, int A, int k,
                                                     int E, int P, int32_t* __restrict__ cnt,
                                                     int32_t* __restrict__ poff,
                                                     int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ inv,
                                                     int2* __restrict__ items,
                                                     int32_t* __restrict__ n_items,
                                                     int2* __restrict__ items2,
                                                     int32_t* __restrict__ n_items2,
                                                     int32_t* __restrict__ cnt_log) {
  __shared__ RouteLds<16, CAP> L;
  __shared__ int st_ids[CAP > 0 ? CAP : 1];
  route_block<16, CAP>(ids, A, k, E, P, cnt, poff, perm, inv, items, n_items, items2, n_items2, cnt_log,
                       L, st_ids);
}

void launch_route(const int32_t* ids, int M, int k, int E, int32_t* cnt, int32_t* poff,
                  int32_t* perm, int32_t* inv, int2* items, int32_t* n_items, int2* items2,
                  int32_t* n_items2, int32_t* cnt_log, hipStream_t s) {
  const int A = M * k, P = moe_max_slots(M, k, E);
  if (A <= kRouteIdsSmall)
    launch_kernel(route_kernel<kRouteIdsSmall>, dim3(1), dim3(1024), 0, s, nullptr, ids, A, k, E, P, cnt, poff,
                  perm, inv, items, n_items, items2, n_items2, cnt_log);
  else
    launch_kernel(route_kernel<0>, dim3(1), dim3(1024), 0, s, nullptr, ids, A, k, E, P, cnt, poff, perm, inv,
                  items, n_items, items2, n_items2, cnt_log);
}

// ---------------------------------------------------------------- grouped GEMMs

__device__ __forceinline__ float silu_f(float v) { return v / (1.0f + __expf(-v)); }

// Grouped expert GEMMs.  A workgroup owns one work item (expert e and a range of
// up to kMoeGroup2 = 128 of its tokens: an expert's 16-token blocks are dealt evenly
// into its items, so 146 tokens make items of 80 and 66 rather than 128 and 18, and
// no workgroup streams a weight tile for a handful of tokens) and a tile of output
// features.  The gate/up GEMM (K = d_model) stages
// weight and token fragment tiles through LDS rings by direct global->LDS copies
// and computes a 128-row x 128-token tile; the down GEMM
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
// (gate and up blocks of 4 feature blocks) x one gate/up work item of up to 128
// tokens; the 8 waves form a 2 x 4 grid of 64-row x 32-token sub-tiles.  Per
// 64-wide k step the workgroup copies 8 weight blocks (two 1 KiB fragment tiles
// each) and up to 8 token blocks straight into LDS: weights into a three-step
// ring (two steps ahead), token rows -- L2 hits -- into a two-step ring (one step
// ahead).  Wave w copies weight block w and token block w; a wave whose token
// block lies past the item's tokens copies none.  The 80 KiB of rings let two
// workgroups share a CU.  Every weight byte is read once per workgroup and shared
// by up to 128 tokens, every token byte once per workgroup and shared by 128
// weight rows: per multiply-add this moves a third less than a 64-token tile.
//
// A token block's 64-wide k step is 16 rows x 128 bytes of row-major h, gathered
// through the permutation.  It is copied as two 8-row halves in which every lane
// moves one 16-byte piece, so each row's 128 bytes come in as one whole cache
// line (a fragment-shaped copy would touch each line twice, 64 bytes at a time,
// and the per-CU rate of line requests is what bounds this kernel).  In LDS half
// h holds rows 8h .. 8h + 7, 128 bytes each, with piece c of row 8h + q stored in
// slot c ^ q ^ h: the MFMA operand read of one piece column (16 rows) then hits
// 16 distinct 16-byte bank groups of the 256-byte bank row (the even and odd rows
// of a half fill opposite 128-byte halves; the two halves differ in the slot's
// lowest bit).
constexpr int kGuRB = 8, kGuTB = 8, kGuKT = 2, kGuWaves = 8;
constexpr int kGuWSlots = 3, kGuXSlots = 2;
constexpr int kGuXHalf = 1024;                  // bytes from one 8-row half to the next
constexpr int kGuXBlock = 2 * kGuXHalf;        // one token block of a k step
constexpr int kGuWBytes = kGuRB * kGuKT * 1024, kGuXBytes = kGuTB * kGuXBlock;
constexpr int kGuLds = kGuWSlots * kGuWBytes + kGuXSlots * kGuXBytes;
constexpr int kGuCopies = kGuRB * kGuKT / kGuWaves;   // weight tile copies per wave per step
static_assert(kMoeGroup2 == 16 * kGuTB, "one token block per wave");

template <bool STREAM>
__device__ __forceinline__ void gate_up_tile_lds(const uint16_t* wgu_e, const uint16_t* h_rm,
                                                 const int32_t* perm, int slot0, int t0, int t1, int F,
                                                 int f0, int d, int lane, int wv, uint16_t* A,
                                                 char* ring) {
  constexpr int WI = 4, WJ = 2;                      // MFMA blocks per wave (rows x tokens)
  const int ntb = min(kGuTB, (t1 - t0 + 15) >> 4);   // token blocks of this item [t0, t1) (>= 1)
  const int nk = d / (32 * kGuKT);
  const bool has_x = wv < ntb;                       // this wave copies a token block
  const uint16_t* wsrc = wgu_e + fm_tile(2 * f0 + wv, 0, d, lane);
  // The token rows are gathered on the fly: in half h of token block wv, lane i
  // copies piece (i % 8) ^ (i / 8) ^ h of the step's 128 bytes of row 8h + i / 8.
  // Padding slots read row 0: their outputs are dropped.
  const uint16_t* xsrc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rr = lane >> 3;
    const int tok = has_x ? perm[slot0 + 16 * wv + 8 * h + rr] : 0;
    xsrc[h] = h_rm + (size_t)max(tok, 0) * d + 8 * ((lane & 7) ^ rr ^ h);
  }
  char* const wring = ring;
  char* const xring = ring + kGuWSlots * kGuWBytes;
  auto issue_w = [&](int step) {
    char* dst = wring + (step % kGuWSlots) * kGuWBytes + wv * kGuKT * 1024;
#pragma unroll
    for (int t = 0; t < kGuKT; ++t) tile_to_lds<STREAM>(wsrc + (step * kGuKT + t) * 512, dst + t * 1024);
  };
  auto issue_x = [&](int step) {
    if (!has_x) return;
    char* dst = xring + (step % kGuXSlots) * kGuXBytes + wv * kGuXBlock;
#pragma unroll
    for (int h = 0; h < 2; ++h) tile_to_lds<false>(xsrc[h] + step * 64, dst + h * kGuXHalf);
  };
  const int wr = wv & 1, wt = wv >> 1;
  const bool has_mma = 2 * wt < ntb;                 // some token block of this wave is real
  f32x4 acc[WI][WJ];
#pragma unroll
  for (int i = 0; i < WI; ++i)
#pragma unroll
    for (int j = 0; j < WJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  lds_char* const lw = lds_launder(wring);
  lds_char* const lx = lds_launder(xring);
  // After step j's barrier the wave copies X(j + XS - 1) then W(j + WS - 1); the
  // prologue runs the same order for j = -(WS - 1) .. -1.  At the top of step s
  // the copies issued after X(s) are W(s + WS - XS) and, for each of the XS - 2
  // steps since, one X and one W step.  When WS > XS, W(s) was issued before X(s)
  // and waiting until only those later copies are in flight covers both; when
  // WS == XS, W(s) is the one right after X(s) and must land too.  A wave without
  // token copies has only W(s + 1) .. W(s + WS - 2) after W(s).  The barrier then
  // makes every wave's copies visible and retires all reads of the slots refilled
  // next.
  constexpr int WS = kGuWSlots, XS = kGuXSlots;
  static_assert(WS >= XS && XS >= 2, "weights run at least as far ahead as token rows");
  constexpr int kStepCopies = 2 + kGuCopies;
  constexpr int kAfterX = (WS > XS ? kGuCopies : 0) + (XS - 2) * kStepCopies;
  constexpr int kAfterW = (WS - 2) * kGuCopies;
  static_assert(kAfterX < 64, "vmcnt range");
#pragma unroll
  for (int j = -(WS - 1); j < 0; ++j) {
    if (j + XS - 1 >= 0 && j + XS - 1 < nk) issue_x(j + XS - 1);
    if (j + WS - 1 < nk) issue_w(j + WS - 1);
  }
  // this lane's operand (token row r, k group g) of k tile t within a token block
  int xoff[kGuKT];
  {
    const int r = lane & 15, g = lane >> 4, rr = r & 7, h = r >> 3;
#pragma unroll
    for (int t = 0; t < kGuKT; ++t) xoff[t] = h * kGuXHalf + rr * 128 + (((4 * t + g) ^ rr ^ h) << 4);
  }
  u32x4 Af[WI][kGuKT], Bf[WJ][kGuKT];
  for (int s = 0; s < nk; ++s) {
    if (s + WS - 2 < nk) {                   // every copy counted above exists
      if (has_x) vm_wait<kAfterX>();
      else vm_wait<kAfterW>();
    } else {
      vm_wait<0>();
    }
    __builtin_amdgcn_s_barrier();
    if (s + XS - 1 < nk) issue_x(s + XS - 1);
    if (s + WS - 1 < nk) issue_w(s + WS - 1);
    if (!has_mma) continue;
    const lds_char* sw = lw + (s % kGuWSlots) * kGuWBytes + lane * 16;
    const lds_char* sx = lx + (s % kGuXSlots) * kGuXBytes;
#pragma unroll
    for (int i = 0; i < WI; ++i)
#pragma unroll
      for (int t = 0; t < kGuKT; ++t) Af[i][t] = ld16_lds(sw + ((wr * WI + i) * kGuKT + t) * 1024);
#pragma unroll
    for (int j = 0; j < WJ; ++j)
#pragma unroll
      for (int t = 0; t < kGuKT; ++t) Bf[j][t] = ld16_lds(sx + (wt * WJ + j) * kGuXBlock + xoff[t]);
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
    if (tb >= ntb || t >= t1) continue;
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

__global__ __launch_bounds__(64 * kGuWaves) void moe_gate_up_kernel(const uint16_t* __restrict__ h_rm,
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
  const int e = it.x, t0 = it.y & 0xffff, t1 = it.y >> 16;
  const int slot0 = poff[e] + t0;
  const uint16_t* wgu_e = wgu + (size_t)e * 2 * F * d;
  // an expert with a single work item streams its weights (read by no other item)
  if (cnt[e] <= kMoeGroup2)
    gate_up_tile_lds<true>(wgu_e, h_rm, perm, slot0, t0, t1, F, fb * (kGuRB / 2), d, lane, wv, A, ring);
  else
    gate_up_tile_lds<false>(wgu_e, h_rm, perm, slot0, t0, t1, F, fb * (kGuRB / 2), d, lane, wv, A, ring);
}

void launch_moe_gate_up(const uint16_t* h_rm, const int32_t* perm, const uint16_t* w_gate_up,
                        const int32_t* cnt, const int32_t* poff, const int2* items2,
                        const int32_t* n_items2, int max_items2, int F, int d, uint16_t* a,
                        hipStream_t s) {
  static LdsLimit limit;
  raise_lds_limit(limit, reinterpret_cast<const void*>(&moe_gate_up_kernel), kGuLds);
  const int blocks = kXcd * ((max_items2 + kXcd - 1) / kXcd) * (F / (16 * kGuRB / 2));
  launch_kernel(moe_gate_up_kernel, dim3(blocks), dim3(64 * kGuWaves), kGuLds, s, nullptr, h_rm, perm,
                w_gate_up, cnt, poff, items2, n_items2, F, d, a);
}

// down: Y[slot][n] = A[slot] . W_d[e][n]^T over K = F.  Workgroup tile: 128 output
// rows x one work item of up to 128 tokens (NT token blocks).  Wave wv owns row
// blocks 2wv, 2wv + 1 and loads their weight fragments straight into registers two
// steps ahead (each weight byte is used by that wave alone); the item's activation
// tiles, shared by the four waves, are copied once per workgroup into a three-step
// LDS ring, wave wv copying token blocks 2wv and 2wv + 1 where they exist.
constexpr int kDnXS = 3;
constexpr int kDnXBytes = 8 * kGuKT * 1024;      // 128 tokens x 64 k
constexpr int kDnLds = kDnXS * kDnXBytes;
static_assert(kMoeGroup2 == 128, "eight token blocks per down work item");

template <bool STREAM, int NT>
__device__ __forceinline__ void down_tile(const uint16_t* wd_e, const uint16_t* A, int slot0, int t0,
                                          int t1, int F, int d, int n0, int lane, int wv, float* Y,
                                          char* ring) {
  const int nblk = d >> 4;
  const int nk = F / (32 * kGuKT);                // >= 1 (F % 64 == 0)
  const int rb0 = (n0 >> 4) + 2 * wv;
  const uint16_t* w0 = wd_e + fm_tile(min(rb0, nblk - 1), 0, F, lane);
  const uint16_t* w1 = wd_e + fm_tile(min(rb0 + 1, nblk - 1), 0, F, lane);
  // wave wv copies token blocks 2wv (when 2wv < NT) and 2wv + 1 (when 2wv + 1 < NT)
  const int ncopy = max(0, min(2, NT - 2 * wv));
  const uint16_t* xsrc = A + fm_tile((slot0 >> 4) + min(2 * wv, NT - 1), 0, F, lane);
  lds_char* const lx = lds_launder(ring);
  typedef u32x4 WSet[4];                           // rows rb0 k0, k1; rows rb0+1 k0, k1
  auto issue = [&](int step, WSet& w) {
    char* dst = ring + (step % kDnXS) * kDnXBytes + 2 * wv * kGuKT * 1024;
    for (int b = 0; b < ncopy; ++b)
#pragma unroll
      for (int t = 0; t < kGuKT; ++t)
        tile_to_lds_untracked(xsrc + ((size_t)b * (F >> 5) + step * kGuKT + t) * 512,
                              dst + (b * kGuKT + t) * 1024);
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
  // iteration's (ncopy * kGuKT copies + 4 loads) may still be in flight unless it
  // issued none.
  // Refilling ring slot (s + 2) % 3 is safe after the barrier: every wave consumed
  // that slot's step s - 1 before arriving.
  auto body = [&](int s, WSet& wc, WSet& wn, bool more, bool last) {
    if (last) vm_wait<0>();
    else if (ncopy == 2) vm_wait<2 * kGuKT + 4>();
    else if (ncopy == 1) vm_wait<kGuKT + 4>();
    else vm_wait<4>();
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
    if (t >= t1) continue;
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
  const int e = it.x, t0 = it.y & 0xffff, t1 = it.y >> 16;
  const int slot0 = poff[e] + t0;
  const int n0 = nb * kDownRows;
  const uint16_t* wd_e = wd + (size_t)e * d * F;
  const int nt = min(8, (t1 - t0 + 15) >> 4);
  const bool single = cnt[e] <= kMoeGroup2;
  // an expert with a single work item streams its weights (read by no other item)
#define DOWN_TILE(NT)                                                                            \
  (single ? down_tile<true, NT>(wd_e, A, slot0, t0, t1, F, d, n0, lane, wv, Y, ring)            \
          : down_tile<false, NT>(wd_e, A, slot0, t0, t1, F, d, n0, lane, wv, Y, ring))
  switch (nt) {
    case 1: DOWN_TILE(1); break;
    case 2: DOWN_TILE(2); break;
    case 3: DOWN_TILE(3); break;
    case 4: DOWN_TILE(4); break;
    case 5: DOWN_TILE(5); break;
    case 6: DOWN_TILE(6); break;
    case 7: DOWN_TILE(7); break;
    default: DOWN_TILE(8); break;
  }
#undef DOWN_TILE
}

int moe_max_items(int M, int k, int E) { return (M * k + kMoeGroup - 1) / kMoeGroup + E; }
int moe_max_items2(int M, int k, int E) { return (M * k + kMoeGroup2 - 1) / kMoeGroup2 + E; }
int moe_max_slots(int M, int k, int E) { return M * k + 15 * E; }

void launch_moe_down(const uint16_t* a, const uint16_t* w_down, const int32_t* cnt,
                     const int32_t* poff, const int2* items2, const int32_t* n_items2, int max_items2,
                     int F, int d, float* Y, hipStream_t s) {
  const int blocks = kXcd * ((max_items2 + kXcd - 1) / kXcd) * ((d + kDownRows - 1) / kDownRows);
  launch_kernel(moe_down_kernel, dim3(blocks), dim3(256), kDnLds, s, nullptr, a, w_down, cnt, poff, items2,
                n_items2, F, d, Y);
}

}  // namespace dg
