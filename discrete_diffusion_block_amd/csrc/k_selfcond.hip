// Self-conditioning signal (DiffusionGemma Technical Report §3.2, decoder forward pass
// and denoising iteration, eq. 5-6; §6 GPU time breakdown, sampling): from the logits L
// of one step, p̂₀ = softmax(L) per canvas row and z = FFW(p̂₀ E), fed to the next step's
// decoder input.  The pages run the softmax and the embedding product in full precision.
//
//  * rowstats: per row the maximum m and S = sum exp(x - m) in fp32 (one pass with an
//    online rescale; fixed reduction order).
//  * sc_embed_gemm: u~[m][n] = sum_v exp(x_mv - m_m) E[v][n], a split-K GEMM with
//    K = V (262144) on bf16 MFMA.  E is exact in bf16; p = exp(x - m) (fp32) enters as
//    the sum of two bf16 operands hi = bf16(p), lo = bf16(p - hi), so the product sees p
//    to 2^-18 relative, and accumulates in fp32 -- the same precision as an fp32 GEMM
//    over this length, at the bf16 rate.  E enters transposed (E^T [d][V] packed once,
//    fragment-major), so each MFMA operand is one contiguous 1 KiB wave load.
//    Workgroup tile: 256 features x 256 canvas rows x one k slice; the waves share
//    the E^T tiles (global->LDS copies, three-step ring) and the p tiles (each wave
//    copies a quarter of the logits chunks into LDS, three-step ring, turns them into p
//    tiles and stores those in a two-step ring); both copy streams run two k steps ahead;
//    each of the four waves owns a 128 x 128 quarter of the outputs (8 x 8 MFMA blocks).  Every global read is a direct global->LDS copy waited for
//    explicitly, so no copy in flight ever holds up the one being waited for.  The row tiles of one (row block, k
//    slice) run consecutively on one XCD, so its logits slice is fetched into that L2
//    once.  Partial sums go to part[split][m][n].
//  * sc_reduce: u = (sum over splits, in split order) / S, written in fp32 (optional)
//    and as bf16 in fragment-major layout for the FFW GEMMs.
#include <math.h>

#include "dg_common.h"
#include "dg_internal.h"

namespace dg {

constexpr float kScLog2e = 1.44269504088896341f;

// exp(x - m) as every self-conditioning kernel evaluates it: 2^(x log2e - m log2e) with
// the exponent formed by one fma from mL = m log2e.
__device__ __forceinline__ float sc_exp(float x, float mL) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(x, kScLog2e, -mL));
}

// ---------------------------------------------------------------- row statistics

__global__ __launch_bounds__(256) void sc_rowstats_kernel(const uint16_t* __restrict__ logits, int V,
                                                          float2* __restrict__ stats) {
  __shared__ float red_m[4], red_s[4];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint16_t* lp = logits + (size_t)row * V;
  float m = -INFINITY, s = 0.f;
  for (int i = 8 * tid; i < V; i += 8 * 256) {   // V % 32 == 0: a piece is wholly in
    const u32x4 v = ld16_stream(lp + i);
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(v[j] << 16);
      x[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
    }
    float pm = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) pm = fmaxf(pm, x[j]);
    if (pm > m) {
      s = (m == -INFINITY) ? 0.f : s * __builtin_amdgcn_exp2f((m - pm) * kScLog2e);
      m = pm;
    }
    const float mL = m * kScLog2e;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += sc_exp(x[j], mL);
  }
  // the row maximum, then every thread's sum rescaled to it and summed in a fixed order
  const float M = [&] {
    const float wm = wave_max(m);
    if (lane == 0) red_m[w] = wm;
    __syncthreads();
    return fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
  }();
  const float sr = (m == -INFINITY) ? 0.f : s * __builtin_amdgcn_exp2f((m - M) * kScLog2e);
  const float ws = wave_sum(sr);
  if (lane == 0) red_s[w] = ws;
  __syncthreads();
  if (tid == 0) {
    const float S = (red_s[0] + red_s[1]) + (red_s[2] + red_s[3]);
    stats[row] = make_float2(M * kScLog2e, 1.0f / S);
  }
}

// ---------------------------------------------------------------- p̂₀ E GEMM

constexpr int kScRB = 16;   // 16-feature blocks of E^T per workgroup
constexpr int kScTB = 16;   // 16-row blocks of canvas rows per workgroup
constexpr int kScASlots = 3, kScPSlots = 2, kScLSlots = 3;
constexpr int kScABytes = kScRB * 1024;         // one 32-wide k step of E^T tiles
constexpr int kScPBytes = kScTB * 2 * 1024;     // one k step of p tiles, hi and lo
constexpr int kScLBytes = kScTB * 1024;         // one k step of logits chunks (16 rows x 64 B each)
constexpr int kScLds = kScASlots * kScABytes + kScPSlots * kScPBytes + kScLSlots * kScLBytes;
constexpr int kScWaves = 4;
constexpr int kScACopies = kScRB / kScWaves;    // E^T tiles each wave copies per step
constexpr int kScPBlocks = kScTB / kScWaves;    // p row blocks each wave computes per step

struct ScArgs {
  const uint16_t* logits;   // bf16 [M][K] row-major
  const float2* stats;      // [M]: (m log2e, 1 / S)
  const uint16_t* et;       // E^T, fragment-major [et_blocks * 16][K]
  float* part;              // [nsplit][M][N]
  int M, N, K;
  int et_blocks;
  int n_row_tiles, n_tok_tiles, nsplit, kslice;
};

__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__global__ __launch_bounds__(64 * kScWaves) void sc_embed_gemm(ScArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char ring[];   // [A slots][P slots][L slots]
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int total = a.n_row_tiles * a.n_tok_tiles * a.nsplit;
  const int per_xcd = (total + kXcd - 1) / kXcd;
  const int L = (int)(blockIdx.x % kXcd) * per_xcd + (int)(blockIdx.x / kXcd);
  if (L >= total) return;                       // uniform per workgroup
  const int row_tile = L % a.n_row_tiles;
  const int grp = L / a.n_row_tiles;
  const int tok_tile = grp % a.n_tok_tiles, split = grp / a.n_tok_tiles;
  const int k0 = split * a.kslice;
  const int nk = (min(a.K, k0 + a.kslice) - k0) >> 5;   // >= 1: the host sizes the slices
  const int rb0 = row_tile * kScRB, tb0 = tok_tile * kScTB;
  const int kb0 = k0 >> 5;

  char* const aring = ring;
  char* const pring = ring + kScASlots * kScABytes;
  char* const lring = pring + kScPSlots * kScPBytes;
  // E^T copy duty: kScACopies blocks from wv * kScACopies of the step (past the matrix:
  // the last block, whose outputs are dropped)
  const uint16_t* asrc[kScACopies];
#pragma unroll
  for (int u = 0; u < kScACopies; ++u)
    asrc[u] = a.et + fm_tile(min(rb0 + wv * kScACopies + u, a.et_blocks - 1), kb0, a.K, lane);
  auto issue_a = [&](int step) {
    char* dst = aring + (step % kScASlots) * kScABytes + wv * kScACopies * 1024;
#pragma unroll
    for (int u = 0; u < kScACopies; ++u) tile_to_lds_untracked(asrc[u] + step * 512, dst + u * 1024);
  };
  // p duty: kScPBlocks row blocks from wv * kScPBlocks of the tile, lane row r, k 8g ..
  // 8g + 7 of each step (rows past M read the last row; their outputs are dropped).  The
  // lane copies its 16 logits bytes of each block into the L slot and reads back the
  // same bytes.
  const uint16_t* lsrc[kScPBlocks];
  float mL[kScPBlocks];
#pragma unroll
  for (int u = 0; u < kScPBlocks; ++u) {
    const int m = min((tb0 + wv * kScPBlocks + u) * 16 + r, a.M - 1);
    lsrc[u] = a.logits + (size_t)m * a.K + k0 + 8 * g;
    mL[u] = a.stats[m].x;
  }
  auto issue_l = [&](int step) {
    char* dst = lring + (step % kScLSlots) * kScLBytes + wv * kScPBlocks * 1024;
#pragma unroll
    for (int u = 0; u < kScPBlocks; ++u) tile_to_lds_untracked(lsrc[u] + step * 32, dst + u * 1024);
  };
  lds_char* const ll = lds_launder(lring);
  auto make_p = [&](int step) {
    char* dst = pring + (step % kScPSlots) * kScPBytes + wv * kScPBlocks * 2 * 1024 + lane * 16;
    const lds_char* src = ll + (step % kScLSlots) * kScLBytes + wv * kScPBlocks * 1024 + lane * 16;
#pragma unroll
    for (int u = 0; u < kScPBlocks; ++u) {
      const u32x4 x = ld16_lds(src + u * 1024);
      u32x4 hi, lo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = sc_exp(__uint_as_float(x[j] << 16), mL[u]);
        const float p1 = sc_exp(__uint_as_float(x[j] & 0xffff0000u), mL[u]);
        const uint32_t h = cvt_pk_bf16(p0, p1);
        hi[j] = h;
        lo[j] = cvt_pk_bf16(p0 - __uint_as_float(h << 16), p1 - __uint_as_float(h & 0xffff0000u));
      }
      *reinterpret_cast<u32x4*>(dst + (2 * u) * 1024) = hi;
      *reinterpret_cast<u32x4*>(dst + (2 * u + 1) * 1024) = lo;
    }
  };

  constexpr int FI = kScRB / 2, FJ = kScTB / 2;   // a 2 x 2 grid of 128 x 128 wave tiles
  const int wr = wv & 1, wt = wv >> 1;
  f32x4 acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Copy order per wave: L(0), A(0), L(1), A(1); then at the top of step s: L(s + 2),
  // A(s + 2) -- both two steps ahead.  Before p(s + 1) is made, vmcnt <= kScStepCopies
  // leaves only step s's copies in flight, so L(s + 1) and A(s + 1) (issued at the top of
  // step s - 1) have landed; the barrier at the top of step s + 1 then publishes A(s + 1)
  // and p(s + 1) of all waves and retires every read of the slots step s + 1 refills
  // (A and p: read by step s's MFMAs; L: read when p(s) was made).
  constexpr int kScStepCopies = kScACopies + kScPBlocks;
  issue_l(0);
  issue_a(0);
  if (nk > 1) {
    issue_l(1);
    issue_a(1);
    vm_wait<kScStepCopies>();
  } else {
    vm_wait<0>();
  }
  make_p(0);
  lds_char* const la = lds_launder(aring);
  lds_char* const lp = lds_launder(pring);
  u32x4 A[FI], Bh[2], Bl[2];
  for (int s = 0; s < nk; ++s) {
    lds_sync();
    if (s + 2 < nk) {
      issue_l(s + 2);
      issue_a(s + 2);
    }
    const lds_char* sa = la + (s % kScASlots) * kScABytes + lane * 16;
    const lds_char* sp = lp + (s % kScPSlots) * kScPBytes + lane * 16;
#pragma unroll
    for (int i = 0; i < FI; ++i) A[i] = ld16_lds(sa + (wr * FI + i) * 1024);
    auto readB = [&](int j) {
      Bh[j & 1] = ld16_lds(sp + (2 * (wt * FJ + j)) * 1024);
      Bl[j & 1] = ld16_lds(sp + (2 * (wt * FJ + j) + 1) * 1024);
    };
    readB(0);
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      if (j + 1 < FJ) readB(j + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FI; ++i) acc[i][j] = mfma16x2(A[i], Bh[j & 1], A[i], Bl[j & 1], acc[i][j]);
    }
    if (s + 1 < nk) {
      if (s + 2 < nk) vm_wait<kScStepCopies>();
      else vm_wait<0>();
      make_p(s + 1);
    }
  }

  float* const base = a.part + (size_t)split * a.M * a.N;
#pragma unroll
  for (int j = 0; j < FJ; ++j) {
    const int m = (tb0 + wt * FJ + j) * 16 + r;
    if (m >= a.M) continue;
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const int n0 = (rb0 + wr * FI + i) * 16 + 4 * g;
      if (n0 >= a.N) continue;   // N % 16 == 0: n0 < N covers n0 .. n0 + 3
      *reinterpret_cast<f32x4*>(base + (size_t)m * a.N + n0) = acc[i][j];
    }
  }
}

// ---------------------------------------------------------------- split reduction

// One thread per 8 features of one row: u = (sum of the split partials in split order) / S.
__global__ __launch_bounds__(256) void sc_reduce_kernel(const float* __restrict__ part, int nsplit,
                                                        const float2* __restrict__ stats, int M, int N,
                                                        uint16_t* __restrict__ u_fm, float* __restrict__ u_out) {
  const int per_row = N >> 3;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * per_row) return;
  const int m = idx / per_row, c = (idx - m * per_row) * 8;
  f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const float* p = part + ((size_t)s * M + m) * N + c;
    v0 += *reinterpret_cast<const f32x4*>(p);
    v1 += *reinterpret_cast<const f32x4*>(p + 4);
  }
  const float inv = stats[m].y;
  v0 *= inv;
  v1 *= inv;
  u32x4 o;
  o.x = pack_bf2(v0[0], v0[1]);
  o.y = pack_bf2(v0[2], v0[3]);
  o.z = pack_bf2(v1[0], v1[1]);
  o.w = pack_bf2(v1[2], v1[3]);
  *reinterpret_cast<u32x4*>(u_fm + fm_index(m, c, N)) = o;
  if (u_out) {
    *reinterpret_cast<f32x4*>(u_out + (size_t)m * N + c) = v0;
    *reinterpret_cast<f32x4*>(u_out + (size_t)m * N + c + 4) = v1;
  }
}

// ---------------------------------------------------------------- host side

int sc_row_tiles(int N) { return (N + 16 * kScRB - 1) / (16 * kScRB); }
int sc_tok_tiles(int M) { return (M + 16 * kScTB - 1) / (16 * kScTB); }

// k slices per (row tile, token tile): as many as one workgroup per CU allows (256
// CUs), each at least 8 k steps long.
int sc_splits(int M, int N, int K) {
  const int tiles = sc_row_tiles(N) * sc_tok_tiles(M);
  int s = std::max(1, 256 / tiles);
  s = std::min(s, std::max(1, K / 256));
  const int steps = K / 32;
  const int per = (steps + s - 1) / s;      // k steps per slice
  return (steps + per - 1) / per;           // no empty slice
}

static int sc_kslice(int K, int nsplit) {
  const int steps = K / 32;
  return (steps + nsplit - 1) / nsplit * 32;
}

void launch_sc_rowstats(const uint16_t* logits, int M, int V, float2* stats, hipStream_t s) {
  launch_kernel(sc_rowstats_kernel, dim3(M), dim3(256), 0, s, nullptr, logits, V, stats);
}

void launch_sc_embed(const uint16_t* logits, const float2* stats, const uint16_t* et, int M, int N, int K,
                     float* part, hipStream_t s) {
  static LdsLimit limit;
  raise_lds_limit(limit, reinterpret_cast<const void*>(&sc_embed_gemm), kScLds);
  ScArgs a{};
  a.logits = logits; a.stats = stats; a.et = et; a.part = part;
  a.M = M; a.N = N; a.K = K;
  a.et_blocks = (N + 15) / 16;
  a.n_row_tiles = sc_row_tiles(N);
  a.n_tok_tiles = sc_tok_tiles(M);
  a.nsplit = sc_splits(M, N, K);
  a.kslice = sc_kslice(K, a.nsplit);
  const int total = a.n_row_tiles * a.n_tok_tiles * a.nsplit;
  const int blocks = kXcd * ((total + kXcd - 1) / kXcd);
  launch_kernel(sc_embed_gemm, dim3(blocks), dim3(64 * kScWaves), (size_t)kScLds, s, nullptr, a);
}

void launch_sc_reduce(const float* part, int nsplit, const float2* stats, int M, int N, uint16_t* u_fm,
                      float* u_out, hipStream_t s) {
  const int n = M * (N / 8);
  launch_kernel(sc_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, s, nullptr, part, nsplit, stats, M, N, u_fm,
                u_out);
}

}  // namespace dg
