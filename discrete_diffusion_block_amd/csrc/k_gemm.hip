// Dense bf16 GEMMs on MFMA (v_mfma_f32_16x16x32_bf16), fp32 accumulation.
//
// Every product is y[m][n] = sum_k x[m][k] * w[n][k].  Both operands live in
// fragment-major layout (weights packed once, activations written that way by
// the kernels that produce them), so every MFMA operand fragment is one
// contiguous 1 KiB wave load straight into registers -- no LDS staging.
// Weight rows sit on the MFMA A side (16 rows per block), tokens on the B side
// (16 tokens per block); a lane then holds 4 consecutive output features of one
// token, so each epilogue is a short vector store.
//
// dense_gemm: a workgroup of 4 waves owns one (WN x 16) feature x (WM x 16)
// token tile and splits K between its waves (interleaved 64-wide k steps),
// then reduces the four partial tiles through LDS in a fixed order.  All token
// tiles of a weight tile run on one XCD, so the weights leave HBM once.
//
// head_gemm: the tied LM head (N = 262144 rows of the embedding) -- 256 x 256
// workgroup tiles with both operands staged through an LDS ring by direct
// global->LDS copies.
#include <type_traits>

#include "dg_common.h"
#include "dg_internal.h"

namespace dg {

enum Epi { EPI_STORE_F32 = 0, EPI_ADD_F32 = 1, EPI_SWIGLU = 2, EPI_QKV = 3 };

struct DenseArgs {
  const uint16_t* x;  // activations, fragment-major [M_pad][K]
  const uint16_t* w;  // packed weights, fragment-major [N_pad][K]
  int M, N, K;
  int nblk;           // 16-row blocks of the packed weight
  float* yf;
  uint16_t* yb;
  int ldy;
  int hq, hd;         // QKV
  KvLayer kv;
  PassGeom g;
  const float2* rope;
  uint16_t* q_out;
};

__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

template <int EPI, int WN>
__device__ __forceinline__ void epilogue(const DenseArgs& a, int blk0, int m, const f32x4 (&v)[WN],
                                         int g) {
  if (m >= a.M) return;
  if constexpr (EPI == EPI_STORE_F32 || EPI == EPI_ADD_F32) {
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      const int n0 = (blk0 + i) * 16 + 4 * g;
      float* dst = a.yf + (size_t)m * a.ldy + n0;
      if (n0 + 3 < a.N) {
        f32x4 o = v[i];
        if constexpr (EPI == EPI_ADD_F32) o += *reinterpret_cast<f32x4*>(dst);
        *reinterpret_cast<f32x4*>(dst) = o;
      } else {
        for (int e = 0; e < 4; ++e)
          if (n0 + e < a.N) dst[e] = (EPI == EPI_ADD_F32 ? dst[e] : 0.f) + v[i][e];
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // packed block 2t = gate rows of features 16t.., block 2t+1 = the matching up rows;
    // the tile's blocks (blk0 even) form WN / 2 such pairs, the last ones possibly past
    // the matrix (their loads were clamped; nothing is written for them)
    static_assert(WN % 2 == 0, "gate/up block pairs");
#pragma unroll
    for (int i = 0; i < WN; i += 2) {
      if (blk0 + i + 1 >= a.nblk) break;
      const int f0 = ((blk0 + i) >> 1) * 16 + 4 * g;
      u32x2 o;
      o.x = pack_bf2(silu(v[i][0]) * v[i + 1][0], silu(v[i][1]) * v[i + 1][1]);
      o.y = pack_bf2(silu(v[i][2]) * v[i + 1][2], silu(v[i][3]) * v[i + 1][3]);
      *reinterpret_cast<u32x2*>(a.yb + fm_index(m, f0, a.ldy)) = o;
    }
  } else {  // EPI_QKV: rows were packed so that lane group g holds features
            // {p, p+1, p+hd/2, p+1+hd/2}, p = 8j + 2g, of head-local block j
    const int hd = a.hd, half = hd >> 1, per = hd >> 4;
    const int b = m / a.g.n, ii = m - b * a.g.n;
    const int pos = a.g.len[b] + ii;
    const int npad = (a.g.n + 15) & ~15;
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      const int blk = blk0 + i;
      if (blk >= a.nblk) continue;
      const int head = blk / per, j = blk - head * per;
      const int p = 8 * j + 2 * g;
      const float x0 = v[i][0], x1 = v[i][1], x2 = v[i][2], x3 = v[i][3];
      if (head < a.hq + a.kv.hkv) {
        const float2 r0 = a.rope[(size_t)m * half + p], r1 = a.rope[(size_t)m * half + p + 1];
        const float y0 = x0 * r0.x - x2 * r0.y, y2 = x2 * r0.x + x0 * r0.y;
        const float y1 = x1 * r1.x - x3 * r1.y, y3 = x3 * r1.x + x1 * r1.y;
        if (head < a.hq) {
          uint16_t* base = a.q_out + ((size_t)b * a.hq + head) * (size_t)npad * hd;
          *reinterpret_cast<uint32_t*>(base + fm_index(ii, p, hd)) = pack_bf2(y0, y1);
          *reinterpret_cast<uint32_t*>(base + fm_index(ii, p + half, hd)) = pack_bf2(y2, y3);
        } else {
          const int kh = head - a.hq;
          uint16_t* base = a.kv.k + ((size_t)kv_seq(a.g, b) * a.kv.hkv + kh) * (size_t)a.kv.max_ctx * hd;
          *reinterpret_cast<uint32_t*>(base + k_index(pos, p, hd)) = pack_bf2(y0, y1);
          *reinterpret_cast<uint32_t*>(base + k_index(pos, p + half, hd)) = pack_bf2(y2, y3);
        }
      } else {
        const int vh = head - a.hq - a.kv.hkv;
        uint16_t* base = a.kv.vt + ((size_t)kv_seq(a.g, b) * a.kv.hkv + vh) * (size_t)hd * a.kv.max_ctx;
        base[v_index(pos, p, hd)] = f2bf(x0);
        base[v_index(pos, p + 1, hd)] = f2bf(x1);
        base[v_index(pos, p + half, hd)] = f2bf(x2);
        base[v_index(pos, p + half + 1, hd)] = f2bf(x3);
      }
    }
  }
}

template <int WN, int WM, int EPI, int NW = 4>
__global__ __launch_bounds__(64 * NW) void dense_gemm(DenseArgs a) {
  extern __shared__ f32x4 red[];  // [NW waves][WN][WM][64 lanes]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  // XCD-aware tile order: block b runs on XCD b % 8, and the token tiles of one
  // weight tile take consecutive ranks on that XCD, so they share its L2 copy
  const int n_tiles = (a.nblk + WN - 1) / WN, m_tiles = (a.M + 16 * WM - 1) / (16 * WM);
  const int rank = blockIdx.x / kXcd;
  const int n_tile = (rank / m_tiles) * kXcd + (int)(blockIdx.x % kXcd);
  if (n_tile >= n_tiles) return;   // uniform per workgroup
  const int blk0 = n_tile * WN;
  const int mb0 = (rank % m_tiles) * WM;

  // fragment tiles (rb, kb): rb clamped to the last real block (dropped in the epilogue)
  const uint16_t* wp[WN];
  const uint16_t* xp[WM];
  const int mblocks = (a.M + 15) >> 4;
#pragma unroll
  for (int i = 0; i < WN; ++i) wp[i] = a.w + fm_tile(min(blk0 + i, a.nblk - 1), 0, a.K, lane);
#pragma unroll
  for (int j = 0; j < WM; ++j) xp[j] = a.x + fm_tile(min(mb0 + j, mblocks - 1), 0, a.K, lane);

  f32x4 acc[WN][WM];
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 A0[WN][2], B0[WM][2], A1[WN][2], B1[WM][2], A2[WN][2], B2[WM][2];
  auto load = [&](u32x4 (&A)[WN][2], u32x4 (&B)[WM][2], int it) {
    const int k = it * 1024;  // two 512-element k tiles per 64-wide step
    // every token tile re-reads these weight tiles, so they go through L2 as usual
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      A[i][0] = ld16(wp[i] + k);
      A[i][1] = ld16(wp[i] + k + 512);
    }
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      B[j][0] = ld16(xp[j] + k);
      B[j][1] = ld16(xp[j] + k + 512);
    }
  };
  auto mma = [&](u32x4 (&A)[WN][2], u32x4 (&B)[WM][2]) {
#pragma unroll
    for (int i = 0; i < WN; ++i)
#pragma unroll
      for (int j = 0; j < WM; ++j) {
        acc[i][j] = mfma16x2(A[i][0], B[j][0], A[i][1], B[j][1], acc[i][j]);
      }
  };

  // wave w takes the 64-wide k steps w, w+NW, w+2NW, ...
  const int nk = a.K >> 6;
  const int nw = w < nk ? (nk - w + NW - 1) / NW : 0;
  pipeline3(nw, [&](int s) { load(A0, B0, w + NW * s); }, [&](int s) { load(A1, B1, w + NW * s); },
            [&](int s) { load(A2, B2, w + NW * s); }, [&] { mma(A0, B0); }, [&] { mma(A1, B1); },
            [&] { mma(A2, B2); });

#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j) red[((w * WN + i) * WM + j) * 64 + lane] = acc[i][j];
  __syncthreads();
  for (int j = w; j < WM; j += NW) {
    f32x4 v[WN];
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      f32x4 s = red[((0 * WN + i) * WM + j) * 64 + lane];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) s += red[((ww * WN + i) * WM + j) * 64 + lane];
      v[i] = s;
    }
    epilogue<EPI, WN>(a, blk0, (mb0 + j) * 16 + r, v, g);
  }
}

// Wide-tile dense GEMM for passes of many rows (several sequences, or long prefill
// chunks): a workgroup owns 256 weight rows x 128 tokens, with both operands staged
// through LDS by direct global->LDS copies (weights in a three-step ring, two steps
// ahead; token tiles in a two-step ring) and read by all four waves.  Wave w computes
// weight rows 64w .. 64w + 63 against the 128 tokens over the whole K, so each
// operand byte from L2 feeds 128 or 256 outputs instead of the small tile's 64.  The
// epilogues are the small tile's, fed one 16-token column (4 weight blocks) at a time.
// Every output accumulates its k steps in order in one wave, which differs from the
// small tile's four interleaved K partials; launch_* picks this kernel by the row
// count alone (kWideMinRows), so a pass's results depend only on its shape.
constexpr int kWideRB = 16, kWideTB = 8, kWideKT = 2;
constexpr int kWideWSlots = 3, kWideXSlots = 2;
constexpr int kWideWBytes = kWideRB * kWideKT * 1024, kWideXBytes = kWideTB * kWideKT * 1024;
constexpr int kWideLds = kWideWSlots * kWideWBytes + kWideXSlots * kWideXBytes;
constexpr int kWideWCopies = kWideRB * kWideKT / 4;   // per wave per step
constexpr int kWideMinRows = 2048;

template <int EPI>
__global__ __launch_bounds__(256) void dense_wide_gemm(DenseArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char ring[];
  constexpr int WI = kWideRB / 4, NB = kWideTB;        // MFMA blocks per wave (rows x tokens)
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int n_row = (a.nblk + kWideRB - 1) / kWideRB, n_tok = (a.M + 16 * kWideTB - 1) / (16 * kWideTB);
  // the token tiles of one weight tile take consecutive ranks on one XCD (shared weights in its L2)
  const int b = blockIdx.x, rank = b / kXcd;
  const int row_tile = (rank / n_tok) * kXcd + b % kXcd, tok_tile = rank % n_tok;
  if (row_tile >= n_row) return;   // uniform per workgroup
  const int rb0 = row_tile * kWideRB, tb0 = tok_tile * kWideTB;
  const int mblocks = (a.M + 15) >> 4;
  const int nk = a.K / (32 * kWideKT);
  constexpr int WB = kWideRB / 4, XB = kWideTB / 4;
  const uint16_t* wsrc[WB];
  const uint16_t* xsrc[XB];
  // blocks past the matrix re-read its last block (their outputs are dropped)
#pragma unroll
  for (int u = 0; u < WB; ++u) wsrc[u] = a.w + fm_tile(min(rb0 + wv * WB + u, a.nblk - 1), 0, a.K, lane);
#pragma unroll
  for (int u = 0; u < XB; ++u) xsrc[u] = a.x + fm_tile(min(tb0 + wv * XB + u, mblocks - 1), 0, a.K, lane);
  char* const wring = ring;
  char* const xring = ring + kWideWSlots * kWideWBytes;
  auto issue_w = [&](int step) {
    char* dst = wring + (step % kWideWSlots) * kWideWBytes + wv * WB * kWideKT * 1024;
#pragma unroll
    for (int u = 0; u < WB; ++u)
#pragma unroll
      for (int t = 0; t < kWideKT; ++t)
        tile_to_lds<false>(wsrc[u] + (step * kWideKT + t) * 512, dst + (u * kWideKT + t) * 1024);
  };
  auto issue_x = [&](int step) {
    char* dst = xring + (step % kWideXSlots) * kWideXBytes + wv * XB * kWideKT * 1024;
#pragma unroll
    for (int u = 0; u < XB; ++u)
#pragma unroll
      for (int t = 0; t < kWideKT; ++t)
        tile_to_lds<false>(xsrc[u] + (step * kWideKT + t) * 512, dst + (u * kWideKT + t) * 1024);
  };
  lds_char* const lw = lds_launder(wring);
  lds_char* const lx = lds_launder(xring);
  f32x4 acc[WI][NB];
#pragma unroll
  for (int i = 0; i < WI; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Copy order: W(0), X(0), W(1), then after step s's barrier X(s + 1), W(s + 2).  At
  // the top of step s the wave's copies of X(s) and W(s) have landed once at most the
  // W(s + 1) batch that follows X(s) is in flight; the barrier then makes every wave's
  // copies visible and retires all reads of the slots refilled next (they held step
  // s - 1).
  issue_w(0);
  issue_x(0);
  if (nk > 1) issue_w(1);
  u32x4 A[WI][kWideKT], B[2][kWideKT];
  for (int s = 0; s < nk; ++s) {
    if (s + 1 < nk) vm_wait<kWideWCopies>();
    else vm_wait<0>();
    __builtin_amdgcn_s_barrier();
    if (s + 1 < nk) issue_x(s + 1);
    if (s + 2 < nk) issue_w(s + 2);
    const lds_char* sw = lw + (s % kWideWSlots) * kWideWBytes + lane * 16;
    const lds_char* sx = lx + (s % kWideXSlots) * kWideXBytes + lane * 16;
#pragma unroll
    for (int i = 0; i < WI; ++i)
#pragma unroll
      for (int t = 0; t < kWideKT; ++t) A[i][t] = ld16_lds(sw + ((wv * WI + i) * kWideKT + t) * 1024);
    auto readB = [&](int j) {
#pragma unroll
      for (int t = 0; t < kWideKT; ++t) B[j & 1][t] = ld16_lds(sx + (j * kWideKT + t) * 1024);
    };
    readB(0);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (j + 1 < NB) readB(j + 1);   // one token column ahead
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < WI; ++i) acc[i][j] = mfma16x2(A[i][0], B[j & 1][0], A[i][1], B[j & 1][1], acc[i][j]);
    }
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    f32x4 v[WI];
#pragma unroll
    for (int i = 0; i < WI; ++i) v[i] = acc[i][j];
    epilogue<EPI, WI>(a, rb0 + wv * WI, (tb0 + j) * 16 + r, v, g);
  }
}

template <int EPI>
static void run_wide(const DenseArgs& a, hipStream_t s, hipEvent_t done = nullptr) {
  static LdsLimit limit;   // the rings exceed the default dynamic-LDS limit
  raise_lds_limit(limit, reinterpret_cast<const void*>(&dense_wide_gemm<EPI>), kWideLds);
  const int n_row = (a.nblk + kWideRB - 1) / kWideRB, n_tok = (a.M + 16 * kWideTB - 1) / (16 * kWideTB);
  const int blocks = kXcd * ((n_row + kXcd - 1) / kXcd) * n_tok;
  launch_kernel(dense_wide_gemm<EPI>, dim3(blocks), dim3(256), kWideLds, s, done, a);
}

template <int WN, int WM, int EPI, int NW = 4>
static void run_dense(const DenseArgs& a, hipStream_t s, hipEvent_t done = nullptr) {
  const int n_tiles = (a.nblk + WN - 1) / WN, m_tiles = (a.M + 16 * WM - 1) / (16 * WM);
  const int blocks = kXcd * ((n_tiles + kXcd - 1) / kXcd) * m_tiles;
  const size_t lds = sizeof(f32x4) * NW * WN * WM * 64;
  // `done` (optional) is signalled by the kernel's own completion
  launch_kernel(dense_gemm<WN, WM, EPI, NW>, dim3(blocks), dim3(64 * NW), lds, s, done, a);
}

void launch_gemm_f32(const uint16_t* x, const uint16_t* w, float* y, int M, int N, int K,
                     bool add, hipStream_t s, hipEvent_t done) {
  DenseArgs a{};
  a.x = x; a.w = w; a.M = M; a.N = N; a.K = K;
  a.nblk = (N + 15) / 16;
  a.yf = y; a.ldy = N;
  // tile shapes measured at the 256-token canvas: narrow outputs (the router)
  // want many small workgroups, wide ones 64 x 64 tiles; passes of many rows take
  // the wide tile
  if (N > 256 && M >= kWideMinRows) {
    if (add)
      run_wide<EPI_ADD_F32>(a, s, done);
    else
      run_wide<EPI_STORE_F32>(a, s, done);
  } else if (add) {
    if (N <= 256)
      run_dense<1, 1, EPI_ADD_F32>(a, s, done);
    else
      run_dense<4, 4, EPI_ADD_F32>(a, s, done);
  } else {
    if (N <= 256)
      run_dense<1, 1, EPI_STORE_F32>(a, s, done);
    else
      run_dense<4, 4, EPI_STORE_F32>(a, s, done);
  }
}

void launch_qkv_rope(const uint16_t* h, const uint16_t* w_qkv, int M, int K, int hq,
                     const KvLayer& kv, const PassGeom& g, const float2* rope_tab,
                     uint16_t* q_out, hipStream_t s) {
  DenseArgs a{};
  a.x = h; a.w = w_qkv; a.M = M; a.K = K;
  a.N = (hq + 2 * kv.hkv) * kv.hd;
  a.nblk = a.N / 16;
  a.hq = hq; a.hd = kv.hd; a.kv = kv; a.g = g; a.rope = rope_tab; a.q_out = q_out;
  if (M >= kWideMinRows)
    run_wide<EPI_QKV>(a, s);
  else
    run_dense<4, 4, EPI_QKV>(a, s);
}

void launch_gemm_swiglu(const uint16_t* h, const uint16_t* w_gate_up, int M, int F, int K,
                        uint16_t* a_out, hipStream_t s) {
  DenseArgs a{};
  a.x = h; a.w = w_gate_up; a.M = M; a.K = K; a.N = 2 * F;
  a.nblk = 2 * (F / 16);
  a.yb = a_out; a.ldy = F;
  // 64-row weight tiles (two gate/up block pairs): one workgroup per CU at 348
  // registers per lane, which leaves room on every CU for the routing kernels and
  // the expert GEMMs that run beside this one (the 32-row tile at 232 registers put
  // two workgroups on each CU and took the registers those kernels need)
  if (M >= kWideMinRows)
    run_wide<EPI_SWIGLU>(a, s);
  else
    run_dense<4, 4, EPI_SWIGLU>(a, s);
}

// ---------------------------------------------------------------- LM head

// Tied LM head, logits[m][v] = h[m] . E[v] in bf16.  Workgroup tile: 256
// vocabulary rows x up to 256 tokens.  A full tile splits over the 4 waves as a
// 2 x 2 grid of 128 x 128 sub-tiles (8 x 8 MFMA blocks each, accumulators in
// AGPRs); a tile with fewer token rows to produce gives wave w vocabulary rows
// 64w .. 64w + 63 against its active token blocks (4 x 4, 8 or 12 MFMA blocks), so
// the MFMA work shrinks with the rows.  When the pass only needs the [MASK] rows
// (count given), h holds those *count rows compacted, and rows[] maps each
// compacted row to its logits row.  Operands are staged through LDS by direct
// global->LDS copies in 64-wide k steps (two 1 KiB fragment tiles per 16-row
// block).  The weight stream comes from HBM, so its ring
// is three steps deep (copies go out two steps ahead); the token tiles are L2 hits
// and ride a two-step ring one step ahead.  Weights are read from HBM exactly once
// and every token tile once per workgroup.  Each accumulator takes its two k tiles
// back to back (a dependent MFMA pair issues at the full rate).
constexpr int kHeadRB = 16;       // 16-row weight blocks per workgroup
constexpr int kHeadTB = 16;       // 16-token blocks per workgroup
constexpr int kHeadKT = 2;        // 32-wide k tiles per step
constexpr int kHeadWSlots = 3, kHeadXSlots = 2;
constexpr int kHeadWBytes = kHeadRB * kHeadKT * 1024;   // one step of weights
constexpr int kHeadXBytes = kHeadTB * kHeadKT * 1024;   // one step of token tiles
constexpr int kHeadLds = kHeadWSlots * kHeadWBytes + kHeadXSlots * kHeadXBytes;
constexpr int kHeadWCopies = kHeadRB * kHeadKT / 4;   // per wave per step
constexpr int kHeadXCopies = kHeadTB * kHeadKT / 4;

__global__ __launch_bounds__(256) void head_gemm(const uint16_t* __restrict__ x,
                                                 const uint16_t* __restrict__ w,
                                                 uint16_t* __restrict__ y, int M, int N, int K,
                                                 int w_blocks, int n_row_tiles, int n_tok_tiles,
                                                 const int32_t* __restrict__ count,
                                                 const int32_t* __restrict__ rows) {
  extern __shared__ __attribute__((aligned(1024))) char ring[];   // [W slots][X slots]
  constexpr int WI = kHeadRB / 4, WJ = kHeadTB;   // MFMA blocks per wave (rows x tokens)
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int b = blockIdx.x, xcd = b % kXcd, rank = b / kXcd;
  const int row_tile = (rank / n_tok_tiles) * kXcd + xcd, tok_tile = rank % n_tok_tiles;
  if (row_tile >= n_row_tiles) return;
  // rows to produce: all M, or the *count [MASK] rows compacted in h
  const int Mc = count ? __builtin_amdgcn_readfirstlane(*count) : M;
  const int rb0 = row_tile * kHeadRB, tb0 = tok_tile * kHeadTB;
  if (tb0 * 16 >= Mc) return;                        // uniform per workgroup
  const int nb = min(kHeadTB, (Mc - tb0 * 16 + 15) >> 4);   // active token blocks of the tile
  const int nk = K / (32 * kHeadKT);

  // copy duty: wave wv copies weight blocks and token blocks wv * (RB / 4) + u;
  // in a slot, block q's k tiles sit at (q * kHeadKT + t) KiB
  constexpr int WB = kHeadRB / 4, XB = kHeadTB / 4;
  const uint16_t* wsrc[WB];
  const uint16_t* xsrc[XB];
#pragma unroll
  for (int u = 0; u < WB; ++u) wsrc[u] = w + fm_tile(min(rb0 + wv * WB + u, w_blocks - 1), 0, K, lane);
  // token blocks past the active ones re-read the last active block (their rows are never used)
#pragma unroll
  for (int u = 0; u < XB; ++u) xsrc[u] = x + fm_tile(tb0 + min(wv * XB + u, nb - 1), 0, K, lane);
  char* const wring = ring;
  char* const xring = ring + kHeadWSlots * kHeadWBytes;
  auto issue_w = [&](int step) {
    char* dst = wring + (step % kHeadWSlots) * kHeadWBytes + wv * WB * kHeadKT * 1024;
#pragma unroll
    for (int u = 0; u < WB; ++u)
#pragma unroll
      for (int t = 0; t < kHeadKT; ++t)
        tile_to_lds<true>(wsrc[u] + (step * kHeadKT + t) * 512, dst + (u * kHeadKT + t) * 1024);
  };
  auto issue_x = [&](int step) {
    char* dst = xring + (step % kHeadXSlots) * kHeadXBytes + wv * XB * kHeadKT * 1024;
#pragma unroll
    for (int u = 0; u < XB; ++u)
#pragma unroll
      for (int t = 0; t < kHeadKT; ++t)
        tile_to_lds<false>(xsrc[u] + (step * kHeadKT + t) * 512, dst + (u * kHeadKT + t) * 1024);
  };

  lds_char* const lw = lds_launder(wring);
  lds_char* const lx = lds_launder(xring);
  // the tile's token-block count, rounded up to a multiple of 4, is a compile-time
  // loop bound: blocks past nb repeat the last active block and are dropped
  auto run = [&](auto nbt) {
    constexpr int NB = decltype(nbt)::value;
    int orow[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int mc = (tb0 + j) * 16 + r;
      orow[j] = (j < nb && mc < Mc) ? (rows ? rows[mc] : mc) : -1;
    }
    f32x4 acc[WI][NB];
#pragma unroll
    for (int i = 0; i < WI; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Copy order: W(0), X(0), W(1), then after step s's barrier X(s + 1), W(s + 2).
    // At the top of step s the wave's copies of X(s) and W(s) have landed once at
    // most the W(s + 1) batch that follows X(s) is in flight; the barrier then makes
    // all waves' copies visible and retires every read of the slots refilled next
    // (they held step s - 1).
    issue_w(0);
    issue_x(0);
    if (nk > 1) issue_w(1);
    u32x4 A[WI][kHeadKT], B[2][kHeadKT];
    static_assert(kHeadKT == 2, "MFMA pairs");
    for (int s = 0; s < nk; ++s) {
      if (s + 1 < nk) vm_wait<kHeadWCopies>();
      else vm_wait<0>();
      __builtin_amdgcn_s_barrier();
      if (s + 1 < nk) issue_x(s + 1);
      if (s + 2 < nk) issue_w(s + 2);
      const lds_char* sw = lw + (s % kHeadWSlots) * kHeadWBytes + lane * 16;
      const lds_char* sx = lx + (s % kHeadXSlots) * kHeadXBytes + lane * 16;
#pragma unroll
      for (int i = 0; i < WI; ++i)
#pragma unroll
        for (int t = 0; t < kHeadKT; ++t) A[i][t] = ld16_lds(sw + ((wv * WI + i) * kHeadKT + t) * 1024);
      auto readB = [&](int j) {
#pragma unroll
        for (int t = 0; t < kHeadKT; ++t) B[j & 1][t] = ld16_lds(sx + (j * kHeadKT + t) * 1024);
      };
      readB(0);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (j + 1 < NB) readB(j + 1);   // one token column ahead
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < WI; ++i)
          acc[i][j] = mfma16x2(A[i][0], B[j & 1][0], A[i][1], B[j & 1][1], acc[i][j]);
      }
    }

#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (orow[j] < 0) continue;
      const size_t m = (size_t)orow[j];
#pragma unroll
      for (int i = 0; i < WI; ++i) {
        const int n0 = (rb0 + wv * WI + i) * 16 + 4 * g;
        if (n0 >= N) continue;   // N is a multiple of 8, so n0 < N covers n0 .. n0 + 3
        u32x2 o;
        o.x = pack_bf2(acc[i][j][0], acc[i][j][1]);
        o.y = pack_bf2(acc[i][j][2], acc[i][j][3]);
        *reinterpret_cast<u32x2*>(y + m * N + n0) = o;
      }
    }
  };
  // A full tile (16 token blocks) takes the 2 x 2 grid of 128 x 128 wave tiles
  // instead: each fragment read from LDS then feeds 8 MFMA blocks, not 4 or 16.
  auto run_full = [&]() {
    constexpr int FI = kHeadRB / 2, FJ = kHeadTB / 2;
    const int wr = wv & 1, wt = wv >> 1;
    // logits rows of this lane's tokens, loaded before the k loop hides their latency
    int orow[FJ];
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const int mc = (tb0 + wt * FJ + j) * 16 + r;
      orow[j] = mc < Mc ? (rows ? rows[mc] : mc) : -1;
    }
    f32x4 acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    issue_w(0);
    issue_x(0);
    if (nk > 1) issue_w(1);
    u32x4 A[FI][kHeadKT], B[2][kHeadKT];
    for (int s = 0; s < nk; ++s) {
      if (s + 1 < nk) vm_wait<kHeadWCopies>();
      else vm_wait<0>();
      __builtin_amdgcn_s_barrier();
      if (s + 1 < nk) issue_x(s + 1);
      if (s + 2 < nk) issue_w(s + 2);
      const lds_char* sw = lw + (s % kHeadWSlots) * kHeadWBytes + lane * 16;
      const lds_char* sx = lx + (s % kHeadXSlots) * kHeadXBytes + lane * 16;
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int t = 0; t < kHeadKT; ++t) A[i][t] = ld16_lds(sw + ((wr * FI + i) * kHeadKT + t) * 1024);
      auto readB = [&](int j) {
#pragma unroll
        for (int t = 0; t < kHeadKT; ++t) B[j & 1][t] = ld16_lds(sx + ((wt * FJ + j) * kHeadKT + t) * 1024);
      };
      readB(0);
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        if (j + 1 < FJ) readB(j + 1);   // one token column ahead
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < FI; ++i)
          acc[i][j] = mfma16x2(A[i][0], B[j & 1][0], A[i][1], B[j & 1][1], acc[i][j]);
      }
    }
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      if (orow[j] < 0) continue;
      const size_t m = (size_t)orow[j];
#pragma unroll
      for (int i = 0; i < FI; ++i) {
        const int n0 = (rb0 + wr * FI + i) * 16 + 4 * g;
        if (n0 >= N) continue;
        u32x2 o;
        o.x = pack_bf2(acc[i][j][0], acc[i][j][1]);
        o.y = pack_bf2(acc[i][j][2], acc[i][j][3]);
        *reinterpret_cast<u32x2*>(y + m * N + n0) = o;
      }
    }
  };
  static_assert(WJ == 16, "token-block classes");
  if (nb <= 4) run(std::integral_constant<int, 4>{});
  else if (nb <= 8) run(std::integral_constant<int, 8>{});
  else if (nb <= 12) run(std::integral_constant<int, 12>{});
  else run_full();
}

void launch_gemm_head(const uint16_t* h, const uint16_t* embed, uint16_t* logits, int M, int N,
                      int K, const int32_t* count, const int32_t* rows, hipStream_t s) {
  constexpr size_t lds = (size_t)kHeadLds;
  static LdsLimit limit;   // the ring exceeds the default dynamic-LDS limit
  raise_lds_limit(limit, reinterpret_cast<const void*>(&head_gemm), (int)lds);
  const int w_blocks = (N + 1 + 15) / 16;   // packed embedding rows: vocab + mask token, padded
  const int n_row = (N + 16 * kHeadRB - 1) / (16 * kHeadRB);
  const int n_tok = (M + 16 * kHeadTB - 1) / (16 * kHeadTB);
  const int blocks = kXcd * ((n_row + kXcd - 1) / kXcd) * n_tok;
  launch_kernel(head_gemm, dim3(blocks), dim3(256), lds, s, nullptr, h, embed, logits, M, N, K, w_blocks,
                n_row, n_tok, count, rows);
}

}  // namespace dg
