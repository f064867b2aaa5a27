// Flash-style attention over the KV cache for both masks of the method:
//  * denoise (bidirectional decoder): every canvas query of sequence b sees the
//    cached keys [lo, len_b) — lo = max(0, len_b - W) on sliding layers, 0 on
//    global ones — plus all canvas keys [len_b, len_b + n);
//  * encoder (prefill / append): query at position p sees keys (p - W, p] on
//    sliding layers, [0, p] on global ones.
// The projection kernel has already written this pass's keys/values into the
// cache at positions len_b .., so every key lives in one contiguous range.
// q, the key cache and the (transposed) value cache are stored in fragment
// tiles, so each operand fragment below is one contiguous 1 KiB wave load.
//
// Work split: a workgroup owns 16 queries of one q head; its NW waves (8; 4 at
// hd 32) take interleaved 32-key chunks of the key range (split-KV) and merge
// their (max, sum, output) partials through LDS in a fixed order.
//
// Layout trick: scores are computed transposed, S^T = K . Q^T, with the key
// rows of each 16-row MFMA block permuted so that a lane ends up holding the
// scores of 8 consecutive keys (8g .. 8g+7 of the chunk) for its query.  Those
// 8 probabilities are exactly the lane's B fragment for O^T += V^T . P^T, and
// V is stored transposed in tiles of 32 keys x 16 hd rows, so the A fragment
// is one 16-byte slot of a contiguous 1 KiB tile.  Softmax state and output rescaling are lane-local (the lane's
// output rows all belong to its query); only the chunk max needs two shuffles.
#include <math.h>

#include "dg_common.h"
#include "dg_internal.h"

namespace dg {


template <int HD, int NW>
__global__ __launch_bounds__(64 * NW) void attention_kernel(const uint16_t* __restrict__ q, int hq,
                                                            KvLayer kv, PassGeom g,
                                                            uint16_t* __restrict__ o) {
  constexpr int NC = HD / 32;   // k-steps of the score MFMA
  constexpr int NB = HD / 16;   // output blocks of 16 hd rows
  __shared__ float Ol[NW][16][HD + 4];
  __shared__ float ml[NW][16][2];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, gq = lane >> 4;
  // XCD-aware order: block bid runs on XCD bid % 8; every workgroup of one
  // (sequence, kv head) pair -- its q heads x query tiles -- runs on the same XCD,
  // so that pair's keys and values leave HBM once
  const int grp = hq / kv.hkv, q_tiles = (g.n + 15) / 16, per_pair = grp * q_tiles;
  const int rank = blockIdx.x / kXcd;
  const int pair = (rank / per_pair) * kXcd + (int)(blockIdx.x % kXcd);
  if (pair >= g.batch * kv.hkv) return;   // uniform per workgroup
  const int b = pair / kv.hkv, kvh = pair - b * kv.hkv;
  const int rem = rank % per_pair;
  const int head = kvh * grp + rem / q_tiles;
  const int i0 = (rem % q_tiles) * 16;
  const int n = g.n, len = g.len[b];
  const float scale = 1.4426950408889634f / sqrtf((float)HD);

  // query fragments: q is fragment-major per (sequence, head), [n_pad][HD]
  const int qi = min(i0 + r, n - 1);
  const int npad = (n + 15) & ~15;
  const uint16_t* qbase = q + ((size_t)b * hq + head) * (size_t)npad * HD;
  u32x4 qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) qf[c] = ld16(qbase + fm_tile(i0 >> 4, c, HD, lane));

  // key range of this lane's query and of the whole 16-query tile
  int lo_q, hi_q, lo_t, hi_t;
  if (g.denoise) {
    lo_q = kv.window > 0 ? max(0, len - kv.window) : 0;
    hi_q = len + n;
    lo_t = lo_q;
    hi_t = hi_q;
  } else {
    const int p = len + qi;
    lo_q = kv.window > 0 ? max(0, p - kv.window + 1) : 0;
    hi_q = p + 1;
    const int pf = len + i0, pl = len + min(i0 + 15, n - 1);
    lo_t = kv.window > 0 ? max(0, pf - kv.window + 1) : 0;
    hi_t = pl + 1;
  }
  const int kc0 = lo_t & ~31;
  const int nchunk = (hi_t - kc0 + 31) >> 5;

  const uint16_t* kbase = kv.k + ((size_t)b * kv.hkv + kvh) * (size_t)kv.max_ctx * HD;
  const uint16_t* vbase = kv.vt + ((size_t)b * kv.hkv + kvh) * (size_t)HD * kv.max_ctx;

  f32x4 acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;

  // One 32-key chunk: K fragments (2 blocks x NC k tiles) and V fragments (NB
  // hd blocks), prefetched one chunk ahead through a two-stage pipeline.
  u32x4 Ka[2][NC], Va[NB], Kb[2][NC], Vb[NB];
  int kca = 0, kcb = 0;
  auto load = [&](u32x4 (&K)[2][NC], u32x4 (&Vt)[NB], int& kcs, int step) {
    kcs = kc0 + 32 * (w + NW * step);
    const uint16_t* kp = kbase + ((size_t)(kcs >> 5) * 2 * NC << 9) + 8 * lane;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int c = 0; c < NC; ++c) K[bb][c] = ld16(kp + ((bb * NC + c) << 9));
    const uint16_t* vp = vbase + ((size_t)(kcs >> 5) * NB << 9) + 8 * lane;
#pragma unroll
    for (int hb = 0; hb < NB; ++hb) Vt[hb] = ld16(vp + (hb << 9));
  };
  auto process = [&](const u32x4 (&K)[2][NC], const u32x4 (&Vt)[NB], int kc) {
    // S^T blocks: block bb row rr <-> key kc + 8*(rr>>2) + 4*bb + (rr&3)
    f32x4 s[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) a = mfma16(K[bb][c], qf[c], a);
      s[bb] = a;
    }
    // lane holds keys kc + 8*gq + e (e = 0..7) for query r
    float sv[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = kc + 8 * gq + e;
      const float v = s[e >> 2][e & 3] * scale;
      sv[e] = (key >= lo_q && key < hi_q) ? v : -INFINITY;
      cmax = fmaxf(cmax, sv[e]);
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
    float p[8];
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = (sv[e] == -INFINITY) ? 0.f : exp2f(sv[e] - m_new);
      ps += p[e];
    }
    l_part = l_part * alpha + ps;
    m_run = m_new;
    // P enters the bf16 PV product as a pair: hi = bf16(P), lo = bf16(P - hi), so the
    // product carries P to ~2^-17 relative (a single bf16 P would add a 2^-9 error to every
    // probability, which near-uniform attention does not average away)
    u32x4 pb, pl;
    {
      float lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) lo[e] = p[e] - bf2f(f2bf(p[e]));
      pb.x = pack_bf2(p[0], p[1]);
      pb.y = pack_bf2(p[2], p[3]);
      pb.z = pack_bf2(p[4], p[5]);
      pb.w = pack_bf2(p[6], p[7]);
      pl.x = pack_bf2(lo[0], lo[1]);
      pl.y = pack_bf2(lo[2], lo[3]);
      pl.z = pack_bf2(lo[4], lo[5]);
      pl.w = pack_bf2(lo[6], lo[7]);
    }
#pragma unroll
    for (int hb = 0; hb < NB; ++hb) {
      acc[hb] *= alpha;
      acc[hb] = mfma16(Vt[hb], pb, acc[hb]);
      acc[hb] = mfma16(Vt[hb], pl, acc[hb]);
    }
  };
  const int nsteps = w < nchunk ? (nchunk - w + NW - 1) / NW : 0;
  pipeline2(nsteps, [&](int t) { load(Ka, Va, kca, t); }, [&](int t) { load(Kb, Vb, kcb, t); },
            [&] { process(Ka, Va, kca); }, [&] { process(Kb, Vb, kcb); });

  float l_row = l_part + __shfl_xor(l_part, 16, 64);
  l_row += __shfl_xor(l_row, 32, 64);
#pragma unroll
  for (int hb = 0; hb < NB; ++hb)
#pragma unroll
    for (int e = 0; e < 4; ++e) Ol[w][r][16 * hb + 4 * gq + e] = acc[hb][e];
  if (gq == 0) {
    ml[w][r][0] = m_run;
    ml[w][r][1] = l_row;
  }
  __syncthreads();

  // merge the NW waves: thread t -> query t / TPQ, hd slice (t % TPQ) * HD / TPQ
  constexpr int TPQ = 4 * NW;                 // threads per query (64 * NW / 16)
  constexpr int CPT = HD / TPQ;               // hd columns per thread
  static_assert(CPT >= 2 && CPT % 2 == 0, "bf16 pairs per thread");
  const int qq = threadIdx.x / TPQ;
  const int d0 = (threadIdx.x % TPQ) * CPT;
  float M = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, ml[ww][qq][0]);
  float sc[NW];
  float L = 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    const float mw = ml[ww][qq][0];
    sc[ww] = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
    L += sc[ww] * ml[ww][qq][1];
  }
  const float invL = L > 0.f ? 1.f / L : 0.f;
  const int iq = i0 + qq;
  if (iq < n) {
    // o is fragment-major [M_pad][hq * HD] (the O projection's activation operand)
    const size_t m = (size_t)b * n + iq;
    const int K = hq * HD;
#pragma unroll
    for (int e = 0; e < CPT; e += 2) {
      float v0 = 0.f, v1 = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        v0 += sc[ww] * Ol[ww][qq][d0 + e];
        v1 += sc[ww] * Ol[ww][qq][d0 + e + 1];
      }
      *reinterpret_cast<uint32_t*>(o + fm_index(m, head * HD + d0 + e, K)) = pack_bf2(v0 * invL, v1 * invL);
    }
  }
}

void launch_attention(const uint16_t* q, int hq, const KvLayer& kv, const PassGeom& g,
                      uint16_t* o, hipStream_t s) {
  const int pairs = g.batch * kv.hkv, per_pair = (hq / kv.hkv) * ((g.n + 15) / 16);
  dim3 grid(kXcd * ((pairs + kXcd - 1) / kXcd) * per_pair);
  // 8 waves split the key range (4 for hd 32, where the merge runs out of columns)
  switch (kv.hd) {
    case 32: launch_kernel(attention_kernel<32, 4>, grid, dim3(256), 0, s, nullptr, q, hq, kv, g, o); break;
    case 64: launch_kernel(attention_kernel<64, 8>, grid, dim3(512), 0, s, nullptr, q, hq, kv, g, o); break;
    default: launch_kernel(attention_kernel<128, 8>, grid, dim3(512), 0, s, nullptr, q, hq, kv, g, o); break;
  }
}

}  // namespace dg
