// Flash-style attention over the KV cache for both masks of the method:
//  * denoise (bidirectional decoder): every canvas query of sequence b sees the
//    cached keys [lo, len_b) — lo = max(0, len_b - W) on sliding layers, 0 on
//    global ones — plus all canvas keys [len_b, len_b + n);
//  * encoder (prefill / append): query at position p sees keys (p - W, p] on
//    sliding layers, [0, p] on global ones.
// The projection kernel has already written this pass's keys/values into the
// cache at positions len_b .., so every key lives in one contiguous range.
//
// Work split.  A workgroup serves one (sequence, kv head) pair: NWV waves, each
// owning 32 query rows (two 16-row MFMA blocks) of one q head of the pair's GQA
// group (4 waves: both q heads of a group, 64 queries of each; 8 waves for long key
// ranges).  Keys stream through LDS in 64-key stages (K and transposed V, copied
// straight from the cache's fragment tiles into a RING-stage ring by direct
// global->LDS loads, one copy per workgroup) and every wave reads each stage: one
// K/V byte from L2 feeds 32 * NWV query rows.  Over long key ranges the loop is
// pipelined: each iteration issues the next stage's score MFMAs before this stage's
// softmax, so the matrix cores work while the VALU computes the exponentials (the same
// arithmetic in the same order, so the same results).  When the pairs alone give too few workgroups to
// fill the chip, the key range of each pair is split over several workgroups
// (split-KV); each writes its unnormalised partial (max, sum, output) and a merge
// kernel combines the splits in a fixed order.
//
// Layout trick (kept from the cache format): scores are computed transposed,
// S^T = K . Q^T, with the key rows of each 16-row block permuted so that a lane
// holds the scores of 8 consecutive keys for its query -- exactly the lane's B
// fragment for O^T += V^T . P^T, with V stored transposed in 32-key x 16-hd tiles.
// Softmax state and output rescaling are lane-local; the stage max needs two
// shuffles.  P enters the bf16 PV product as a pair hi = bf16(P), lo = bf16(P - hi)
// (~2^-17 relative), because near-uniform attention does not average a single
// bf16 rounding of P away.
#include <math.h>

#include "dg_common.h"
#include "dg_internal.h"

namespace dg {

struct AttnArgs {
  const uint16_t* q;      // fragment-major per (sequence, q head): [npad16][HD]
  uint16_t* o;            // fragment-major [M_pad][hq * HD] (written when nsplit == 1)
  float* part_o;          // [nsplit][batch][hq][npad32][HD] unnormalised partial outputs
  float2* part_ml;        // [nsplit][batch][hq][npad32] (max in log2 units, sum)
  KvLayer kv;
  PassGeom g;
  int hq;
  int grp;                // q heads per kv head
  int qt32;               // 32-query tiles per head: ceil(n / 32)
  int wg_per_pair;        // ceil(grp * qt32 / NWV)
  int nsplit;
};

constexpr int kAttnStageKeys = 64;

template <int HD, int NWV, int RING, bool PIPE = false>
__global__ __launch_bounds__(64 * NWV, 8 / NWV) void attention_kernel(AttnArgs a) {
  constexpr int NC = HD / 32;                 // k-steps of the score MFMA
  constexpr int NB = HD / 16;                 // 16-row output blocks of hd
  constexpr int KCH = 2 * NC * 1024;          // bytes of one 32-key K chunk (2 key blocks x NC tiles)
  constexpr int VCH = NB * 1024;              // bytes of one 32-key transposed-V chunk
  constexpr int STAGE = 2 * (KCH + VCH);      // one 64-key stage: K chunk 0, K chunk 1, V chunk 0, V chunk 1
  constexpr int COPIES = STAGE / 1024 / NWV;  // 1 KiB copies per wave per stage
  static_assert(STAGE % (1024 * NWV) == 0, "whole copies per wave");
  static_assert(RING == 2 || RING == 3 || (PIPE && RING == 4), "stages in the ring");
  extern __shared__ __attribute__((aligned(1024))) char ring[];   // [RING][STAGE]

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, gq = lane >> 4;
  const PassGeom& g = a.g;
  const KvLayer& kv = a.kv;

  // unit -> (pair, workgroup of the pair, split); XCD x owns a contiguous range of the
  // units, so all workgroups of one pair share an XCD's L2 copy of its keys and values
  int unit;
  {
    const int x = blockIdx.x % kXcd, rank = blockIdx.x / kXcd;
    const long T = (long)g.batch * kv.hkv * a.wg_per_pair * a.nsplit;
    const long u0 = (long)x * T / kXcd, u1 = (long)(x + 1) * T / kXcd;
    if (rank >= u1 - u0) return;              // uniform per workgroup
    unit = (int)(u0 + rank);
  }
  const int split = unit % a.nsplit;
  const int wgp = (unit / a.nsplit) % a.wg_per_pair;
  const int pair = unit / (a.nsplit * a.wg_per_pair);
  const int b = pair / kv.hkv, kvh = pair - b * kv.hkv;
  const int n = g.n, len = g.len[b];
  const bool den = !seq_encodes(g, b);        // this sequence denoises (else: causal encoder)
  const int ngroups = a.grp * a.qt32;
  const int rg0 = wgp * NWV;
  const int rg = rg0 + w;
  const bool active = rg < ngroups;
  const int head = kvh * a.grp + (active ? rg / a.qt32 : 0);
  const int q0 = active ? (rg % a.qt32) * 32 : 0;

  // key range of the workgroup (the union over its waves' queries), in 64-key stages
  int lo_t, hi_t;
  if (den) {
    lo_t = kv.window > 0 ? max(0, len - kv.window) : 0;
    hi_t = len + n;
  } else {
    int qmin = n, qmax = -1;
    for (int j = 0; j < NWV && rg0 + j < ngroups; ++j) {
      const int qq = ((rg0 + j) % a.qt32) * 32;
      qmin = min(qmin, qq);
      qmax = max(qmax, min(qq + 31, n - 1));
    }
    lo_t = kv.window > 0 ? max(0, len + qmin - kv.window + 1) : 0;
    hi_t = len + qmax + 1;
  }
  const int st0 = lo_t / kAttnStageKeys;
  const int nst = (hi_t - st0 * kAttnStageKeys + kAttnStageKeys - 1) / kAttnStageKeys;
  const int s_begin = st0 + (int)((long)nst * split / a.nsplit);
  const int s_end = st0 + (int)((long)nst * (split + 1) / a.nsplit);

  // this lane's two queries (blocks qb = 0, 1: queries q0 + 16 qb + r) and their fragments
  const int npad16 = (n + 15) & ~15;
  const uint16_t* qbase = a.q + ((size_t)b * a.hq + head) * (size_t)npad16 * HD;
  u32x4 qf[2][NC];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int blk = min((q0 >> 4) + qb, (n - 1) >> 4);     // padded rows read the last block
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[qb][c] = ld16(qbase + fm_tile(blk, c, HD, lane));
  }
  int lo_q[2], hi_q[2];                       // visible key range of each of the lane's queries
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (den) {
      lo_q[qb] = lo_t;
      hi_q[qb] = hi_t;
    } else {
      const int p = len + q0 + 16 * qb + r;
      lo_q[qb] = kv.window > 0 ? max(0, p - kv.window + 1) : 0;
      hi_q[qb] = p + 1;
    }
  }
  // the wave's whole 32-query range, for deciding which stages need no mask at all
  const int p_first = len + q0, p_last = len + min(q0 + 31, n - 1);

  const uint16_t* kbase = kv.k + ((size_t)kv_seq(g, b) * kv.hkv + kvh) * (size_t)kv.max_ctx * HD;
  const uint16_t* vbase = kv.vt + ((size_t)kv_seq(g, b) * kv.hkv + kvh) * (size_t)HD * kv.max_ctx;
  // stage st: K chunks 2 st, 2 st + 1 (contiguous), then V chunks 2 st, 2 st + 1
  auto issue = [&](int st, int slot) {
    char* dst = ring + slot * STAGE;
    const uint16_t* ks = kbase + (size_t)(2 * st) * (KCH / 2);
    const uint16_t* vs = vbase + (size_t)(2 * st) * (VCH / 2);
#pragma unroll
    for (int c = 0; c < COPIES; ++c) {
      const int t = w * COPIES + c;           // 1 KiB tile index within the stage
      const uint16_t* src = t < 2 * KCH / 1024 ? ks + t * 512 : vs + (t - 2 * KCH / 1024) * 512;
      tile_to_lds<false>(src + 8 * lane, dst + t * 1024);
    }
  };

  f32x4 acc[2][NB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int i = 0; i < NB; ++i) acc[qb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_part[2] = {0.f, 0.f};
  const float scale = 1.4426950408889634f / sqrtf((float)HD);   // softmax in log2 units
  lds_char* const lr = lds_launder(ring);

  // one stage's scores S^T = K . Q^T of both 32-key chunks for both query blocks
  // (s[qb][chunk][bb]), then its online softmax and the P.V product; the two steps are
  // separate so that the pipelined loop can issue the next stage's score MFMAs before
  // this stage's softmax (the matrix cores work while the VALU runs the softmax)
  auto scores = [&](int st, f32x4 (&s)[2][2][2]) {
    const lds_char* sk = lr + ((st - s_begin) % RING) * STAGE + lane * 16;
    // scores of both 32-key chunks for both query blocks: s[qb][chunk][bb]
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        u32x4 kf[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) kf[c] = ld16_lds(sk + ch * KCH + ((bb * NC + c) << 10));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NC; ++c) t = mfma16(kf[c], qf[qb][c], t);
          s[qb][ch][bb] = t;
        }
      }
  };
  auto softmax_pv = [&](int st, f32x4 (&s)[2][2][2]) {
    const lds_char* sv = lr + ((st - s_begin) % RING) * STAGE + lane * 16 + 2 * KCH;
    const int kc0 = st * kAttnStageKeys;
    // lane holds keys kc0 + 32 ch + 8 gq + e (e = 0..7: bb = e / 4, row e % 4) for query r
    const bool nomask = den ? (kc0 >= lo_t && kc0 + kAttnStageKeys <= hi_t)
                                  : (kc0 + kAttnStageKeys - 1 <= p_first &&
                                     (kv.window == 0 || p_last - kc0 < kv.window));
    u32x4 ph[2][2], pl[2][2];
    float alpha[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float sv16[16];
      float cmax = -INFINITY;
#pragma unroll
      for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = s[qb][ch][e >> 2][e & 3] * scale;
          const int key = kc0 + 32 * ch + 8 * gq + e;
          // branch-free: a select per key, no short-circuit control flow
          const bool vis = nomask | ((key >= lo_q[qb]) & (key < hi_q[qb]));
          const float x = vis ? v : -INFINITY;
          sv16[8 * ch + e] = x;
          cmax = fmaxf(cmax, x);
        }
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
      const float m_new = fmaxf(m_run[qb], cmax);
      // v_exp_f32 directly (results below 2^-126 flush to zero; exp2(-inf) = 0, so a
      // masked key needs no select once the subtracted max is finite)
      const float m_sub = (m_new == -INFINITY) ? 0.f : m_new;
      alpha[qb] = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
      float p[16];
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = __builtin_amdgcn_exp2f(sv16[e] - m_sub);
        ps += p[e];
      }
      l_part[qb] = l_part[qb] * alpha[qb] + ps;
      m_run[qb] = m_new;
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x0 = p[8 * ch + 2 * j], x1 = p[8 * ch + 2 * j + 1];
          hi[j] = cvt_pk_bf16(x0, x1);
          lo[j] = cvt_pk_bf16(x0 - __uint_as_float(hi[j] << 16), x1 - __uint_as_float(hi[j] & 0xffff0000u));
        }
        ph[qb][ch] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        pl[qb][ch] = u32x4{lo[0], lo[1], lo[2], lo[3]};
      }
    }
    // rescale the outputs only when some lane's running max moved
    if (__builtin_amdgcn_ballot_w64(alpha[0] != 1.f || alpha[1] != 1.f)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int hb = 0; hb < NB; ++hb) acc[qb][hb] *= alpha[qb];
    }
#pragma unroll
    for (int hb = 0; hb < NB; ++hb) {
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        const u32x4 vf = ld16_lds(sv + ch * VCH + (hb << 10));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          acc[qb][hb] = mfma16(vf, ph[qb][ch], acc[qb][hb]);
          acc[qb][hb] = mfma16(vf, pl[qb][ch], acc[qb][hb]);
        }
      }
    }
  };

  if constexpr (!PIPE) {
    // RING - 1 stages in flight: stage st is copied RING - 1 iterations ahead of its use.
    // At the top of iteration st the wave's later copies are those of the stages after
    // st already issued (at most RING - 2 of them); waiting until only they remain lands
    // stage st, and the barrier makes every wave's copies visible and retires all reads
    // of the slot refilled next (stage st - 1's).
#pragma unroll
    for (int j = 0; j < RING - 1; ++j)
      if (s_begin + j < s_end) issue(s_begin + j, j);
    for (int st = s_begin; st < s_end; ++st) {
      if (RING == 3 && st + 1 < s_end) vm_wait<COPIES>();
      else vm_wait<0>();
      __builtin_amdgcn_s_barrier();
      if (st + RING - 1 < s_end) issue(st + RING - 1, (st + RING - 1 - s_begin) % RING);
      if (!active) continue;
      f32x4 sc[2][2][2];
      scores(st, sc);
      softmax_pv(st, sc);
    }
  } else {
    // Pipelined: iteration st computes stage st + 1's scores, then stage st's softmax and
    // P.V.  Four slots: stage st + 3 is copied in iteration st into the slot of stage
    // st - 1, whose K (scores in iteration st - 2) and V (iteration st - 1) every wave has
    // finished with at the barrier.  At the top of iteration st stage st + 1 must have
    // landed: the only later copies are stage st + 2's (issued in iteration st - 1).
    static_assert(RING == 4, "the pipelined loop keeps two stages ahead in four slots");
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (s_begin + j < s_end) issue(s_begin + j, j);
    if (s_begin + 2 < s_end) vm_wait<2 * COPIES>();
    else if (s_begin + 1 < s_end) vm_wait<COPIES>();
    else vm_wait<0>();
    __builtin_amdgcn_s_barrier();
    f32x4 sa[2][2][2], sb[2][2][2];
    if (active && s_begin < s_end) scores(s_begin, sa);
    for (int st = s_begin; st < s_end; ++st) {
      if (st + 2 < s_end) vm_wait<COPIES>();
      else vm_wait<0>();
      __builtin_amdgcn_s_barrier();
      if (st + 3 < s_end) issue(st + 3, (st + 3 - s_begin) % RING);
      if (!active) continue;
      if (st + 1 < s_end) scores(st + 1, sb);
      softmax_pv(st, sa);
#pragma unroll
      for (int i = 0; i < 8; ++i) (&sa[0][0][0])[i] = (&sb[0][0][0])[i];
    }
  }
  if (!active) return;

  // each lane's query: the four lanes of a query (gq = 0..3) hold disjoint keys' sums
  const int npad32 = a.qt32 * 32;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l_row = l_part[qb] + __shfl_xor(l_part[qb], 16, 64);
    l_row += __shfl_xor(l_row, 32, 64);
    const int iq = q0 + 16 * qb + r;
    if (a.nsplit == 1) {
      if (iq >= n) continue;
      const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
      const size_t m = (size_t)b * n + iq;
      const int K = a.hq * HD;
#pragma unroll
      for (int hb = 0; hb < NB; ++hb) {
        const int c = head * HD + 16 * hb + 4 * gq;
        u32x2 o2;
        o2.x = cvt_pk_bf16(acc[qb][hb][0] * inv, acc[qb][hb][1] * inv);
        o2.y = cvt_pk_bf16(acc[qb][hb][2] * inv, acc[qb][hb][3] * inv);
        *reinterpret_cast<u32x2*>(a.o + fm_index(m, c, K)) = o2;
      }
    } else {
      const size_t row = (((size_t)split * g.batch + b) * a.hq + head) * npad32 + iq;
      if (gq == 0) a.part_ml[row] = make_float2(m_run[qb], l_row);
#pragma unroll
      for (int hb = 0; hb < NB; ++hb)
        *reinterpret_cast<f32x4*>(a.part_o + row * HD + 16 * hb + 4 * gq) = acc[qb][hb];
    }
  }
}

// Merge of the split-KV partials: one thread per 8 output features of one (sequence,
// head, query); the splits are combined in split order.  Every load a thread needs is
// issued before the first is used (the split count is bounded by kAttnMaxSplits and the
// loops are unrolled over that bound), so the merge costs about one memory round trip
// rather than one per split.
constexpr int kAttnMaxSplits = 16;

template <int HD>
__global__ __launch_bounds__(256) void attention_merge_kernel(const float* __restrict__ part_o,
                                                              const float2* __restrict__ part_ml, int nsplit,
                                                              int batch, int hq, int n, int npad32,
                                                              uint16_t* __restrict__ o) {
  constexpr int TPR = HD / 8;
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long rows = (long)batch * hq * n;
  if (t >= rows * TPR) return;
  const int c8 = (int)(t % TPR) * 8;
  long rr = t / TPR;
  const int iq = (int)(rr % n);
  rr /= n;
  const int head = (int)(rr % hq), b = (int)(rr / hq);
  const size_t base = ((size_t)b * hq + head) * npad32 + iq;
  const size_t stride = (size_t)batch * hq * npad32;
  float2 ml[kAttnMaxSplits];
  f32x4 v0[kAttnMaxSplits], v1[kAttnMaxSplits];
#pragma unroll
  for (int s = 0; s < kAttnMaxSplits; ++s) {
    if (s < nsplit) {
      ml[s] = part_ml[s * stride + base];
      const float* po = part_o + (s * stride + base) * HD + c8;
      v0[s] = *reinterpret_cast<const f32x4*>(po);
      v1[s] = *reinterpret_cast<const f32x4*>(po + 4);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kAttnMaxSplits; ++s)
    if (s < nsplit) M = fmaxf(M, ml[s].x);
  float L = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kAttnMaxSplits; ++s) {
    if (s >= nsplit || ml[s].x == -INFINITY) continue;
    const float f = exp2f(ml[s].x - M);
    L += ml[s].y * f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += v0[s][e] * f;
      acc[4 + e] += v1[s][e] * f;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const size_t m = (size_t)b * n + iq;
  u32x4 out;
  out.x = cvt_pk_bf16(acc[0] * inv, acc[1] * inv);
  out.y = cvt_pk_bf16(acc[2] * inv, acc[3] * inv);
  out.z = cvt_pk_bf16(acc[4] * inv, acc[5] * inv);
  out.w = cvt_pk_bf16(acc[6] * inv, acc[7] * inv);
  *reinterpret_cast<u32x4*>(o + fm_index(m, head * HD + c8, hq * HD)) = out;
}

template <int HD, int NWV, int RING, bool PIPE = false>
static void run_attention(const uint16_t* q, int hq, const KvLayer& kv, const PassGeom& g, int max_keys,
                          uint16_t* o, float* part_o, float2* part_ml, hipStream_t s) {
  constexpr int STAGE = 2 * (2 * (HD / 32) * 1024 + (HD / 16) * 1024);
  static LdsLimit limit;
  raise_lds_limit(limit, reinterpret_cast<const void*>(&attention_kernel<HD, NWV, RING, PIPE>), RING * STAGE);
  AttnArgs a{};
  a.q = q; a.o = o; a.part_o = part_o; a.part_ml = part_ml;
  a.kv = kv; a.g = g; a.hq = hq;
  a.grp = hq / kv.hkv;
  a.qt32 = (g.n + 31) / 32;
  a.wg_per_pair = (a.grp * a.qt32 + NWV - 1) / NWV;
  const int pairs = g.batch * kv.hkv;
  const int base_wgs = pairs * a.wg_per_pair;
  // split the key range when the pairs alone leave CUs idle: aim at ~2 workgroups per
  // CU, keep at least two 64-key stages per split, and stay within the partial buffer
  const int stages = (max_keys + kAttnStageKeys - 1) / kAttnStageKeys + 1;
  int nsplit = (512 + base_wgs - 1) / base_wgs;
  nsplit = min(nsplit, max(1, stages / 2));
  nsplit = min(nsplit, max(1, kAttnMaxSplitRows / (g.batch * a.qt32 * 32)));
  nsplit = min(nsplit, kAttnMaxSplits);
  if (!part_o) nsplit = 1;
  a.nsplit = max(1, nsplit);
  const long units = (long)base_wgs * a.nsplit;
  const int blocks = (int)(kXcd * ((units + kXcd - 1) / kXcd));
  launch_kernel(attention_kernel<HD, NWV, RING, PIPE>, dim3(blocks), dim3(64 * NWV), RING * STAGE, s, nullptr, a);
  if (a.nsplit > 1) {
    const long threads = (long)g.batch * hq * g.n * (HD / 8);
    launch_kernel(attention_merge_kernel<HD>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, nullptr,
                  part_o, part_ml, a.nsplit, g.batch, hq, g.n, a.qt32 * 32, o);
  }
}

// Long key ranges (global layers over a long prefix) take their own workgroup shape:
// 8 waves share each K/V stage (half the copies per query), and the pipelined loop
// issues the next stage's score MFMAs before this stage's softmax, with four ring slots
// so that each copy still goes out two stages ahead of its use.
constexpr int kAttnLongKeys = 4096, kAttnWavesLong = 8, kAttnRingLong = 4;

void launch_attention(const uint16_t* q, int hq, const KvLayer& kv, const PassGeom& g, uint16_t* o,
                      float* part_o, float2* part_ml, hipStream_t s) {
  int max_keys = 0;   // the longest key range of any sequence of the pass
  for (int bb = 0; bb < g.batch; ++bb) {
    const int keys = !seq_encodes(g, bb) ? (kv.window > 0 ? min(g.len[bb], kv.window) : g.len[bb]) + g.n
                               : (kv.window > 0 ? min(g.len[bb] + g.n, kv.window + 63) : g.len[bb] + g.n);
    max_keys = max(max_keys, keys);
  }
  constexpr int NWL = kAttnWavesLong, RL = kAttnRingLong;
  const bool lng = max_keys >= kAttnLongKeys;
  switch (kv.hd) {
    case 32:
      if (lng) run_attention<32, NWL, RL, true>(q, hq, kv, g, max_keys, o, part_o, part_ml, s);
      else run_attention<32, 4, 2>(q, hq, kv, g, max_keys, o, part_o, part_ml, s);
      break;
    case 64:
      if (lng) run_attention<64, NWL, RL, true>(q, hq, kv, g, max_keys, o, part_o, part_ml, s);
      else run_attention<64, 4, 2>(q, hq, kv, g, max_keys, o, part_o, part_ml, s);
      break;
    default:
      if (lng) run_attention<128, NWL, RL, true>(q, hq, kv, g, max_keys, o, part_o, part_ml, s);
      else run_attention<128, 4, 2>(q, hq, kv, g, max_keys, o, part_o, part_ml, s);
      break;
  }
}

}  // namespace dg
