// Entropy-bounded sampler (DiffusionGemma Technical Report §3.3): per masked
// canvas row, entropy and argmax of softmax(logits); then the masked positions
// are accepted in order of increasing entropy while the running entropy sum
// stays within the budget gamma (at least one per step).
//
// Pass 1 streams the bf16 logits once (HBM-bound: 512 KiB per 262144-wide
// row): one 256-thread workgroup per (row, kSampleChunk-logit chunk) computes the
// chunk's lowest argmax and, for the logits y = x / tau at the sampling
// temperature tau (1 unless annealed, §3.3), the chunk max m_c of y,
// s_c = sum exp(y - m_c) and t_c = sum exp(y - m_c) (m_c - y).  Rows that are not
// [MASK] are skipped.
// Pass 2 (one workgroup per sequence) merges the chunks of each row in index
// order, H = log S + T / S, ranks the masked rows by (H, position), takes the
// running fp64 sum in rank order, and commits the argmax of the first k* rows --
// when that decision is certified: no entropy gap or running sum that decides it
// lies within the fast pass's error bound of the boundary.  Otherwise the sequence
// is deferred to the canonical entropy Ĥ (a fixed sequence of IEEE float64
// operations and exact integer sums, reproducible bit for bit by any implementation
// that follows it): pass 3 computes its integer sums for the deferred sequences'
// masked rows only, and pass 4 takes their decision on Ĥ.  Either way the committed
// set is the one the rule gives on Ĥ.
//
// The uniform ("multinomial") variant (Technical Report §3.2, multinomial diffusion;
// §3.3): every position of a canvas is a candidate (accepted tokens stay revisable),
// and every position outside the accepted set is re-noised to a uniformly random token.
// A sequence whose canvas was complete before the call (done step set) is left alone.
#include <math.h>

#include "dg_common.h"
#include "dg_internal.h"

namespace dg {

// Merge two (max, argmax, s, t) partials of disjoint logit sets, each with
// s = sum exp(x - m) and t = sum exp(x - m) (m - x): rescale both to the larger max.
// An empty partial has m = -inf, s = t = 0.  Equal maxima keep the lower index.
__device__ __forceinline__ void merge_part(float& m, int& a, float& s, float& t, float m2, int a2,
                                           float s2, float t2) {
  const float M = fmaxf(m, m2);
  float s1 = 0.f, t1 = 0.f;
  if (m != -INFINITY) {
    const float f = __expf(m - M);
    s1 = s * f;
    t1 = (t + (M - m) * s) * f;
  }
  if (m2 != -INFINITY) {
    const float f = __expf(m2 - M);
    s1 += s2 * f;
    t1 += (t2 + (M - m2) * s2) * f;
  }
  if (m2 > m || (m2 == m && a2 < a)) a = a2;
  m = M;
  s = s1;
  t = t1;
}

// One workgroup per (masked row, kSampleChunk logits).  Each thread loads its
// kSampleChunk / 2048 16-byte pieces up front (all in flight at once, streamed past
// the caches); the workgroup first agrees on the chunk maximum M (one barrier), then
// every thread sums exp(x - M) and exp(x - M) (M - x) over its own pieces against that
// common M, so the partials combine by plain sums (no per-level rescaling), and only
// the lanes holding M search their own elements for its lowest index.  Per element
// the work is kept to one instruction per step:
//  * the max of the high bf16 halves is taken on the raw 32-bit words (the low half
//    only perturbs mantissa bits below the bf16 ulp) and masked once at the end;
//  * exp(x - M) = 2^-(M - x) log2 e with d' = (M - x) log2 e formed by one fma, so
//    t = sum e (M - x) accumulates e d' and is divided by log2 e once.
__global__ __launch_bounds__(256) void sample_partials_kernel(const uint16_t* __restrict__ logits,
                                                              const int32_t* __restrict__ canvas,
                                                              int vocab, int nchunks, float inv_tau,
                                                              int C, int all_rows,
                                                              const int32_t* __restrict__ frozen,
                                                              float4* __restrict__ part,
                                                              int* __restrict__ part_arg) {
  __shared__ float wmax[4];
  __shared__ float4 wsum[4];
  const int row = blockIdx.y, ch = blockIdx.x;
  if (all_rows ? (frozen && frozen[row / C] != 0) : canvas[row] != vocab) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c0 = ch * kSampleChunk;
  const int c1 = min(vocab, c0 + kSampleChunk);
  const uint16_t* lp = logits + (size_t)row * vocab;
  constexpr int NL = kSampleChunk / (256 * 8);
  // pieces past the end of the vocabulary hold bf16 -1.0e30 (0xf14a): it never wins
  // the max, its exp underflows to exactly 0 and (M - x) log2 e stays finite, so it
  // adds nothing to s or t (logits are finite and far inside the fp32 range)
  constexpr uint32_t kPad = 0xf14af14au;
  u32x4 v[NL];
  if (c1 - c0 == kSampleChunk) {               // every chunk but a ragged last one
#pragma unroll
    for (int i = 0; i < NL; ++i) v[i] = ld16_stream(lp + c0 + (i * 256 + tid) * 8);
  } else {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e0 = c0 + (i * 256 + tid) * 8;   // vocab % 8 == 0: a piece is wholly in or out
      v[i] = e0 < c1 ? ld16_stream(lp + e0) : u32x4{kPad, kPad, kPad, kPad};
    }
  }
  float mh = -INFINITY, ml = -INFINITY;
#pragma unroll
  for (int i = 0; i < NL; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mh = fmaxf(mh, __uint_as_float(v[i][j]));
      ml = fmaxf(ml, __uint_as_float(v[i][j] << 16));
    }
  const float m = fmaxf(__uint_as_float(__float_as_uint(mh) & 0xffff0000u), ml);
  // each pass below unpacks the halves again rather than keeping them from the pass
  // before (the empty asm hides that they are the same words): keeping them would
  // cost 32 more registers and a third of the resident workgroups
#pragma unroll
  for (int i = 0; i < NL; ++i) asm volatile("" : "+v"(v[i]));
  const float wm = wave_max(m);
  if (lane == 0) wmax[w] = wm;
  __syncthreads();
  const float M = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  // lowest index holding M: only lanes whose own maximum equals it look, scanning
  // their elements from the highest index down so the last hit is the lowest
  int a = INT_MAX;
  if (m == M) {
#pragma unroll
    for (int i = NL - 1; i >= 0; --i)
#pragma unroll
      for (int j = 7; j >= 0; --j) {
        const uint32_t u = v[i][j >> 1];
        const float x = __uint_as_float(j & 1 ? (u & 0xffff0000u) : (u << 16));
        if (x == M) a = c0 + (i * 256 + tid) * 8 + j;
      }
  }
#pragma unroll
  for (int i = 0; i < NL; ++i) asm volatile("" : "+v"(v[i]));
  constexpr float kLog2e = 1.44269504088896341f;
  const float kL = kLog2e * inv_tau;            // exactly log2 e at tau = 1
  const float mL = M * kL;
  float s = 0.f, t = 0.f;
#pragma unroll
  for (int i = 0; i < NL; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float xl = __uint_as_float(v[i][j] << 16), xh = __uint_as_float(v[i][j] & 0xffff0000u);
      const float dl = __builtin_fmaf(xl, -kL, mL), dh = __builtin_fmaf(xh, -kL, mL);
      const float el = __builtin_amdgcn_exp2f(-dl), eh = __builtin_amdgcn_exp2f(-dh);
      s += el;
      t = __builtin_fmaf(el, dl, t);
      s += eh;
      t = __builtin_fmaf(eh, dh, t);
    }
  t *= 1.0f / kLog2e;
  s = wave_sum(s);
  t = wave_sum(t);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a = min(a, __shfl_xor(a, o, 64));
  if (lane == 0) wsum[w] = make_float4(s, t, __int_as_float(a), 0.f);
  __syncthreads();
  if (tid == 0) {
    const float4 p0 = wsum[0], p1 = wsum[1], p2 = wsum[2], p3 = wsum[3];
    part[(size_t)row * nchunks + ch] =
        make_float4(M * inv_tau, (p0.x + p1.x) + (p2.x + p3.x), (p0.y + p1.y) + (p2.y + p3.y), M);
    part_arg[(size_t)row * nchunks + ch] =
        min(min(__float_as_int(p0.z), __float_as_int(p1.z)), min(__float_as_int(p2.z), __float_as_int(p3.z)));
  }
}

void launch_sample_partials(const uint16_t* logits, const int32_t* canvas, int batch, int C, int vocab,
                            float inv_tau, int all_rows, const int32_t* frozen, float4* part, int* part_arg,
                            hipStream_t s) {
  const int nchunks = (vocab + kSampleChunk - 1) / kSampleChunk;
  launch_kernel(sample_partials_kernel, dim3(nchunks, batch * C), dim3(256), 0, s, nullptr, logits, canvas,
                vocab, nchunks, inv_tau, C, all_rows, frozen, part, part_arg);
}

// ---------------------------------------------------------------- uniform tokens
//
// Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
// 1, 2, 3", SC 2011): ten rounds, each taking the full 128-bit products of words 0 and 2
// with the two round multipliers, crossing the halves over the pairs and XOR-ing in the
// other words and the key, which advances by the two Weyl increments between rounds.
// The token of (seed, draw, sequence, position) is floor(x V / 2^64) for x the first
// output word of the block at counter (position, sequence, draw, 0) under key (seed, 0).
__device__ __forceinline__ uint64_t philox_first_word(uint64_t x0, uint64_t x1, uint64_t x2, uint64_t k0) {
  constexpr uint64_t kMul0 = 0xD2E7470EE14C6C93ull, kMul1 = 0xCA5A826395121157ull;
  constexpr uint64_t kBump0 = 0x9E3779B97F4A7C15ull, kBump1 = 0xBB67AE8584CAA73Bull;
  uint64_t x3 = 0, k1 = 0;
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint64_t hi0 = __umul64hi(kMul0, x0), lo0 = kMul0 * x0;
    const uint64_t hi1 = __umul64hi(kMul1, x2), lo1 = kMul1 * x2;
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
    k0 += kBump0;
    k1 += kBump1;
  }
  return x0;
}

__device__ __forceinline__ int uniform_token(uint64_t seed, int draw, int seq, int pos, int vocab) {
  return (int)__umul64hi(philox_first_word((uint64_t)pos, (uint64_t)seq, (uint64_t)draw, seed), (uint64_t)vocab);
}

__global__ __launch_bounds__(256) void uniform_canvas_kernel(int32_t* __restrict__ canvas, int batch, int C,
                                                             int vocab, uint64_t seed, int draw) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= batch * C) return;
  canvas[i] = uniform_token(seed, draw, i / C, i % C, vocab);
}

void launch_uniform_canvas(int32_t* canvas, int batch, int C, int vocab, uint64_t seed, int draw, hipStream_t s) {
  launch_kernel(uniform_canvas_kernel, dim3((batch * C + 255) / 256), dim3(256), 0, s, nullptr, canvas, batch, C,
                vocab, seed, draw);
}

// Order key of a masked row: (H, row) as one unsigned 64-bit integer that compares
// like the pair -- the fp32 bits of H mapped to an order-preserving unsigned form
// (-0 taken as +0, NaN as +inf) above the row index.
__device__ __forceinline__ uint64_t eb_key(float H, int row) {
  if (H != H) H = INFINITY;
  const uint32_t u = __float_as_uint(H + 0.0f);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (uint64_t)o << 32 | (uint32_t)row;
}

// ---------------------------------------------------------------- canonical entropy
//
// Ĥ of a row of bf16 logits x at temperature tau:
//   u = (m - x) * (1 / tau) in float64 (m = the row maximum, tau the float32 value);
//   e^-u by k = rint(u / ln2), r = (u - k ln2_hi) - k ln2_lo (Cody and Waite's
//   two-part reduction; ln2_hi holds ln 2 to 32 significant bits, so k ln2_hi is
//   exact), e^-r = sum_{i<=12} (-r)^i / i! in Horner form, times 2^-k; 0 for u >= 30;
//   S = sum rint(e 2^40), T = sum rint((e u) 2^40) as exact 64-bit integers;
//   Ĥ = float32(max(0, (log S' - 40 ln2) + T' / S')) with S', T' the float64 values
//   hi * 2^32 + lo of S, T, and log a = j ln2 + 2 s (1 + z/3 + ... + z^12/25) for
//   a = f 2^j, f in [sqrt(1/2), sqrt(2)), s = (f - 1) / (f + 1), z = s^2.
// Every operation is one IEEE float64 add, subtract, multiply or divide rounded to
// nearest even (the pragma keeps the compiler from fusing a multiply and an add),
// rint, an exact scaling by a power of two, or an integer add, so the result does
// not depend on the machine or the summation order.  |Ĥ - H| <= 3e-6.
constexpr double kLn2 = 0x1.62e42fefa39efp-1;        // nearest double to ln 2
constexpr double kLn2Hi = 0x1.62e42fee00000p-1;      // ln 2 to 32 significant bits
constexpr double kLn2Lo = 0x1.a39ef35793c76p-33;     // nearest double to ln 2 - kLn2Hi
constexpr double kInvLn2 = 0x1.71547652b82fep+0;     // nearest double to 1 / ln 2
constexpr double kSqrtHalf = 0x1.6a09e667f3bcdp-1;   // nearest double to sqrt(1/2)
constexpr double kCanonQ = 1099511627776.0;          // 2^40
constexpr double kCanonUMax = 30.0;

__device__ __forceinline__ double canon_exp_neg(double u) {
#pragma clang fp contract(off)
  if (!(u < kCanonUMax)) return 0.0;
  const double k = rint(u * kInvLn2);
  const double r = (u - k * kLn2Hi) - k * kLn2Lo;
  const double y = -r;
  // 1 / i! for i = 12 .. 0, each the correctly rounded quotient
  double p = 1.0 / 479001600.0;
  p = p * y + 1.0 / 39916800.0;
  p = p * y + 1.0 / 3628800.0;
  p = p * y + 1.0 / 362880.0;
  p = p * y + 1.0 / 40320.0;
  p = p * y + 1.0 / 5040.0;
  p = p * y + 1.0 / 720.0;
  p = p * y + 1.0 / 120.0;
  p = p * y + 1.0 / 24.0;
  p = p * y + 1.0 / 6.0;
  p = p * y + 0.5;
  p = p * y + 1.0;
  p = p * y + 1.0;
  return ldexp(p, -(int)k);
}

__device__ __forceinline__ double canon_log(double a) {
#pragma clang fp contract(off)
  int j = 0;
  double f = frexp(a, &j);
  if (f < kSqrtHalf) {
    f = f * 2.0;
    j -= 1;
  }
  const double s = (f - 1.0) / (f + 1.0);
  const double z = s * s;
  // 1 / (2i + 1) for i = 12 .. 0
  double p = 1.0 / 25.0;
  p = p * z + 1.0 / 23.0;
  p = p * z + 1.0 / 21.0;
  p = p * z + 1.0 / 19.0;
  p = p * z + 1.0 / 17.0;
  p = p * z + 1.0 / 15.0;
  p = p * z + 1.0 / 13.0;
  p = p * z + 1.0 / 11.0;
  p = p * z + 1.0 / 9.0;
  p = p * z + 1.0 / 7.0;
  p = p * z + 1.0 / 5.0;
  p = p * z + 1.0 / 3.0;
  p = p * z + 1.0;
  return (double)j * kLn2 + (2.0 * s) * p;
}

__device__ __forceinline__ double u64_to_f64(uint64_t v) {
#pragma clang fp contract(off)
  return (double)(uint32_t)(v >> 32) * 4294967296.0 + (double)(uint32_t)v;
}

__device__ __forceinline__ float canon_entropy(uint64_t S, uint64_t T) {
#pragma clang fp contract(off)
  const double Sf = u64_to_f64(S), Tf = u64_to_f64(T);
  constexpr double kC40 = 40.0 * kLn2;
  const double h = (canon_log(Sf) - kC40) + Tf / Sf;
  return (float)(h > 0.0 ? h : 0.0);
}

// Pass 3: exact integer sums (S, T) of one (row, kSampleChunk-logit chunk) for the
// canonical entropy, for the masked rows of the sequences pass 2 deferred (flag set);
// every other workgroup returns at once.  The row maximum is the largest raw chunk
// maximum pass 1 recorded.
__global__ __launch_bounds__(256) void canon_partials_kernel(const uint16_t* __restrict__ logits,
                                                             const int32_t* __restrict__ canvas, int C,
                                                             int vocab, int nchunks, float tau, int all_rows,
                                                             const float4* __restrict__ part,
                                                             const int32_t* __restrict__ flag,
                                                             const float* __restrict__ Hf,
                                                             const float2* __restrict__ win,
                                                             ulonglong2* __restrict__ cpart) {
  __shared__ uint64_t red[2][4];
  const int row = blockIdx.y, ch = blockIdx.x, b = row / C;
  const int f = flag[b];
  if (f == 0 || (!all_rows && canvas[row] != vocab)) return;   // uniform per workgroup
  if (f == 2) {                                 // only the rows of the boundary window
    const float h = Hf[row];
    const float2 w = win[b];
    if (!(h >= w.x && h <= w.y)) return;
  }
  float m = -INFINITY;
  for (int c = 0; c < nchunks; ++c) m = fmaxf(m, part[(size_t)row * nchunks + c].w);
  const double md = (double)m, inv = 1.0 / (double)tau;
  const int c0 = ch * kSampleChunk, c1 = min(vocab, c0 + kSampleChunk);
  const uint16_t* lp = logits + (size_t)row * vocab;
  uint64_t S = 0, T = 0;
  for (int i = c0 + 8 * threadIdx.x; i < c1; i += 8 * 256) {   // vocab % 8 == 0
    const u32x4 v = ld16(lp + i);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w = v[j >> 1];
      const double x = (double)__uint_as_float(j & 1 ? (w & 0xffff0000u) : (w << 16));
      double u, e;
      {
#pragma clang fp contract(off)
        u = (md - x) * inv;
        e = canon_exp_neg(u);
        S += (uint64_t)rint(e * kCanonQ);
        T += (uint64_t)rint((e * u) * kCanonQ);
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    S += __shfl_xor(S, o, 64);
    T += __shfl_xor(T, o, 64);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][w] = S;
    red[1][w] = T;
  }
  __syncthreads();
  if (threadIdx.x == 0)
    cpart[(size_t)row * nchunks + ch] =
        make_ulonglong2(red[0][0] + red[0][1] + red[0][2] + red[0][3], red[1][0] + red[1][1] + red[1][2] + red[1][3]);
}

void launch_canon_partials(const uint16_t* logits, const int32_t* canvas, int batch, int C, int vocab,
                           float tau, int all_rows, const float4* part, const int32_t* flag, const float* Hf,
                           const float2* win, ulonglong2* cpart, hipStream_t s) {
  const int nchunks = (vocab + kSampleChunk - 1) / kSampleChunk;
  launch_kernel(canon_partials_kernel, dim3(nchunks, batch * C), dim3(256), 0, s, nullptr, logits, canvas, C,
                vocab, nchunks, tau, all_rows, part, flag, Hf, win, cpart);
}

// ---------------------------------------------------------------- selection

// Bound on |H_fast - Ĥ| used to certify a fast decision.  The fast pass sums exp
// terms in fp32 along chains of at most ~80 roundings (64 per thread, 6 + 2 in the
// workgroup, <= 8 in the chunk merge), so S and T carry a relative error below
// ~1e-5 each; with T / S <= log V ~ 12.5 that bounds |H_fast - H| by ~2.6e-4, and
// |Ĥ - H| <= 3e-6.  The float64 running sums over <= 1024 entropies below 16 add at
// most ~2e-9 of rounding, bounded by kSumSlack.
constexpr double kCertEps = 5e-4;
constexpr double kSumSlack = 1e-8;

enum SelMode { SEL_FAST = 0, SEL_CANON = 1, SEL_GIVEN = 2 };

struct SelArgs {
  const float4* part;        // SEL_FAST: fp32 chunk partials (tempered max, s, t, raw max)
  const int* part_arg;       //           and chunk argmaxes
  int nchunks;
  const ulonglong2* cpart;   // SEL_CANON: exact integer chunk sums (S, T)
  const float* H_in;         // SEL_GIVEN: entropies and argmaxes given
  const int32_t* amax_in;
  int32_t* canvas;
  int C, vocab;
  float gamma;
  uint64_t commit;           // bit b: sequence b commits (accepts) every candidate row
  float* H_out;
  int32_t* amax_out;
  int32_t* n_masked;
  int32_t* prev_amax;        // adaptive stop (NULL: off)
  float e_stop;
  int step;
  int32_t* done_step;
  int32_t* flag;             // [batch]: SEL_FAST sets 0 (decided), 1 (deferred: every masked row's Ĥ is
                             // needed) or 2 (deferred: only the order of the rows in a window at the
                             // budget boundary is open; k* is already certain)
  int32_t* moved;            // [batch]: SEL_FAST's count of moved argmaxes, for SEL_CANON
  int32_t* amax_ws;          // [batch][C]: every masked row's argmax, for SEL_CANON
  float* Hf_ws;              // [batch][C]: every masked row's fast entropy
  float2* win;               // [batch]: the window [lo, hi] of fast entropies whose Ĥ decides (flag 2)
  int32_t* kstar_ws;         // [batch]: the certain k* (flag 2)
  int uniform;               // uniform variant: every row a candidate, the rest re-noised
  uint64_t seed;             //   with the tokens of (seed, draw)
  int draw;
};

template <int TPR, int MODE>   // threads per canvas row (chunk merge and rank count)
__global__ __launch_bounds__(1024) void eb_select_kernel(SelArgs A) {
  __shared__ __attribute__((aligned(16))) uint64_t keys[1024];
  __shared__ __attribute__((aligned(16))) float sortedH[1024];
  __shared__ float Hpos[1024];
  __shared__ int rank_s[1024];
  __shared__ int nm_s, kstar_s;
  __shared__ int decided_s;
  const int b = blockIdx.x;
  if (MODE == SEL_CANON && A.flag[b] == 0) return;   // decided by the fast pass
  const int C = A.C;
  // the row's TPR threads are adjacent lanes
  const int r = threadIdx.x / TPR, sub = threadIdx.x % TPR;
  const size_t ridx = (size_t)b * C + r;
  // candidate rows ("masked" below): the [MASK] rows, or in the uniform variant every row
  // of a sequence not yet complete (its done step is read before any thread writes it)
  const bool frozen = A.uniform && A.done_step && A.done_step[b] != 0;
  const bool masked = r < C && !frozen && (A.uniform || A.canvas[ridx] == A.vocab);
  // phase 1: entropy and argmax of each masked row
  float H = INFINITY;
  int a = 0;
  float hf = 0.f;         // SEL_CANON, flag 2: the row's fast entropy
  bool in_win = true;     // SEL_CANON, flag 2: the row lies in the boundary window
  if (MODE == SEL_FAST) {
    // the row's threads merge interleaved subsets of its chunks, then combine
    // through shuffles
    const int nchunks = A.nchunks;
    float M = -INFINITY, S = 0.f, T = 0.f;
    a = INT_MAX;
    if (masked) {
      const float4* pr = A.part + ridx * nchunks;
      const int* pa = A.part_arg + ridx * nchunks;
      int k = sub;
      for (; k + 3 * TPR < nchunks; k += 4 * TPR) {
        float4 p[4];
        int q[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          p[u] = pr[k + u * TPR];
          q[u] = pa[k + u * TPR];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) merge_part(M, a, S, T, p[u].x, q[u], p[u].y, p[u].z);
      }
      for (; k < nchunks; k += TPR) {
        const float4 p = pr[k];
        merge_part(M, a, S, T, p.x, pa[k], p.y, p.z);
      }
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) {
      const float m2 = __shfl_xor(M, o, 64), s2 = __shfl_xor(S, o, 64), t2 = __shfl_xor(T, o, 64);
      const int a2 = __shfl_xor(a, o, 64);
      merge_part(M, a, S, T, m2, a2, s2, t2);
    }
    // H >= 0 exactly; the fp32 partials can leave a rounding residue of ~1e-7 below
    if (masked) H = fmaxf(logf(S) + T / S, 0.f);
  } else if (MODE == SEL_CANON) {
    // flag 1: every masked row's Ĥ; flag 2: Ĥ of the window rows only (their sums are the
    // only ones pass 3 computed), the fast entropy elsewhere
    if (masked && A.flag[b] == 2) {
      hf = A.Hf_ws[ridx];
      in_win = hf >= A.win[b].x && hf <= A.win[b].y;
    }
    uint64_t S = 0, T = 0;
    if (masked && in_win)
      for (int k = sub; k < A.nchunks; k += TPR) {
        const ulonglong2 p = A.cpart[ridx * A.nchunks + k];
        S += p.x;
        T += p.y;
      }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) {
      S += __shfl_xor(S, o, 64);
      T += __shfl_xor(T, o, 64);
    }
    if (masked) {
      H = in_win ? canon_entropy(S, T) : hf;
      a = A.amax_ws[ridx];
    }
  } else if (masked) {
    H = A.H_in[ridx];
    a = A.amax_in[ridx];
  }
  if (masked && (a < 0 || a >= A.vocab)) a = min(max(a, 0), A.vocab - 1);
  // unmasked rows (and the padding up to a multiple of 8) take the largest key,
  // which no masked row's key exceeds, so they are never counted below one
  const int Cp = (C + 7) & ~7;
  uint64_t key = masked ? eb_key(H, r) : ~0ull;
  // flag 2: rows below the window precede every window row (in position order), rows
  // above it follow every masked row; only the window rows are ranked by (Ĥ, position)
  if (MODE == SEL_CANON && masked && !in_win) key = hf < A.win[b].x ? (uint64_t)r : ~0ull;
  if (sub == 0 && r < Cp) keys[r] = key;
  if (sub == 0 && r < C) Hpos[r] = H;
  // adaptive stop (prev_amax given; §3.3): the rows whose argmax moved since the
  // previous step (SEL_CANON takes the fast pass's count: prev_amax holds this
  // step's argmaxes by then)
  int n_moved = 1;
  if (A.prev_amax) {
    if (MODE == SEL_CANON)
      n_moved = A.moved[b];
    else
      n_moved = __syncthreads_count(masked && sub == 0 && a != A.prev_amax[ridx]);
  }
  const int nm_all = __syncthreads_count(masked && sub == 0);
  // phase 2: rank of each masked row = #{masked j : key_j < key_r}; the row's TPR
  // threads count interleaved pairs of keys (one 16-byte LDS read per pair)
  if (masked) {
    // the row's threads can hold H differing in the last bit (their shuffle merges
    // round in different orders), so all of them rank the key thread 0 stored
    const uint64_t key = keys[r];
    const ulonglong2* k2 = reinterpret_cast<const ulonglong2*>(keys);
    int rank = 0;
    for (int q = sub; q < Cp / 2; q += TPR) {
      const ulonglong2 kk = k2[q];
      rank += (kk.x < key) + (kk.y < key);
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) rank += __shfl_xor(rank, o, 64);
    if (sub == 0) {
      sortedH[rank] = (H != H) ? INFINITY : H;
      rank_s[r] = rank;
    }
  }
  if (threadIdx.x == 0) nm_s = nm_all;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int n = nm_s;
    const double g = (double)A.gamma;
    bool cert = true;       // SEL_FAST: the fast entropies decide
    bool order_only = true; // SEL_FAST, not cert: only the order at the boundary is open
    bool stop = false;
    float2 window = make_float2(0.f, 0.f);
    if (A.prev_amax && n_moved == 0 && n > 0) {
      // mean entropy of the masked rows: float64 running sum in position order
      double hs = 0.0;
      for (int i = 0; i < C; ++i)
        if (A.uniform || A.canvas[(size_t)b * C + i] == A.vocab) hs += (double)Hpos[i];
      const double mean = hs / n;
      stop = mean < (double)A.e_stop;
      if (MODE == SEL_FAST && fabs(mean - (double)A.e_stop) <= kCertEps + kSumSlack) cert = order_only = false;
    }
    int ks;
    if (MODE == SEL_CANON && A.flag[b] == 2) {
      ks = A.kstar_ws[b];                     // certain; the ranking above settled the order
    } else if (((A.commit >> b) & 1) || stop || n == 0) {
      ks = n;
    } else {
      // running fp64 sum in rank order (S_k of the first k rows); k_nat = the number
      // of leading running sums within gamma (the sums never decrease)
      double S = 0.0, S_at = 0.0;
      int k = 0;
      const float4* s4 = reinterpret_cast<const float4*>(sortedH);
      bool over = false;
      for (int j = 0; j < n && !over; j += 4) {
        const float4 h = s4[j >> 2];
        const float hv[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (over || j + u >= n) break;
          S += (double)hv[u];
          if (S <= g) {
            k = j + u + 1;
            S_at = S;
          } else {
            over = true;
          }
        }
      }
      ks = k < 1 ? 1 : k;
      if (MODE == SEL_FAST) {
        // certified when no Ĥ within kCertEps of each fast H changes the set:
        // the ks-th and (ks+1)-th entropies are more than 2 eps apart, and the
        // running sums at ks (when within gamma) and at ks + 1 stay on their side
        // of gamma by more than eps per term
        const double S_ks = k >= 1 ? S_at : (double)sortedH[0];
        if (ks < n) {
          const double next = S_ks + (double)sortedH[ks];
          if ((double)sortedH[ks] - (double)sortedH[ks - 1] <= 2.0 * kCertEps) {
            cert = false;
            // rows with a fast entropy below h_ks - 2 eps are in whatever the Ĥ, rows above
            // h_(ks+1) + 2 eps out: only the rows between need Ĥ
            window = make_float2((float)((double)sortedH[ks - 1] - 2.0 * kCertEps),
                                 (float)((double)sortedH[ks] + 2.0 * kCertEps));
          }
          if (next - g <= (ks + 1) * kCertEps + kSumSlack) cert = order_only = false;
        }
        if (k >= 1 && g - S_at <= k * kCertEps + kSumSlack) cert = order_only = false;
      }
    }
    if (MODE == SEL_FAST && A.flag) {
      A.flag[b] = cert ? 0 : (order_only ? 2 : 1);
      if (!cert) {
        A.moved[b] = n_moved;
        if (order_only) {
          // widen by a float32 ulp on each side so that the rounding of the bounds to
          // float can only add rows to the window
          A.win[b] = make_float2(nextafterf(window.x, -INFINITY), nextafterf(window.y, INFINITY));
          A.kstar_ws[b] = ks;
        }
        ks = 0;                               // the canonical pass decides
      }
    }
    kstar_s = ks;
    const bool decided = cert || MODE != SEL_FAST || !A.flag;
    decided_s = decided;
    if (decided) {
      A.n_masked[b] = n - ks;
      // complete: no [MASK] left; in the uniform variant, the stop fired or the last step
      const bool complete = A.uniform ? (n > 0 && (((A.commit >> b) & 1) || stop)) : n - ks == 0;
      if (A.done_step && complete && A.done_step[b] == 0) A.done_step[b] = A.step + 1;
    }
  }
  __syncthreads();
  if (sub == 0 && r < C) {
    if (A.H_out) A.H_out[ridx] = masked ? H : __int_as_float(0x7fc00000);   // NaN on unmasked rows
    if (MODE != SEL_CANON) {
      if (A.amax_out) A.amax_out[ridx] = masked ? a : -1;                   // -1 on unmasked rows
      if (A.prev_amax) A.prev_amax[ridx] = masked ? a : -1;
      if (A.amax_ws && masked) A.amax_ws[ridx] = a;
      if (A.Hf_ws && masked) A.Hf_ws[ridx] = H;
    }
    if (masked && rank_s[r] < kstar_s)
      A.canvas[ridx] = a;
    else if (A.uniform && masked && decided_s)
      A.canvas[ridx] = uniform_token(A.seed, A.draw, b, r, A.vocab);
  }
}

template <int MODE>
static void run_select(const SelArgs& a, int batch, hipStream_t s) {
  const int rows64 = ((a.C + 63) / 64) * 64;
  if (4 * rows64 <= 1024)
    launch_kernel(eb_select_kernel<4, MODE>, dim3(batch), dim3(4 * rows64), 0, s, nullptr, a);
  else
    launch_kernel(eb_select_kernel<1, MODE>, dim3(batch), dim3(rows64), 0, s, nullptr, a);
}

void launch_eb_select(const float4* part, const int* part_arg, int nchunks, const float* H_in,
                      const int32_t* amax_in, int32_t* canvas, int batch, int C, int vocab,
                      float gamma, uint64_t commit, float* H_out, int32_t* amax_out,
                      int32_t* n_masked, int32_t* prev_amax, float e_stop, int step, int32_t* done_step,
                      int32_t* flag, int32_t* moved, int32_t* amax_ws, float* Hf_ws, float2* win,
                      int32_t* kstar_ws, int uniform, uint64_t seed, int draw, hipStream_t s) {
  SelArgs a{};
  a.uniform = uniform; a.seed = seed; a.draw = draw;
  a.part = part; a.part_arg = part_arg; a.nchunks = nchunks;
  a.Hf_ws = Hf_ws; a.win = win; a.kstar_ws = kstar_ws;
  a.H_in = H_in; a.amax_in = amax_in;
  a.canvas = canvas; a.C = C; a.vocab = vocab; a.gamma = gamma; a.commit = commit;
  a.H_out = H_out; a.amax_out = amax_out; a.n_masked = n_masked;
  a.prev_amax = prev_amax; a.e_stop = e_stop; a.step = step; a.done_step = done_step;
  a.flag = flag; a.moved = moved; a.amax_ws = amax_ws;
  if (part) run_select<SEL_FAST>(a, batch, s);
  else run_select<SEL_GIVEN>(a, batch, s);
}

void launch_eb_select_canon(const ulonglong2* cpart, int nchunks, int32_t* canvas, int batch, int C, int vocab,
                            float gamma, uint64_t commit, float* H_out, int32_t* amax_out, int32_t* n_masked,
                            int32_t* prev_amax, float e_stop, int step, int32_t* done_step,
                            int32_t* flag, int32_t* moved, int32_t* amax_ws, float* Hf_ws, float2* win,
                            int32_t* kstar_ws, int uniform, uint64_t seed, int draw, hipStream_t s) {
  SelArgs a{};
  a.uniform = uniform; a.seed = seed; a.draw = draw;
  a.cpart = cpart; a.nchunks = nchunks;
  a.Hf_ws = Hf_ws; a.win = win; a.kstar_ws = kstar_ws;
  a.canvas = canvas; a.C = C; a.vocab = vocab; a.gamma = gamma; a.commit = commit;
  a.H_out = H_out; a.amax_out = amax_out; a.n_masked = n_masked;
  a.prev_amax = prev_amax; a.e_stop = e_stop; a.step = step; a.done_step = done_step;
  a.flag = flag; a.moved = moved; a.amax_ws = amax_ws;
  run_select<SEL_CANON>(a, batch, s);
}

}  // namespace dg
