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
// running fp64 sum in rank order, and commits the argmax of the first k* rows.
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
                                                              float4* __restrict__ part,
                                                              int* __restrict__ part_arg) {
  __shared__ float wmax[4];
  __shared__ float4 wsum[4];
  const int row = blockIdx.y, ch = blockIdx.x;
  if (canvas[row] != vocab) return;
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
        make_float4(M * inv_tau, (p0.x + p1.x) + (p2.x + p3.x), (p0.y + p1.y) + (p2.y + p3.y), 0.f);
    part_arg[(size_t)row * nchunks + ch] =
        min(min(__float_as_int(p0.z), __float_as_int(p1.z)), min(__float_as_int(p2.z), __float_as_int(p3.z)));
  }
}

void launch_sample_partials(const uint16_t* logits, const int32_t* canvas, int rows, int vocab,
                            float inv_tau, float4* part, int* part_arg, hipStream_t s) {
  const int nchunks = (vocab + kSampleChunk - 1) / kSampleChunk;
  launch_kernel(sample_partials_kernel, dim3(nchunks, rows), dim3(256), 0, s, nullptr, logits, canvas,
                vocab, nchunks, inv_tau, part, part_arg);
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

template <int TPR>   // threads per canvas row (chunk merge and rank count)
__global__ __launch_bounds__(1024) void eb_select_kernel(const float4* __restrict__ part,
                                                         const int* __restrict__ part_arg,
                                                         int nchunks, const float* __restrict__ H_in,
                                                         const int32_t* __restrict__ amax_in,
                                                         int32_t* __restrict__ canvas, int C,
                                                         int vocab, float gamma, int commit_all,
                                                         float* __restrict__ H_out,
                                                         int32_t* __restrict__ amax_out,
                                                         int32_t* __restrict__ n_masked,
                                                         int32_t* __restrict__ prev_amax, float e_stop,
                                                         int step, int32_t* __restrict__ done_step) {
  __shared__ __attribute__((aligned(16))) uint64_t keys[1024];
  __shared__ double hsum[16];
  __shared__ __attribute__((aligned(16))) float sortedH[1024];
  __shared__ int rank_s[1024];
  __shared__ int nm_s, kstar_s;
  const int b = blockIdx.x;
  // the row's TPR threads are adjacent lanes
  const int r = threadIdx.x / TPR, sub = threadIdx.x % TPR;
  const size_t ridx = (size_t)b * C + r;
  const bool masked = r < C && canvas[ridx] == vocab;
  // phase 1: entropy and argmax of each masked row; the row's threads merge
  // interleaved subsets of its chunks, then combine through shuffles
  float H = INFINITY;
  int a = 0;
  if (part) {
    float M = -INFINITY, S = 0.f, T = 0.f;
    a = INT_MAX;
    if (masked) {
      const float4* pr = part + ridx * nchunks;
      const int* pa = part_arg + ridx * nchunks;
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
  } else if (masked) {
    H = H_in[ridx];
    a = amax_in[ridx];
  }
  if (masked && (a < 0 || a >= vocab)) a = min(max(a, 0), vocab - 1);
  // unmasked rows (and the padding up to a multiple of 8) take the largest key,
  // which no masked row's key exceeds, so they are never counted below one
  const int Cp = (C + 7) & ~7;
  const uint64_t key = masked ? eb_key(H, r) : ~0ull;
  if (sub == 0 && r < Cp) keys[r] = key;
  // adaptive stop (prev_amax given; §3.3): the masked rows' entropies summed in fp64
  // (per wave, then the waves in order) and the rows whose argmax moved since the
  // previous step counted
  bool moved = false;
  if (prev_amax) {
    const double hv = wave_sum_d((masked && sub == 0) ? (double)H : 0.0);
    if ((threadIdx.x & 63) == 0) hsum[threadIdx.x >> 6] = hv;
    moved = masked && sub == 0 && a != prev_amax[ridx];
  }
  const int nm_all = __syncthreads_count(masked && sub == 0);
  const int n_moved = prev_amax ? __syncthreads_count(moved) : 1;
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
    bool stop = false;
    if (n_moved == 0 && n > 0) {
      double hs = 0.0;
      for (int w = 0; w < (int)(blockDim.x >> 6); ++w) hs += hsum[w];
      stop = hs / n < (double)e_stop;
    }
    int ks;
    if (commit_all || stop || n == 0) {
      ks = n;
    } else {
      // running fp64 sum in rank order; entries are read four at a time
      double S = 0.0;
      int k = 0;
      bool over = false;
      const float4* s4 = reinterpret_cast<const float4*>(sortedH);
      for (int j = 0; j < n && !over; j += 4) {
        const float4 h = s4[j >> 2];
        const float hv[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (over || j + u >= n) break;
          S += (double)hv[u];
          if (S <= (double)gamma)
            k = j + u + 1;
          else
            over = true;
        }
      }
      ks = k < 1 ? 1 : k;
    }
    kstar_s = ks;
    n_masked[b] = n - ks;
    if (done_step && n - ks == 0 && done_step[b] == 0) done_step[b] = step + 1;
  }
  __syncthreads();
  if (sub == 0 && r < C) {
    if (H_out) H_out[ridx] = masked ? H : __int_as_float(0x7fc00000);   // NaN on unmasked rows
    if (amax_out) amax_out[ridx] = masked ? a : -1;                       // -1 on unmasked rows
    if (prev_amax) prev_amax[ridx] = masked ? a : -1;
    if (masked && rank_s[r] < kstar_s) canvas[ridx] = a;
  }
}

void launch_eb_select(const float4* part, const int* part_arg, int nchunks, const float* H_in,
                      const int32_t* amax_in, int32_t* canvas, int batch, int C, int vocab,
                      float gamma, int commit_all, float* H_out, int32_t* amax_out,
                      int32_t* n_masked, int32_t* prev_amax, float e_stop, int step, int32_t* done_step,
                      hipStream_t s) {
  const int rows64 = ((C + 63) / 64) * 64;
  if (4 * rows64 <= 1024)
    launch_kernel(eb_select_kernel<4>, dim3(batch), dim3(4 * rows64), 0, s, nullptr, part, part_arg, nchunks,
                  H_in, amax_in, canvas, C, vocab, gamma, commit_all, H_out, amax_out, n_masked, prev_amax,
                  e_stop, step, done_step);
  else
    launch_kernel(eb_select_kernel<1>, dim3(batch), dim3(rows64), 0, s, nullptr, part, part_arg, nchunks,
                  H_in, amax_in, canvas, C, vocab, gamma, commit_all, H_out, amax_out, n_masked, prev_amax,
                  e_stop, step, done_step);
}

}  // namespace dg
