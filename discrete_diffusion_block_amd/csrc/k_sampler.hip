// Entropy-bounded sampler (DiffusionGemma Technical Report §3.3): per masked
// canvas row, entropy and argmax of softmax(logits); then the masked positions
// are accepted in order of increasing entropy while the running entropy sum
// stays within the budget gamma (at least one per step).
//
// Pass 1 streams the bf16 logits once (HBM-bound: 512 KiB per 262144-wide
// row): one 256-thread workgroup per (row, kSampleChunk-logit chunk) computes the
// chunk max m_c, its lowest argmax, s_c = sum exp(x - m_c) and
// t_c = sum exp(x - m_c) (m_c - x).  Rows that are not [MASK] are skipped.
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
// the caches) and reduces them to a thread-local (max, s, t) in two register passes;
// the workgroup merges the 256 partials, and only the lanes holding the chunk maximum
// search their own elements for its lowest index.  The pass is VALU-bound at about
// ten operations per logit, so every per-element step is kept to one instruction:
//  * the max of the high bf16 halves is taken on the raw 32-bit words (the low half
//    only perturbs mantissa bits below the bf16 ulp) and masked once at the end;
//  * exp(x - m) = 2^-(m - x) log2 e with d' = (m - x) log2 e formed by one fma, so
//    t = sum e (m - x) accumulates e d' and is divided by log2 e once.
__global__ __launch_bounds__(256) void sample_partials_kernel(const uint16_t* __restrict__ logits,
                                                              const int32_t* __restrict__ canvas,
                                                              int vocab, int nchunks,
                                                              float4* __restrict__ part,
                                                              int* __restrict__ part_arg) {
  __shared__ float4 wp[4];
  __shared__ int wa[4];
  __shared__ float chunk_max;
  const int row = blockIdx.y, ch = blockIdx.x;
  if (canvas[row] != vocab) return;
  const int tid = threadIdx.x;
  const int c0 = ch * kSampleChunk;
  const int c1 = min(vocab, c0 + kSampleChunk);
  const uint16_t* lp = logits + (size_t)row * vocab;
  constexpr int NL = kSampleChunk / (256 * 8);
  // pieces past the end of the vocabulary hold bf16 -1.0e30 (0xf14a): it never wins
  // the max, its exp underflows to exactly 0 and (m - x) log2 e stays finite, so it
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
  constexpr float kLog2e = 1.44269504088896341f;
  const float mL = m * kLog2e;
  float s = 0.f, t = 0.f;
#pragma unroll
  for (int i = 0; i < NL; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float xl = __uint_as_float(v[i][j] << 16), xh = __uint_as_float(v[i][j] & 0xffff0000u);
      const float dl = __builtin_fmaf(xl, -kLog2e, mL), dh = __builtin_fmaf(xh, -kLog2e, mL);
      const float el = __builtin_amdgcn_exp2f(-dl), eh = __builtin_amdgcn_exp2f(-dh);
      s += el;
      t = __builtin_fmaf(el, dl, t);
      s += eh;
      t = __builtin_fmaf(eh, dh, t);
    }
  t *= 1.0f / kLog2e;
  // (max, s, t) over the workgroup: xor butterfly within each wave, then the waves;
  // the thread keeps its own maximum m for the argmax search below
  float mm = m, ss = s, tt = t;
  int a = INT_MAX;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(mm, o, 64), s2 = __shfl_xor(ss, o, 64), t2 = __shfl_xor(tt, o, 64);
    merge_part(mm, a, ss, tt, m2, INT_MAX, s2, t2);
  }
  if ((tid & 63) == 0) wp[tid >> 6] = make_float4(mm, ss, tt, 0.f);
  __syncthreads();
  if (tid == 0) {
    float M = wp[0].x, S = wp[0].y, T = wp[0].z;
    int A = INT_MAX;
#pragma unroll
    for (int w = 1; w < 4; ++w) merge_part(M, A, S, T, wp[w].x, INT_MAX, wp[w].y, wp[w].z);
    chunk_max = M;
    wp[0] = make_float4(M, S, T, 0.f);
  }
  __syncthreads();
  // lowest index holding the chunk maximum: only lanes whose own maximum equals it look
  const float M = chunk_max;
  if (m == M) {
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t w = v[i][j >> 1];
        const float x = __uint_as_float(j & 1 ? (w & 0xffff0000u) : (w << 16));
        if (x == M && a == INT_MAX) a = c0 + (i * 256 + tid) * 8 + j;
      }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a = min(a, __shfl_xor(a, o, 64));
  if ((tid & 63) == 0) wa[tid >> 6] = a;
  __syncthreads();
  if (tid == 0) {
    const int A = min(min(wa[0], wa[1]), min(wa[2], wa[3]));
    part[(size_t)row * nchunks + ch] = wp[0];
    part_arg[(size_t)row * nchunks + ch] = A;
  }
}

void launch_sample_partials(const uint16_t* logits, const int32_t* canvas, int rows, int vocab,
                            float4* part, int* part_arg, hipStream_t s) {
  const int nchunks = (vocab + kSampleChunk - 1) / kSampleChunk;
  launch_kernel(sample_partials_kernel, dim3(nchunks, rows), dim3(256), 0, s, nullptr, logits, canvas,
                vocab, nchunks, part, part_arg);
}

template <int TPR>   // threads per canvas row in the chunk merge
__global__ __launch_bounds__(1024) void eb_select_kernel(const float4* __restrict__ part,
                                                         const int* __restrict__ part_arg,
                                                         int nchunks, const float* __restrict__ H_in,
                                                         const int32_t* __restrict__ amax_in,
                                                         int32_t* __restrict__ canvas, int C,
                                                         int vocab, float gamma, int commit_all,
                                                         float* __restrict__ H_out,
                                                         int32_t* __restrict__ amax_out,
                                                         int32_t* __restrict__ n_masked) {
  __shared__ __attribute__((aligned(16))) float Hs[1024];
  __shared__ __attribute__((aligned(16))) float sortedH[1024];
  __shared__ float Hrow[1024];
  __shared__ int arow[1024];
  __shared__ int nm_s, kstar_s;
  const int b = blockIdx.x;
  // phase 1: entropy and argmax of each row; the row's TPR threads (adjacent lanes)
  // merge interleaved subsets of its chunks, then combine through shuffles
  {
    const int r = threadIdx.x / TPR, sub = threadIdx.x % TPR;
    const size_t ridx = (size_t)b * C + r;
    const bool rmasked = r < C && canvas[ridx] == vocab;
    float H = INFINITY;
    int a = 0;
    if (part) {
      float M = -INFINITY, S = 0.f, T = 0.f;
      a = INT_MAX;
      if (rmasked) {
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
      if (rmasked) H = fmaxf(logf(S) + T / S, 0.f);
    } else if (rmasked) {
      H = H_in[ridx];
      a = amax_in[ridx];
    }
    if (rmasked && (a < 0 || a >= vocab)) a = min(max(a, 0), vocab - 1);
    if (sub == 0 && r < C) {
      Hrow[r] = rmasked ? H : __int_as_float(0x7fc00000);
      arow[r] = rmasked ? a : -1;
    }
  }
  __syncthreads();
  // phase 2: one thread per row
  const int c = threadIdx.x;
  const size_t idx = (size_t)b * C + c;
  const bool masked = c < C && arow[c] >= 0;
  const float H = c < C ? Hrow[c] : 0.f;
  const int a = c < C ? arow[c] : -1;
  const float key = (masked && !(H != H)) ? H : INFINITY;
  // unmasked positions hold NaN, which no comparison below counts
  if (c < C) Hs[c] = masked ? key : __int_as_float(0x7fc00000);
  const int nm_all = __syncthreads_count(masked);
  int rank = 0;
  if (masked) {
    // rank = #{j : (H_j, j) < (H_c, c)}, four broadcast LDS reads at a time
    const float4* H4 = reinterpret_cast<const float4*>(Hs);
    const int C4 = C >> 2;
    for (int q = 0; q < C4; ++q) {
      const float4 h = H4[q];
      const int j = 4 * q;
      rank += (h.x < key || (h.x == key && j < c)) + (h.y < key || (h.y == key && j + 1 < c)) +
              (h.z < key || (h.z == key && j + 2 < c)) + (h.w < key || (h.w == key && j + 3 < c));
    }
    for (int j = 4 * C4; j < C; ++j) {
      const float hj = Hs[j];
      rank += (hj < key || (hj == key && j < c));
    }
    sortedH[rank] = key;
  }
  if (c == 0) nm_s = nm_all;
  __syncthreads();
  if (c == 0) {
    const int n = nm_s;
    int ks;
    if (commit_all || n == 0) {
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
  }
  __syncthreads();
  if (c < C) {
    if (H_out) H_out[idx] = H;          // NaN on unmasked rows
    if (amax_out) amax_out[idx] = a;    // -1 on unmasked rows
    if (masked && rank < kstar_s) canvas[idx] = a;
  }
}

void launch_eb_select(const float4* part, const int* part_arg, int nchunks, const float* H_in,
                      const int32_t* amax_in, int32_t* canvas, int batch, int C, int vocab,
                      float gamma, int commit_all, float* H_out, int32_t* amax_out,
                      int32_t* n_masked, hipStream_t s) {
  const int rows64 = ((C + 63) / 64) * 64;
  if (4 * rows64 <= 1024)
    launch_kernel(eb_select_kernel<4>, dim3(batch), dim3(4 * rows64), 0, s, nullptr, part, part_arg, nchunks,
                  H_in, amax_in, canvas, C, vocab, gamma, commit_all, H_out, amax_out, n_masked);
  else
    launch_kernel(eb_select_kernel<1>, dim3(batch), dim3(rows64), 0, s, nullptr, part, part_arg, nchunks,
                  H_in, amax_in, canvas, C, vocab, gamma, commit_all, H_out, amax_out, n_masked);
}

}  // namespace dg
