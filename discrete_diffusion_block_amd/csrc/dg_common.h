// Shared device helpers for the gfx950 kernels: bf16 bit conversions, MFMA
// fragment types, wave reductions.  Everything here is wave64 / CDNA4 specific.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace dg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> bf16 (round to nearest even) in one instruction, packed low first.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ bf16x8 as_bf8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l supplies A[l%16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l%16] (any common
// permutation of the 32 k-slots is allowed as long as A and B agree) and holds
// D[4*(l/16) + i][l%16], i = 0..3.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(a), as_bf8(b), c, 0, 0, 0);
}

// Two k tiles into one accumulator, issued back to back.  A dependent MFMA pair
// forwards its accumulator and issues at the full rate (~16 clocks), while
// consecutive MFMAs on different accumulators cost ~28 clocks each on this core
// (measured), so every GEMM issues its MFMAs as such pairs; the scheduling
// barrier stops the compiler from interleaving pairs back into that slow order.
__device__ __forceinline__ f32x4 mfma16x2(u32x4 a0, u32x4 b0, u32x4 a1, u32x4 b1, f32x4 c) {
  c = mfma16(a0, b0, c);
  c = mfma16(a1, b1, c);
  __builtin_amdgcn_sched_barrier(0);
  return c;
}

// Two-stage software pipeline over n steps with no branch in the steady state:
// load_a(i)/load_b(i) fill register set A/B with step i, mma_a()/mma_b() consume
// them.  Keeping the loop body branch-free lets the compiler wait only for the
// set it is about to use (vmcnt > 0) while the other set's loads stay in flight.
template <class LA, class LB, class MA, class MB>
__device__ __forceinline__ void pipeline2(int n, LA load_a, LB load_b, MA mma_a, MB mma_b) {
  // sched_barrier(0) keeps the scheduler from sinking a prefetch below the MFMAs
  // that wait on the other set, which would leave only one set in flight.
  if (n <= 0) return;
  load_a(0);
  int s = 0;
  for (; s + 2 < n; s += 2) {
    load_b(s + 1);
    __builtin_amdgcn_sched_barrier(0);
    mma_a();
    __builtin_amdgcn_sched_barrier(0);
    load_a(s + 2);
    __builtin_amdgcn_sched_barrier(0);
    mma_b();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (s + 1 < n) {
    load_b(s + 1);
    __builtin_amdgcn_sched_barrier(0);
    mma_a();
    mma_b();
  } else {
    mma_a();
  }
}

// Three-stage variant: two register sets are in flight while the third is
// consumed.  The steady-state loop is entered only after both prologue loads
// were issued unconditionally: the compiler's wait-count analysis merges every
// path into the loop header, and a path with fewer loads in flight would make
// it wait for the whole pipeline at the top of each trip.
template <class L0, class L1, class L2, class M0, class M1, class M2>
__device__ __forceinline__ void pipeline3(int n, L0 l0, L1 l1, L2 l2, M0 m0, M1 m1, M2 m2) {
  if (n <= 0) return;
  // last r = n - s steps (1..4) with steps s, s+1 (those < n) already loaded; s % 3 == 0
  auto tail = [&](int s, int r) {
    if (r >= 3) l2(s + 2);
    __builtin_amdgcn_sched_barrier(0);
    m0();
    if (r == 4) l0(s + 3);
    __builtin_amdgcn_sched_barrier(0);
    if (r >= 2) m1();
    if (r >= 3) m2();
    if (r == 4) m0();
  };
  if (n < 5) {
    l0(0);
    if (n > 1) l1(1);
    tail(0, n);
    return;
  }
  l0(0);
  l1(1);
  __builtin_amdgcn_sched_barrier(0);
  int s = 0;
  for (; s + 4 < n; s += 3) {
    l2(s + 2);
    __builtin_amdgcn_sched_barrier(0);
    m0();
    __builtin_amdgcn_sched_barrier(0);
    l0(s + 3);
    __builtin_amdgcn_sched_barrier(0);
    m1();
    __builtin_amdgcn_sched_barrier(0);
    l1(s + 4);
    __builtin_amdgcn_sched_barrier(0);
    m2();
    __builtin_amdgcn_sched_barrier(0);
  }
  tail(s, n - s);
}

// Four-stage variant: three register sets are in flight while the fourth is
// consumed; same structure as pipeline3.
template <class L0, class L1, class L2, class L3, class M0, class M1, class M2, class M3>
__device__ __forceinline__ void pipeline4(int n, L0 l0, L1 l1, L2 l2, L3 l3, M0 m0, M1 m1, M2 m2,
                                          M3 m3) {
  if (n <= 0) return;
  // last r = n - s steps (1..7) with steps s .. s+2 (those < n) already loaded; s % 4 == 0
  auto tail = [&](int s, int r) {
    if (r > 3) l3(s + 3);
    __builtin_amdgcn_sched_barrier(0);
    m0();
    if (r > 1) {
      if (r > 4) l0(s + 4);
      __builtin_amdgcn_sched_barrier(0);
      m1();
    }
    if (r > 2) {
      if (r > 5) l1(s + 5);
      __builtin_amdgcn_sched_barrier(0);
      m2();
    }
    if (r > 3) {
      if (r > 6) l2(s + 6);
      __builtin_amdgcn_sched_barrier(0);
      m3();
    }
    if (r > 4) m0();
    if (r > 5) m1();
    if (r > 6) m2();
  };
  if (n < 8) {
    l0(0);
    if (n > 1) l1(1);
    if (n > 2) l2(2);
    tail(0, n);
    return;
  }
  l0(0);
  l1(1);
  l2(2);
  __builtin_amdgcn_sched_barrier(0);
  int s = 0;
  for (; s + 7 < n; s += 4) {
    l3(s + 3);
    __builtin_amdgcn_sched_barrier(0);
    m0();
    __builtin_amdgcn_sched_barrier(0);
    l0(s + 4);
    __builtin_amdgcn_sched_barrier(0);
    m1();
    __builtin_amdgcn_sched_barrier(0);
    l1(s + 5);
    __builtin_amdgcn_sched_barrier(0);
    m2();
    __builtin_amdgcn_sched_barrier(0);
    l2(s + 6);
    __builtin_amdgcn_sched_barrier(0);
    m3();
    __builtin_amdgcn_sched_barrier(0);
  }
  tail(s, n - s);
}

// 16-byte load that bypasses cache retention (weights are streamed exactly once).
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Direct global -> LDS copy of one 1 KiB fragment tile by one wave: lane l moves
// the 16 bytes at src (its own slot of the tile) to lds_tile + 16 l, without
// passing through registers.  NT marks the source as streamed once.  Completion
// is tracked by the wave's vmcnt; the compiler does not order LDS reads after
// these copies, so callers wait (vm_wait) and barrier explicitly.
template <bool NT>
__device__ __forceinline__ void tile_to_lds(const uint16_t* src, void* lds_tile) {
  __builtin_amdgcn_global_load_lds(src, lds_tile, 16, 0, NT ? 2 : 0);
}

// The same copy issued from inline asm.  The compiler's wait-count bookkeeping then
// never sees it, which keeps its waits for the caller's ordinary loads precise (with
// LDS copies in its model it falls back to waiting for every outstanding load); the
// caller waits for the copy itself with vm_wait.  The asm writes no register, so no
// register the compiler allocates depends on the copy's completion.
__device__ __forceinline__ void tile_to_lds_untracked(const uint16_t* src, void* lds_tile) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_tile);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m)
               : "memory", "m0");
}

// LDS written only by direct copies looks never-stored to the optimizer, which may
// then drop or hoist reads of it; reading through a laundered LDS-address-space
// pointer keeps every read where it is written.
typedef __attribute__((address_space(3))) char lds_char;
__device__ __forceinline__ lds_char* lds_launder(void* p) {
  lds_char* q = (lds_char*)p;
  asm volatile("" : "+v"(q));
  return q;
}
__device__ __forceinline__ u32x4 ld16_lds(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
}

// s_waitcnt vmcnt(N): wait until at most N vector-memory loads of this wave are in flight.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroups are dispatched round-robin over the XCDs (8 on MI355X), each with
// its own L2.  xcd_swizzle(b, n) renumbers a 1-D grid of n blocks (n a multiple
// of kXcd) so that consecutive logical indices run on the same XCD: blocks that
// share data should be given consecutive logical indices.
constexpr int kXcd = 8;
__device__ __forceinline__ int xcd_swizzle(int b, int n) {
  return (b % kXcd) * (n / kXcd) + b / kXcd;
}

// ---------------------------------------------------------------- layouts
//
// Fragment-major ("F-major") layout of a bf16 matrix X[R][K] (R padded to a
// multiple of 16, K a multiple of 32): the matrix is cut into 16-row x 32-col
// tiles of 512 elements (1 KiB), stored row-block-major with the k tiles of a
// row block consecutive.  Inside a tile, lane l of a wave owns the 8 elements
// (row l%16, cols 8*(l/16) .. +7) at element offset 8*l -- exactly the operand
// fragment of v_mfma_f32_16x16x32_bf16.  Loading a fragment is therefore one
// fully contiguous 1 KiB wave load, which the vector memory path serves about
// four times faster than the 16-rows-by-64-bytes pattern of a row-major read.
__host__ __device__ __forceinline__ size_t fm_index(size_t r, int c, int K) {
  return (((r >> 4) * (size_t)(K >> 5) + (size_t)(c >> 5)) << 9) +
         ((size_t)((((c & 31) >> 3) << 4) + (int)(r & 15)) << 3) + (c & 7);
}
// Start of the fragment tile (row block rb, k block kb) plus this lane's slot.
__device__ __forceinline__ size_t fm_tile(size_t rb, int kb, int K, int lane) {
  return ((rb * (size_t)(K >> 5) + (size_t)kb) << 9) + ((size_t)lane << 3);
}

// Key cache of one (layer, sequence, kv head): positions in chunks of 32, each
// chunk two 16-key blocks (bb) whose row r holds key 8*(r/4) + 4*bb + r%4 of
// the chunk, hd split in 32-wide k tiles.  With that key order, the scores a
// lane receives from S^T = K Q^T are 8 consecutive keys of the chunk, which is
// the lane's operand fragment for O^T += V^T P^T.
__host__ __device__ __forceinline__ size_t k_index(int p, int c, int hd) {
  const int pp = p & 31, bb = (pp >> 2) & 1, r = ((pp >> 3) << 2) | (pp & 3);
  return (((size_t)((p >> 5) * 2 + bb) * (size_t)(hd >> 5) + (size_t)(c >> 5)) << 9) +
         ((size_t)((((c & 31) >> 3) << 4) + r) << 3) + (c & 7);
}
// Value cache, stored transposed: for each 32-key chunk and 16-wide hd block, a
// tile whose lane l holds V[keys 8*(l/16) .. +7 of the chunk][hd row l%16].
__host__ __device__ __forceinline__ size_t v_index(int p, int c, int hd) {
  return (((size_t)(p >> 5) * (size_t)(hd >> 4) + (size_t)(c >> 4)) << 9) +
         ((size_t)((((p & 31) >> 3) << 4) + (c & 15)) << 3) + (p & 7);
}

// Work-unit schedule for the grouped expert GEMMs: n_items work items x nfb
// feature tiles, numbered item-major (u = item * nfb + fb).  XCD x (= blockIdx.x %
// kXcd) owns the contiguous range [x*T/kXcd, (x+1)*T/kXcd) of the T = n_items * nfb
// units, so every XCD gets the same number of workgroups to within one, the feature
// tiles of an item run back to back on one XCD (its token rows stay in that L2), and
// the neighbouring items of one expert -- consecutive in the list -- share weight
// tiles there.  Returns false for blocks beyond this XCD's share; the grid needs
// kXcd * ceil(T / kXcd) blocks.
__device__ __forceinline__ bool xcd_item_schedule(int n_items, int nfb, int* item, int* fb) {
  const int x = blockIdx.x % kXcd, rank = blockIdx.x / kXcd;
  const long T = (long)n_items * nfb;
  const long u0 = (long)x * T / kXcd, u1 = (long)(x + 1) * T / kXcd;
  if (rank >= u1 - u0) return false;
  const int u = (int)(u0 + rank);
  *item = u / nfb;
  *fb = u - *item * nfb;
  return true;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Block-wide sum of one float per thread (blockDim.x multiple of 64, <= 1024);
// fixed reduction tree, so the result is deterministic.  `red` needs 16 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}

}  // namespace dg
