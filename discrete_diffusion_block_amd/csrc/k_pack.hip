// One-time weight packing: row-major bf16 matrices -> fragment-major tiles,
// with the row orders the GEMM epilogues expect baked in.
//  * plain:   packed row p = source row p (rows past R are zero).
//  * qkv:     within each head of hd rows, packed 16-row block j row r holds
//             source feature 8j + 2(r/4) + r%2 + ((r/2)%2) * hd/2, so a lane's
//             four output rows are the rotary pairs (i, i+hd/2), (i+1, i+1+hd/2).
//  * gate_up: packed block 2t = gate rows 16t.., block 2t+1 = up rows F+16t..,
//             so one 32-row wave tile carries matching gate and up features.
//  * transpose: the packed matrix is the source's transpose (the embedding as the
//             k-major operand of the self-conditioning product).
#include "dg_common.h"
#include "dg_internal.h"

namespace dg {

__device__ __forceinline__ int packed_source_row(int kind, int p, int param) {
  if (kind == 1) {  // qkv, param = head_dim
    const int hd = param, head = p / hd, q = p - head * hd;
    const int j = q >> 4, r = q & 15;
    return head * hd + 8 * j + 2 * (r >> 2) + (r & 1) + ((r >> 1) & 1) * (hd >> 1);
  }
  if (kind == 2) {  // gate_up, param = F
    const int t = p >> 5, q = (p >> 4) & 1, r = p & 15;
    return q * param + 16 * t + r;
  }
  return p;
}

// One thread per 8 consecutive columns of one packed row.
__global__ void pack_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int nmat,
                            int R, int K, int Rpad, int kind, int param) {
  const size_t per_mat = (size_t)Rpad * (K >> 3);
  const size_t total = per_mat * nmat;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const int mat = (int)(i / per_mat);
    const size_t rem = i - (size_t)mat * per_mat;
    const int p = (int)(rem / (K >> 3));
    const int c = (int)(rem - (size_t)p * (K >> 3)) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (p < R) {
      const int srow = packed_source_row(kind, p, param);
      v = ld16(src + ((size_t)mat * R + srow) * K + c);
    }
    *reinterpret_cast<u32x4*>(dst + (size_t)mat * Rpad * K + fm_index(p, c, K)) = v;
  }
}

void launch_pack(const uint16_t* src, uint16_t* dst, int nmat, int R, int K, int kind, int param,
                 hipStream_t s) {
  const int Rpad = (R + 15) / 16 * 16;
  const size_t total = (size_t)nmat * Rpad * (K / 8);
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
  launch_kernel(pack_kernel, dim3(blocks), dim3(256), 0, s, nullptr, src, dst, nmat, R, K, Rpad, kind, param);
}

// One thread per 8 consecutive packed columns (source rows c .. c + 7) of one packed
// row p (source column p); one-time work, so the strided gather is acceptable.
__global__ void pack_transpose_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int rows,
                                      int cols, int Rpad) {
  const size_t total = (size_t)Rpad * (rows >> 3);
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % (size_t)(rows >> 3)) * 8;
    const int p = (int)(i / (size_t)(rows >> 3));
    u32x4 v = {0u, 0u, 0u, 0u};
    if (p < cols) {
      uint16_t e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = src[(size_t)(c + j) * cols + p];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (uint32_t)e[2 * j] | ((uint32_t)e[2 * j + 1] << 16);
    }
    *reinterpret_cast<u32x4*>(dst + fm_index(p, c, rows)) = v;
  }
}

void launch_pack_transpose(const uint16_t* src, uint16_t* dst, int rows, int cols, hipStream_t s) {
  const int Rpad = (cols + 15) / 16 * 16;
  const size_t total = (size_t)Rpad * (rows / 8);
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
  launch_kernel(pack_transpose_kernel, dim3(blocks), dim3(256), 0, s, nullptr, src, dst, rows, cols, Rpad);
}

// Row-major bf16 activations -> fragment-major (test tap support).
void launch_pack_rows(const uint16_t* src, uint16_t* dst, int R, int K, hipStream_t s) {
  launch_pack(src, dst, 1, R, K, 0, 0, s);
}

}  // namespace dg
