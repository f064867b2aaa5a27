// Internal launchers of the engine's kernels (not part of the C ABI).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dg.h"

namespace dg {

// Geometry of one transformer pass: `batch` sequences of `n` tokens each; row
// m = b * n + i holds token i of sequence b at position len[b] + i.
struct PassGeom {
  int batch;
  int n;
  int denoise;               // 1: bidirectional canvas over the cached prefix; 0: causal encoder
  int len[DG_MAX_BATCH];
};

// KV-cache view of one layer.
struct KvLayer {
  uint16_t* k;               // [max_batch][Hkv][max_ctx][hd]
  uint16_t* vt;              // [max_batch][Hkv][hd][max_ctx]
  int hkv, hd, max_ctx;
  int window;                // 0 = global layer
};

// Every kernel launch goes through launch_kernel.  The engine's profiler may park a
// timing event in next_launch_events(); the next launch then has it signalled by
// its own completion (no marker packet after the kernel) and clears it.  `done`
// (optional) is likewise signalled by the kernel's completion, for another stream
// to wait on.
struct LaunchEvents {
  hipEvent_t stop = nullptr;
};
inline LaunchEvents& next_launch_events() {
  static thread_local LaunchEvents e;
  return e;
}
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                          hipEvent_t done, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
  LaunchEvents& ev = next_launch_events();
  hipEvent_t stop = done;
  if (ev.stop) {
    stop = ev.stop;
    ev = LaunchEvents{};
  }
  hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, nullptr, stop, 0u, static_cast<KArgs>(args)...);
  if (done && stop != done) (void)hipEventRecord(done, s);
}

// ---- embed / norm / prep ----
// also clears zero[0 .. nzero)
void launch_prep(const PassGeom& g, int hd, float theta, float2* rope_tab, int d, float t,
                 float* temb, int32_t* zero, int nzero, hipStream_t s);
void launch_embed_norm(const int32_t* tokens, const uint16_t* embed, const float* temb,
                       const float* gain, float eps, float* x, uint16_t* h, int M, int d, int vocab,
                       hipStream_t s);
// h: fragment-major; h_rm (optional): the same values row-major [M][d]
void launch_rmsnorm(const float* x, const float* gain, float eps, uint16_t* h, uint16_t* h_rm, int M,
                    int d, hipStream_t s, hipEvent_t done = nullptr);
// rows_out given: only the [MASK] rows of canvas (mask id mask_id) are normed,
// compacted into h (the order of arrival); rows_out lists their row indices and
// *count (zero on entry) their number
void launch_combine(float* x, const float* ys, const float* Y, const float* wts, const int32_t* inv,
                    int M, int k, int d, const float* next_gain, float eps, uint16_t* h,
                    const int32_t* canvas, int mask_id, int32_t* rows_out, int32_t* count, hipStream_t s);

// ---- dense GEMMs ----
// y = x . w^T with fp32 output (store) or fp32 accumulate into y (add).
void launch_gemm_f32(const uint16_t* x, const uint16_t* w, float* y, int M, int N, int K,
                     bool add, hipStream_t s,
                     hipEvent_t done = nullptr);
// q/k/v projection with RoPE; q -> q_out [M][Hq][hd], k/v -> cache at the pass positions.
void launch_qkv_rope(const uint16_t* h, const uint16_t* w_qkv, int M, int K, int hq,
                     const KvLayer& kv, const PassGeom& g, const float2* rope_tab,
                     uint16_t* q_out, hipStream_t s);
// shared-expert gate/up projection with fused SwiGLU: a[M][F] = silu(h Wg^T) * (h Wu^T).
void launch_gemm_swiglu(const uint16_t* h, const uint16_t* w_gate_up, int M, int F, int K,
                        uint16_t* a, hipStream_t s);
// tied LM head: logits bf16 [M][N] = h . E[0:N]^T
// count given: h holds *count rows compacted, rows[i] the logits row of row i
void launch_gemm_head(const uint16_t* h, const uint16_t* embed, uint16_t* logits, int M, int N,
                      int K, const int32_t* count, const int32_t* rows, hipStream_t s);

// ---- attention ----
void launch_attention(const uint16_t* q, int hq, const KvLayer& kv, const PassGeom& g,
                      uint16_t* o, hipStream_t s);

// ---- MoE ----
void launch_topk(const float* r, int M, int E, int k, int32_t* ids, float* w, hipStream_t s);
constexpr int kMoeGroup = 64;        // tokens per work item of the routing test tap's list
constexpr int kMoeGroup2 = 128;      // tokens per expert GEMM work item
int moe_max_items(int M, int k, int E);
int moe_max_items2(int M, int k, int E);
int moe_max_slots(int M, int k, int E);   // padded slot space: M*k + 15*E
// items: (expert, first token) of every kMoeGroup-token group; items2 (optional)
// the same for kMoeGroup2-token groups
void launch_route(const int32_t* ids, int M, int k, int E, int32_t* cnt, int32_t* poff,
                  int32_t* perm, int32_t* inv, int2* items, int32_t* n_items, int2* items2,
                  int32_t* n_items2, int32_t* cnt_log, hipStream_t s);

// x rows are gathered per slot from h_rm (row-major [M][d]) through perm; work
// items of kMoeGroup2 tokens
void launch_moe_gate_up(const uint16_t* h_rm, const int32_t* perm, const uint16_t* w_gate_up,
                        const int32_t* cnt, const int32_t* poff, const int2* items2,
                        const int32_t* n_items2, int max_items2, int F, int d, uint16_t* a,
                        hipStream_t s);
// work items of kMoeGroup2 tokens
void launch_moe_down(const uint16_t* a, const uint16_t* w_down, const int32_t* cnt,
                     const int32_t* poff, const int2* items2, const int32_t* n_items2, int max_items2,
                     int F, int d, float* Y, hipStream_t s);

// ---- weight packing ----
void launch_pack(const uint16_t* src, uint16_t* dst, int nmat, int R, int K, int kind, int param,
                 hipStream_t s);

// ---- sampler ----
constexpr int kSampleChunk = 16384;  // logits per workgroup in the first sampler pass (multiple of 2048)
// inv_tau = 1 / sampling temperature (1 = the plain distribution)
void launch_sample_partials(const uint16_t* logits, const int32_t* canvas, int rows, int vocab,
                            float inv_tau, float4* part, int* part_arg, hipStream_t s);
// prev_amax (optional, [batch][C] in/out): the previous step's argmax, for the
// adaptive stop at e_stop; done_step (optional, [batch]): set to step + 1 where it is
// 0 and the call leaves no [MASK] row
void launch_eb_select(const float4* part, const int* part_arg, int nchunks, const float* H_in,
                      const int32_t* amax_in, int32_t* canvas, int batch, int C, int vocab,
                      float gamma, int commit_all, float* H_out, int32_t* amax_out,
                      int32_t* n_masked, int32_t* prev_amax, float e_stop, int step, int32_t* done_step,
                      hipStream_t s);
void launch_copy16(const void* src, void* dst, size_t n_bytes, hipStream_t s);
void launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t s);

}  // namespace dg
