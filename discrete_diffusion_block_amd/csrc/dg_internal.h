// Internal launchers of the engine's kernels (not part of the C ABI).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "dg.h"

namespace dg {

// Geometry of one transformer pass: `batch` sequences of `n` tokens each; row
// m = b * n + i holds token i of sequence b at position len[b] + i.
struct PassGeom {
  int batch;
  int n;
  int denoise;               // 1: some sequence denoises its canvas (the pass ends in the head)
  uint64_t enc;              // bit b: sequence b runs the causal encoder (prefill / KV update);
                             // the others the bidirectional denoiser over the cached prefix
  int len[DG_MAX_BATCH];
  float t[DG_MAX_BATCH];     // denoising time of each denoising sequence
  int kvshift[DG_MAX_BATCH]; // pass sequence b keeps its keys/values in cache sequence
                             // b - kvshift[b] (0: its own; a pass may run two segments of
                             // one cached sequence as two pass sequences)
};
__host__ __device__ inline int kv_seq(const PassGeom& g, int b) { return b - g.kvshift[b]; }
__host__ __device__ inline bool seq_encodes(const PassGeom& g, int b) { return (g.enc >> b) & 1; }
inline uint64_t all_sequences(int batch) { return batch >= 64 ? ~0ull : ((1ull << batch) - 1); }

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

// Raises a kernel's dynamic-LDS limit to `bytes` on the current device, once per
// device (the attribute is per device; each device gets its own bit).  Safe to call
// from several threads: a second concurrent setter repeats an idempotent call.
struct LdsLimit {
  std::atomic<uint64_t> devices{0};
};
inline void raise_lds_limit(LdsLimit& st, const void* fn, int bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return;
  const uint64_t bit = 1ull << (dev & 63);
  if (st.devices.load(std::memory_order_acquire) & bit) return;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess)
    st.devices.fetch_or(bit, std::memory_order_release);
}

// ---- embed / norm / prep ----
// also clears zero[0 .. nzero)
void launch_prep(const PassGeom& g, int hd, float theta, float2* rope_tab, int d,
                 float* temb, int32_t* zero, int nzero, hipStream_t s);
// temb (optional): [batch][d], sequence b's timestep embedding, added to the rows of the
// sequences whose bit in enc is clear (rows m = b * n + i); z (optional): the
// self-conditioning signal, fp32 row-major [M][d], added to the same rows
void launch_embed_norm(const int32_t* tokens, const uint16_t* embed, const float* temb, const float* z,
                       int n, uint64_t enc, const float* gain, float eps, float* x, uint16_t* h, int M, int d,
                       int vocab, hipStream_t s);
// h: fragment-major; h_rm (optional): the same values row-major [M][d]
void launch_rmsnorm(const float* x, const float* gain, float eps, uint16_t* h, uint16_t* h_rm, int M,
                    int d, hipStream_t s, hipEvent_t done = nullptr);
// rows_out given: only the [MASK] rows of canvas (mask id mask_id) are normed,
// compacted into h (the order of arrival); rows_out lists their row indices and
// *count (zero on entry) their number
// rows_out given: only the rows of sequences whose bit in skip is clear (rows m = b * n +
// i), and of those only the [MASK] rows when canvas is given, are normed, compacted
void launch_combine(float* x, const float* ys, const float* Y, const float* wts, const int32_t* inv,
                    int M, int k, int d, const float* next_gain, float eps, uint16_t* h,
                    const int32_t* canvas, int mask_id, uint64_t skip, int n, int32_t* rows_out, int32_t* count,
                    int row_base, hipStream_t s);

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
// split-KV partials: nsplit * batch * (queries rounded up to 32) stays within this many
// rows per q head (part_o holds kAttnMaxSplitRows * hq * hd floats, part_ml as many
// float2 / hd); part_o NULL: no split
constexpr int kAttnMaxSplitRows = 4096;
void launch_attention(const uint16_t* q, int hq, const KvLayer& kv, const PassGeom& g, uint16_t* o,
                      float* part_o, float2* part_ml, hipStream_t s);

// ---- MoE ----
void launch_topk(const float* r, int M, int E, int k, int32_t* ids, float* w, hipStream_t s);
// the given expert ids (forced [M][k]) in place of the top-k; weights from r
void launch_forced_route(const float* r, int M, int E, int k, const int32_t* forced, int32_t* ids, float* w,
                         hipStream_t s);
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
// Fragment-major copy of the transpose of row-major src [rows][cols]: packed [cols][rows].
void launch_pack_transpose(const uint16_t* src, uint16_t* dst, int rows, int cols, hipStream_t s);

// ---- sampler ----
constexpr int kSampleChunk = 16384;  // logits per workgroup in the first sampler pass (multiple of 2048)
// inv_tau = 1 / sampling temperature (1 = the plain distribution).  all_rows: every
// row is a candidate (uniform variant), except those of sequences with frozen[b] != 0
// (frozen optional); otherwise the [MASK] rows.
void launch_sample_partials(const uint16_t* logits, const int32_t* canvas, int batch, int C, int vocab,
                            float inv_tau, int all_rows, const int32_t* frozen, float4* part, int* part_arg,
                            hipStream_t s);
// A canvas [batch][C] of the uniformly random tokens of (seed, draw).
void launch_uniform_canvas(int32_t* canvas, int batch, int C, int vocab, uint64_t seed, int draw, hipStream_t s);
// Pass 2: merge the chunk partials (part given) or take the given entropies and
// argmaxes (H_in / amax_in), rank, and commit.  prev_amax (optional, [batch][C]
// in/out): the previous step's argmax, for the adaptive stop at e_stop; done_step
// (optional, [batch]): set to step + 1 where it is 0 and the call leaves no [MASK]
// row.  With part given and flag non-NULL, a sequence whose decision is not
// certified under the fast entropies' error bound is left undecided: flag[b] = 1,
// moved[b] = its count of moved argmaxes, amax_ws = its argmaxes (for the canonical
// passes below); decided sequences get flag[b] = 0.  uniform: every row of a sequence
// whose done_step is 0 is a candidate, and the decided sequences' rows outside the
// accepted set take the uniformly random tokens of (seed, draw); done_step is set when
// the stop fires or its commit bit is set.  commit: bit b set = sequence b commits every
// candidate row (the last step of a block).
void launch_eb_select(const float4* part, const int* part_arg, int nchunks, const float* H_in,
                      const int32_t* amax_in, int32_t* canvas, int batch, int C, int vocab,
                      float gamma, uint64_t commit, float* H_out, int32_t* amax_out,
                      int32_t* n_masked, int32_t* prev_amax, float e_stop, int step, int32_t* done_step,
                      int32_t* flag, int32_t* moved, int32_t* amax_ws, float* Hf_ws, float2* win,
                      int32_t* kstar_ws, int uniform, uint64_t seed, int draw, hipStream_t s);
// Pass 3: exact integer sums of the canonical entropy for the masked rows of the
// flagged sequences -- all of them (flag 1) or those whose fast entropy Hf lies in the
// sequence's window win (flag 2) (tau: the temperature; part: pass 1's partials, for
// the row max).
void launch_canon_partials(const uint16_t* logits, const int32_t* canvas, int batch, int C, int vocab,
                           float tau, int all_rows, const float4* part, const int32_t* flag, const float* Hf,
                           const float2* win, ulonglong2* cpart, hipStream_t s);
// Pass 4: the decision of the flagged sequences on the canonical entropy.
void launch_eb_select_canon(const ulonglong2* cpart, int nchunks, int32_t* canvas, int batch, int C, int vocab,
                            float gamma, uint64_t commit, float* H_out, int32_t* amax_out, int32_t* n_masked,
                            int32_t* prev_amax, float e_stop, int step, int32_t* done_step,
                            int32_t* flag, int32_t* moved, int32_t* amax_ws, float* Hf_ws, float2* win,
                            int32_t* kstar_ws, int uniform, uint64_t seed, int draw, hipStream_t s);
// ---- self-conditioning (p̂₀ = softmax of each logits row, u = p̂₀ E, z = FFW(u)) ----
// k slices of the p̂₀ E product for M rows, N = d features, K = V (the partial buffer
// holds sc_splits * M * N floats).
int sc_splits(int M, int N, int K);
// stats[m] = (m log2e, 1 / S): the row maximum and the softmax denominator, fp32.
void launch_sc_rowstats(const uint16_t* logits, int M, int V, float2* stats, hipStream_t s);
// part[split][m][n] = sum over the split's k of exp(x_mk - max_m) E^T[n][k]; et: E^T
// packed fragment-major ([N][K]).
void launch_sc_embed(const uint16_t* logits, const float2* stats, const uint16_t* et, int M, int N, int K,
                     float* part, hipStream_t s);
// u = (sum of the partials) / S: bf16 fragment-major into u_fm, fp32 row-major into
// u_out when given.
void launch_sc_reduce(const float* part, int nsplit, const float2* stats, int M, int N, uint16_t* u_fm,
                      float* u_out, hipStream_t s);
void launch_copy16(const void* src, void* dst, size_t n_bytes, hipStream_t s);
// blocks x 256 threads, iters rounds of 4 dependent MFMA pairs per wave; out: blocks * 256 floats
void launch_mfma_rate(int blocks, int iters, float* out, hipStream_t s);
// streaming read of n_bytes (multiple of 16) by blocks x 256 threads; out: blocks * 256 words
void launch_read_rate(const void* src, size_t n_bytes, int blocks, uint32_t* out, hipStream_t s);
// A per-sequence element offset, passed by value.
struct SeqOffsets {
  int64_t v[DG_MAX_BATCH];
};
// For each sequence with its bit in enc set: copy its canvas row to out + off.v[b] (out
// may be NULL) and refill the row with mask_id.
void launch_serve_finish(int32_t* canvas, int batch, int C, int32_t mask_id, uint64_t enc, int32_t* out,
                         const SeqOffsets& off, hipStream_t s);
void launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t s);

}  // namespace dg
