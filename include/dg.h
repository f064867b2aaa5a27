/*
 * dg.h — C ABI of the block-parallel diffusion denoising engine (MI355X / gfx950).
 *
 * The engine implements the inference hot path of block diffusion decoding as
 * described in the DiffusionGemma Technical Report (§3.1 block-AR generation,
 * §3.2 the denoising framework at inference time, §3.3 the entropy-bounded
 * sampler) with the architecture listed in "DiffusionGemma 深度解析" (core
 * architecture parameters: 30 layers, sliding window 1024, canvas 256, vocab
 * 262K, 128 experts with top-8 routing plus one shared expert, absorbing [MASK]
 * whose id equals the vocabulary size, timestep embedding on the decoder input).
 *
 * Conventions shared by every call:
 *  - Pointers named d_* are device memory owned by the caller.  bf16 tensors are
 *    passed as uint16_t (raw bfloat16 bits), row-major, contiguous.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it: it never synchronises the host, never allocates and
 *    never frees.  Device-side faults surface at the caller's next sync.
 *  - Arguments and shapes are validated before anything is enqueued; on an
 *    error nothing is written and the status says why (dg_last_error() gives a
 *    thread-local detail string).
 *  - Token ids are int32; [MASK] = vocab.  Canvas tokens that are not [MASK]
 *    are committed and are never changed by any call.
 *  - A dg_ctx is immutable after dg_create and may be shared by threads; calls
 *    that run concurrently need distinct workspaces and KV caches.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DG_MAX_BATCH 64

typedef enum dg_status {
  DG_OK = 0,
  DG_ERR_INVALID_ARG = -1,   /* NULL pointer, negative size, out-of-range value */
  DG_ERR_SHAPE = -2,         /* a model dimension the kernels do not support */
  DG_ERR_WORKSPACE = -3,     /* workspace smaller than dg_workspace_size() */
  DG_ERR_KV_CAPACITY = -4,   /* the pass would write beyond max_ctx */
  DG_ERR_HIP = -5,           /* a HIP launch failed (detail in dg_last_error) */
  DG_ERR_UNSUPPORTED = -6
} dg_status;

/* Model shapes.  Supported: d_model % 64 == 0, head_dim in {32, 64, 128},
 * n_q_heads % n_kv_heads == 0, expert_ffn % 64 == 0, shared_ffn % 64 == 0,
 * n_experts <= 256, top_k <= min(n_experts, 16), canvas <= 1024,
 * max_ctx % 64 == 0, 1 <= max_batch <= DG_MAX_BATCH. */
typedef struct dg_config {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim;
  int32_t n_experts, top_k, expert_ffn, shared_ffn;
  int32_t vocab;         /* V; the [MASK] token id is V (embedding has V+1 rows) */
  int32_t canvas;        /* C, tokens denoised in parallel per sequence */
  int32_t window;        /* sliding-window length W of non-global layers */
  int32_t global_every;  /* 0: all layers slide; g > 0: layer l is global iff (l+1) % g == 0 */
  int32_t max_batch, max_ctx;
  float rms_eps, rope_theta;
} dg_config;

/* Weight packing.  The engine reads every bf16 weight matrix in a
 * fragment-major layout: 16-row x 32-column tiles of 1 KiB, row-block-major,
 * the 8 elements (row l%16, columns 8*(l/16)..+7) of a tile at element offset
 * 8*l -- the operand fragment of one MFMA for lane l -- so each fragment is one
 * contiguous wave load.  Rows are padded to a multiple of 16 (with zeros).
 * dg_pack_weight converts n_mats consecutive row-major [rows][cols] matrices
 * into that layout (dst holds n_mats * dg_packed_elems(rows, cols) elements):
 *   DG_PACK_PLAIN    rows in order;
 *   DG_PACK_QKV      param = head_dim: within each head the rows are ordered so
 *                    that each lane receives the rotary pairs (i, i + hd/2);
 *   DG_PACK_GATE_UP  param = F, rows = 2F: 16-row block 2t = gate rows 16t..,
 *                    block 2t+1 = up rows F+16t..
 * The source is not modified; the call only enqueues a kernel on `stream`. */
typedef enum dg_pack_kind { DG_PACK_PLAIN = 0, DG_PACK_QKV = 1, DG_PACK_GATE_UP = 2 } dg_pack_kind;
dg_status dg_packed_elems(int rows, int cols, size_t* elems);
dg_status dg_pack_weight(int kind, const uint16_t* d_src, uint16_t* d_dst, int n_mats, int rows,
                         int cols, int param, void* stream);

/* Weights of one layer (device pointers, borrowed for the ctx's lifetime).
 * Norm gains are fp32 [d]; every matrix is bf16, packed with dg_pack_weight
 * from the row-major shape given here. */
typedef struct dg_layer_weights {
  const float* attn_norm;      /* fp32 [d] RMSNorm gain before attention */
  const uint16_t* w_qkv;       /* QKV-packed [(Hq + 2 Hkv) * hd][d]: q heads, k heads, v heads */
  const uint16_t* w_o;         /* plain-packed [d][Hq * hd] */
  const float* ffn_norm;       /* fp32 [d] RMSNorm gain before the MoE block */
  const uint16_t* w_router;    /* plain-packed [E][d] (rows padded to 16) */
  const uint16_t* w_gate_up;   /* GATE_UP-packed, E matrices [2F][d] (F gate rows, F up rows) */
  const uint16_t* w_down;      /* plain-packed, E matrices [d][F] */
  const uint16_t* ws_gate_up;  /* shared expert, GATE_UP-packed [2Fs][d] */
  const uint16_t* ws_down;     /* shared expert, plain-packed [d][Fs] */
} dg_layer_weights;

typedef struct dg_weights {
  const uint16_t* embed;              /* plain-packed [V+1][d]; tied: logits use rows 0..V-1 */
  const float* final_norm;            /* fp32 [d] */
  const dg_layer_weights* layers;     /* HOST array of n_layers entries (copied by dg_create) */
} dg_weights;

/* KV cache (caller-owned device buffers, zero-filled before first use), each
 * n_layers * max_batch * n_kv_heads blocks of max_ctx * head_dim bf16, in the
 * block order [layer][sequence][kv head].  Inside a block:
 *   k (post-RoPE keys): 32-position chunks, each two 16-row tiles per 32-wide
 *     hd slice; position p of a chunk is row 4*(p/8) + p%4 of tile (p/4)%2,
 *     element (row r, dim c) of a tile at 8*(16*((c%32)/8) + r) + c%8;
 *   v (values, transposed): per 32-position chunk and 16-wide hd slice a tile
 *     with element (position p, dim c) at 8*(16*((p%32)/8) + c%16) + p%8.
 * (Both are the MFMA operand fragments of the attention kernel.)
 * len[b] is the host-side count of committed positions of sequence b; the
 * library advances it when it enqueues a prefill/append, so no device read-back
 * is ever needed.  Slots len[b] .. len[b]+C-1 also serve as scratch for the
 * canvas keys/values of a denoising step. */
typedef struct dg_kv {
  uint16_t* k;
  uint16_t* v;
  int64_t len[DG_MAX_BATCH];
} dg_kv;

typedef struct dg_ctx dg_ctx;

/* Create an engine for cfg with the given weights (pointers are borrowed; the
 * dg_layer_weights array itself is copied).  Validates shapes.  Allocates only
 * the ctx's host-side state. */
dg_status dg_create(const dg_config* cfg, const dg_weights* w, dg_ctx** out);
void dg_destroy(dg_ctx* ctx);

/* Bytes of device workspace needed by any call on `batch` sequences. */
dg_status dg_workspace_size(const dg_ctx* ctx, int batch, size_t* bytes);
/* Bytes of each of the k and v cache buffers for cfg. */
dg_status dg_kv_size(const dg_config* cfg, size_t* bytes_each);

const char* dg_status_string(dg_status s);
const char* dg_last_error(void);

/* Causal encoder pass (DiffusionGemma Technical Report §3.1, context encoding
 * into the KV cache, eq. 3; and the append of a finished canvas, eq. 4).
 * d_tokens: int32 [batch][n], ids in [0, V].  Token i of sequence b sits at
 * position kv->len[b] + i; key j is visible to query i iff j <= i and (global
 * layer or i - j < W).  Writes K/V of those positions in every layer and
 * advances kv->len[b] by n.  Long inputs are processed in chunks (causal
 * encoding splits exactly).  Errors: DG_ERR_KV_CAPACITY if len+n > max_ctx. */
dg_status dg_prefill_kv(dg_ctx* ctx, dg_kv* kv, const int32_t* d_tokens, int batch, int n,
                        void* d_ws, size_t ws_bytes, void* stream);

/* One denoising forward pass of the bidirectional decoder (Technical Report
 * §3.2 decoder forward pass; "DiffusionGemma 深度解析": timestep embedding).
 * d_canvas: int32 [batch][C] (committed ids or [MASK]); t in [0, 1] is the
 * diffusion time whose sinusoidal embedding is added to the canvas inputs.
 * Canvas query c of sequence b sits at position len[b] + c and sees the last
 * min(len[b], W) cached keys of a sliding layer (all len[b] of a global layer)
 * plus all C canvas keys.  Output d_logits: bf16 [batch][C][V].
 * Errors: DG_ERR_KV_CAPACITY if len[b] + C > max_ctx. */
dg_status dg_denoise_step(dg_ctx* ctx, const dg_kv* kv, const int32_t* d_canvas, int batch,
                          float t, uint16_t* d_logits, void* d_ws, size_t ws_bytes, void* stream);

/* Entropy-bounded unmasking (Technical Report §3.3).  For every [MASK] row of
 * d_logits (bf16 [batch][canvas][vocab]): H = -sum p log p of softmax(row) and
 * the argmax (lowest id among exact maxima).  Masked positions are ordered by
 * (H asc, position asc); with S_k the running fp64 sum of H (fp32 values) in
 * that order, the first k* = max(1, max{k : S_k <= gamma}) positions get their
 * argmax committed (all of them when commit_all != 0).  Rows that are not
 * [MASK] are neither read nor written.
 * Outputs: d_canvas updated in place; d_entropy (fp32 [batch][canvas], NaN on
 * rows that were not masked) and d_argmax (int32, -1 on such rows) may be NULL;
 * d_n_masked (int32 [batch]) = masked rows left after the commit.
 * Workspace: dg_sample_workspace_size().  Needs no ctx. */
dg_status dg_sample_workspace_size(int batch, int canvas, int vocab, size_t* bytes);
dg_status dg_sample_eb(const uint16_t* d_logits, int32_t* d_canvas, int batch, int canvas,
                       int vocab, float gamma, int commit_all, float* d_entropy,
                       int32_t* d_argmax, int32_t* d_n_masked, void* d_ws, size_t ws_bytes,
                       void* stream);

/* dg_sample_eb with the two extras of the Technical Report's default sampler (§3.3):
 *  - temperature annealing: H is the entropy of softmax(row / temperature)
 *    (temperature finite and > 0; 1 gives dg_sample_eb; the argmax does not depend
 *    on it);
 *  - adaptive stopping, when d_prev_argmax (int32 [batch][canvas], in/out) is not
 *    NULL: it holds the previous step's argmax of every row (-1 where there was
 *    none: fill it with -1 before a block's first step) and is overwritten with
 *    this step's (-1 on rows that were not [MASK]).  A sequence whose [MASK] rows
 *    have a mean H (fp64) below e_stop and every argmax equal to the previous
 *    step's commits all of them in this call.
 * d_done_step (int32 [batch], may be NULL): an entry that is 0 is set to step + 1
 * when this call leaves its sequence with no [MASK] row.  Other arguments, outputs
 * and the workspace as for dg_sample_eb.  Errors: DG_ERR_INVALID_ARG for a
 * temperature that is not finite and > 0, a NaN gamma or e_stop, or step < 0. */
dg_status dg_sample_eb_ex(const uint16_t* d_logits, int32_t* d_canvas, int batch, int canvas,
                          int vocab, float gamma, int commit_all, float temperature, float e_stop,
                          int32_t* d_prev_argmax, int step, int32_t* d_done_step,
                          float* d_entropy, int32_t* d_argmax, int32_t* d_n_masked, void* d_ws,
                          size_t ws_bytes, void* stream);

/* Generate one block per sequence (Technical Report §3.1–§3.3): fill d_canvas
 * (int32 [batch][C]) with [MASK]; for s = 0..steps-1 run the denoising pass at
 * t_s = 1 - s/steps and dg_sample_eb (commit_all on the last step); then, if
 * append_kv, run the causal append pass over the finished canvas (len += C).
 * The denoising passes here compute the head only for the rows that are still
 * [MASK] (the only rows the sampler reads; committed tokens are never revised),
 * so the head's work shrinks as the block fills in.
 * d_logits: bf16 [batch][C][V] scratch owned by the caller; row c holds the
 * logits of the last step in which position c was [MASK].  d_n_masked: int32
 * [batch], holds the masked count after the last step (0). */
dg_status dg_generate_block(dg_ctx* ctx, dg_kv* kv, int32_t* d_canvas, int batch, int steps,
                            float gamma, int append_kv, uint16_t* d_logits, int32_t* d_n_masked,
                            void* d_ws, size_t ws_bytes, void* stream);

/* dg_generate_block with the Technical Report's default sampler (§3.3) on the
 * absorbing canvas: up to max_steps steps at t_s = 1 - s/max_steps, entropies at
 * the temperature tau_min + (tau_max - tau_min) t_s (annealed linearly from tau_max
 * to tau_min; both finite and > 0), and the adaptive stop with threshold e_stop
 * (< 0: off; see dg_sample_eb_ex), which commits a sequence's remaining positions
 * at once; the last step commits whatever is left.  d_done_step (int32 [batch],
 * out): the number of steps after which each canvas was complete.  The previous
 * argmax lives in the workspace.  Once a canvas is complete its later steps change
 * nothing, but their denoising passes still run: nothing is skipped on the device
 * and the host never waits. */
dg_status dg_generate_block_ex(dg_ctx* ctx, dg_kv* kv, int32_t* d_canvas, int batch, int max_steps,
                               float gamma, float tau_max, float tau_min, float e_stop,
                               int append_kv, uint16_t* d_logits, int32_t* d_n_masked,
                               int32_t* d_done_step, void* d_ws, size_t ws_bytes, void* stream);

/* ---- measurement helpers (diagnostics; not thread-safe) ---- */

/* Kernel kinds the engine launches, for per-kind event timing. */
typedef enum dg_kernel_kind {
  DG_K_PREP = 0, DG_K_EMBED, DG_K_QKV, DG_K_ATTENTION, DG_K_O_PROJ, DG_K_NORM, DG_K_ROUTER,
  DG_K_TOPK, DG_K_ROUTE, DG_K_MOE_GATE_UP, DG_K_MOE_DOWN, DG_K_SHARED_GATE_UP, DG_K_SHARED_DOWN,
  DG_K_COMBINE, DG_K_HEAD, DG_K_SAMPLE_PASS1, DG_K_SAMPLE_SELECT, DG_K_FILL,
  DG_K_COUNT
} dg_kernel_kind;

/* Start timing the kernel launches made through ctx (dg_prefill_kv,
 * dg_denoise_step, dg_generate_block), up to `capacity` launches (events are
 * created here).  Each timed launch gets a start event recorded on its stream
 * just ahead of it (it fires as the stream's previous work completes) and a stop
 * event signalled by the kernel's own completion.  kind_mask selects the kinds
 * timed (bit DG_K_x); 0 times every kind.  Not thread-safe. */
dg_status dg_profile_begin(dg_ctx* ctx, int capacity, uint32_t kind_mask);
/* Stop, wait for the recorded events, and return per kind the summed kernel
 * milliseconds and launch counts (arrays of DG_K_COUNT entries). */
dg_status dg_profile_end(dg_ctx* ctx, double* ms, int32_t* count);
/* Byte offset, inside a workspace sized for `batch`, of an int32 [n_layers][E]
 * log of the per-expert token counts of the most recent pass through each layer. */
dg_status dg_workspace_moe_counts(const dg_ctx* ctx, int batch, size_t* offset);

/* ---- kernel taps for tests (not part of the stable contract) ---- */

/* Router selection alone: r fp32 [M][E] (E a multiple of 4 in [4, 256], rows
 * 16-byte aligned) -> ids int32 [M][k] (by logit desc, id asc) and weights fp32
 * [M][k] (softmax over the k selected logits). */
dg_status dg_test_router_topk(const float* d_r, int M, int E, int k, int32_t* d_ids,
                              float* d_w, void* stream);

/* Router top-k + the token->expert counting sort, as run in a layer.  Outputs:
 * ids/w as dg_test_router_topk; cnt int32 [E]; poff int32 [E+1] (16-aligned
 * padded slot offsets); perm int32 [M*k + 15E] (token of each padded slot, -1 on
 * padding); inv int32 [M*k] (slot of assignment m*k+j); items int32x2
 * [(M*k+63)/64 + E] -- (expert, first token) of every group of up to 64 of an
 * expert's tokens, experts ascending -- and n_items int32 [1]. */
dg_status dg_test_route(const float* d_r, int M, int E, int k, int32_t* d_ids, float* d_w,
                        int32_t* d_cnt, int32_t* d_poff, int32_t* d_perm, int32_t* d_inv,
                        int32_t* d_items, int32_t* d_n_items, void* stream);

/* Entropy-bounded selection alone on given fp32 entropies and argmax ids:
 * same rule and outputs as dg_sample_eb, with d_entropy and d_argmax as inputs
 * (read on [MASK] rows only). */
dg_status dg_test_eb_select(const float* d_entropy, const int32_t* d_argmax, int32_t* d_canvas,
                            int batch, int canvas, int vocab, float gamma, int commit_all,
                            int32_t* d_n_masked, void* stream);

/* bf16 GEMM y[M][N] = x[M][K] . w[N][K]^T, fp32 row-major out (K % 64 == 0);
 * x and w both plain-packed (fragment-major, rows padded to 16). */
dg_status dg_test_gemm(const uint16_t* d_x, const uint16_t* d_w, float* d_y, int M, int N, int K,
                       void* stream);

/* Plain device copy of n_bytes (a positive multiple of 16) from d_src to d_dst
 * with 16-byte loads and stores: a kernel of known traffic, for calibrating the
 * hardware byte counters against which the other kernels are measured. */
dg_status dg_test_copy(const void* d_src, void* d_dst, size_t n_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
