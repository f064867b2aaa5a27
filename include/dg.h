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
 *  - Threads: a dg_ctx may be shared by threads once dg_create has returned.
 *    Calls that run concurrently need distinct workspaces and KV caches (and
 *    their own logits/canvas buffers); each call forks the shared expert onto the
 *    ctx's side stream with a fork/join event pair of its own (taken from a
 *    mutex-guarded pool), so concurrent calls serialise on that stream but never
 *    share an event.  The measurement helpers (dg_profile_*) and the test taps
 *    that change a ctx (dg_test_force_routing) are not thread-safe.
 *  - Device: a ctx belongs to the device current at dg_create (its weights live
 *    there); call it with that device current.
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
 *   DG_PACK_TRANSPOSE the packed matrix is the transpose [cols][rows] of the
 *                    source (n_mats = 1, rows % 32 == 0; dst holds
 *                    dg_packed_elems(cols, rows) elements) -- the embedding rows
 *                    0..V-1 as the self-conditioning product's operand.
 * The source is not modified; the call only enqueues a kernel on `stream`. */
typedef enum dg_pack_kind { DG_PACK_PLAIN = 0, DG_PACK_QKV = 1, DG_PACK_GATE_UP = 2,
                            DG_PACK_TRANSPOSE = 3 } dg_pack_kind;
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
  /* Self-conditioning (Technical Report §3.2, eq. 5-6): all three NULL (no
   * self-conditioning) or all set; needs vocab % 32 == 0. */
  const uint16_t* embed_t;            /* TRANSPOSE-packed embedding rows 0..V-1: [d][V] */
  const uint16_t* sc_gate_up;         /* GATE_UP-packed [2Fs][d], Fs = shared_ffn */
  const uint16_t* sc_down;            /* plain-packed [d][Fs] */
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
 * dg_layer_weights array itself is copied).  Validates shapes.  Allocates the
 * ctx's host-side state and creates its side stream on the current device (no
 * device memory); without a usable device it still succeeds and every call then
 * keeps all work on the caller's stream. */
dg_status dg_create(const dg_config* cfg, const dg_weights* w, dg_ctx** out);
void dg_destroy(dg_ctx* ctx);

/* Bytes of device workspace needed by any call on `batch` sequences. */
dg_status dg_workspace_size(const dg_ctx* ctx, int batch, size_t* bytes);
/* Bytes of each of the k and v cache buffers for cfg. */
dg_status dg_kv_size(const dg_config* cfg, size_t* bytes_each);

const char* dg_status_string(dg_status s);
const char* dg_last_error(void);
/* Digest of the sources this library was built from (16 hex digits; "unstamped"
 * when the build did not define it).  The Python binding compares it with the
 * sources next to it and refuses a library built from others. */
const char* dg_source_digest(void);

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

/* dg_sample_eb for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same rule,
 * kernels, arguments and outputs, but no workspace argument -- the sampler's scratch
 * is a static 4 MiB array inside the library (one per device, held until the process
 * ends; enough for about 7000 canvas rows of 262144 logits).  Calls whose
 * dg_sample_workspace_size exceeds 4 MiB fail with DG_ERR_WORKSPACE before anything
 * is enqueued.  The call allocates and frees nothing.  Every call on a device shares
 * that device's scratch: calls that overlap in time on one device (other streams,
 * other threads) race and must be serialised by the caller. */
dg_status dg_sample_eb_noalloc(const uint16_t* d_logits, int32_t* d_canvas, int batch, int canvas,
                               int vocab, float gamma, int commit_all, float* d_entropy,
                               int32_t* d_argmax, int32_t* d_n_masked, void* stream);

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

/* n_blocks consecutive blocks per sequence (Technical Report §3.1–§3.3, the block
 * loop): block j fills d_canvas + j * batch * C (int32 [n_blocks][batch][C], out) as
 * dg_generate_block does, and its KV append runs fused into block j + 1's first
 * denoising pass: one pass over 2 * batch * C rows in which the first batch * C rows
 * (block j, causal, at len) write their keys/values before the attention of every
 * layer and the other rows (block j + 1's canvas, at len + C) attend to them.  Every
 * row's arithmetic is that of the separate passes, so canvases, logits and the KV
 * cache equal n_blocks calls of dg_generate_block(append_kv = 1) bit for bit, as long
 * as the fused pass (2 * batch * C rows) and the separate ones fall on the same side
 * of 2048 rows, where the dense GEMMs change tile shape and with it their fp32
 * summation order (always so for batch 1 and 2 at C = 256).  When C > 256 or
 * 2 * batch > DG_MAX_BATCH the passes stay separate.  The last block is
 * appended by its own pass if append_last.  d_logits and d_n_masked as for
 * dg_generate_block (the last block's).  Errors: as dg_generate_block, and
 * DG_ERR_KV_CAPACITY when len + n_blocks * C exceeds max_ctx. */
dg_status dg_generate_blocks(dg_ctx* ctx, dg_kv* kv, int32_t* d_canvas, int batch, int n_blocks, int steps,
                             float gamma, int append_last, uint16_t* d_logits, int32_t* d_n_masked,
                             void* d_ws, size_t ws_bytes, void* stream);

/* dg_generate_block with the Technical Report's default sampler (§3.3) on the
 * absorbing canvas: up to max_steps steps at t_s = 1 - s/max_steps, entropies at
 * the temperature tau_min + (tau_max - tau_min) t_s (annealed linearly from tau_max
 * to tau_min; both finite and > 0), and the adaptive stop with threshold e_stop
 * (< 0: off; see dg_sample_eb_ex), which commits a sequence's remaining positions
 * at once; the last step commits whatever is left.  d_done_step (int32 [batch],
 * out): the number of steps after which each canvas was complete.  The previous
 * argmax lives in the workspace.  Once a canvas is complete its later steps change
 * nothing.  With the stop on (e_stop >= 0) and max_steps > 2 the call skips them:
 * after each step's sampler it copies d_done_step into pinned host memory, and
 * before it enqueues step s it waits for the copy of step s - 2 and ends the step
 * loop (then runs the append pass) once every sequence is complete, so at most one
 * pass runs after the last canvas completes.  The host then blocks until the device
 * is within two steps of the call's end; such a call cannot be captured into a
 * graph.  With the stop off the host never waits.  The skipped steps would change
 * neither the canvas, d_n_masked, d_done_step nor the KV cache. */
dg_status dg_generate_block_ex(dg_ctx* ctx, dg_kv* kv, int32_t* d_canvas, int batch, int max_steps,
                               float gamma, float tau_max, float tau_min, float e_stop,
                               int append_kv, uint16_t* d_logits, int32_t* d_n_masked,
                               int32_t* d_done_step, void* d_ws, size_t ws_bytes, void* stream);

/* ---- uniform ("multinomial") variant (Technical Report §2.1; §3.2, canvas
 * initialisation and multinomial diffusion; §3.3) ----
 * The canvas starts as uniformly random tokens; at every step every position is a
 * candidate, so tokens accepted at an earlier step of the same canvas can change;
 * the accepted positions take their argmax and all others are re-noised uniformly.
 * Random tokens: Philox4x64-10 (Salmon, Moraes, Dror and Shaw, SC 2011), counter
 * (position, sequence, draw, 0), key (seed, 0); token = floor(x * vocab / 2^64) for x
 * the block's first output word.  Draw 0 is the initial canvas; the generator below
 * re-noises after step s with draw s + 1. */

/* Fill d_canvas (int32 [batch][canvas], device) with the tokens of (seed, draw).
 * Errors: DG_ERR_INVALID_ARG for a NULL pointer, sizes < 1, more than 2^30 positions
 * or draw < 0. */
dg_status dg_uniform_canvas(int32_t* d_canvas, int batch, int canvas, int vocab, uint64_t seed, int draw,
                            void* stream);

/* dg_sample_eb_ex for the uniform variant.  Every row of a sequence is a candidate
 * (d_canvas may hold any token ids; [MASK] plays no part): the accepted rows are the
 * first k* of all rows in (Ĥ, position) order, by the same rule, and take their
 * argmax; every other row takes the token of (seed, draw, its sequence, its
 * position).  d_done_step (int32 [batch], may be NULL): a sequence whose entry is not
 * 0 is complete and is neither read nor written (its entropy/argmax outputs hold NaN
 * and -1 and its d_n_open 0); an entry that is 0 is set to step + 1 when the
 * adaptive stop fires or commit_all (the sequence is then complete).  d_n_open (int32
 * [batch], out): the number of re-noised rows.  d_prev_argmax, temperature, e_stop,
 * d_entropy, d_argmax and the workspace as for dg_sample_eb_ex (the stop's mean runs
 * over every row).  Errors as for dg_sample_eb_ex, and DG_ERR_INVALID_ARG for
 * draw < 0. */
dg_status dg_sample_eb_uniform(const uint16_t* d_logits, int32_t* d_canvas, int batch, int canvas,
                               int vocab, float gamma, int commit_all, float temperature, float e_stop,
                               int32_t* d_prev_argmax, int step, int32_t* d_done_step, uint64_t seed,
                               int draw, float* d_entropy, int32_t* d_argmax, int32_t* d_n_open,
                               void* d_ws, size_t ws_bytes, void* stream);

/* dg_generate_block_ex for the uniform variant: d_canvas starts as the tokens of
 * (seed, draw 0); step s (t_s = 1 - s/max_steps, temperature annealed as in
 * dg_generate_block_ex) runs the denoising pass with the head over every row and
 * dg_sample_eb_uniform with draw s + 1 (commit_all on the last step); a canvas is
 * complete when the stop fires or after the last step and is not changed afterwards.
 * Then the append pass if append_kv.  d_n_open: int32 [batch] (0 at the end);
 * d_done_step: int32 [batch], the number of steps after which each canvas was
 * complete.  With the stop on, the steps after every canvas is complete are skipped
 * as in dg_generate_block_ex; d_logits then holds the last pass that ran (its rows of
 * complete canvases are scratch either way).  Errors as for dg_generate_block_ex. */
dg_status dg_generate_block_uniform(dg_ctx* ctx, dg_kv* kv, int32_t* d_canvas, int batch, int max_steps,
                                    float gamma, float tau_max, float tau_min, float e_stop, uint64_t seed,
                                    int append_kv, uint16_t* d_logits, int32_t* d_n_open,
                                    int32_t* d_done_step, void* d_ws, size_t ws_bytes, void* stream);

/* ---- self-conditioning (Technical Report §3.2, decoder forward pass and denoising
 * iteration, eq. 5-6; §6, sampling) ----
 * The decoder's third input z [C][d] feeds its previous prediction back: from a
 * step's logits L, p̂₀ = softmax(L) per row and z = FFW(p̂₀ E), E the embedding rows
 * 0..V-1, FFW = W_down (silu(W_gate u) * (W_up u)) a SwiGLU network of width
 * shared_ffn; z is added to the canvas rows' input (token embedding + timestep
 * embedding) of the next step, and is 0 at a canvas's first step.  The softmax and
 * the product p̂₀ E run at fp32 precision (p̂₀ carried to 2^-18 relative, fp32
 * accumulation); u = p̂₀ E enters the FFW rounded to bf16 like every GEMM input.
 * The ctx needs the self-conditioning weights (dg_weights.embed_t, sc_gate_up,
 * sc_down); otherwise these calls return DG_ERR_UNSUPPORTED. */

/* z (fp32 [batch][C][d], out) from d_logits (bf16 [batch][C][V], every row read);
 * d_u (fp32 [batch][C][d], may be NULL): p̂₀ E before its bf16 rounding.  Workspace:
 * dg_workspace_size of the ctx. */
dg_status dg_self_cond(dg_ctx* ctx, const uint16_t* d_logits, int batch, float* d_z, float* d_u, void* d_ws,
                       size_t ws_bytes, void* stream);

/* dg_denoise_step with the self-conditioning signal d_z (fp32 [batch][C][d], NULL: z = 0,
 * the plain pass) added to the canvas rows' input. */
dg_status dg_denoise_step_sc(dg_ctx* ctx, const dg_kv* kv, const int32_t* d_canvas, int batch, float t,
                             const float* d_z, uint16_t* d_logits, void* d_ws, size_t ws_bytes, void* stream);

/* dg_generate_block_ex (uniform = 0) or dg_generate_block_uniform (uniform = 1, with
 * seed) with self-conditioning: step 0 runs with z = 0, and after every step but the
 * last z is recomputed from that step's logits for the next one; the head computes
 * every canvas row at every step.  z lives in the workspace.  With the stop on, the
 * steps after every canvas is complete are skipped as in dg_generate_block_ex. */
dg_status dg_generate_block_sc(dg_ctx* ctx, dg_kv* kv, int32_t* d_canvas, int batch, int max_steps, float gamma,
                               float tau_max, float tau_min, float e_stop, int uniform, uint64_t seed,
                               int append_kv, uint16_t* d_logits, int32_t* d_n, int32_t* d_done_step,
                               void* d_ws, size_t ws_bytes, void* stream);

/* ---- mixed batches and continuous batching (Technical Report §6, eliminating CPU-GPU
 * synchronisation; multi-user throughput) ----
 * A served batch holds two kinds of forward pass -- denoising steps and KV-cache updates
 * (the causal encoding of a finished canvas) -- that need different attention masks; a
 * per-sequence causal flag selects the mask, so both run in one pass. */

/* One pass over `batch` sequences of C tokens (d_tokens int32 [batch][C]): sequence b with
 * h_encode[b] != 0 runs the causal encoder and appends the K/V of its C tokens (kv->len[b]
 * += C, as dg_prefill_kv); every other one runs the denoising pass over its canvas at time
 * h_t[b] in [0, 1] (as dg_denoise_step) and gets the logits rows of its canvas.  The head
 * computes only the rows of the denoising sequences; the logits rows of the encoding ones
 * are left as they were.  h_encode, h_t: host arrays [batch] (h_t and d_logits may be NULL
 * when every sequence encodes).  Errors as for dg_denoise_step and dg_prefill_kv. */
dg_status dg_mixed_step(dg_ctx* ctx, dg_kv* kv, const int32_t* d_tokens, int batch, const int32_t* h_encode,
                        const float* h_t, uint16_t* d_logits, void* d_ws, size_t ws_bytes, void* stream);

/* dg_sample_eb with a commit-all flag per sequence (h_commit_all, host int32 [batch],
 * batch <= DG_MAX_BATCH): the sequences at the last step of their block commit every
 * [MASK] row, the others follow the entropy bound.  A sequence with no [MASK] row (one
 * whose canvas is being appended) is left unchanged. */
dg_status dg_sample_eb_seq(const uint16_t* d_logits, int32_t* d_canvas, int batch, int canvas, int vocab,
                           float gamma, const int32_t* h_commit_all, float* d_entropy, int32_t* d_argmax,
                           int32_t* d_n_masked, void* d_ws, size_t ws_bytes, void* stream);

/* Continuous batching of block generation: n_passes mixed passes over `batch` sequences,
 * each cycling through `steps` denoising steps of its canvas (t = 1 - phase/steps, the
 * entropy-bounded sampler with gamma, every remaining [MASK] row committed at phase
 * steps - 1) and one pass (phase == steps) that appends the finished canvas, whose canvas
 * row then restarts all-[MASK].  h_phase (host int32 [batch], in/out): each sequence's
 * phase in [0, steps], advanced by n_passes (mod steps + 1); d_canvas must hold the state
 * that phase implies (at a sequence's first call: all [MASK] at a phase below steps).  The
 * schedule is fixed on the host, so the loop enqueues every pass without waiting.
 * d_out (int32 [batch][out_blocks][C], may be NULL): sequence b's finished canvases in
 * a ring, block i of sequence b at slot i % out_blocks, i counted in h_out_count[b] (host
 * int32 [batch], in/out).  d_logits: bf16 [batch][C][V] scratch; d_n_masked: int32 [batch].
 * Errors: DG_ERR_INVALID_ARG for bad phases or sizes, DG_ERR_KV_CAPACITY when the
 * appends of the call would pass max_ctx (checked before anything is enqueued). */
dg_status dg_serve(dg_ctx* ctx, dg_kv* kv, int32_t* d_canvas, int batch, int steps, float gamma, int n_passes,
                   int32_t* h_phase, uint16_t* d_logits, int32_t* d_n_masked, int32_t* d_out, int out_blocks,
                   int32_t* h_out_count, void* d_ws, size_t ws_bytes, void* stream);

/* ---- measurement helpers (diagnostics; not thread-safe) ---- */

/* Kernel kinds the engine launches, for per-kind event timing. */
typedef enum dg_kernel_kind {
  DG_K_PREP = 0, DG_K_EMBED, DG_K_QKV, DG_K_ATTENTION, DG_K_O_PROJ, DG_K_NORM, DG_K_ROUTER,
  DG_K_TOPK, DG_K_ROUTE, DG_K_MOE_GATE_UP, DG_K_MOE_DOWN, DG_K_SHARED_GATE_UP, DG_K_SHARED_DOWN,
  DG_K_COMBINE, DG_K_HEAD, DG_K_SAMPLE_PASS1, DG_K_SAMPLE_SELECT, DG_K_FILL,
  DG_K_SAMPLE_CANON, DG_K_SAMPLE_SELECT_CANON, DG_K_ATTENTION_GLOBAL,
  DG_K_SC_STATS, DG_K_SC_EMBED, DG_K_SC_REDUCE, DG_K_SC_FFW,
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
/* Attention launches of global layers are timed as DG_K_ATTENTION_GLOBAL, those of
 * sliding-window layers as DG_K_ATTENTION. */
/* dg_sample_eb with its launches timed by ctx's profiler (a measurement tap: the
 * sampler itself needs no ctx). */
dg_status dg_test_sample_eb_profiled(dg_ctx* ctx, const uint16_t* d_logits, int32_t* d_canvas, int batch,
                                     int canvas, int vocab, float gamma, int commit_all, int32_t* d_n_masked,
                                     void* d_ws, size_t ws_bytes, void* stream);
/* Byte offset, inside a workspace sized for `batch`, of an int32 [n_layers][E]
 * log of the per-expert token counts of the most recent pass through each layer. */
dg_status dg_workspace_moe_counts(const dg_ctx* ctx, int batch, size_t* offset);

/* ---- kernel taps for tests (not part of the stable contract) ---- */

/* Teacher-forced routing: while d_ids is not NULL, layer l of every pass through
 * ctx takes the expert ids d_ids[l][m][0..top_k) (int32 [n_layers][M][top_k],
 * M = batch * tokens of each following pass -- the caller gives one array per
 * pass, so a prefill must fit one pass: at most max(canvas, 512) tokens) in that
 * order instead of the router's top-k; the weights are still the softmax of the
 * engine's own router logits at those ids.  Ids are clamped to [0, E).  NULL
 * restores the router.  For parity tests that must not depend on near-tied
 * routing decisions; not thread-safe. */
dg_status dg_test_force_routing(dg_ctx* ctx, const int32_t* d_ids);

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
 * expert's tokens, experts ascending -- and n_items int32 [1]; items2 int32x2
 * [(M*k+127)/128 + E] and n_items2 int32 [1] -- the expert GEMMs' work items: an
 * expert with c tokens gets n = ceil(c/128) items, item i holding its 16-token
 * blocks [floor(i*b/n), floor((i+1)*b/n)) of b = ceil(c/16), as (expert,
 * t0 | t1 << 16) with [t0, t1) the item's tokens. */
dg_status dg_test_route(const float* d_r, int M, int E, int k, int32_t* d_ids, float* d_w,
                        int32_t* d_cnt, int32_t* d_poff, int32_t* d_perm, int32_t* d_inv,
                        int32_t* d_items, int32_t* d_n_items, int32_t* d_items2, int32_t* d_n_items2,
                        void* stream);

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

/* Achievable bf16 matrix-core rate, for reporting measured peaks beside the vendor
 * figures: `blocks` workgroups of 256 threads; each wave issues `iters` rounds of 8
 * v_mfma_f32_16x16x32_bf16 (16384 flop each; a dependent pair on each of 4
 * accumulators) on register operands and touches no memory until it writes
 * d_out[blocks * 256] (float, caller-owned): per lane 4 * 4 * 64 * iters, exact for
 * iters < 2^14.  Work = blocks * 4 * 8 * iters * 16384 flop.  Errors: DG_ERR_INVALID_ARG for blocks outside 1..65536, iters outside
 * 1..2^20 or a NULL d_out. */
dg_status dg_test_mfma_rate(int blocks, int iters, float* d_out, void* stream);

/* Achievable HBM read rate, for the same report: `blocks` workgroups of 256 threads
 * stream d_src (n_bytes, a positive multiple of 16; caller-owned) once, thread t
 * reading the 16-byte words t, t + S, t + 2S, ... (S = blocks * 256) four at a time,
 * and write the first 32-bit lane of their XOR to d_out[t] (uint32 [blocks * 256],
 * caller-owned).  Errors: DG_ERR_INVALID_ARG for NULL buffers, a byte count that is
 * zero or not a multiple of 16, or blocks outside 1..65536. */
dg_status dg_test_read_rate(const void* d_src, size_t n_bytes, int blocks, uint32_t* d_out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
