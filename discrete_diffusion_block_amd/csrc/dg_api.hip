// C ABI of the engine: argument validation, workspace carving and the
// per-pass kernel schedule.  Everything is enqueued on the caller's stream;
// nothing here synchronises, allocates device memory or reads back.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <new>
#include <string>
#include <vector>

#include "dg.h"
#include "dg_common.h"
#include "dg_internal.h"

using namespace dg;

// Optional per-launch event timing (dg_profile_begin/end).
struct Prof {
  bool on = false;
  uint32_t mask = 0;            // kinds timed (bit per dg_kernel_kind)
  std::vector<hipEvent_t> ev;   // two per record
  std::vector<int> kind;
  size_t used = 0;
};

struct dg_ctx {
  dg_config cfg;
  const uint16_t* embed;
  const float* final_norm;
  std::vector<dg_layer_weights> layers;
  mutable Prof prof;
  // Side stream for the shared expert, which runs concurrently with the routed
  // experts' routing chain; forked from and joined back into the caller's stream
  // with events.  Created on first use, on the device current at that time.
  mutable hipStream_t side = nullptr;
  mutable hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  mutable int side_dev = -1;
};

namespace {

thread_local std::string g_err;

dg_status fail(dg_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

dg_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return DG_OK;
}

// Brackets one launch with profiling events when profiling is on.
struct Timed {
  const dg_ctx* c;
  int kind;
  hipStream_t s;
  bool on;
  // The start event is a marker ahead of the launch (it fires once the stream's
  // previous work is done, i.e. as the kernel can begin); the stop event rides on the
  // launch itself (next_launch_events) and fires at the kernel's completion.
  Timed(const dg_ctx* c_, int k, hipStream_t s_) : c(c_), kind(k), s(s_) {
    on = c && c->prof.on && (c->prof.mask >> k & 1u) && c->prof.used < c->prof.kind.size();
    if (on) {
      (void)hipEventRecord(c->prof.ev[2 * c->prof.used], s);
      next_launch_events() = LaunchEvents{c->prof.ev[2 * c->prof.used + 1]};
    }
  }
  ~Timed() {
    if (on) {
      // a statement that launched nothing leaves its stop event unused: not counted
      const bool used = next_launch_events().stop == nullptr;
      next_launch_events() = LaunchEvents{};
      c->prof.kind[c->prof.used++] = used ? kind : -1;
    }
  }
};
#define DG_TIMED(ctx, kind, stmt) \
  do {                            \
    Timed _timed(ctx, kind, s);   \
    stmt;                         \
  } while (0)
#define DG_TIMED_ON(ctx, kind, strm, stmt) \
  do {                                     \
    Timed _timed(ctx, kind, strm);         \
    stmt;                                  \
  } while (0)

// The side stream for the current device, or nullptr (work then stays on the
// caller's stream) if it cannot be set up or the context moved to another device.
hipStream_t side_stream(const dg_ctx* ctx) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  if (ctx->side) return ctx->side_dev == dev ? ctx->side : nullptr;
  hipStream_t st = nullptr;
  hipEvent_t a = nullptr, b = nullptr;
  if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
  // both events only order work between two queues of this device: no system-scope
  // (host-visibility) fence is needed when they are signalled
  constexpr unsigned kFlags = hipEventDisableTiming | hipEventDisableSystemFence;
  if (hipEventCreateWithFlags(&a, kFlags) != hipSuccess || hipEventCreateWithFlags(&b, kFlags) != hipSuccess) {
    if (a) (void)hipEventDestroy(a);
    (void)hipStreamDestroy(st);
    return nullptr;
  }
  ctx->side = st;
  ctx->ev_fork = a;
  ctx->ev_join = b;
  ctx->side_dev = dev;
  return st;
}

constexpr int kPrefillChunk = 512;   // tokens per sequence per encoder pass
constexpr int kPassCounters = 16;    // device counters cleared at the start of every pass
constexpr size_t kAlign = 256;

struct Ws {
  float* x;        // residual stream, fp32 row-major [M][d]
  uint16_t* h;     // normed activations, fragment-major [M_pad][d]
  uint16_t* h_rm;  // the FFN-normed activations again, row-major [M][d] (expert row gathers)
  uint16_t* q;     // queries, fragment-major per (sequence, head) [n_pad][hd]
  uint16_t* o;     // attention output, fragment-major [M_pad][Hq*hd]
  float2* rope;
  float* temb;
  float* r;        // router logits fp32 [M][E]
  int32_t* ids;
  float* wts;
  int32_t* cnt;
  int32_t* poff;   // padded (16-aligned) slot offsets [E+1]
  int32_t* perm;   // token of each padded slot (-1 on padding)
  int32_t* inv;    // padded slot of each assignment
  int2* items;
  int32_t* n_items;
  int2* items2;
  int32_t* n_items2;
  int32_t* prev_amax;  // [batch][C]: the previous step's argmax (adaptive stop)
  int32_t* cnt_log;
  int32_t* rows;   // logits row of each compacted [MASK] row (head restricted to masked rows)
  int32_t* counters;   // [0]: compacted [MASK] rows; cleared at the start of every pass
  uint16_t* A;     // expert SwiGLU outputs, fragment-major [P_pad][F]
  float* Y;        // expert outputs fp32 [P][d]
  uint16_t* As;    // shared-expert SwiGLU output, fragment-major [M_pad][Fs]
  float* ys;       // shared-expert output fp32 row-major [M][d]
  float4* part;
  int* part_arg;
};

struct Carver {
  char* base;
  size_t off = 0;
  template <class T>
  T* take(size_t count) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

int sample_chunks(int vocab) { return (vocab + kSampleChunk - 1) / kSampleChunk; }

size_t carve_sampler(Carver& cv, int batch, int canvas, int vocab, Ws* ws) {
  const size_t rows = (size_t)batch * canvas;
  ws->part = cv.take<float4>(rows * sample_chunks(vocab));
  ws->part_arg = cv.take<int>(rows * sample_chunks(vocab));
  return cv.off;
}

size_t round16(size_t v) { return (v + 15) / 16 * 16; }

size_t carve(const dg_config& c, int batch, char* base, Ws* ws) {
  const size_t n = (size_t)std::max(c.canvas, kPrefillChunk);
  const size_t M = (size_t)batch * n;
  const size_t Mp = round16(M);
  const size_t qd = (size_t)c.n_q_heads * c.head_dim;
  const size_t P = (size_t)moe_max_slots((int)M, c.top_k, c.n_experts);
  Carver cv{base};
  ws->x = cv.take<float>(M * c.d_model);
  ws->h = cv.take<uint16_t>(Mp * c.d_model);
  ws->h_rm = cv.take<uint16_t>(M * c.d_model);
  ws->q = cv.take<uint16_t>((size_t)batch * round16(n) * qd);
  ws->o = cv.take<uint16_t>(Mp * qd);
  ws->rope = cv.take<float2>(M * (c.head_dim / 2));
  ws->temb = cv.take<float>(c.d_model);
  ws->r = cv.take<float>(M * c.n_experts);
  ws->ids = cv.take<int32_t>(M * c.top_k);
  ws->wts = cv.take<float>(M * c.top_k);
  ws->cnt = cv.take<int32_t>(c.n_experts);
  ws->poff = cv.take<int32_t>(c.n_experts + 1);
  ws->perm = cv.take<int32_t>(P);
  ws->inv = cv.take<int32_t>(M * c.top_k);
  ws->items = cv.take<int2>(moe_max_items((int)M, c.top_k, c.n_experts));
  ws->n_items = cv.take<int32_t>(1);
  ws->items2 = cv.take<int2>(moe_max_items2((int)M, c.top_k, c.n_experts));
  ws->n_items2 = cv.take<int32_t>(1);
  ws->cnt_log = cv.take<int32_t>((size_t)c.n_layers * c.n_experts);
  ws->rows = cv.take<int32_t>(M);
  ws->counters = cv.take<int32_t>(kPassCounters);
  ws->A = cv.take<uint16_t>(round16(P) * c.expert_ffn);
  ws->Y = cv.take<float>(P * c.d_model);
  ws->As = cv.take<uint16_t>(Mp * c.shared_ffn);
  ws->ys = cv.take<float>(M * c.d_model);
  ws->prev_amax = cv.take<int32_t>((size_t)batch * c.canvas);
  carve_sampler(cv, batch, c.canvas, c.vocab, ws);
  return cv.off + kAlign;
}

dg_status validate_config(const dg_config* c) {
  if (!c) return fail(DG_ERR_INVALID_ARG, "config is NULL");
  if (c->n_layers < 1) return fail(DG_ERR_SHAPE, "n_layers must be >= 1");
  if (c->d_model < 64 || c->d_model % 64) return fail(DG_ERR_SHAPE, "d_model must be a positive multiple of 64");
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
    return fail(DG_ERR_SHAPE, "head_dim must be 32, 64 or 128");
  if (c->n_q_heads < 1 || c->n_kv_heads < 1 || c->n_q_heads % c->n_kv_heads)
    return fail(DG_ERR_SHAPE, "n_q_heads must be a positive multiple of n_kv_heads");
  if ((c->n_q_heads * c->head_dim) % 64) return fail(DG_ERR_SHAPE, "n_q_heads * head_dim must be a multiple of 64");
  if (c->n_experts < 4 || c->n_experts > 256 || c->n_experts % 4)
    return fail(DG_ERR_SHAPE, "n_experts must be a multiple of 4 in [4, 256]");
  if (c->top_k < 1 || c->top_k > 16 || c->top_k > c->n_experts)
    return fail(DG_ERR_SHAPE, "top_k must be in [1, min(16, n_experts)]");
  if (c->expert_ffn < 64 || c->expert_ffn % 64) return fail(DG_ERR_SHAPE, "expert_ffn must be a positive multiple of 64");
  if (c->shared_ffn < 64 || c->shared_ffn % 64) return fail(DG_ERR_SHAPE, "shared_ffn must be a positive multiple of 64");
  if (c->vocab < 8 || c->vocab % 8) return fail(DG_ERR_SHAPE, "vocab must be a positive multiple of 8");
  if (c->canvas < 1 || c->canvas > 1024) return fail(DG_ERR_SHAPE, "canvas must be in [1, 1024]");
  if (c->window < 1) return fail(DG_ERR_SHAPE, "window must be >= 1");
  if (c->global_every < 0) return fail(DG_ERR_SHAPE, "global_every must be >= 0");
  if (c->max_batch < 1 || c->max_batch > DG_MAX_BATCH) return fail(DG_ERR_SHAPE, "max_batch must be in [1, %d]", DG_MAX_BATCH);
  if (c->max_ctx < c->canvas || c->max_ctx % 64) return fail(DG_ERR_SHAPE, "max_ctx must be a multiple of 64 and >= canvas");
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) return fail(DG_ERR_SHAPE, "rms_eps must be >= 0 and rope_theta > 0");
  return DG_OK;
}

bool is_global(const dg_config& c, int l) { return c.global_every > 0 && (l + 1) % c.global_every == 0; }

size_t layer_kv_elems(const dg_config& c) {
  return (size_t)c.max_batch * c.n_kv_heads * c.max_ctx * c.head_dim;
}

KvLayer kv_layer(const dg_ctx* ctx, const dg_kv* kv, int l) {
  const dg_config& c = ctx->cfg;
  KvLayer v;
  v.k = kv->k + (size_t)l * layer_kv_elems(c);
  v.vt = kv->v + (size_t)l * layer_kv_elems(c);
  v.hkv = c.n_kv_heads;
  v.hd = c.head_dim;
  v.max_ctx = c.max_ctx;
  v.window = is_global(c, l) ? 0 : c.window;
  return v;
}

// One transformer pass over batch x n tokens (denoise: + final norm + tied head).
// masked_head (denoise passes): the head computes only the rows whose canvas token is
// [MASK] -- the only rows the sampler reads -- and leaves the other logits rows as
// they were.
dg_status run_pass(const dg_ctx* ctx, const dg_kv* kv, const PassGeom& g, const int32_t* tokens,
                   float t, uint16_t* logits, const Ws& ws, hipStream_t s, bool masked_head = false) {
  const dg_config& c = ctx->cfg;
  const int M = g.batch * g.n;
  const int d = c.d_model, hq = c.n_q_heads, hd = c.head_dim, E = c.n_experts, k = c.top_k;
  const float eps = c.rms_eps;
  const int nl = c.n_layers;
  DG_TIMED(ctx, DG_K_PREP, launch_prep(g, hd, c.rope_theta, ws.rope, d, t, g.denoise ? ws.temb : nullptr,
                                       ws.counters, kPassCounters, s));
  DG_TIMED(ctx, DG_K_EMBED,
           launch_embed_norm(tokens, ctx->embed, g.denoise ? ws.temb : nullptr, ctx->layers[0].attn_norm,
                             eps, ws.x, ws.h, M, d, c.vocab, s));
  for (int l = 0; l < nl; ++l) {
    const dg_layer_weights& L = ctx->layers[l];
    const KvLayer kvl = kv_layer(ctx, kv, l);
    DG_TIMED(ctx, DG_K_QKV, launch_qkv_rope(ws.h, L.w_qkv, M, d, hq, kvl, g, ws.rope, ws.q, s));
    // In the encoder only the keys/values are observable; the last layer's
    // attention output and FFN feed nothing, so they are not computed.
    if (!g.denoise && l == nl - 1) break;
    DG_TIMED(ctx, DG_K_ATTENTION, launch_attention(ws.q, hq, kvl, g, ws.o, s));
    DG_TIMED(ctx, DG_K_O_PROJ, launch_gemm_f32(ws.o, L.w_o, ws.x, M, d, hq * hd, /*add=*/true, s));
    // The shared expert depends only on h: it runs on the side stream while the
    // routed experts' routing chain (small, latency-bound kernels) runs here.  It
    // reads h and writes As and ys, which nothing on this stream touches before
    // the join; the combine kernel adds ys.  The fork and join events are
    // signalled by the kernels' own completion (no marker packets on the queues).
    hipStream_t s2 = side_stream(ctx);
    const bool fork = s2 != nullptr;
    if (!fork) s2 = s;
    DG_TIMED(ctx, DG_K_NORM,
             launch_rmsnorm(ws.x, L.ffn_norm, eps, ws.h, ws.h_rm, M, d, s, fork ? ctx->ev_fork : nullptr));
    if (fork) (void)hipStreamWaitEvent(s2, ctx->ev_fork, 0);
    DG_TIMED_ON(ctx, DG_K_SHARED_GATE_UP, s2,
                launch_gemm_swiglu(ws.h, L.ws_gate_up, M, c.shared_ffn, d, ws.As, s2));
    DG_TIMED_ON(ctx, DG_K_SHARED_DOWN, s2,
                launch_gemm_f32(ws.As, L.ws_down, ws.ys, M, d, c.shared_ffn, /*add=*/false, s2,
                                fork ? ctx->ev_join : nullptr));
    DG_TIMED(ctx, DG_K_ROUTER, launch_gemm_f32(ws.h, L.w_router, ws.r, M, E, d, /*add=*/false, s));
    DG_TIMED(ctx, DG_K_TOPK, launch_topk(ws.r, M, E, k, ws.ids, ws.wts, s));
    DG_TIMED(ctx, DG_K_ROUTE,
             launch_route(ws.ids, M, k, E, ws.cnt, ws.poff, ws.perm, ws.inv, ws.items, ws.n_items, ws.items2,
                          ws.n_items2,
                          ws.cnt_log + (size_t)l * E, s));
    DG_TIMED(ctx, DG_K_MOE_GATE_UP,
             launch_moe_gate_up(ws.h_rm, ws.perm, L.w_gate_up, ws.cnt, ws.poff, ws.items2, ws.n_items2,
                                moe_max_items2(M, k, E),
                                c.expert_ffn, d, ws.A, s));
    DG_TIMED(ctx, DG_K_MOE_DOWN,
             launch_moe_down(ws.A, L.w_down, ws.cnt, ws.poff, ws.items2, ws.n_items2, moe_max_items2(M, k, E),
                             c.expert_ffn, d, ws.Y, s));
    if (fork) (void)hipStreamWaitEvent(s, ctx->ev_join, 0);
    const float* next_gain = (l + 1 < nl) ? ctx->layers[l + 1].attn_norm : (g.denoise ? ctx->final_norm : nullptr);
    const bool compact = masked_head && g.denoise && l == nl - 1;
    DG_TIMED(ctx, DG_K_COMBINE,
             launch_combine(ws.x, ws.ys, ws.Y, ws.wts, ws.inv, M, k, d, next_gain, eps, ws.h,
                            compact ? tokens : nullptr, c.vocab, compact ? ws.rows : nullptr, ws.counters, s));
  }
  const bool compact = masked_head && g.denoise;
  if (g.denoise)
    DG_TIMED(ctx, DG_K_HEAD, launch_gemm_head(ws.h, ctx->embed, logits, M, c.vocab, d,
                                              compact ? ws.counters : nullptr, compact ? ws.rows : nullptr, s));
  return check_launch("transformer pass");
}

dg_status check_kv(const dg_ctx* ctx, const dg_kv* kv, int batch) {
  if (!kv || !kv->k || !kv->v) return fail(DG_ERR_INVALID_ARG, "KV cache pointers are NULL");
  if (batch < 1 || batch > ctx->cfg.max_batch) return fail(DG_ERR_INVALID_ARG, "batch must be in [1, max_batch=%d]", ctx->cfg.max_batch);
  for (int b = 0; b < batch; ++b)
    if (kv->len[b] < 0 || kv->len[b] > ctx->cfg.max_ctx) return fail(DG_ERR_INVALID_ARG, "kv->len[%d] out of range", b);
  return DG_OK;
}

dg_status get_ws(const dg_ctx* ctx, int batch, void* d_ws, size_t ws_bytes, Ws* ws) {
  const size_t need = carve(ctx->cfg, batch, nullptr, ws);
  if (!d_ws) return fail(DG_ERR_INVALID_ARG, "workspace is NULL");
  if (ws_bytes < need) return fail(DG_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  char* base = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(d_ws) + kAlign - 1) / kAlign * kAlign);
  carve(ctx->cfg, batch, base, ws);
  return DG_OK;
}

dg_status denoise_impl(dg_ctx* ctx, const dg_kv* kv, const int32_t* d_canvas, int batch, float t,
                       uint16_t* d_logits, const Ws& ws, hipStream_t s, bool masked_head = false) {
  PassGeom g{};
  g.batch = batch;
  g.n = ctx->cfg.canvas;
  g.denoise = 1;
  for (int b = 0; b < batch; ++b) {
    if (kv->len[b] + ctx->cfg.canvas > ctx->cfg.max_ctx)
      return fail(DG_ERR_KV_CAPACITY, "sequence %d: len %lld + canvas %d exceeds max_ctx %d", b,
                  (long long)kv->len[b], ctx->cfg.canvas, ctx->cfg.max_ctx);
    g.len[b] = (int)kv->len[b];
  }
  return run_pass(ctx, kv, g, d_canvas, t, d_logits, ws, s, masked_head);
}

dg_status prefill_impl(dg_ctx* ctx, dg_kv* kv, const int32_t* d_tokens, int batch, int n,
                       const Ws& ws, hipStream_t s) {
  for (int b = 0; b < batch; ++b)
    if (kv->len[b] + n > ctx->cfg.max_ctx)
      return fail(DG_ERR_KV_CAPACITY, "sequence %d: len %lld + %d tokens exceeds max_ctx %d", b,
                  (long long)kv->len[b], n, ctx->cfg.max_ctx);
  if (n == 0) return DG_OK;
  const int chunk = std::max(ctx->cfg.canvas, kPrefillChunk);
  if (batch == 1 || n <= chunk) {
    for (int s0 = 0; s0 < n; s0 += chunk) {
      PassGeom g{};
      g.batch = batch;
      g.n = std::min(chunk, n - s0);
      g.denoise = 0;
      for (int b = 0; b < batch; ++b) g.len[b] = (int)kv->len[b] + s0;
      // a chunk's tokens are a strided slice when batch > 1; only batch == 1 can chunk in place
      dg_status st = run_pass(ctx, kv, g, d_tokens + s0, 0.f, nullptr, ws, s);
      if (st != DG_OK) return st;
    }
  } else {
    // batch > 1 and n > chunk: one sequence at a time, chunked
    for (int b = 0; b < batch; ++b) {
      for (int s0 = 0; s0 < n; s0 += chunk) {
        PassGeom g{};
        g.batch = 1;
        g.n = std::min(chunk, n - s0);
        g.denoise = 0;
        g.len[0] = (int)kv->len[b] + s0;
        dg_kv one = *kv;
        const size_t seq_k = (size_t)ctx->cfg.n_kv_heads * ctx->cfg.max_ctx * ctx->cfg.head_dim;
        // view of sequence b: offset the cache base by b sequences within each layer
        one.k = kv->k + (size_t)b * seq_k;
        one.v = kv->v + (size_t)b * seq_k;
        dg_status st = run_pass(ctx, &one, g, d_tokens + (size_t)b * n + s0, 0.f, nullptr, ws, s);
        if (st != DG_OK) return st;
      }
    }
  }
  for (int b = 0; b < batch; ++b) kv->len[b] += n;
  return DG_OK;
}

// Sampler extras of the Technical Report (§3.3): temperature, and the adaptive stop
// state (prev_amax NULL: off).
struct SampleOpts {
  float temperature = 1.0f;
  float e_stop = -1.0f;
  int32_t* prev_amax = nullptr;
  int step = 0;
  int32_t* done_step = nullptr;
};

dg_status sample_impl(const uint16_t* d_logits, int32_t* d_canvas, int batch, int canvas, int vocab,
                      float gamma, int commit_all, float* d_entropy, int32_t* d_argmax,
                      int32_t* d_n_masked, const Ws& ws, hipStream_t s, const dg_ctx* ctx = nullptr,
                      const SampleOpts& o = SampleOpts{}) {
  DG_TIMED(ctx, DG_K_SAMPLE_PASS1,
           launch_sample_partials(d_logits, d_canvas, batch * canvas, vocab, 1.0f / o.temperature, ws.part,
                                  ws.part_arg, s));
  DG_TIMED(ctx, DG_K_SAMPLE_SELECT,
           launch_eb_select(ws.part, ws.part_arg, sample_chunks(vocab), nullptr, nullptr, d_canvas, batch,
                            canvas, vocab, gamma, commit_all, d_entropy, d_argmax, d_n_masked, o.prev_amax,
                            o.e_stop, o.step, o.done_step, s));
  return check_launch("sampler");
}

}  // namespace

extern "C" {

const char* dg_status_string(dg_status s) {
  switch (s) {
    case DG_OK: return "ok";
    case DG_ERR_INVALID_ARG: return "invalid argument";
    case DG_ERR_SHAPE: return "unsupported shape";
    case DG_ERR_WORKSPACE: return "workspace too small";
    case DG_ERR_KV_CAPACITY: return "KV cache capacity exceeded";
    case DG_ERR_HIP: return "HIP error";
    case DG_ERR_UNSUPPORTED: return "unsupported";
  }
  return "unknown status";
}

const char* dg_last_error(void) { return g_err.c_str(); }

dg_status dg_create(const dg_config* cfg, const dg_weights* w, dg_ctx** out) {
  if (!out) return fail(DG_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  dg_status st = validate_config(cfg);
  if (st != DG_OK) return st;
  if (!w || !w->embed || !w->final_norm || !w->layers) return fail(DG_ERR_INVALID_ARG, "weights are NULL");
  for (int l = 0; l < cfg->n_layers; ++l) {
    const dg_layer_weights& L = w->layers[l];
    if (!L.attn_norm || !L.w_qkv || !L.w_o || !L.ffn_norm || !L.w_router || !L.w_gate_up || !L.w_down ||
        !L.ws_gate_up || !L.ws_down)
      return fail(DG_ERR_INVALID_ARG, "layer %d has a NULL weight", l);
  }
  dg_ctx* c = new (std::nothrow) dg_ctx;
  if (!c) return fail(DG_ERR_INVALID_ARG, "out of host memory");
  c->cfg = *cfg;
  c->embed = w->embed;
  c->final_norm = w->final_norm;
  c->layers.assign(w->layers, w->layers + cfg->n_layers);
  *out = c;
  return DG_OK;
}

void dg_destroy(dg_ctx* ctx) {
  if (!ctx) return;
  for (hipEvent_t e : ctx->prof.ev) (void)hipEventDestroy(e);
  if (ctx->side) {
    (void)hipStreamSynchronize(ctx->side);
    (void)hipStreamDestroy(ctx->side);
    (void)hipEventDestroy(ctx->ev_fork);
    (void)hipEventDestroy(ctx->ev_join);
  }
  delete ctx;
}

dg_status dg_workspace_size(const dg_ctx* ctx, int batch, size_t* bytes) {
  if (!ctx || !bytes) return fail(DG_ERR_INVALID_ARG, "NULL argument");
  if (batch < 1 || batch > ctx->cfg.max_batch) return fail(DG_ERR_INVALID_ARG, "batch out of range");
  Ws ws;
  *bytes = carve(ctx->cfg, batch, nullptr, &ws);
  return DG_OK;
}

dg_status dg_kv_size(const dg_config* cfg, size_t* bytes_each) {
  if (!bytes_each) return fail(DG_ERR_INVALID_ARG, "NULL argument");
  dg_status st = validate_config(cfg);
  if (st != DG_OK) return st;
  *bytes_each = (size_t)cfg->n_layers * layer_kv_elems(*cfg) * sizeof(uint16_t);
  return DG_OK;
}

dg_status dg_prefill_kv(dg_ctx* ctx, dg_kv* kv, const int32_t* d_tokens, int batch, int n,
                        void* d_ws, size_t ws_bytes, void* stream) {
  if (!ctx) return fail(DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_kv(ctx, kv, batch);
  if (st != DG_OK) return st;
  if (n < 0) return fail(DG_ERR_INVALID_ARG, "n must be >= 0");
  if (n > 0 && !d_tokens) return fail(DG_ERR_INVALID_ARG, "tokens are NULL");
  Ws ws;
  st = get_ws(ctx, batch, d_ws, ws_bytes, &ws);
  if (st != DG_OK) return st;
  return prefill_impl(ctx, kv, d_tokens, batch, n, ws, (hipStream_t)stream);
}

dg_status dg_denoise_step(dg_ctx* ctx, const dg_kv* kv, const int32_t* d_canvas, int batch, float t,
                          uint16_t* d_logits, void* d_ws, size_t ws_bytes, void* stream) {
  if (!ctx) return fail(DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_kv(ctx, kv, batch);
  if (st != DG_OK) return st;
  if (!d_canvas || !d_logits) return fail(DG_ERR_INVALID_ARG, "canvas or logits is NULL");
  if (!(t >= 0.f && t <= 1.f)) return fail(DG_ERR_INVALID_ARG, "t must be in [0, 1]");
  Ws ws;
  st = get_ws(ctx, batch, d_ws, ws_bytes, &ws);
  if (st != DG_OK) return st;
  return denoise_impl(ctx, kv, d_canvas, batch, t, d_logits, ws, (hipStream_t)stream);
}

dg_status dg_sample_workspace_size(int batch, int canvas, int vocab, size_t* bytes) {
  if (!bytes || batch < 1 || canvas < 1 || canvas > 1024 || vocab < 8 || vocab % 8)
    return fail(DG_ERR_INVALID_ARG, "bad sampler sizes");
  Carver cv{nullptr};
  Ws ws;
  *bytes = carve_sampler(cv, batch, canvas, vocab, &ws) + kAlign;
  return DG_OK;
}

dg_status dg_sample_eb_ex(const uint16_t* d_logits, int32_t* d_canvas, int batch, int canvas, int vocab,
                          float gamma, int commit_all, float temperature, float e_stop,
                          int32_t* d_prev_argmax, int step, int32_t* d_done_step, float* d_entropy,
                          int32_t* d_argmax, int32_t* d_n_masked, void* d_ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  dg_status st = dg_sample_workspace_size(batch, canvas, vocab, &need);
  if (st != DG_OK) return st;
  if (!d_logits || !d_canvas || !d_n_masked || !d_ws) return fail(DG_ERR_INVALID_ARG, "NULL pointer");
  if (gamma != gamma) return fail(DG_ERR_INVALID_ARG, "gamma is NaN");
  if (!(temperature > 0.0f) || temperature > 3.0e38f) return fail(DG_ERR_INVALID_ARG, "temperature must be finite and > 0");
  if (e_stop != e_stop) return fail(DG_ERR_INVALID_ARG, "e_stop is NaN");
  if (step < 0) return fail(DG_ERR_INVALID_ARG, "step must be >= 0");
  if (ws_bytes < need) return fail(DG_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  char* base = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(d_ws) + kAlign - 1) / kAlign * kAlign);
  Carver cv{base};
  Ws ws;
  carve_sampler(cv, batch, canvas, vocab, &ws);
  SampleOpts o;
  o.temperature = temperature;
  o.e_stop = e_stop;
  o.prev_amax = d_prev_argmax;
  o.step = step;
  o.done_step = d_done_step;
  return sample_impl(d_logits, d_canvas, batch, canvas, vocab, gamma, commit_all, d_entropy, d_argmax,
                     d_n_masked, ws, (hipStream_t)stream, nullptr, o);
}

dg_status dg_sample_eb(const uint16_t* d_logits, int32_t* d_canvas, int batch, int canvas, int vocab,
                       float gamma, int commit_all, float* d_entropy, int32_t* d_argmax,
                       int32_t* d_n_masked, void* d_ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  dg_status st = dg_sample_workspace_size(batch, canvas, vocab, &need);
  if (st != DG_OK) return st;
  if (!d_logits || !d_canvas || !d_n_masked || !d_ws) return fail(DG_ERR_INVALID_ARG, "NULL pointer");
  if (gamma != gamma) return fail(DG_ERR_INVALID_ARG, "gamma is NaN");
  if (ws_bytes < need) return fail(DG_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  char* base = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(d_ws) + kAlign - 1) / kAlign * kAlign);
  Carver cv{base};
  Ws ws;
  carve_sampler(cv, batch, canvas, vocab, &ws);
  return sample_impl(d_logits, d_canvas, batch, canvas, vocab, gamma, commit_all, d_entropy, d_argmax,
                     d_n_masked, ws, (hipStream_t)stream);
}

dg_status dg_generate_block(dg_ctx* ctx, dg_kv* kv, int32_t* d_canvas, int batch, int steps,
                            float gamma, int append_kv, uint16_t* d_logits, int32_t* d_n_masked,
                            void* d_ws, size_t ws_bytes, void* stream) {
  if (!ctx) return fail(DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_kv(ctx, kv, batch);
  if (st != DG_OK) return st;
  if (!d_canvas || !d_logits || !d_n_masked) return fail(DG_ERR_INVALID_ARG, "NULL pointer");
  if (steps < 1) return fail(DG_ERR_INVALID_ARG, "steps must be >= 1");
  if (gamma != gamma) return fail(DG_ERR_INVALID_ARG, "gamma is NaN");
  const dg_config& c = ctx->cfg;
  for (int b = 0; b < batch; ++b)
    if (kv->len[b] + c.canvas > c.max_ctx)
      return fail(DG_ERR_KV_CAPACITY, "sequence %d: len %lld + canvas %d exceeds max_ctx %d", b,
                  (long long)kv->len[b], c.canvas, c.max_ctx);
  Ws ws;
  st = get_ws(ctx, batch, d_ws, ws_bytes, &ws);
  if (st != DG_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  DG_TIMED(ctx, DG_K_FILL, launch_fill_i32(d_canvas, c.vocab, (size_t)batch * c.canvas, s));
  for (int step = 0; step < steps; ++step) {
    const float t = 1.0f - (float)step / (float)steps;
    st = denoise_impl(ctx, kv, d_canvas, batch, t, d_logits, ws, s, /*masked_head=*/true);
    if (st != DG_OK) return st;
    st = sample_impl(d_logits, d_canvas, batch, c.canvas, c.vocab, gamma, step == steps - 1, nullptr,
                     nullptr, d_n_masked, ws, s, ctx);
    if (st != DG_OK) return st;
  }
  if (append_kv) return prefill_impl(ctx, kv, d_canvas, batch, c.canvas, ws, s);
  return DG_OK;
}

dg_status dg_generate_block_ex(dg_ctx* ctx, dg_kv* kv, int32_t* d_canvas, int batch, int max_steps,
                               float gamma, float tau_max, float tau_min, float e_stop, int append_kv,
                               uint16_t* d_logits, int32_t* d_n_masked, int32_t* d_done_step, void* d_ws,
                               size_t ws_bytes, void* stream) {
  if (!ctx) return fail(DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_kv(ctx, kv, batch);
  if (st != DG_OK) return st;
  if (!d_canvas || !d_logits || !d_n_masked || !d_done_step) return fail(DG_ERR_INVALID_ARG, "NULL pointer");
  if (max_steps < 1) return fail(DG_ERR_INVALID_ARG, "max_steps must be >= 1");
  if (gamma != gamma || e_stop != e_stop) return fail(DG_ERR_INVALID_ARG, "gamma or e_stop is NaN");
  if (!(tau_max > 0.0f) || !(tau_min > 0.0f) || tau_max > 3.0e38f || tau_min > 3.0e38f)
    return fail(DG_ERR_INVALID_ARG, "temperatures must be finite and > 0");
  const dg_config& c = ctx->cfg;
  for (int b = 0; b < batch; ++b)
    if (kv->len[b] + c.canvas > c.max_ctx)
      return fail(DG_ERR_KV_CAPACITY, "sequence %d: len %lld + canvas %d exceeds max_ctx %d", b,
                  (long long)kv->len[b], c.canvas, c.max_ctx);
  Ws ws;
  st = get_ws(ctx, batch, d_ws, ws_bytes, &ws);
  if (st != DG_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  DG_TIMED(ctx, DG_K_FILL, launch_fill_i32(d_canvas, c.vocab, (size_t)batch * c.canvas, s));
  DG_TIMED(ctx, DG_K_FILL, launch_fill_i32(ws.prev_amax, -1, (size_t)batch * c.canvas, s));
  DG_TIMED(ctx, DG_K_FILL, launch_fill_i32(d_done_step, 0, (size_t)batch, s));
  for (int step = 0; step < max_steps; ++step) {
    const float t = 1.0f - (float)step / (float)max_steps;
    SampleOpts o;
    o.temperature = tau_min + (tau_max - tau_min) * t;
    if (!(o.temperature > 0.0f)) return fail(DG_ERR_INVALID_ARG, "annealed temperature must stay > 0");
    o.e_stop = e_stop;
    o.prev_amax = ws.prev_amax;
    o.step = step;
    o.done_step = d_done_step;
    st = denoise_impl(ctx, kv, d_canvas, batch, t, d_logits, ws, s, /*masked_head=*/true);
    if (st != DG_OK) return st;
    st = sample_impl(d_logits, d_canvas, batch, c.canvas, c.vocab, gamma, step == max_steps - 1, nullptr,
                     nullptr, d_n_masked, ws, s, ctx, o);
    if (st != DG_OK) return st;
  }
  if (append_kv) return prefill_impl(ctx, kv, d_canvas, batch, c.canvas, ws, s);
  return DG_OK;
}

dg_status dg_packed_elems(int rows, int cols, size_t* elems) {
  if (!elems || rows < 1 || cols < 32 || cols % 32) return fail(DG_ERR_INVALID_ARG, "bad packing shape");
  *elems = round16((size_t)rows) * (size_t)cols;
  return DG_OK;
}

dg_status dg_pack_weight(int kind, const uint16_t* d_src, uint16_t* d_dst, int n_mats, int rows, int cols,
                         int param, void* stream) {
  if (!d_src || !d_dst || n_mats < 1 || rows < 1 || cols < 32 || cols % 32)
    return fail(DG_ERR_INVALID_ARG, "bad packing arguments");
  if (kind == DG_PACK_QKV) {
    if ((param != 32 && param != 64 && param != 128) || rows % param)
      return fail(DG_ERR_INVALID_ARG, "qkv packing needs rows = heads * head_dim");
  } else if (kind == DG_PACK_GATE_UP) {
    if (param < 16 || param % 16 || rows != 2 * param)
      return fail(DG_ERR_INVALID_ARG, "gate/up packing needs rows = 2 * F, F % 16 == 0");
  } else if (kind != DG_PACK_PLAIN) {
    return fail(DG_ERR_INVALID_ARG, "unknown packing kind");
  }
  launch_pack(d_src, d_dst, n_mats, rows, cols, kind, param, (hipStream_t)stream);
  return check_launch("pack");
}

dg_status dg_profile_begin(dg_ctx* ctx, int capacity, uint32_t kind_mask) {
  if (!ctx || capacity < 1) return fail(DG_ERR_INVALID_ARG, "bad profiling arguments");
  if (kind_mask >> DG_K_COUNT) return fail(DG_ERR_INVALID_ARG, "kind_mask names an unknown kernel kind");
  Prof& p = ctx->prof;
  p.mask = kind_mask ? kind_mask : (1u << DG_K_COUNT) - 1u;
  for (hipEvent_t e : p.ev) (void)hipEventDestroy(e);
  p.ev.assign(2 * (size_t)capacity, nullptr);
  for (auto& e : p.ev)
    if (hipEventCreate(&e) != hipSuccess) return fail(DG_ERR_HIP, "hipEventCreate failed");
  p.kind.assign(capacity, -1);
  p.used = 0;
  p.on = true;
  return DG_OK;
}

dg_status dg_profile_end(dg_ctx* ctx, double* ms, int32_t* count) {
  if (!ctx || !ms || !count) return fail(DG_ERR_INVALID_ARG, "NULL argument");
  Prof& p = ctx->prof;
  p.on = false;
  for (int k = 0; k < DG_K_COUNT; ++k) {
    ms[k] = 0.0;
    count[k] = 0;
  }
  for (size_t i = 0; i < p.used; ++i) {
    if (p.kind[i] < 0) continue;
    if (hipEventSynchronize(p.ev[2 * i + 1]) != hipSuccess) return fail(DG_ERR_HIP, "event sync failed");
    float t = 0.f;
    if (hipEventElapsedTime(&t, p.ev[2 * i], p.ev[2 * i + 1]) != hipSuccess)
      return fail(DG_ERR_HIP, "event timing failed");
    ms[p.kind[i]] += t;
    count[p.kind[i]] += 1;
  }
  for (hipEvent_t e : p.ev) (void)hipEventDestroy(e);
  p.ev.clear();
  p.kind.clear();
  p.used = 0;
  return DG_OK;
}

dg_status dg_workspace_moe_counts(const dg_ctx* ctx, int batch, size_t* offset) {
  if (!ctx || !offset || batch < 1 || batch > ctx->cfg.max_batch) return fail(DG_ERR_INVALID_ARG, "bad arguments");
  Ws ws;
  carve(ctx->cfg, batch, reinterpret_cast<char*>(kAlign), &ws);   // offsets relative to an aligned base
  *offset = reinterpret_cast<uintptr_t>(ws.cnt_log) - kAlign;
  return DG_OK;
}

dg_status dg_test_router_topk(const float* d_r, int M, int E, int k, int32_t* d_ids, float* d_w,
                              void* stream) {
  if (!d_r || !d_ids || !d_w || M < 1 || E < 4 || E > 256 || E % 4 || k < 1 || k > 16 || k > E)
    return fail(DG_ERR_INVALID_ARG, "bad router arguments");
  launch_topk(d_r, M, E, k, d_ids, d_w, (hipStream_t)stream);
  return check_launch("router top-k");
}

dg_status dg_test_route(const float* d_r, int M, int E, int k, int32_t* d_ids, float* d_w,
                        int32_t* d_cnt, int32_t* d_poff, int32_t* d_perm, int32_t* d_inv,
                        int32_t* d_items, int32_t* d_n_items, void* stream) {
  if (!d_r || !d_ids || !d_w || !d_cnt || !d_poff || !d_perm || !d_inv || !d_items || !d_n_items ||
      M < 1 || E < 4 || E > 256 || E % 4 || k < 1 || k > 16 || k > E)
    return fail(DG_ERR_INVALID_ARG, "bad routing arguments");
  hipStream_t s = (hipStream_t)stream;
  launch_topk(d_r, M, E, k, d_ids, d_w, s);
  launch_route(d_ids, M, k, E, d_cnt, d_poff, d_perm, d_inv, reinterpret_cast<int2*>(d_items), d_n_items,
               nullptr, nullptr, nullptr, s);
  return check_launch("route");
}

dg_status dg_test_eb_select(const float* d_entropy, const int32_t* d_argmax, int32_t* d_canvas,
                            int batch, int canvas, int vocab, float gamma, int commit_all,
                            int32_t* d_n_masked, void* stream) {
  if (!d_entropy || !d_argmax || !d_canvas || !d_n_masked || batch < 1 || canvas < 1 || canvas > 1024 ||
      vocab < 1 || gamma != gamma)
    return fail(DG_ERR_INVALID_ARG, "bad selection arguments");
  launch_eb_select(nullptr, nullptr, 0, d_entropy, d_argmax, d_canvas, batch, canvas, vocab, gamma,
                   commit_all, nullptr, nullptr, d_n_masked, nullptr, -1.0f, 0, nullptr, (hipStream_t)stream);
  return check_launch("eb select");
}

dg_status dg_test_gemm(const uint16_t* d_x, const uint16_t* d_w, float* d_y, int M, int N, int K,
                       void* stream) {
  if (!d_x || !d_w || !d_y || M < 1 || N < 4 || N % 4 || K < 64 || K % 64)
    return fail(DG_ERR_INVALID_ARG, "bad GEMM arguments");
  launch_gemm_f32(d_x, d_w, d_y, M, N, K, false, (hipStream_t)stream);
  return check_launch("gemm");
}

dg_status dg_test_copy(const void* d_src, void* d_dst, size_t n_bytes, void* stream) {
  if (!d_src || !d_dst || n_bytes == 0 || n_bytes % 16)
    return fail(DG_ERR_INVALID_ARG, "copy needs non-NULL buffers and a positive multiple of 16 bytes");
  launch_copy16(d_src, d_dst, n_bytes, (hipStream_t)stream);
  return check_launch("copy");
}

}  // extern "C"
