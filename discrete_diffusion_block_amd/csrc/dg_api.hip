// C ABI of the engine: argument validation, workspace carving and the
// per-pass kernel schedule.  Everything is enqueued on the caller's stream;
// nothing here allocates device memory.  Only the block generators with the
// adaptive stop on read back (a few words of pinned host memory, two steps
// behind the device) and wait on the device for them.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <string>
#include <utility>
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

struct StopProbe;

struct dg_ctx {
  dg_config cfg;
  const uint16_t* embed;
  const float* final_norm;
  std::vector<dg_layer_weights> layers;
  // self-conditioning weights (all NULL: none)
  const uint16_t* embed_t = nullptr;
  const uint16_t* sc_gate_up = nullptr;
  const uint16_t* sc_down = nullptr;
  mutable Prof prof;
  // Side stream for the shared expert, which runs concurrently with the routed
  // experts' routing chain; forked from and joined back into the caller's stream
  // with events.  Created by dg_create on the device current then (side_dev);
  // calls made on another device keep all work on the caller's stream.  Calls
  // from several threads may enqueue on it at once: each call forks and joins
  // with an event pair of its own, and every item a call puts on the side stream
  // waits only for work its own call enqueued earlier, so the calls serialise
  // there without ever waiting on each other in a cycle.
  hipStream_t side = nullptr;
  int side_dev = -1;
  // Fork/join event pairs, one per call in flight (taken at the start of a call,
  // given back at its end; a pair given back may still be pending on the device,
  // which is fine: a wait refers to the record that preceded it).
  mutable std::mutex ev_mu;
  mutable std::vector<std::pair<hipEvent_t, hipEvent_t>> ev_free;
  mutable std::vector<std::pair<hipEvent_t, hipEvent_t>> ev_all;
  // Forced routing (test tap, not thread-safe): when set, layer l of every pass
  // takes its expert ids from force_ids + l * M * k instead of the router's top-k.
  const int32_t* force_ids = nullptr;
  // Stop probes of the block generators (see StopProbe), one per call in flight;
  // guarded by ev_mu.
  mutable std::vector<StopProbe*> probes;
};

// Host view of the adaptive stop inside one block-generator call.  After the
// sampler of step s the generator copies the per-sequence completion steps into
// pinned host memory (slot s % kStopLag) and records an event; before it enqueues
// step s it waits for the event of step s - kStopLag and ends the loop once every
// sequence is complete.  The device then runs at most one pass after the stop (the
// one already enqueued), and the host stays kStopLag steps ahead of the device.
constexpr int kStopLag = 2;
struct StopProbe {
  int dev = -1;
  bool busy = false;
  int32_t* host = nullptr;                 // pinned [kStopLag][DG_MAX_BATCH]
  hipEvent_t ev[kStopLag] = {};
  bool recorded[kStopLag] = {};
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

// Fork/join events of one call: the side stream and an event pair for the current
// device, or a null side stream (all work then stays on the caller's stream) when
// the call runs on another device than the ctx's or the events cannot be made.
struct SideFork {
  const dg_ctx* ctx = nullptr;
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  explicit SideFork(const dg_ctx* c) : ctx(c) {
    int dev = -1;
    if (!c->side || hipGetDevice(&dev) != hipSuccess || dev != c->side_dev) return;
    std::lock_guard<std::mutex> lk(c->ev_mu);
    if (c->ev_free.empty()) {
      // both events only order work between two queues of this device: no
      // system-scope (host-visibility) fence is needed when they are signalled
      constexpr unsigned kFlags = hipEventDisableTiming | hipEventDisableSystemFence;
      hipEvent_t a = nullptr, b = nullptr;
      if (hipEventCreateWithFlags(&a, kFlags) != hipSuccess) return;
      if (hipEventCreateWithFlags(&b, kFlags) != hipSuccess) {
        (void)hipEventDestroy(a);
        return;
      }
      c->ev_all.emplace_back(a, b);
      c->ev_free.emplace_back(a, b);
    }
    fork = c->ev_free.back().first;
    join = c->ev_free.back().second;
    c->ev_free.pop_back();
    side = c->side;
  }
  ~SideFork() {
    if (!side) return;
    std::lock_guard<std::mutex> lk(ctx->ev_mu);
    ctx->ev_free.emplace_back(fork, join);
  }
  SideFork(const SideFork&) = delete;
  SideFork& operator=(const SideFork&) = delete;
};

// A probe for the current device whose earlier copies have all landed (a probe
// given back by an earlier call may still have a copy in flight on that call's
// stream, which must not land in this call's slots), or a new one; NULL when none
// can be made (the generator then runs every step).
StopProbe* acquire_probe(const dg_ctx* c) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lk(c->ev_mu);
  for (StopProbe* p : c->probes) {
    if (p->busy || p->dev != dev) continue;
    bool idle = true;
    for (int i = 0; i < kStopLag; ++i)
      if (p->recorded[i] && hipEventQuery(p->ev[i]) != hipSuccess) idle = false;
    if (idle) {
      p->busy = true;
      return p;
    }
  }
  (void)hipGetLastError();
  StopProbe* p = new (std::nothrow) StopProbe;
  if (!p) return nullptr;
  p->dev = dev;
  bool ok = hipHostMalloc((void**)&p->host, sizeof(int32_t) * kStopLag * DG_MAX_BATCH, hipHostMallocDefault) ==
            hipSuccess;
  for (int i = 0; ok && i < kStopLag; ++i) ok = hipEventCreateWithFlags(&p->ev[i], hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    for (int i = 0; i < kStopLag; ++i)
      if (p->ev[i]) (void)hipEventDestroy(p->ev[i]);
    if (p->host) (void)hipHostFree(p->host);
    delete p;
    (void)hipGetLastError();
    return nullptr;
  }
  p->busy = true;
  c->probes.push_back(p);
  return p;
}

struct ProbeLease {
  const dg_ctx* c;
  StopProbe* p;
  ProbeLease(const dg_ctx* c_, bool want) : c(c_), p(want ? acquire_probe(c_) : nullptr) {}
  ~ProbeLease() {
    if (!p) return;
    std::lock_guard<std::mutex> lk(c->ev_mu);
    p->busy = false;
  }
  ProbeLease(const ProbeLease&) = delete;
  ProbeLease& operator=(const ProbeLease&) = delete;
};

constexpr int kPrefillChunk = 512;   // tokens per sequence per encoder pass
constexpr int kPassCounters = 16;    // device counters cleared at the start of every pass
constexpr size_t kAlign = 256;

struct Ws {
  float* x;        // residual stream, fp32 row-major [M][d]
  uint16_t* h;     // normed activations, fragment-major [M_pad][d]
  uint16_t* h_rm;  // the FFN-normed activations again, row-major [M][d] (expert row gathers)
  uint16_t* q;     // queries, fragment-major per (sequence, head) [n_pad][hd]
  uint16_t* o;     // attention output, fragment-major [M_pad][Hq*hd]
  float* att_po;   // attention split-KV partial outputs [kAttnMaxSplitRows * Hq][hd]
  float2* att_pml; // and their (max, sum) [kAttnMaxSplitRows * Hq]
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
  ulonglong2* cpart;   // canonical-entropy integer chunk sums
  int32_t* sflag;      // [batch]: sequence deferred to the canonical entropy
  int32_t* smoved;     // [batch]
  int32_t* samax;      // [batch][C]
  float* shf;          // [batch][C]: fast entropies
  float2* swin;        // [batch]: boundary windows
  int32_t* skstar;     // [batch]
  // self-conditioning (carved only when the ctx has its weights): rows = batch * C
  float2* sc_stats;    // [rows]: (max log2e, 1 / S)
  float* sc_part;      // [splits][rows][d]: partial sums of p̂₀ E
  uint16_t* sc_u;      // p̂₀ E in bf16, fragment-major [rows_pad][d]
  uint16_t* sc_act;    // FFW activation, fragment-major [rows_pad][Fs]
  float* sc_z;         // the signal, fp32 row-major [rows][d]
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
  ws->cpart = cv.take<ulonglong2>(rows * sample_chunks(vocab));
  ws->sflag = cv.take<int32_t>(batch);
  ws->smoved = cv.take<int32_t>(batch);
  ws->samax = cv.take<int32_t>(rows);
  ws->shf = cv.take<float>(rows);
  ws->swin = cv.take<float2>(batch);
  ws->skstar = cv.take<int32_t>(batch);
  return cv.off;
}

size_t round16(size_t v) { return (v + 15) / 16 * 16; }

size_t carve(const dg_config& c, int batch, char* base, Ws* ws, bool self_cond) {
  const size_t n = (size_t)std::max(c.canvas, kPrefillChunk);
  const size_t M = (size_t)batch * n;
  const size_t Mp = round16(M);
  const size_t qd = (size_t)c.n_q_heads * c.head_dim;
  const size_t P = (size_t)moe_max_slots((int)M, c.top_k, c.n_experts);
  Carver cv{base};
  // first, so that its offset is the same for every batch (dg_workspace_moe_counts)
  ws->cnt_log = cv.take<int32_t>((size_t)c.n_layers * c.n_experts);
  ws->x = cv.take<float>(M * c.d_model);
  ws->h = cv.take<uint16_t>(Mp * c.d_model);
  ws->h_rm = cv.take<uint16_t>(M * c.d_model);
  ws->q = cv.take<uint16_t>((size_t)batch * round16(n) * qd);
  ws->o = cv.take<uint16_t>(Mp * qd);
  ws->att_po = cv.take<float>((size_t)kAttnMaxSplitRows * qd);
  ws->att_pml = cv.take<float2>((size_t)kAttnMaxSplitRows * c.n_q_heads);
  ws->rope = cv.take<float2>(M * (c.head_dim / 2));
  ws->temb = cv.take<float>((size_t)DG_MAX_BATCH * c.d_model);   // a fused block pass has 2 sequences per slot
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
  ws->rows = cv.take<int32_t>(M);
  ws->counters = cv.take<int32_t>(kPassCounters);
  ws->A = cv.take<uint16_t>(round16(P) * c.expert_ffn);
  ws->Y = cv.take<float>(P * c.d_model);
  ws->As = cv.take<uint16_t>(Mp * c.shared_ffn);
  ws->ys = cv.take<float>(M * c.d_model);
  ws->prev_amax = cv.take<int32_t>((size_t)batch * c.canvas);
  carve_sampler(cv, batch, c.canvas, c.vocab, ws);
  ws->sc_stats = nullptr;
  ws->sc_part = ws->sc_z = nullptr;
  ws->sc_u = ws->sc_act = nullptr;
  if (self_cond) {
    const size_t rows = (size_t)batch * c.canvas;
    ws->sc_stats = cv.take<float2>(rows);
    ws->sc_part = cv.take<float>((size_t)sc_splits((int)rows, c.d_model, c.vocab) * rows * c.d_model);
    ws->sc_u = cv.take<uint16_t>(round16(rows) * c.d_model);
    ws->sc_act = cv.take<uint16_t>(round16(rows) * c.shared_ffn);
    ws->sc_z = cv.take<float>(rows * c.d_model);
  }
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
// split > 0 (a fused block pass): the pass's first `split` sequences are KV updates and
// the others denoising canvases; attention runs as one launch per group (each with the
// key splitting it gets in a pass of its own), and the head's output rows count from
// the first denoising row.
PassGeom sub_geom(const PassGeom& g, int s0, int s1) {
  PassGeom h{};
  h.batch = s1 - s0;
  h.n = g.n;
  h.enc = (g.enc >> s0) & all_sequences(s1 - s0);
  h.denoise = h.enc != all_sequences(s1 - s0);
  for (int b = s0; b < s1; ++b) {
    h.len[b - s0] = g.len[b];
    h.t[b - s0] = g.t[b];
    h.kvshift[b - s0] = g.kvshift[b] - s0;   // the same cache sequence: (b - s0) - h.kvshift = b - g.kvshift
  }
  return h;
}

dg_status run_pass(const dg_ctx* ctx, const dg_kv* kv, const PassGeom& g, const int32_t* tokens,
                   uint16_t* logits, const Ws& ws, hipStream_t s, bool masked_head = false,
                   const float* z = nullptr, int split = 0) {
  const dg_config& c = ctx->cfg;
  for (int b = 0; b < g.batch; ++b)
    if (kv_seq(g, b) < 0 || kv_seq(g, b) >= c.max_batch)
      return fail(DG_ERR_INVALID_ARG, "pass sequence %d maps to cache sequence %d", b, kv_seq(g, b));
  const int M = g.batch * g.n;
  const int d = c.d_model, hq = c.n_q_heads, hd = c.head_dim, E = c.n_experts, k = c.top_k;
  const float eps = c.rms_eps;
  const int nl = c.n_layers;
  SideFork sf(ctx);
  DG_TIMED(ctx, DG_K_PREP, launch_prep(g, hd, c.rope_theta, ws.rope, d, g.denoise ? ws.temb : nullptr,
                                       ws.counters, kPassCounters, s));
  DG_TIMED(ctx, DG_K_EMBED,
           launch_embed_norm(tokens, ctx->embed, g.denoise ? ws.temb : nullptr, g.denoise ? z : nullptr, g.n, g.enc,
                             ctx->layers[0].attn_norm, eps, ws.x, ws.h, M, d, c.vocab, s));
  for (int l = 0; l < nl; ++l) {
    const dg_layer_weights& L = ctx->layers[l];
    const KvLayer kvl = kv_layer(ctx, kv, l);
    DG_TIMED(ctx, DG_K_QKV, launch_qkv_rope(ws.h, L.w_qkv, M, d, hq, kvl, g, ws.rope, ws.q, s));
    // In the encoder only the keys/values are observable; the last layer's
    // attention output and FFN feed nothing, so they are not computed.
    if (!g.denoise && l == nl - 1) break;
    if (split > 0 && split < g.batch) {
      const size_t q_seq = (size_t)hq * ((g.n + 15) & ~15) * hd;    // one sequence's q
      for (int part = 0; part < 2; ++part) {
        const int s0 = part ? split : 0, s1 = part ? g.batch : split;
        DG_TIMED(ctx, kvl.window == 0 ? DG_K_ATTENTION_GLOBAL : DG_K_ATTENTION,
                 launch_attention(ws.q + s0 * q_seq, hq, kvl, sub_geom(g, s0, s1),
                                  ws.o + (size_t)s0 * g.n * hq * hd, ws.att_po, ws.att_pml, s));
      }
    } else {
      DG_TIMED(ctx, kvl.window == 0 ? DG_K_ATTENTION_GLOBAL : DG_K_ATTENTION,
               launch_attention(ws.q, hq, kvl, g, ws.o, ws.att_po, ws.att_pml, s));
    }
    DG_TIMED(ctx, DG_K_O_PROJ, launch_gemm_f32(ws.o, L.w_o, ws.x, M, d, hq * hd, /*add=*/true, s));
    // The shared expert depends only on h: it runs on the side stream while the
    // routed experts' routing chain (small, latency-bound kernels) runs here.  It
    // reads h and writes As and ys, which nothing on this stream touches before
    // the join; the combine kernel adds ys.  The fork and join events are
    // signalled by the kernels' own completion (no marker packets on the queues).
    hipStream_t s2 = sf.side;
    const bool fork = s2 != nullptr;
    if (!fork) s2 = s;
    DG_TIMED(ctx, DG_K_NORM,
             launch_rmsnorm(ws.x, L.ffn_norm, eps, ws.h, ws.h_rm, M, d, s, fork ? sf.fork : nullptr));
    if (fork) (void)hipStreamWaitEvent(s2, sf.fork, 0);
    DG_TIMED_ON(ctx, DG_K_SHARED_GATE_UP, s2,
                launch_gemm_swiglu(ws.h, L.ws_gate_up, M, c.shared_ffn, d, ws.As, s2));
    DG_TIMED_ON(ctx, DG_K_SHARED_DOWN, s2,
                launch_gemm_f32(ws.As, L.ws_down, ws.ys, M, d, c.shared_ffn, /*add=*/false, s2,
                                fork ? sf.join : nullptr));
    DG_TIMED(ctx, DG_K_ROUTER, launch_gemm_f32(ws.h, L.w_router, ws.r, M, E, d, /*add=*/false, s));
    if (ctx->force_ids)
      DG_TIMED(ctx, DG_K_TOPK,
               launch_forced_route(ws.r, M, E, k, ctx->force_ids + (size_t)l * M * k, ws.ids, ws.wts, s));
    else
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
    if (fork) (void)hipStreamWaitEvent(s, sf.join, 0);
    const float* next_gain = (l + 1 < nl) ? ctx->layers[l + 1].attn_norm : (g.denoise ? ctx->final_norm : nullptr);
    // the head's rows: those of the denoising sequences (all of them, or only their
    // [MASK] rows), compacted when that is not every row
    const bool compact = (masked_head || g.enc != 0) && g.denoise && l == nl - 1;
    DG_TIMED(ctx, DG_K_COMBINE,
             launch_combine(ws.x, ws.ys, ws.Y, ws.wts, ws.inv, M, k, d, next_gain, eps, ws.h,
                            compact && masked_head ? tokens : nullptr, c.vocab, g.enc, g.n,
                            compact ? ws.rows : nullptr, ws.counters, split * g.n, s));
  }
  const bool compact = (masked_head || g.enc != 0) && g.denoise;
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
  const size_t need = carve(ctx->cfg, batch, nullptr, ws, ctx->embed_t != nullptr);
  if (!d_ws) return fail(DG_ERR_INVALID_ARG, "workspace is NULL");
  if (ws_bytes < need) return fail(DG_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  char* base = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(d_ws) + kAlign - 1) / kAlign * kAlign);
  carve(ctx->cfg, batch, base, ws, ctx->embed_t != nullptr);
  return DG_OK;
}

dg_status denoise_impl(dg_ctx* ctx, const dg_kv* kv, const int32_t* d_canvas, int batch, float t,
                       uint16_t* d_logits, const Ws& ws, hipStream_t s, bool masked_head = false,
                       const float* z = nullptr) {
  PassGeom g{};
  g.batch = batch;
  g.n = ctx->cfg.canvas;
  g.denoise = 1;
  g.enc = 0;
  for (int b = 0; b < batch; ++b) {
    if (kv->len[b] + ctx->cfg.canvas > ctx->cfg.max_ctx)
      return fail(DG_ERR_KV_CAPACITY, "sequence %d: len %lld + canvas %d exceeds max_ctx %d", b,
                  (long long)kv->len[b], ctx->cfg.canvas, ctx->cfg.max_ctx);
    g.len[b] = (int)kv->len[b];
    g.t[b] = t;
  }
  return run_pass(ctx, kv, g, d_canvas, d_logits, ws, s, masked_head, z);
}

// Self-conditioning signal z (and u = p̂₀ E in fp32 when u_out is given) of the
// batch * C logits rows (Technical Report §3.2, eq. 5-6).
dg_status self_cond_impl(const dg_ctx* ctx, const uint16_t* logits, int batch, float* z, float* u_out,
                         const Ws& ws, hipStream_t s) {
  const dg_config& c = ctx->cfg;
  const int M = batch * c.canvas, d = c.d_model, V = c.vocab;
  DG_TIMED(ctx, DG_K_SC_STATS, launch_sc_rowstats(logits, M, V, ws.sc_stats, s));
  DG_TIMED(ctx, DG_K_SC_EMBED, launch_sc_embed(logits, ws.sc_stats, ctx->embed_t, M, d, V, ws.sc_part, s));
  DG_TIMED(ctx, DG_K_SC_REDUCE,
           launch_sc_reduce(ws.sc_part, sc_splits(M, d, V), ws.sc_stats, M, d, ws.sc_u, u_out, s));
  DG_TIMED(ctx, DG_K_SC_FFW, launch_gemm_swiglu(ws.sc_u, ctx->sc_gate_up, M, c.shared_ffn, d, ws.sc_act, s));
  DG_TIMED(ctx, DG_K_SC_FFW, launch_gemm_f32(ws.sc_act, ctx->sc_down, z, M, d, c.shared_ffn, /*add=*/false, s));
  return check_launch("self-conditioning");
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
      g.enc = all_sequences(batch);
      for (int b = 0; b < batch; ++b) g.len[b] = (int)kv->len[b] + s0;
      // a chunk's tokens are a strided slice when batch > 1; only batch == 1 can chunk in place
      dg_status st = run_pass(ctx, kv, g, d_tokens + s0, nullptr, ws, s);
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
        g.enc = 1;
        g.len[0] = (int)kv->len[b] + s0;
        dg_kv one = *kv;
        const size_t seq_k = (size_t)ctx->cfg.n_kv_heads * ctx->cfg.max_ctx * ctx->cfg.head_dim;
        // view of sequence b: offset the cache base by b sequences within each layer
        one.k = kv->k + (size_t)b * seq_k;
        one.v = kv->v + (size_t)b * seq_k;
        dg_status st = run_pass(ctx, &one, g, d_tokens + (size_t)b * n + s0, nullptr, ws, s);
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
  // uniform variant (Technical Report §3.2, multinomial diffusion): every position a
  // candidate, the others re-noised with the tokens of (seed, draw)
  int uniform = 0;
  uint64_t seed = 0;
  int draw = 0;
};

// commit: bit b set = sequence b commits every candidate row (the last step of its block)
uint64_t commit_mask(bool all) { return all ? ~0ull : 0ull; }

dg_status sample_impl(const uint16_t* d_logits, int32_t* d_canvas, int batch, int canvas, int vocab,
                      float gamma, uint64_t commit, float* d_entropy, int32_t* d_argmax,
                      int32_t* d_n_masked, const Ws& ws, hipStream_t s, const dg_ctx* ctx = nullptr,
                      const SampleOpts& o = SampleOpts{}) {
  DG_TIMED(ctx, DG_K_SAMPLE_PASS1,
           launch_sample_partials(d_logits, d_canvas, batch, canvas, vocab, 1.0f / o.temperature, o.uniform,
                                  o.uniform ? o.done_step : nullptr, ws.part, ws.part_arg, s));
  DG_TIMED(ctx, DG_K_SAMPLE_SELECT,
           launch_eb_select(ws.part, ws.part_arg, sample_chunks(vocab), nullptr, nullptr, d_canvas, batch,
                            canvas, vocab, gamma, commit, d_entropy, d_argmax, d_n_masked, o.prev_amax,
                            o.e_stop, o.step, o.done_step, ws.sflag, ws.smoved, ws.samax, ws.shf, ws.swin,
                            ws.skstar, o.uniform, o.seed, o.draw, s));
  // sequences whose decision the fast entropies could not certify: canonical entropy
  // (every workgroup of a decided sequence returns at once)
  DG_TIMED(ctx, DG_K_SAMPLE_CANON,
           launch_canon_partials(d_logits, d_canvas, batch, canvas, vocab, o.temperature, o.uniform, ws.part,
                                 ws.sflag, ws.shf, ws.swin, ws.cpart, s));
  DG_TIMED(ctx, DG_K_SAMPLE_SELECT_CANON,
           launch_eb_select_canon(ws.cpart, sample_chunks(vocab), d_canvas, batch, canvas, vocab, gamma,
                                  commit, d_entropy, d_argmax, d_n_masked, o.prev_amax, o.e_stop, o.step,
                                  o.done_step, ws.sflag, ws.smoved, ws.samax, ws.shf, ws.swin, ws.skstar,
                                  o.uniform, o.seed, o.draw, s));
  return check_launch("sampler");
}

// ---- static scratch for the sampler variant that allocates nothing ----
//
// dg_sample_eb_noalloc keeps the sampler's workspace in this file-scope device array
// (each device holds its own copy from module load until the process ends).  Host code
// never names the array when it needs its memory: the name is a host-side stand-in;
// the device address comes from hipGetSymbolAddress, once per device, kept below.
constexpr size_t kScratchBytes = size_t(4) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call per device).
dg_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(DG_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(DG_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DG_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DG_OK;
}

// Validation and workspace carving shared by the sampler entry points.
dg_status sample_checked(const uint16_t* d_logits, int32_t* d_canvas, int batch, int canvas, int vocab,
                         float gamma, int commit_all, float* d_entropy, int32_t* d_argmax, int32_t* d_n,
                         void* d_ws, size_t ws_bytes, void* stream, const SampleOpts& o) {
  size_t need = 0;
  dg_status st = dg_sample_workspace_size(batch, canvas, vocab, &need);
  if (st != DG_OK) return st;
  if (!d_logits || !d_canvas || !d_n || !d_ws) return fail(DG_ERR_INVALID_ARG, "NULL pointer");
  if (gamma != gamma) return fail(DG_ERR_INVALID_ARG, "gamma is NaN");
  if (!(o.temperature > 0.0f) || o.temperature > 3.0e38f)
    return fail(DG_ERR_INVALID_ARG, "temperature must be finite and > 0");
  if (o.e_stop != o.e_stop) return fail(DG_ERR_INVALID_ARG, "e_stop is NaN");
  if (o.step < 0) return fail(DG_ERR_INVALID_ARG, "step must be >= 0");
  if (ws_bytes < need) return fail(DG_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  char* base = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(d_ws) + kAlign - 1) / kAlign * kAlign);
  Carver cv{base};
  Ws ws;
  carve_sampler(cv, batch, canvas, vocab, &ws);
  return sample_impl(d_logits, d_canvas, batch, canvas, vocab, gamma, commit_mask(commit_all), d_entropy, d_argmax, d_n, ws,
                     (hipStream_t)stream, nullptr, o);
}

// The annealed, adaptively stopped block generation of the Technical Report (§3.3) on the
// absorbing canvas (uniform 0: all [MASK] at the start, masked rows only in the head) or
// the uniform variant (§3.2: uniformly random tokens at the start, draw s + 1 re-noises
// after step s, every row in the head).
dg_status generate_annealed(dg_ctx* ctx, dg_kv* kv, int32_t* d_canvas, int batch, int max_steps, float gamma,
                            float tau_max, float tau_min, float e_stop, int uniform, uint64_t seed, int append_kv,
                            uint16_t* d_logits, int32_t* d_n, int32_t* d_done_step, void* d_ws, size_t ws_bytes,
                            void* stream, bool self_cond = false) {
  if (!ctx) return fail(DG_ERR_INVALID_ARG, "ctx is NULL");
  if (self_cond && !ctx->embed_t)
    return fail(DG_ERR_UNSUPPORTED, "the ctx was created without self-conditioning weights");
  dg_status st = check_kv(ctx, kv, batch);
  if (st != DG_OK) return st;
  if (!d_canvas || !d_logits || !d_n || !d_done_step) return fail(DG_ERR_INVALID_ARG, "NULL pointer");
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
  if (uniform)
    DG_TIMED(ctx, DG_K_FILL, launch_uniform_canvas(d_canvas, batch, c.canvas, c.vocab, seed, 0, s));
  else
    DG_TIMED(ctx, DG_K_FILL, launch_fill_i32(d_canvas, c.vocab, (size_t)batch * c.canvas, s));
  DG_TIMED(ctx, DG_K_FILL, launch_fill_i32(ws.prev_amax, -1, (size_t)batch * c.canvas, s));
  DG_TIMED(ctx, DG_K_FILL, launch_fill_i32(d_done_step, 0, (size_t)batch, s));
  // with the adaptive stop on, the passes after every canvas is complete are skipped
  ProbeLease probe(ctx, e_stop >= 0.0f && max_steps > kStopLag);
  for (int step = 0; step < max_steps; ++step) {
    if (probe.p && step >= kStopLag) {
      const int slot = step % kStopLag;   // written after the sampler of step - kStopLag
      const hipError_t e = hipEventSynchronize(probe.p->ev[slot]);
      if (e != hipSuccess) return fail(DG_ERR_HIP, "stop probe: %s", hipGetErrorString(e));
      const int32_t* h = probe.p->host + slot * DG_MAX_BATCH;
      bool all = true;
      for (int b = 0; b < batch; ++b) all = all && h[b] != 0;
      if (all) break;
    }
    const float t = 1.0f - (float)step / (float)max_steps;
    SampleOpts o;
    o.temperature = tau_min + (tau_max - tau_min) * t;
    if (!(o.temperature > 0.0f)) return fail(DG_ERR_INVALID_ARG, "annealed temperature must stay > 0");
    o.e_stop = e_stop;
    o.prev_amax = ws.prev_amax;
    o.step = step;
    o.done_step = d_done_step;
    o.uniform = uniform;
    o.seed = seed;
    o.draw = step + 1;
    // with self-conditioning every row's logits feed z; otherwise the absorbing canvas
    // needs only its [MASK] rows
    st = denoise_impl(ctx, kv, d_canvas, batch, t, d_logits, ws, s, /*masked_head=*/!uniform && !self_cond,
                      self_cond && step > 0 ? ws.sc_z : nullptr);
    if (st != DG_OK) return st;
    if (self_cond && step + 1 < max_steps) {
      st = self_cond_impl(ctx, d_logits, batch, ws.sc_z, nullptr, ws, s);
      if (st != DG_OK) return st;
    }
    st = sample_impl(d_logits, d_canvas, batch, c.canvas, c.vocab, gamma, commit_mask(step == max_steps - 1), nullptr,
                     nullptr, d_n, ws, s, ctx, o);
    if (st != DG_OK) return st;
    if (probe.p && step + kStopLag < max_steps) {   // read before step + kStopLag is enqueued
      const int slot = step % kStopLag;
      hipError_t e = hipMemcpyAsync(probe.p->host + slot * DG_MAX_BATCH, d_done_step, sizeof(int32_t) * batch,
                                    hipMemcpyDeviceToHost, s);
      if (e == hipSuccess) e = hipEventRecord(probe.p->ev[slot], s);
      if (e != hipSuccess) return fail(DG_ERR_HIP, "stop probe: %s", hipGetErrorString(e));
      probe.p->recorded[slot] = true;
    }
  }
  if (append_kv) return prefill_impl(ctx, kv, d_canvas, batch, c.canvas, ws, s);
  return DG_OK;
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

#ifndef DG_SOURCE_DIGEST
#define DG_SOURCE_DIGEST "unstamped"
#endif
const char* dg_source_digest(void) { return DG_SOURCE_DIGEST; }

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
  const int n_sc = (w->embed_t != nullptr) + (w->sc_gate_up != nullptr) + (w->sc_down != nullptr);
  if (n_sc != 0 && n_sc != 3) return fail(DG_ERR_INVALID_ARG, "self-conditioning weights: set all three or none");
  if (n_sc == 3 && cfg->vocab % 32) return fail(DG_ERR_SHAPE, "self-conditioning needs vocab % 32 == 0");
  dg_ctx* c = new (std::nothrow) dg_ctx;
  if (!c) return fail(DG_ERR_INVALID_ARG, "out of host memory");
  c->cfg = *cfg;
  c->embed = w->embed;
  c->final_norm = w->final_norm;
  c->layers.assign(w->layers, w->layers + cfg->n_layers);
  c->embed_t = w->embed_t;
  c->sc_gate_up = w->sc_gate_up;
  c->sc_down = w->sc_down;
  int dev = -1;
  hipStream_t side = nullptr;
  if (hipGetDevice(&dev) == hipSuccess && hipStreamCreateWithFlags(&side, hipStreamNonBlocking) == hipSuccess) {
    c->side = side;
    c->side_dev = dev;
  }
  (void)hipGetLastError();   // no device (or no side stream) is not an error: work stays on one stream
  *out = c;
  return DG_OK;
}

void dg_destroy(dg_ctx* ctx) {
  if (!ctx) return;
  for (hipEvent_t e : ctx->prof.ev) (void)hipEventDestroy(e);
  if (ctx->side) {
    (void)hipStreamSynchronize(ctx->side);
    (void)hipStreamDestroy(ctx->side);
  }
  for (auto& e : ctx->ev_all) {
    (void)hipEventDestroy(e.first);
    (void)hipEventDestroy(e.second);
  }
  for (StopProbe* p : ctx->probes) {
    for (int i = 0; i < kStopLag; ++i) {
      if (p->recorded[i]) (void)hipEventSynchronize(p->ev[i]);   // its copy lands before the memory goes
      (void)hipEventDestroy(p->ev[i]);
    }
    (void)hipHostFree(p->host);
    delete p;
  }
  delete ctx;
}

dg_status dg_workspace_size(const dg_ctx* ctx, int batch, size_t* bytes) {
  if (!ctx || !bytes) return fail(DG_ERR_INVALID_ARG, "NULL argument");
  if (batch < 1 || batch > ctx->cfg.max_batch) return fail(DG_ERR_INVALID_ARG, "batch out of range");
  Ws ws;
  *bytes = carve(ctx->cfg, batch, nullptr, &ws, ctx->embed_t != nullptr);
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
  SampleOpts o;
  o.temperature = temperature;
  o.e_stop = e_stop;
  o.prev_amax = d_prev_argmax;
  o.step = step;
  o.done_step = d_done_step;
  return sample_checked(d_logits, d_canvas, batch, canvas, vocab, gamma, commit_all, d_entropy, d_argmax,
                        d_n_masked, d_ws, ws_bytes, stream, o);
}

dg_status dg_sample_eb_uniform(const uint16_t* d_logits, int32_t* d_canvas, int batch, int canvas, int vocab,
                               float gamma, int commit_all, float temperature, float e_stop,
                               int32_t* d_prev_argmax, int step, int32_t* d_done_step, uint64_t seed, int draw,
                               float* d_entropy, int32_t* d_argmax, int32_t* d_n_open, void* d_ws,
                               size_t ws_bytes, void* stream) {
  if (draw < 0) return fail(DG_ERR_INVALID_ARG, "draw must be >= 0");
  SampleOpts o;
  o.temperature = temperature;
  o.e_stop = e_stop;
  o.prev_amax = d_prev_argmax;
  o.step = step;
  o.done_step = d_done_step;
  o.uniform = 1;
  o.seed = seed;
  o.draw = draw;
  return sample_checked(d_logits, d_canvas, batch, canvas, vocab, gamma, commit_all, d_entropy, d_argmax,
                        d_n_open, d_ws, ws_bytes, stream, o);
}

dg_status dg_uniform_canvas(int32_t* d_canvas, int batch, int canvas, int vocab, uint64_t seed, int draw,
                            void* stream) {
  if (!d_canvas) return fail(DG_ERR_INVALID_ARG, "NULL pointer");
  if (batch < 1 || canvas < 1 || vocab < 1 || draw < 0 || (int64_t)batch * canvas > (int64_t)1 << 30)
    return fail(DG_ERR_INVALID_ARG, "bad canvas sizes or draw");
  launch_uniform_canvas(d_canvas, batch, canvas, vocab, seed, draw, (hipStream_t)stream);
  return check_launch("uniform canvas");
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
  return sample_impl(d_logits, d_canvas, batch, canvas, vocab, gamma, commit_mask(commit_all), d_entropy, d_argmax,
                     d_n_masked, ws, (hipStream_t)stream);
}

dg_status dg_sample_eb_noalloc(const uint16_t* d_logits, int32_t* d_canvas, int batch, int canvas, int vocab,
                               float gamma, int commit_all, float* d_entropy, int32_t* d_argmax,
                               int32_t* d_n_masked, void* stream) {
  size_t need = 0;
  dg_status st = dg_sample_workspace_size(batch, canvas, vocab, &need);
  if (st != DG_OK) return st;
  if (need > kScratchBytes)
    return fail(DG_ERR_WORKSPACE,
                "%d x %d rows of %d logits need %zu bytes of sampler scratch, beyond the library's static %zu "
                "bytes: call dg_sample_eb with a workspace",
                batch, canvas, vocab, need, kScratchBytes);
  if (!d_logits || !d_canvas || !d_n_masked) return fail(DG_ERR_INVALID_ARG, "NULL pointer");
  if (gamma != gamma) return fail(DG_ERR_INVALID_ARG, "gamma is NaN");
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != DG_OK) return st;
  // the same kernels as dg_sample_eb; every scratch word they read this call was
  // written earlier in this call, so nothing needs clearing first
  return dg_sample_eb(d_logits, d_canvas, batch, canvas, vocab, gamma, commit_all, d_entropy, d_argmax, d_n_masked,
                      ws, kScratchBytes, stream);
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
    st = sample_impl(d_logits, d_canvas, batch, c.canvas, c.vocab, gamma, commit_mask(step == steps - 1), nullptr,
                     nullptr, d_n_masked, ws, s, ctx);
    if (st != DG_OK) return st;
  }
  if (append_kv) return prefill_impl(ctx, kv, d_canvas, batch, c.canvas, ws, s);
  return DG_OK;
}

dg_status dg_generate_blocks(dg_ctx* ctx, dg_kv* kv, int32_t* d_canvas, int batch, int n_blocks, int steps,
                             float gamma, int append_last, uint16_t* d_logits, int32_t* d_n_masked, void* d_ws,
                             size_t ws_bytes, void* stream) {
  if (!ctx) return fail(DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_kv(ctx, kv, batch);
  if (st != DG_OK) return st;
  if (!d_canvas || !d_logits || !d_n_masked) return fail(DG_ERR_INVALID_ARG, "NULL pointer");
  if (steps < 1 || n_blocks < 1) return fail(DG_ERR_INVALID_ARG, "steps and n_blocks must be >= 1");
  if (gamma != gamma) return fail(DG_ERR_INVALID_ARG, "gamma is NaN");
  const dg_config& c = ctx->cfg;
  const int C = c.canvas;
  for (int b = 0; b < batch; ++b)
    if (kv->len[b] + (int64_t)n_blocks * C > c.max_ctx)
      return fail(DG_ERR_KV_CAPACITY, "sequence %d: len %lld + %d blocks of %d exceeds max_ctx %d", b,
                  (long long)kv->len[b], n_blocks, C, c.max_ctx);
  Ws ws;
  st = get_ws(ctx, batch, d_ws, ws_bytes, &ws);
  if (st != DG_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  // the append of block j - 1 and the first step of block j share one pass when both
  // fit the workspace's rows and the pass's sequence slots
  const bool fuse = 2 * C <= std::max(C, kPrefillChunk) && 2 * batch <= DG_MAX_BATCH;
  for (int j = 0; j < n_blocks; ++j) {
    int32_t* cv = d_canvas + (size_t)j * batch * C;
    DG_TIMED(ctx, DG_K_FILL, launch_fill_i32(cv, c.vocab, (size_t)batch * C, s));
    for (int step = 0; step < steps; ++step) {
      const float t = 1.0f - (float)step / (float)steps;
      if (step == 0 && j > 0 && fuse) {
        // sequences 0 .. batch-1: the causal append of block j - 1 at len; sequences
        // batch .. 2 batch-1: block j's canvas at len + C, in the same cache sequences
        PassGeom g{};
        g.batch = 2 * batch;
        g.n = C;
        g.denoise = 1;
        g.enc = all_sequences(batch);
        for (int b = 0; b < batch; ++b) {
          g.len[b] = (int)kv->len[b];
          g.len[batch + b] = (int)kv->len[b] + C;
          g.t[batch + b] = t;
          g.kvshift[batch + b] = batch;
        }
        st = run_pass(ctx, kv, g, d_canvas + (size_t)(j - 1) * batch * C, d_logits, ws, s, /*masked_head=*/true,
                      nullptr, /*split=*/batch);
        if (st != DG_OK) return st;
        for (int b = 0; b < batch; ++b) kv->len[b] += C;
      } else {
        if (step == 0 && j > 0) {
          st = prefill_impl(ctx, kv, d_canvas + (size_t)(j - 1) * batch * C, batch, C, ws, s);
          if (st != DG_OK) return st;
        }
        st = denoise_impl(ctx, kv, cv, batch, t, d_logits, ws, s, /*masked_head=*/true);
        if (st != DG_OK) return st;
      }
      st = sample_impl(d_logits, cv, batch, C, c.vocab, gamma, commit_mask(step == steps - 1), nullptr, nullptr,
                       d_n_masked, ws, s, ctx);
      if (st != DG_OK) return st;
    }
  }
  if (append_last) return prefill_impl(ctx, kv, d_canvas + (size_t)(n_blocks - 1) * batch * C, batch, C, ws, s);
  return DG_OK;
}

dg_status dg_generate_block_ex(dg_ctx* ctx, dg_kv* kv, int32_t* d_canvas, int batch, int max_steps,
                               float gamma, float tau_max, float tau_min, float e_stop, int append_kv,
                               uint16_t* d_logits, int32_t* d_n_masked, int32_t* d_done_step, void* d_ws,
                               size_t ws_bytes, void* stream) {
  return generate_annealed(ctx, kv, d_canvas, batch, max_steps, gamma, tau_max, tau_min, e_stop, 0, 0, append_kv,
                           d_logits, d_n_masked, d_done_step, d_ws, ws_bytes, stream);
}

dg_status dg_generate_block_uniform(dg_ctx* ctx, dg_kv* kv, int32_t* d_canvas, int batch, int max_steps,
                                    float gamma, float tau_max, float tau_min, float e_stop, uint64_t seed,
                                    int append_kv, uint16_t* d_logits, int32_t* d_n_open, int32_t* d_done_step,
                                    void* d_ws, size_t ws_bytes, void* stream) {
  return generate_annealed(ctx, kv, d_canvas, batch, max_steps, gamma, tau_max, tau_min, e_stop, 1, seed,
                           append_kv, d_logits, d_n_open, d_done_step, d_ws, ws_bytes, stream);
}

dg_status dg_mixed_step(dg_ctx* ctx, dg_kv* kv, const int32_t* d_tokens, int batch, const int32_t* h_encode,
                        const float* h_t, uint16_t* d_logits, void* d_ws, size_t ws_bytes, void* stream) {
  if (!ctx) return fail(DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_kv(ctx, kv, batch);
  if (st != DG_OK) return st;
  if (!d_tokens || !h_encode) return fail(DG_ERR_INVALID_ARG, "tokens or encode flags are NULL");
  const dg_config& c = ctx->cfg;
  PassGeom g{};
  g.batch = batch;
  g.n = c.canvas;
  for (int b = 0; b < batch; ++b) {
    if (kv->len[b] + c.canvas > c.max_ctx)
      return fail(DG_ERR_KV_CAPACITY, "sequence %d: len %lld + canvas %d exceeds max_ctx %d", b,
                  (long long)kv->len[b], c.canvas, c.max_ctx);
    g.len[b] = (int)kv->len[b];
    if (h_encode[b]) {
      g.enc |= 1ull << b;
    } else {
      if (!h_t || !d_logits) return fail(DG_ERR_INVALID_ARG, "a denoising sequence needs t and logits");
      if (!(h_t[b] >= 0.f && h_t[b] <= 1.f)) return fail(DG_ERR_INVALID_ARG, "t[%d] must be in [0, 1]", b);
      g.t[b] = h_t[b];
      g.denoise = 1;
    }
  }
  Ws ws;
  st = get_ws(ctx, batch, d_ws, ws_bytes, &ws);
  if (st != DG_OK) return st;
  st = run_pass(ctx, kv, g, d_tokens, d_logits, ws, (hipStream_t)stream);
  if (st != DG_OK) return st;
  for (int b = 0; b < batch; ++b)
    if (h_encode[b]) kv->len[b] += c.canvas;
  return DG_OK;
}

dg_status dg_sample_eb_seq(const uint16_t* d_logits, int32_t* d_canvas, int batch, int canvas, int vocab,
                           float gamma, const int32_t* h_commit_all, float* d_entropy, int32_t* d_argmax,
                           int32_t* d_n_masked, void* d_ws, size_t ws_bytes, void* stream) {
  if (!h_commit_all) return fail(DG_ERR_INVALID_ARG, "commit flags are NULL");
  if (batch < 1 || batch > DG_MAX_BATCH) return fail(DG_ERR_INVALID_ARG, "batch must be in [1, %d]", DG_MAX_BATCH);
  size_t need = 0;
  dg_status st = dg_sample_workspace_size(batch, canvas, vocab, &need);
  if (st != DG_OK) return st;
  if (!d_logits || !d_canvas || !d_n_masked || !d_ws) return fail(DG_ERR_INVALID_ARG, "NULL pointer");
  if (gamma != gamma) return fail(DG_ERR_INVALID_ARG, "gamma is NaN");
  if (ws_bytes < need) return fail(DG_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  uint64_t commit = 0;
  for (int b = 0; b < batch; ++b)
    if (h_commit_all[b]) commit |= 1ull << b;
  char* base = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(d_ws) + kAlign - 1) / kAlign * kAlign);
  Carver cv{base};
  Ws ws;
  carve_sampler(cv, batch, canvas, vocab, &ws);
  return sample_impl(d_logits, d_canvas, batch, canvas, vocab, gamma, commit, d_entropy, d_argmax, d_n_masked, ws,
                     (hipStream_t)stream);
}

dg_status dg_serve(dg_ctx* ctx, dg_kv* kv, int32_t* d_canvas, int batch, int steps, float gamma, int n_passes,
                   int32_t* h_phase, uint16_t* d_logits, int32_t* d_n_masked, int32_t* d_out, int out_blocks,
                   int32_t* h_out_count, void* d_ws, size_t ws_bytes, void* stream) {
  if (!ctx) return fail(DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_kv(ctx, kv, batch);
  if (st != DG_OK) return st;
  if (!d_canvas || !d_logits || !d_n_masked || !h_phase) return fail(DG_ERR_INVALID_ARG, "NULL pointer");
  if (steps < 1 || n_passes < 0) return fail(DG_ERR_INVALID_ARG, "steps must be >= 1 and n_passes >= 0");
  if (gamma != gamma) return fail(DG_ERR_INVALID_ARG, "gamma is NaN");
  if (d_out && (out_blocks < 1 || !h_out_count))
    return fail(DG_ERR_INVALID_ARG, "an output ring needs out_blocks >= 1 and the block counts");
  const dg_config& c = ctx->cfg;
  for (int b = 0; b < batch; ++b) {
    if (h_phase[b] < 0 || h_phase[b] > steps) return fail(DG_ERR_INVALID_ARG, "phase[%d] outside [0, steps]", b);
    if (d_out && h_out_count[b] < 0) return fail(DG_ERR_INVALID_ARG, "out_count[%d] < 0", b);
    // the appends this call makes, plus one canvas of denoising scratch after the last
    const int64_t first = (steps - h_phase[b] + (steps + 1)) % (steps + 1);   // passes to its next append
    const int64_t appends = n_passes > first ? 1 + (n_passes - 1 - first) / (steps + 1) : 0;
    if (kv->len[b] + (appends + 1) * c.canvas > c.max_ctx)
      return fail(DG_ERR_KV_CAPACITY, "sequence %d: len %lld + %lld appended canvases exceeds max_ctx %d", b,
                  (long long)kv->len[b], (long long)appends, c.max_ctx);
  }
  Ws ws;
  st = get_ws(ctx, batch, d_ws, ws_bytes, &ws);
  if (st != DG_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  for (int p = 0; p < n_passes; ++p) {
    PassGeom g{};
    g.batch = batch;
    g.n = c.canvas;
    uint64_t commit = 0;
    SeqOffsets off{};
    for (int b = 0; b < batch; ++b) {
      g.len[b] = (int)kv->len[b];
      if (h_phase[b] == steps) {
        g.enc |= 1ull << b;
        if (d_out) off.v[b] = ((int64_t)b * out_blocks + h_out_count[b] % out_blocks) * c.canvas;
      } else {
        g.t[b] = 1.0f - (float)h_phase[b] / (float)steps;
        g.denoise = 1;
        if (h_phase[b] == steps - 1) commit |= 1ull << b;
      }
    }
    st = run_pass(ctx, kv, g, d_canvas, d_logits, ws, s, /*masked_head=*/true);
    if (st != DG_OK) return st;
    if (g.denoise) {
      // the appending sequences' canvases hold no [MASK] row: the sampler leaves them alone
      st = sample_impl(d_logits, d_canvas, batch, c.canvas, c.vocab, gamma, commit, nullptr, nullptr, d_n_masked, ws,
                       s, ctx);
      if (st != DG_OK) return st;
    }
    if (g.enc) {
      DG_TIMED(ctx, DG_K_FILL, launch_serve_finish(d_canvas, batch, c.canvas, c.vocab, g.enc, d_out, off, s));
      for (int b = 0; b < batch; ++b)
        if ((g.enc >> b) & 1) {
          kv->len[b] += c.canvas;
          if (d_out) ++h_out_count[b];
        }
    }
    for (int b = 0; b < batch; ++b) h_phase[b] = (h_phase[b] + 1) % (steps + 1);
  }
  return check_launch("serve");
}

dg_status dg_generate_block_sc(dg_ctx* ctx, dg_kv* kv, int32_t* d_canvas, int batch, int max_steps, float gamma,
                               float tau_max, float tau_min, float e_stop, int uniform, uint64_t seed,
                               int append_kv, uint16_t* d_logits, int32_t* d_n, int32_t* d_done_step,
                               void* d_ws, size_t ws_bytes, void* stream) {
  return generate_annealed(ctx, kv, d_canvas, batch, max_steps, gamma, tau_max, tau_min, e_stop, uniform ? 1 : 0,
                           seed, append_kv, d_logits, d_n, d_done_step, d_ws, ws_bytes, stream, /*self_cond=*/true);
}

dg_status dg_self_cond(dg_ctx* ctx, const uint16_t* d_logits, int batch, float* d_z, float* d_u, void* d_ws,
                       size_t ws_bytes, void* stream) {
  if (!ctx) return fail(DG_ERR_INVALID_ARG, "ctx is NULL");
  if (!ctx->embed_t) return fail(DG_ERR_UNSUPPORTED, "the ctx was created without self-conditioning weights");
  if (!d_logits || !d_z) return fail(DG_ERR_INVALID_ARG, "logits or z is NULL");
  if (batch < 1 || batch > ctx->cfg.max_batch) return fail(DG_ERR_INVALID_ARG, "batch must be in [1, max_batch]");
  Ws ws;
  dg_status st = get_ws(ctx, batch, d_ws, ws_bytes, &ws);
  if (st != DG_OK) return st;
  return self_cond_impl(ctx, d_logits, batch, d_z, d_u, ws, (hipStream_t)stream);
}

dg_status dg_denoise_step_sc(dg_ctx* ctx, const dg_kv* kv, const int32_t* d_canvas, int batch, float t,
                             const float* d_z, uint16_t* d_logits, void* d_ws, size_t ws_bytes, void* stream) {
  if (!ctx) return fail(DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_kv(ctx, kv, batch);
  if (st != DG_OK) return st;
  if (!d_canvas || !d_logits) return fail(DG_ERR_INVALID_ARG, "canvas or logits is NULL");
  if (!(t >= 0.f && t <= 1.f)) return fail(DG_ERR_INVALID_ARG, "t must be in [0, 1]");
  Ws ws;
  st = get_ws(ctx, batch, d_ws, ws_bytes, &ws);
  if (st != DG_OK) return st;
  return denoise_impl(ctx, kv, d_canvas, batch, t, d_logits, ws, (hipStream_t)stream, false, d_z);
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
  } else if (kind == DG_PACK_TRANSPOSE) {
    if (n_mats != 1 || rows % 32) return fail(DG_ERR_INVALID_ARG, "transpose packing needs n_mats = 1, rows % 32 == 0");
    launch_pack_transpose(d_src, d_dst, rows, cols, (hipStream_t)stream);
    return check_launch("pack");
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

dg_status dg_test_sample_eb_profiled(dg_ctx* ctx, const uint16_t* d_logits, int32_t* d_canvas, int batch,
                                     int canvas, int vocab, float gamma, int commit_all, int32_t* d_n_masked,
                                     void* d_ws, size_t ws_bytes, void* stream) {
  if (!ctx) return fail(DG_ERR_INVALID_ARG, "ctx is NULL");
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
  return sample_impl(d_logits, d_canvas, batch, canvas, vocab, gamma, commit_mask(commit_all), nullptr, nullptr, d_n_masked, ws,
                     (hipStream_t)stream, ctx);
}

dg_status dg_workspace_moe_counts(const dg_ctx* ctx, int batch, size_t* offset) {
  if (!ctx || !offset || batch < 1 || batch > ctx->cfg.max_batch) return fail(DG_ERR_INVALID_ARG, "bad arguments");
  Ws ws;
  carve(ctx->cfg, batch, reinterpret_cast<char*>(kAlign), &ws, ctx->embed_t != nullptr);   // offsets relative to an aligned base
  *offset = reinterpret_cast<uintptr_t>(ws.cnt_log) - kAlign;
  return DG_OK;
}

dg_status dg_test_force_routing(dg_ctx* ctx, const int32_t* d_ids) {
  if (!ctx) return fail(DG_ERR_INVALID_ARG, "ctx is NULL");
  ctx->force_ids = d_ids;
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
                        int32_t* d_items, int32_t* d_n_items, int32_t* d_items2, int32_t* d_n_items2,
                        void* stream) {
  if (!d_r || !d_ids || !d_w || !d_cnt || !d_poff || !d_perm || !d_inv || !d_items || !d_n_items ||
      !d_items2 || !d_n_items2 || M < 1 || E < 4 || E > 256 || E % 4 || k < 1 || k > 16 || k > E)
    return fail(DG_ERR_INVALID_ARG, "bad routing arguments");
  hipStream_t s = (hipStream_t)stream;
  launch_topk(d_r, M, E, k, d_ids, d_w, s);
  launch_route(d_ids, M, k, E, d_cnt, d_poff, d_perm, d_inv, reinterpret_cast<int2*>(d_items), d_n_items,
               reinterpret_cast<int2*>(d_items2), d_n_items2, nullptr, s);
  return check_launch("route");
}

dg_status dg_test_eb_select(const float* d_entropy, const int32_t* d_argmax, int32_t* d_canvas,
                            int batch, int canvas, int vocab, float gamma, int commit_all,
                            int32_t* d_n_masked, void* stream) {
  if (!d_entropy || !d_argmax || !d_canvas || !d_n_masked || batch < 1 || canvas < 1 || canvas > 1024 ||
      vocab < 1 || gamma != gamma)
    return fail(DG_ERR_INVALID_ARG, "bad selection arguments");
  launch_eb_select(nullptr, nullptr, 0, d_entropy, d_argmax, d_canvas, batch, canvas, vocab, gamma,
                   commit_mask(commit_all), nullptr, nullptr, d_n_masked, nullptr, -1.0f, 0, nullptr, nullptr, nullptr,
                   nullptr, nullptr, nullptr, nullptr, 0, 0, 0, (hipStream_t)stream);
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

dg_status dg_test_mfma_rate(int blocks, int iters, float* d_out, void* stream) {
  if (!d_out || blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 20))
    return fail(DG_ERR_INVALID_ARG, "rate test needs 1..65536 blocks, 1..2^20 rounds and an output buffer");
  launch_mfma_rate(blocks, iters, d_out, (hipStream_t)stream);
  return check_launch("mfma rate");
}

dg_status dg_test_read_rate(const void* d_src, size_t n_bytes, int blocks, uint32_t* d_out, void* stream) {
  if (!d_src || !d_out || n_bytes == 0 || n_bytes % 16 || blocks < 1 || blocks > 65536)
    return fail(DG_ERR_INVALID_ARG, "read test needs buffers, a positive multiple of 16 bytes and 1..65536 blocks");
  launch_read_rate(d_src, n_bytes, blocks, d_out, (hipStream_t)stream);
  return check_launch("read rate");
}

}  // extern "C"
