"""Oracle for the block-parallel denoising step — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct CPU implementation in numpy float64 of what the
engine computes.  Only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import it; the engine never does, and it imports nothing from the
engine.  Inputs (weights, prompts, logits) are produced elsewhere and passed in.

Sources (the DiffusionGemma pages):
  * DiffusionGemma Technical Report (translated), §3.1 block-AR generation: the
    context is encoded causally into a KV cache (eq. 3); a 256-token canvas is
    denoised while attending to that cache and bidirectionally to itself; the
    finished canvas is encoded causally and its keys/values appended (eq. 4).
  * same report, §3.3 sampler: tokens are accepted in order of increasing
    entropy while an entropy budget holds.
  * same report, §3.4 efficiency metrics (tokens per forward counts the K-1
    extra append passes).
  * "DiffusionGemma 深度解析" (ai-master.cc), architecture parameters (30 layers,
    sliding window 1024, canvas 256, vocab 262K, 128 experts top-8 + 1 shared,
    timestep embedding added to the decoder input) and the absorbing [MASK]
    forward process ([MASK] id = vocabulary size, absorb rate t/T).

Readings taken where the pages are silent (each one is listed with its reason
in the design notes of the repository):
  * RMSNorm (eps 1e-6, learned gain), pre-norm residual blocks, final norm.
  * RoPE, theta 10000, rotate-half pairing (i, i + hd/2), absolute positions.
  * Sinusoidal timestep embedding [sin(1000 t f_i), cos(1000 t f_i)],
    f_i = 10000^(-i/(d/2)), added to canvas rows only.
  * Router: experts ordered by (logit desc, id asc), top-k, softmax over the
    k selected logits; shared expert added with weight 1; SwiGLU experts.
  * Tied head: logits = h_final · E[0:V]^T; [MASK] (row V) is never predicted.
  * Denoise attention: every canvas query sees the cached prefix keys of the
    layer (sliding layers: the last min(P, W); global layers: all P) and all
    C canvas keys.  Encoder (prefill/append): key j visible to query i iff
    j <= i and (global layer or i - j < W).
  * Sampler: per masked row, argmax (lowest id on ties) and entropy
    H = -sum p log p of softmax(logits / tau) (tau = 1 unless annealed).  Selection: masked positions ordered
    by (H asc, position asc); S_k = running fp64 sum of H in that order;
    commit the first k* = max(1, max{k : S_k <= gamma}) positions, or all
    when commit_all (the last step of a block).
  * Precision contract ("bf16 compute, fp32 accumulate"): with rnd=True the
    oracle rounds to bfloat16 (RNE, via fp32) exactly the values the engine
    stores as bf16 — normed activations, q/k/v, attention output, SwiGLU
    output, final normed state — and computes everything else in float64.
    Decisions (router top-k, argmax, entropy order) are thereby taken on
    inputs of the engine's precision.  rnd=False gives the pure float64 model.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np

# --------------------------------------------------------------------------------------
# bfloat16 rounding (round to nearest even, through fp32 as the engine does)
# --------------------------------------------------------------------------------------


def bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 value (ties to even); returns float64."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    out = u.astype(np.uint32).view(np.float32).astype(np.float64)
    nan = np.isnan(f)
    if np.any(nan):
        out[nan] = np.nan
    return out


def _ident(x):
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------------------
# Building blocks
# --------------------------------------------------------------------------------------


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(g, np.float64)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary position embedding, rotate-half pairing.  x: [n][H][hd], pos: [n]."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]        # [n][half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def timestep_embedding(t: float, d: int) -> np.ndarray:
    """Sinusoidal embedding of the diffusion time t in [0, 1]: [sin(1000 t f), cos(1000 t f)]."""
    half = d // 2
    f = 10000.0 ** (-np.arange(half, dtype=np.float64) / half)
    a = 1000.0 * float(t) * f
    return np.concatenate([np.sin(a), np.cos(a)])


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """Masked softmax attention with grouped KV heads.

    q: [nq][Hq][hd]; k, v: [nk][Hkv][hd]; allowed: bool [nq][nk].
    q head h reads kv head h // (Hq / Hkv).  Scale 1/sqrt(hd).  Returns [nq][Hq][hd].
    """
    nq, hq, hd = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    out = np.zeros((nq, hq, hd))
    for h in range(hq):
        kh = k[:, h // grp, :]
        vh = v[:, h // grp, :]
        s = (q[:, h, :] @ kh.T) / math.sqrt(hd)                          # [nq][nk]
        s = np.where(allowed, s, -np.inf)
        m = np.max(s, axis=1, keepdims=True)
        p = np.exp(s - m)
        p = p / np.sum(p, axis=1, keepdims=True)
        out[:, h, :] = p @ vh
    return out


def silu(a: np.ndarray) -> np.ndarray:
    return a / (1.0 + np.exp(-a))


def swiglu_ffn(h: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray,
               rnd=_ident) -> np.ndarray:
    """(silu(h W_g^T) * (h W_u^T)) W_d^T.  h: [n][d]; W_g, W_u: [F][d]; W_d: [d][F]."""
    g = h @ np.asarray(w_gate, np.float64).T
    u = h @ np.asarray(w_up, np.float64).T
    a = rnd(silu(g) * u)
    return a @ np.asarray(w_down, np.float64).T


def router_topk(r: np.ndarray, k: int):
    """Top-k experts per row by (logit desc, id asc); weights = softmax over the k chosen logits.

    r: [n][E].  Returns ids int [n][k] (rank order) and weights float64 [n][k].
    A NaN logit is read as -inf (it ranks with -inf, below every number; the
    pages do not cover non-finite logits), and -0 ties with +0 as numbers do.
    """
    r = np.asarray(r, dtype=np.float64)
    r = np.where(np.isnan(r), -np.inf, r)
    n, e = r.shape
    ids = np.zeros((n, k), dtype=np.int64)
    for i in range(n):
        order = sorted(range(e), key=lambda j: (-r[i, j], j))
        ids[i] = order[:k]
    sel = np.take_along_axis(r, ids, axis=1)
    w = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = w / w.sum(axis=1, keepdims=True)
    return ids, w


def moe_ffn(h2: np.ndarray, lw: dict, cfg, rnd=_ident):
    """Routed experts + shared expert.  h2: [n][d] -> [n][d].

    Router logits r = h2 W_r^T; each token's top-k experts are applied with the
    softmax weights and summed (in rank order), then the shared expert is added.
    Returns (y, ids, weights, router_logits).
    """
    n = h2.shape[0]
    F = cfg.expert_ffn
    r = h2 @ np.asarray(lw["w_router"], np.float64).T
    ids, w = router_topk(r, cfg.top_k)
    y = np.zeros((n, cfg.d_model))
    per_tok = np.zeros((n, cfg.top_k, cfg.d_model))
    for e in range(cfg.n_experts):
        tok, slot = np.nonzero(ids == e)
        if tok.size == 0:
            continue
        wgu = lw["w_gate_up"][e]
        out = swiglu_ffn(h2[tok], wgu[:F], wgu[F:], lw["w_down"][e], rnd)
        per_tok[tok, slot] = out
    for j in range(cfg.top_k):
        y += w[:, j:j + 1] * per_tok[:, j, :]
    Fs = cfg.shared_ffn
    y += swiglu_ffn(h2, lw["ws_gate_up"][:Fs], lw["ws_gate_up"][Fs:], lw["ws_down"], rnd)
    return y, ids, w, r


# --------------------------------------------------------------------------------------
# KV cache and the transformer passes
# --------------------------------------------------------------------------------------


class KVCache:
    """Per layer, per sequence: keys/values of every committed position (post-RoPE)."""

    def __init__(self, cfg, batch: int):
        self.cfg = cfg
        self.batch = batch
        e = np.zeros((0, cfg.n_kv_heads, cfg.head_dim))
        self.k = [[e.copy() for _ in range(batch)] for _ in range(cfg.n_layers)]
        self.v = [[e.copy() for _ in range(batch)] for _ in range(cfg.n_layers)]
        self.len = [0] * batch


def _split_qkv(qkv: np.ndarray, cfg):
    n = qkv.shape[0]
    hq, hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    q = qkv[:, :hq * hd].reshape(n, hq, hd)
    k = qkv[:, hq * hd:(hq + hkv) * hd].reshape(n, hkv, hd)
    v = qkv[:, (hq + hkv) * hd:].reshape(n, hkv, hd)
    return q, k, v


def _layer(x, pos, lw, cfg, rnd, keys_of, trace=None):
    """One pre-norm block.  keys_of(k_new, v_new) -> (K, V, allowed) for this layer."""
    n = x.shape[0]
    h = rnd(rms_norm(x, lw["attn_norm"], cfg.rms_eps))
    q, k, v = _split_qkv(h @ np.asarray(lw["w_qkv"], np.float64).T, cfg)
    q = rnd(rope(q, pos, cfg.rope_theta))
    k = rnd(rope(k, pos, cfg.rope_theta))
    v = rnd(v)
    K, V, allowed = keys_of(k, v)
    o = rnd(attention(q, K, V, allowed)).reshape(n, -1)
    x = x + o @ np.asarray(lw["w_o"], np.float64).T
    h2 = rnd(rms_norm(x, lw["ffn_norm"], cfg.rms_eps))
    y, ids, w, r = moe_ffn(h2, lw, cfg, rnd)
    if trace is not None:
        trace.append({"h": h, "q": q, "k": k, "v": v, "o": o, "h2": h2, "router": r,
                      "ids": ids, "w": w, "y": y})
    return x + y, k, v


def _embed_rows(weights, tokens) -> np.ndarray:
    return np.asarray(weights["embed"][np.asarray(tokens, dtype=np.int64)], dtype=np.float64)


def prefill_kv(cfg, weights: dict, kv: KVCache, tokens: np.ndarray, rnd: bool = True,
               trace: Optional[list] = None) -> None:
    """Causal encoder pass over tokens [B][n] at positions len..len+n-1; appends K/V.

    DiffusionGemma Technical Report §3.1: the context (and later each finished
    canvas) is encoded with causal attention and its keys/values are appended.
    Sliding layers restrict query i to keys i-W < j <= i.
    """
    R = bf16 if rnd else _ident
    tokens = np.asarray(tokens)
    B, n = tokens.shape
    for b in range(B):
        start = kv.len[b]
        pos = np.arange(start, start + n)
        x = _embed_rows(weights, tokens[b])
        for l in range(cfg.n_layers):
            glob = cfg.is_global(l)

            def keys_of(k_new, v_new, l=l, glob=glob):
                kv.k[l][b] = np.concatenate([kv.k[l][b][:start], k_new], axis=0)
                kv.v[l][b] = np.concatenate([kv.v[l][b][:start], v_new], axis=0)
                j = np.arange(start + n)[None, :]
                i = pos[:, None]
                allowed = (j <= i) & (glob | (i - j < cfg.window))
                return kv.k[l][b], kv.v[l][b], allowed

            x, _, _ = _layer(x, pos, weights["layers"][l], cfg, R, keys_of,
                             trace[b] if trace is not None else None)
        kv.len[b] = start + n


def denoise_step(cfg, weights: dict, kv: KVCache, canvas: np.ndarray, t: float,
                 rnd: bool = True, trace: Optional[list] = None) -> np.ndarray:
    """Bidirectional decoder pass over the canvas [B][C]; returns logits float64 [B][C][V].

    DiffusionGemma Technical Report §3.1–3.2: the canvas attends to the cached
    context and bidirectionally within itself; "DiffusionGemma 深度解析": a
    timestep embedding conditions the denoiser.  Canvas K/V are not cached.
    """
    R = bf16 if rnd else _ident
    canvas = np.asarray(canvas)
    B, C = canvas.shape
    V = cfg.vocab
    logits = np.zeros((B, C, V))
    E = np.asarray(weights["embed"][:V], np.float64)
    temb = timestep_embedding(t, cfg.d_model)
    for b in range(B):
        P = kv.len[b]
        pos = np.arange(P, P + C)
        x = _embed_rows(weights, canvas[b]) + temb[None, :]
        for l in range(cfg.n_layers):
            lo = 0 if cfg.is_global(l) else max(0, P - cfg.window)

            def keys_of(k_new, v_new, l=l, lo=lo):
                K = np.concatenate([kv.k[l][b][lo:P], k_new], axis=0)
                Vv = np.concatenate([kv.v[l][b][lo:P], v_new], axis=0)
                return K, Vv, np.ones((C, K.shape[0]), dtype=bool)

            x, _, _ = _layer(x, pos, weights["layers"][l], cfg, R, keys_of,
                             trace[b] if trace is not None else None)
        hf = R(rms_norm(x, weights["final_norm"], cfg.rms_eps))
        logits[b] = hf @ E.T
    return logits


# --------------------------------------------------------------------------------------
# Sampler: entropy, argmax, entropy-bounded selection
# --------------------------------------------------------------------------------------


def entropy_argmax(rows: np.ndarray, tau: float = 1.0):
    """Per row of logits: (H, argmax).  H = -sum p log p with p = softmax(row / tau), in
    float64 (tau > 0 is the sampling temperature of DiffusionGemma Technical Report §3.3,
    "temperature annealing"; tau = 1 is the plain distribution).

    argmax is the lowest index among exact maxima of the row (the same for every tau).
    """
    raw = np.asarray(rows, dtype=np.float64)
    a = np.argmax(raw, axis=-1)
    x = raw / float(tau)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    p = e / np.sum(e, axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0, p * np.log(p), 0.0)
    return -np.sum(plogp, axis=-1), a


def eb_select(H32: np.ndarray, masked: List[int], gamma: float, commit_all: bool) -> List[int]:
    """Entropy-bounded selection (DiffusionGemma Technical Report §3.3).

    Masked positions are ordered by (entropy asc, position asc).  The running
    sum S_k of the entropies in that order is accumulated in float64; the first
    k* = max(1, max{k : S_k <= gamma}) positions are chosen (all when
    commit_all).  H32 holds float32 entropies (the decision precision).
    """
    order = sorted(masked, key=lambda i: (float(np.float32(H32[i])), i))
    if commit_all or not order:
        return order
    s = 0.0
    k = 0
    for j, i in enumerate(order):
        s += float(np.float32(H32[i]))
        if s <= float(np.float32(gamma)):
            k = j + 1
        else:
            break
    return order[:max(1, k)]


def temperature(t: float, tau_max: float, tau_min: float) -> float:
    """Technical Report §3.3, temperature annealing: the temperature moves linearly along
    the denoising time t in [0, 1], from tau_max at t = 1 (the start of a block) to
    tau_min at t = 0."""
    return tau_min + (tau_max - tau_min) * t


def adaptive_stop(H32: np.ndarray, amax: np.ndarray, prev_amax: np.ndarray, masked: List[int],
                  e_stop: float) -> bool:
    """Technical Report §3.3, adaptive stopping, on the masked rows of one canvas (the only
    rows the absorbing sampler predicts): true when their mean entropy is below e_stop and
    every one of them has the same most likely token as at the previous step.  The mean
    is the exactly rounded float64 sum of the float32 entropies divided by their number."""
    if not masked:
        return False
    mean = math.fsum(float(np.float32(H32[i])) for i in masked) / len(masked)
    return mean < e_stop and all(int(amax[i]) == int(prev_amax[i]) for i in masked)


def sample_eb(logits: np.ndarray, canvas: np.ndarray, gamma: float, commit_all: bool,
              mask_id: int, tau: float = 1.0, e_stop: Optional[float] = None,
              prev_amax: Optional[np.ndarray] = None):
    """One sampler call on logits [B][C][V] (values as the engine stores them: bf16).

    Returns (new_canvas, H32 [B][C] (NaN on unmasked rows), argmax [B][C] (-1 on
    unmasked rows), n_masked [B] after the commit, committed list per batch).
    Committed tokens are never revised: only [MASK] rows are read or written.
    Entropies are taken at temperature tau.  With e_stop given, a sequence whose masked
    rows pass adaptive_stop against prev_amax [B][C] (the previous step's argmax, -1
    where there was none) commits all of them.
    """
    canvas = np.array(canvas, dtype=np.int64, copy=True)
    B, C = canvas.shape
    H32 = np.full((B, C), np.nan, dtype=np.float32)
    amax = np.full((B, C), -1, dtype=np.int64)
    n_masked = np.zeros(B, dtype=np.int64)
    committed = []
    for b in range(B):
        masked = [i for i in range(C) if canvas[b, i] == mask_id]
        if masked:
            H, a = entropy_argmax(logits[b, masked], tau)
            H32[b, masked] = H.astype(np.float32)
            amax[b, masked] = a
        stop = e_stop is not None and adaptive_stop(H32[b], amax[b], prev_amax[b], masked, e_stop)
        sel = eb_select(H32[b], masked, gamma, commit_all or stop)
        for i in sel:
            canvas[b, i] = amax[b, i]
        committed.append(sel)
        n_masked[b] = len(masked) - len(sel)
    return canvas, H32, amax, n_masked, committed


def generate_block(cfg, weights: dict, kv: KVCache, batch: int, steps: int, gamma: float,
                   append: bool = True, rnd: bool = True, record: Optional[list] = None):
    """Denoise one all-[MASK] canvas per sequence for `steps` steps, then append its K/V.

    Step s uses t_s = 1 - s/steps (DiffusionGemma Technical Report §3.2: t runs
    from 1 towards 0 in increments 1/N); the last step commits every remaining
    masked position.  Returns the final canvas [B][C].
    """
    canvas = np.full((batch, cfg.canvas), cfg.mask_id, dtype=np.int64)
    for s in range(steps):
        t = 1.0 - s / steps
        logits = denoise_step(cfg, weights, kv, canvas, t, rnd)
        stored = bf16(logits) if rnd else logits
        new, H32, amax, n_masked, committed = sample_eb(stored, canvas, gamma, s == steps - 1,
                                                        cfg.mask_id)
        if record is not None:
            record.append({"t": t, "canvas_in": canvas.copy(), "logits": logits, "H": H32,
                           "argmax": amax, "n_masked": n_masked, "committed": committed})
        canvas = new
    if append:
        prefill_kv(cfg, weights, kv, canvas, rnd)
    return canvas


def generate_block_annealed(cfg, weights: dict, kv: KVCache, batch: int, max_steps: int, gamma: float,
                            tau_max: float, tau_min: float, e_stop: float, append: bool = True,
                            rnd: bool = True, record: Optional[list] = None):
    """The Technical Report's sampler (§3.3) on the absorbing canvas: up to max_steps steps
    with t_s = 1 - s/max_steps, entropies at the annealed temperature
    temperature(t_s, tau_max, tau_min), and the adaptive stop, which commits every masked
    position of a sequence at once; the last step commits the rest.  Steps after a
    sequence is complete change nothing for it.  Returns (canvas [B][C], steps [B]): the
    step count after which each canvas was complete."""
    canvas = np.full((batch, cfg.canvas), cfg.mask_id, dtype=np.int64)
    prev = np.full((batch, cfg.canvas), -1, dtype=np.int64)
    done_at = np.zeros(batch, dtype=np.int64)
    for s in range(max_steps):
        t = 1.0 - s / max_steps
        tau = temperature(t, tau_max, tau_min)
        logits = denoise_step(cfg, weights, kv, canvas, t, rnd)
        stored = bf16(logits) if rnd else logits
        new, H32, amax, n_masked, committed = sample_eb(stored, canvas, gamma, s == max_steps - 1,
                                                        cfg.mask_id, tau, e_stop, prev)
        if record is not None:
            record.append({"t": t, "tau": tau, "canvas_in": canvas.copy(), "H": H32, "argmax": amax,
                           "n_masked": n_masked, "committed": committed})
        for b in range(batch):
            if done_at[b] == 0 and n_masked[b] == 0:
                done_at[b] = s + 1
        prev = amax
        canvas = new
    if append:
        prefill_kv(cfg, weights, kv, canvas, rnd)
    return canvas, done_at


# --------------------------------------------------------------------------------------
# Absorbing forward process (training-side; checked, not on the engine's path)
# --------------------------------------------------------------------------------------


def absorbing_forward(x: np.ndarray, t: float, T: float, u: np.ndarray, mask_id: int):
    """"DiffusionGemma 深度解析", absorbing diffusion: each token becomes [MASK] with
    probability t/T.  u holds one U[0,1) draw per position (passed in), so the
    same u couples all t: a position masked at t stays masked at every t' > t.
    """
    m = np.asarray(u) < (t / T)
    out = np.where(m, mask_id, np.asarray(x))
    return out, m


def to_numpy_weights(w) -> Dict:
    """Torch tensors (bf16/fp32, any device) -> numpy float32 (exact upcast of bf16)."""
    def cv(t):
        return t.detach().float().cpu().numpy()
    return {"embed": cv(w["embed"]), "final_norm": cv(w["final_norm"]),
            "layers": [{k: cv(v) for k, v in lw.items()} for lw in w["layers"]]}
