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
  * Self-conditioning: z = SwiGLU(softmax(L) E) from a step's logits, added to the
    canvas rows' input at the next step (0 at the first).
  * Mixed batches: each sequence runs its own pass (denoising, or the causal KV update
    of a finished canvas) in one batch; serving cycles each sequence through N steps and
    an append.
  * Uniform ("multinomial") variant: the canvas starts as uniformly random tokens;
    every position is a candidate at every step; accepted positions take their
    argmax and the rest are re-noised uniformly (Philox4x64-10 tokens).
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
                 rnd: bool = True, trace: Optional[list] = None,
                 z: Optional[np.ndarray] = None) -> np.ndarray:
    """Bidirectional decoder pass over the canvas [B][C]; returns logits float64 [B][C][V].

    DiffusionGemma Technical Report §3.1–3.2: the canvas attends to the cached
    context and bidirectionally within itself; "DiffusionGemma 深度解析": a
    timestep embedding conditions the denoiser.  Canvas K/V are not cached.
    z [B][C][d] (optional): the self-conditioning signal, added to the canvas rows'
    input with the timestep embedding (see self_condition).
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
        if z is not None:
            x = x + np.asarray(z[b], np.float64)
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
# Self-conditioning
# --------------------------------------------------------------------------------------
#
# DiffusionGemma Technical Report §3.2 (decoder forward pass; denoising iteration, eq. 5-6)
# and §6 (GPU time breakdown, sampling): the decoder has a third input z_t in R^{C x d}
# that feeds its previous prediction back.  After each step the clean-token probabilities
# p̂₀ = softmax(L_t) over the vocabulary give z_{t - dt} = FFW(p̂₀ E), E the token embedding
# matrix [V][d], FFW a feed-forward network; the embedding product and the softmax run in
# full precision.  Readings: z enters the decoder added to the canvas rows' input
# embedding (beside the timestep embedding); z = 0 at a canvas's first step (training
# conditions half its data on z = 0); p̂₀ is the plain softmax (temperature 1: the
# temperature only shapes the transition); FFW is a SwiGLU network d -> Fs -> d (Fs =
# the shared expert's width) with its own weights, computed like the model's other
# feed-forward networks (its input p̂₀E and its activation stored in bf16); with
# self-conditioning every canvas row's logits are computed at every step.

def self_condition(logits: np.ndarray, embed: np.ndarray, sc: dict, rnd: bool = True):
    """z [n][d] (and u = p̂₀ E, float64 [n][d]) from rows of logits [n][V] (the values the
    decoder stored).  p̂₀ = softmax of each row in float64; u = p̂₀ · E[0:V]; z = SwiGLU
    with sc["sc_gate_up"] ([2 Fs][d]: Fs gate rows, then Fs up rows) and sc["sc_down"]
    ([d][Fs]) on u rounded to bf16."""
    R = bf16 if rnd else _ident
    L = np.asarray(logits, np.float64)
    V = L.shape[-1]
    e = np.exp(L - L.max(axis=-1, keepdims=True))
    p = e / e.sum(axis=-1, keepdims=True)
    u = p @ np.asarray(embed[:V], np.float64)
    wgu = np.asarray(sc["sc_gate_up"], np.float64)
    Fs = wgu.shape[0] // 2
    z = swiglu_ffn(R(u), wgu[:Fs], wgu[Fs:], sc["sc_down"], R)
    return z, u


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


# --------------------------------------------------------------------------------------
# Canonical decision entropy
# --------------------------------------------------------------------------------------
#
# The entropy-bounded sampler (DiffusionGemma Technical Report §3.3) turns entropies
# into an integer decision: the order of the masked positions and the point where the
# running entropy sum passes the budget.  Two correct float implementations of
# -sum p log p (different exp/log code, different summation order) differ in the last
# bits, so the decision is taken on one canonical value: Ĥ, a fixed function of the
# row's bf16 logits built only from IEEE float64 add, subtract, multiply, divide,
# round-to-nearest-even, exact power-of-two scaling and integer addition, each in a
# fixed order, so that any implementation that follows it gets the same bits.
#   1. m = max of the row; u_v = (m - x_v) * (1 / tau)   (float64; tau as float32)
#   2. e_v = exp(-u_v), evaluated as: k = rint(u / ln2);
#      r = (u - k ln2_hi) - k ln2_lo (Cody and Waite's two-part reduction, ln2_hi with
#      enough trailing zero bits that k ln2_hi is exact); e^-r by the Taylor series
#      sum_{i<=12} (-r)^i / i! in Horner form (one rounding per multiply and per add);
#      e = that * 2^-k.  Terms with u >= 30 are 0.
#   3. s_v = rint(e_v 2^40), t_v = rint((e_v u_v) 2^40), summed exactly as integers
#      (order-independent): S = sum s_v, T = sum t_v.  The dropped fraction is at most
#      V 2^-41 <= 1.2e-7 of the leading term.
#   4. Ĥ = float32(max(0, (log(S) - 40 ln2) + T / S)), with S and T converted to
#      float64 as hi * 2^32 + lo (one rounding), and log(a) = j ln2 + 2 atanh(s) for
#      a = f 2^j, f in [sqrt(1/2), sqrt(2)), s = (f - 1) / (f + 1), atanh by its series
#      s (1 + z/3 + z^2/5 + ... + z^12/25), z = s^2, in Horner form.
# |Ĥ - H| stays below ~3e-6 for V <= 2^23 (quantisation 1.2e-7 relative in S and T,
# the u >= 30 tail V e^-30 (1 + 30) <= 8e-7, the float32 rounding of the result
# <= 8e-7); the pins check it against -sum p log p.

def _from_decimal(x) -> float:
    return float(x)          # Decimal -> float is correctly rounded


def _canon_constants():
    from decimal import Context, Decimal
    from fractions import Fraction
    ctx = Context(prec=80)
    ln2 = Decimal(2).ln(ctx)
    ln2_d = _from_decimal(ln2)
    # ln2_hi: ln 2 truncated to 32 significant bits (21 trailing zero bits of the
    # 53-bit significand), so k * ln2_hi is exact for every k < 2^21
    mant, exp = math.frexp(ln2_d)
    hi = math.ldexp(math.floor(math.ldexp(mant, 32)), exp - 32)
    lo = _from_decimal(ctx.subtract(ln2, Decimal(hi)))
    inv_ln2 = _from_decimal(ctx.divide(Decimal(1), ln2))
    sqrt_half = _from_decimal(Decimal("0.5").sqrt(ctx))
    exp_c = [float(Fraction(1, math.factorial(i))) for i in range(13)]
    log_c = [float(Fraction(1, 2 * i + 1)) for i in range(13)]
    return ln2_d, hi, lo, inv_ln2, sqrt_half, exp_c, log_c


_LN2, _LN2_HI, _LN2_LO, _INV_LN2, _SQRT_HALF, _EXP_C, _LOG_C = _canon_constants()
_CANON_UMAX = 30.0
_CANON_Q = 2.0 ** 40


def canon_exp_neg(u: np.ndarray) -> np.ndarray:
    """e^-u for float64 u >= 0 by the fixed sequence of step 2 above (0 for u >= 30)."""
    u = np.asarray(u, dtype=np.float64)
    k = np.rint(u * _INV_LN2)
    r = (u - k * _LN2_HI) - k * _LN2_LO
    y = -r
    p = np.full_like(y, _EXP_C[12])
    for c in reversed(_EXP_C[:12]):
        p = p * y
        p = p + c
    e = np.ldexp(p, -np.clip(k, 0, 2000).astype(np.int64))
    return np.where(u < _CANON_UMAX, e, 0.0)


def canon_log(a: np.ndarray) -> np.ndarray:
    """Natural log of float64 a >= 1 by the fixed sequence of step 4 above."""
    a = np.asarray(a, dtype=np.float64)
    f, j = np.frexp(a)
    low = f < _SQRT_HALF
    f = np.where(low, f * 2.0, f)
    j = np.where(low, j - 1, j).astype(np.float64)
    s = (f - 1.0) / (f + 1.0)
    z = s * s
    p = np.full_like(z, _LOG_C[12])
    for c in reversed(_LOG_C[:12]):
        p = p * z
        p = p + c
    return j * _LN2 + (2.0 * s) * p


def _u64_to_f64(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.uint64)
    hi = (v >> np.uint64(32)).astype(np.float64)
    lo = (v & np.uint64(0xFFFFFFFF)).astype(np.float64)
    return hi * 4294967296.0 + lo


def entropy_canonical_sums(rows: np.ndarray, tau: float = 1.0):
    """Steps 1-3 above: the exact integer sums (S, T) per row (uint64)."""
    x = np.asarray(rows, dtype=np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    inv = 1.0 / float(np.float32(tau))
    u = (m - x) * inv
    e = canon_exp_neg(u)
    qs = np.rint(e * _CANON_Q).astype(np.uint64)
    qt = np.rint((e * u) * _CANON_Q).astype(np.uint64)
    return qs.sum(axis=-1, dtype=np.uint64), qt.sum(axis=-1, dtype=np.uint64)


def entropy_canonical(rows: np.ndarray, tau: float = 1.0) -> np.ndarray:
    """The canonical decision entropy Ĥ (float32) of each row of bf16 logits at
    temperature tau; see the steps above.  V must stay below 2^23."""
    rows = np.asarray(rows, dtype=np.float64)
    assert rows.shape[-1] < (1 << 23)
    S, T = entropy_canonical_sums(rows, tau)
    Sf, Tf = _u64_to_f64(S), _u64_to_f64(T)
    h = (canon_log(Sf) - 40.0 * _LN2) + Tf / Sf
    return np.maximum(h, 0.0).astype(np.float32)


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
    """Technical Report §3.3, adaptive stopping, on the candidate rows of one canvas (the
    masked rows for the absorbing sampler, every row for the uniform variant): true when
    their mean entropy is below e_stop and every one of them has the same most likely
    token as at the previous step.  The mean is the float64 running sum of the float32
    entropies in position order, divided by their number (a fixed order, so that the
    decision is reproducible bit for bit)."""
    if not masked:
        return False
    acc = 0.0
    for i in sorted(masked):
        acc += float(np.float32(H32[i]))
    mean = acc / len(masked)
    return mean < float(np.float32(e_stop)) and all(int(amax[i]) == int(prev_amax[i]) for i in masked)


def sample_eb(logits: np.ndarray, canvas: np.ndarray, gamma: float, commit_all: bool,
              mask_id: int, tau: float = 1.0, e_stop: Optional[float] = None,
              prev_amax: Optional[np.ndarray] = None):
    """One sampler call on logits [B][C][V] (values as the engine stores them: bf16).

    Returns (new_canvas, H32 [B][C] (NaN on unmasked rows), argmax [B][C] (-1 on
    unmasked rows), n_masked [B] after the commit, committed list per batch).
    Committed tokens are never revised: only [MASK] rows are read or written.
    Entropies are taken at temperature tau; the decisions (order, budget, stop) use the
    canonical entropy Ĥ (entropy_canonical), which H32 holds.  With e_stop given, a
    sequence whose masked rows pass adaptive_stop against prev_amax [B][C] (the previous
    step's argmax, -1 where there was none) commits all of them.
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
            rows = np.asarray(logits[b, masked], dtype=np.float64)
            H32[b, masked] = entropy_canonical(rows, tau)
            amax[b, masked] = np.argmax(rows, axis=-1)
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
                            rnd: bool = True, record: Optional[list] = None,
                            self_cond: Optional[dict] = None):
    """The Technical Report's sampler (§3.3) on the absorbing canvas: up to max_steps steps
    with t_s = 1 - s/max_steps, entropies at the annealed temperature
    temperature(t_s, tau_max, tau_min), and the adaptive stop, which commits every masked
    position of a sequence at once; the last step commits the rest.  Steps after a
    sequence is complete change nothing for it.  With self_cond (self-conditioning weights,
    see self_condition) each step's decoder takes z from the previous step's logits (z = 0
    at the first step).  Returns (canvas [B][C], steps [B]): the step count after which
    each canvas was complete."""
    canvas = np.full((batch, cfg.canvas), cfg.mask_id, dtype=np.int64)
    prev = np.full((batch, cfg.canvas), -1, dtype=np.int64)
    done_at = np.zeros(batch, dtype=np.int64)
    z = np.zeros((batch, cfg.canvas, cfg.d_model)) if self_cond is not None else None
    for s in range(max_steps):
        t = 1.0 - s / max_steps
        tau = temperature(t, tau_max, tau_min)
        logits = denoise_step(cfg, weights, kv, canvas, t, rnd, z=z)
        stored = bf16(logits) if rnd else logits
        z_in = z
        if self_cond is not None:
            z = np.stack([self_condition(stored[b], weights["embed"], self_cond, rnd)[0] for b in range(batch)])
        new, H32, amax, n_masked, committed = sample_eb(stored, canvas, gamma, s == max_steps - 1,
                                                        cfg.mask_id, tau, e_stop, prev)
        if record is not None:
            record.append({"t": t, "tau": tau, "canvas_in": canvas.copy(), "H": H32, "argmax": amax,
                           "n_masked": n_masked, "committed": committed, "z_in": z_in})
        for b in range(batch):
            if done_at[b] == 0 and n_masked[b] == 0:
                done_at[b] = s + 1
        prev = amax
        canvas = new
    if append:
        prefill_kv(cfg, weights, kv, canvas, rnd)
    return canvas, done_at


# --------------------------------------------------------------------------------------
# Mixed batches and continuous batching
# --------------------------------------------------------------------------------------
#
# DiffusionGemma Technical Report §6 (eliminating CPU-GPU synchronisation; multi-user
# throughput): a served batch holds two kinds of forward pass -- denoising steps, and KV
# cache updates (the causal encoding of a finished canvas) -- that need different attention
# masks and may share one batch; a per-sequence causal-attention flag selects the mask.
# Rows of different sequences never interact, so the plain definition of a mixed batch is
# every sequence's own pass.  Readings for the serving loop: each sequence cycles through
# N denoising steps of an all-[MASK] canvas (t_s = 1 - s/N, the entropy-bounded sampler,
# the last step commits every remaining position) and one pass that appends the finished
# canvas, after which its canvas starts again all-[MASK]; a sequence's phase is the step it
# is at (N: the append); the schedule is fixed, so nothing needs the device's state.


def _kv_one(kv: KVCache, b: int) -> KVCache:
    one = KVCache.__new__(KVCache)
    one.cfg, one.batch = kv.cfg, 1
    one.k = [[kv.k[l][b]] for l in range(len(kv.k))]
    one.v = [[kv.v[l][b]] for l in range(len(kv.v))]
    one.len = [kv.len[b]]
    return one


def _kv_put(kv: KVCache, b: int, one: KVCache) -> None:
    for l in range(len(kv.k)):
        kv.k[l][b] = one.k[l][0]
        kv.v[l][b] = one.v[l][0]
    kv.len[b] = one.len[0]


def mixed_step(cfg, weights: dict, kv: KVCache, tokens: np.ndarray, encode, t, rnd: bool = True,
               trace: Optional[list] = None) -> np.ndarray:
    """One batch of both kinds of pass: sequence b with encode[b] runs the causal encoder over
    its C tokens and appends their K/V (prefill_kv); every other one runs the denoising pass
    over its canvas at its own time t[b] (denoise_step).  Returns logits [B][C][V] (NaN on
    the rows of encoding sequences).  trace (optional): one list per sequence, as for
    prefill_kv and denoise_step."""
    tokens = np.asarray(tokens)
    B, C = tokens.shape
    logits = np.full((B, C, cfg.vocab), np.nan)
    for b in range(B):
        one = _kv_one(kv, b)
        tr = [trace[b]] if trace is not None else None
        if encode[b]:
            prefill_kv(cfg, weights, one, tokens[b:b + 1], rnd, trace=tr)
        else:
            logits[b] = denoise_step(cfg, weights, one, tokens[b:b + 1], float(t[b]), rnd, trace=tr)[0]
        _kv_put(kv, b, one)
    return logits


def serve(cfg, weights: dict, kv: KVCache, batch: int, steps: int, gamma: float, n_passes: int, phase,
          rnd: bool = True, record: Optional[list] = None):
    """Continuous batching of block generation: n_passes mixed passes, sequence b starting at
    phase[b] in [0, steps) with an all-[MASK] canvas (a later start shortens only its first
    canvas, which still ends with the commit-all step).  Each pass runs every sequence's
    current phase in one mixed_step (denoising at t = 1 - phase/steps, or the append at
    phase = steps), then the sampler on each denoising sequence (sample_eb; commit_all at
    phase steps - 1); an appended canvas is recorded and restarts all-[MASK].  Returns
    (canvas [B][C], finished: per sequence the list of appended canvases, phase [B]).
    record (optional) gets per pass: the canvas and phases it started from, the encode
    flags and times, and the routing trace."""
    C, V = cfg.canvas, cfg.vocab
    phase = np.array(phase, dtype=np.int64).copy()
    assert ((phase >= 0) & (phase < steps)).all(), "a sequence starts at a denoising step"
    canvas = np.full((batch, C), cfg.mask_id, dtype=np.int64)
    finished = [[] for _ in range(batch)]
    for _ in range(n_passes):
        enc = phase == steps
        t = np.where(enc, 0.0, 1.0 - phase / steps)
        tr = [[] for _ in range(batch)] if record is not None else None
        if record is not None:
            record.append({"canvas_in": canvas.copy(), "phase": phase.copy(), "encode": enc.copy(), "t": t.copy(),
                           "trace": tr})
        logits = mixed_step(cfg, weights, kv, canvas, enc, t, rnd, trace=tr)
        stored = bf16(logits) if rnd else logits
        for b in range(batch):
            if enc[b]:
                finished[b].append(canvas[b].copy())
                canvas[b] = cfg.mask_id
            else:
                new, *_ = sample_eb(stored[b:b + 1], canvas[b:b + 1], gamma, bool(phase[b] == steps - 1),
                                    cfg.mask_id)
                canvas[b] = new[0]
        phase = (phase + 1) % (steps + 1)
    return canvas, finished, phase


# --------------------------------------------------------------------------------------
# Uniform ("multinomial") variant
# --------------------------------------------------------------------------------------
#
# DiffusionGemma Technical Report §2.1 (the corruption path ends in the uniform prior
# over the vocabulary), §3.2 ("canvas initialisation": the canvas starts as uniformly
# random tokens; "multinomial diffusion": tokens accepted at an earlier step of the
# current canvas can still change) and §3.3 (tokens are accepted in order of increasing
# entropy under the bound; every other position is re-noised uniformly at random).
# Readings: every position of the canvas is a candidate at every step; an accepted
# position takes its most likely token (lowest id on ties), as in the absorbing sampler;
# the last step accepts every position; a canvas is complete when the adaptive stop fires
# or after the last step, and is not touched afterwards.
#
# Random tokens: Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers:
# as easy as 1, 2, 3", SC 2011) with counter (position, sequence, draw, 0) and key
# (seed, 0); draw 0 fills the initial canvas, draw s + 1 re-noises after step s.  The
# first output word x gives the token floor(x V / 2^64).

_U64 = (1 << 64) - 1
_PHILOX_MUL = (0xD2E7470EE14C6C93, 0xCA5A826395121157)   # the two round multipliers
_PHILOX_BUMP = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)  # the Weyl key increments


def philox4x64(counter, key, rounds: int = 10):
    """One Philox4x64 block: four 64-bit output words for a 4-word counter and 2-word key.
    Each round multiplies words 0 and 2 by the two constants (full 128-bit products),
    swaps the halves across the pairs and XORs in the other words and the key; the key
    advances by the Weyl increments between rounds."""
    x0, x1, x2, x3 = (int(v) & _U64 for v in counter)
    k0, k1 = (int(v) & _U64 for v in key)
    for _ in range(rounds):
        p0 = _PHILOX_MUL[0] * x0
        p1 = _PHILOX_MUL[1] * x2
        x0, x1, x2, x3 = (p1 >> 64) ^ x1 ^ k0, p1 & _U64, (p0 >> 64) ^ x3 ^ k1, p0 & _U64
        k0 = (k0 + _PHILOX_BUMP[0]) & _U64
        k1 = (k1 + _PHILOX_BUMP[1]) & _U64
    return x0, x1, x2, x3


def uniform_token(seed: int, draw: int, seq: int, pos: int, vocab: int) -> int:
    """The uniformly random token of (seed, draw, sequence, position) in [0, vocab)."""
    x = philox4x64((pos, seq, draw, 0), (seed, 0))[0]
    return (x * int(vocab)) >> 64


def uniform_canvas(seed: int, draw: int, batch: int, C: int, vocab: int) -> np.ndarray:
    """A canvas [B][C] of uniformly random tokens (draw 0: the initial canvas)."""
    return np.array([[uniform_token(seed, draw, b, i, vocab) for i in range(C)] for b in range(batch)],
                    dtype=np.int64)


def sample_eb_uniform(logits: np.ndarray, canvas: np.ndarray, gamma: float, commit_all: bool,
                      seed: int, draw: int, tau: float = 1.0, e_stop: Optional[float] = None,
                      prev_amax: Optional[np.ndarray] = None, frozen: Optional[np.ndarray] = None):
    """One sampler call of the uniform variant on logits [B][C][V] (bf16 values).

    Every position is a candidate: Ĥ and argmax of every row at temperature tau; the
    accepted positions are eb_select's over all of them (all when commit_all, or when
    the adaptive stop fires against prev_amax); each accepted position takes its argmax
    and every other one uniform_token(seed, draw, b, position).  A frozen sequence
    (complete before this call) is neither read nor written.  Returns (new_canvas,
    H32 [B][C] (NaN where frozen), argmax [B][C] (-1 where frozen), n_open [B] = the
    number of re-noised positions, accepted list per batch, complete [B])."""
    canvas = np.array(canvas, dtype=np.int64, copy=True)
    B, C = canvas.shape
    V = logits.shape[-1]
    H32 = np.full((B, C), np.nan, dtype=np.float32)
    amax = np.full((B, C), -1, dtype=np.int64)
    n_open = np.zeros(B, dtype=np.int64)
    complete = np.zeros(B, dtype=bool)
    accepted = []
    for b in range(B):
        if frozen is not None and frozen[b]:
            accepted.append([])
            continue
        rows = np.asarray(logits[b], dtype=np.float64)
        H32[b] = entropy_canonical(rows, tau)
        amax[b] = np.argmax(rows, axis=-1)
        cand = list(range(C))
        stop = e_stop is not None and adaptive_stop(H32[b], amax[b], prev_amax[b], cand, e_stop)
        sel = eb_select(H32[b], cand, gamma, commit_all or stop)
        keep = set(sel)
        for i in range(C):
            canvas[b, i] = amax[b, i] if i in keep else uniform_token(seed, draw, b, i, V)
        accepted.append(sel)
        n_open[b] = C - len(sel)
        complete[b] = bool(commit_all or stop)
    return canvas, H32, amax, n_open, accepted, complete


def generate_block_uniform(cfg, weights: dict, kv: KVCache, batch: int, max_steps: int, gamma: float,
                           seed: int, tau_max: float = 1.0, tau_min: float = 1.0,
                           e_stop: Optional[float] = None, append: bool = True, rnd: bool = True,
                           record: Optional[list] = None, self_cond: Optional[dict] = None):
    """One canvas per sequence by the uniform variant: the canvas starts as
    uniform_canvas(seed, 0, ...); step s (t_s = 1 - s/max_steps, temperature
    temperature(t_s, tau_max, tau_min)) runs the decoder over the whole canvas and
    sample_eb_uniform with draw s + 1; the last step accepts every position.  With
    self_cond, z as in generate_block_annealed.  Returns (canvas [B][C], steps [B]): the
    step count after which each canvas was complete."""
    C, V = cfg.canvas, cfg.vocab
    canvas = uniform_canvas(seed, 0, batch, C, V)
    prev = np.full((batch, C), -1, dtype=np.int64)
    done_at = np.zeros(batch, dtype=np.int64)
    z = np.zeros((batch, C, cfg.d_model)) if self_cond is not None else None
    for s in range(max_steps):
        t = 1.0 - s / max_steps
        tau = temperature(t, tau_max, tau_min)
        frozen = done_at > 0
        logits = denoise_step(cfg, weights, kv, canvas, t, rnd, z=z)
        stored = bf16(logits) if rnd else logits
        z_in = z
        if self_cond is not None:
            z = np.stack([self_condition(stored[b], weights["embed"], self_cond, rnd)[0] for b in range(batch)])
        new, H32, amax, n_open, accepted, complete = sample_eb_uniform(
            stored, canvas, gamma, s == max_steps - 1, seed, s + 1, tau, e_stop, prev, frozen)
        if record is not None:
            record.append({"t": t, "tau": tau, "canvas_in": canvas.copy(), "H": H32, "argmax": amax,
                           "n_open": n_open, "accepted": accepted, "complete": complete, "z_in": z_in})
        for b in range(batch):
            if not frozen[b] and complete[b]:
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
