"""Seeded synthetic inputs: model shapes, random-init weights, prompts, logits.

This module holds no arithmetic of the method itself.  It only draws random
numbers and lays them out; the engine and the oracle both consume what it
returns (the same tensors, copied between host and device), so neither side
ever generates its own inputs.

Shapes follow the architecture parameters listed on the DiffusionGemma pages
("DiffusionGemma 深度解析", core architecture parameters: 30 layers, sliding
window 1024, canvas 256, vocabulary 262K, 128 experts with 8 active plus one
shared expert).  No trained weights exist here: every weight is N(0, 0.02^2)
rounded to bfloat16 (round-to-nearest-even), every RMSNorm gain is
1 + N(0, 0.1^2) so that a dropped gain is visible in tests.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import torch


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    expert_ffn: int
    shared_ffn: int
    vocab: int                # V; the [MASK] id is V
    canvas: int = 256         # C
    window: int = 1024        # sliding-window length of the causal encoder
    global_every: int = 0     # 0: every layer slides; g: layer l is global iff (l+1) % g == 0
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0

    @property
    def mask_id(self) -> int:
        return self.vocab

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def is_global(self, layer: int) -> bool:
        return self.global_every > 0 and (layer + 1) % self.global_every == 0


# The workloads the engine is exercised on (all synthetic, random-init).
CONFIGS: Dict[str, ModelConfig] = {
    # tiny end-to-end case the oracle finishes in seconds
    "tiny": ModelConfig(n_layers=2, d_model=256, n_q_heads=8, n_kv_heads=4, head_dim=32,
                        n_experts=8, top_k=2, expert_ffn=128, shared_ffn=128, vocab=4096,
                        canvas=32, window=1024),
    # one MoE layer at the full per-layer shape (25.2B total / 3.8B active sizing)
    "layer": ModelConfig(n_layers=1, d_model=2816, n_q_heads=16, n_kv_heads=8, head_dim=128,
                         n_experts=128, top_k=8, expert_ffn=704, shared_ffn=2112, vocab=262144,
                         canvas=256, window=1024),
    # full 30-layer model, tied 262144-row embedding / head
    "full": ModelConfig(n_layers=30, d_model=2816, n_q_heads=16, n_kv_heads=8, head_dim=128,
                        n_experts=128, top_k=8, expert_ffn=704, shared_ffn=2112, vocab=262144,
                        canvas=256, window=1024),
    # same model, every 6th layer attends globally (long-context batched workload)
    "long": ModelConfig(n_layers=30, d_model=2816, n_q_heads=16, n_kv_heads=8, head_dim=128,
                        n_experts=128, top_k=8, expert_ffn=704, shared_ffn=2112, vocab=262144,
                        canvas=256, window=1024, global_every=6),
}

# Seeds of the input streams (fixed so that every run sees the same data).
SEED_WEIGHTS = 0
SEED_PROMPT = 1
SEED_LOGITS = 2
SEED_MASKED = 3

LAYER_KEYS = ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_router", "w_gate_up", "w_down",
              "ws_gate_up", "ws_down")


def layer_shapes(cfg: ModelConfig) -> Dict[str, tuple]:
    d, hd, F, Fs, E = cfg.d_model, cfg.head_dim, cfg.expert_ffn, cfg.shared_ffn, cfg.n_experts
    return {
        "attn_norm": (d,),
        "w_qkv": (cfg.qkv_rows, d),                 # rows: q heads, then k heads, then v heads
        "w_o": (d, cfg.n_q_heads * hd),
        "ffn_norm": (d,),
        "w_router": (E, d),
        "w_gate_up": (E, 2 * F, d),                 # per expert: F gate rows, then F up rows
        "w_down": (E, d, F),
        "ws_gate_up": (2 * Fs, d),
        "ws_down": (d, Fs),
    }


def _gen(seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal_bf16(shape, std, gen, device) -> torch.Tensor:
    """N(0, std^2) drawn in fp32, rounded to bfloat16 (RNE), drawn in row slabs to bound memory."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    n = flat.numel()
    slab = 1 << 26
    for s in range(0, n, slab):
        e = min(n, s + slab)
        flat[s:e] = (torch.randn(e - s, generator=gen, device=device, dtype=torch.float32) * std).to(torch.bfloat16)
    return out


def _gain(n, gen, device) -> torch.Tensor:
    return 1.0 + 0.1 * torch.randn(n, generator=gen, device=device, dtype=torch.float32)


def make_weights(cfg: ModelConfig, seed: int = SEED_WEIGHTS, device: str = "cpu",
                 std: float = 0.02, layers: Optional[List[int]] = None, with_embed: bool = True) -> dict:
    """Random-init weights.  Returns {"embed", "final_norm", "layers": [dict per layer]}.

    Each tensor has its own generator seeded from (seed, tensor index), so a
    layer's weights do not depend on which other layers were drawn.
    embed is [V+1][d] bf16; row V is the [MASK] embedding (the head uses rows 0..V-1).
    Norm gains are fp32, every matrix is bf16 and row-major as listed in layer_shapes().
    with_embed=False leaves out embed and final_norm (None), for drawing layers one at a
    time.
    """
    shapes = layer_shapes(cfg)
    w = {
        "embed": _normal_bf16((cfg.vocab + 1, cfg.d_model), std, _gen(seed * 1000003 + 1, device), device)
        if with_embed else None,
        "final_norm": _gain(cfg.d_model, _gen(seed * 1000003 + 2, device), device) if with_embed else None,
        "layers": [],
    }
    todo = range(cfg.n_layers) if layers is None else layers
    for l in todo:
        lw = {}
        for i, key in enumerate(LAYER_KEYS):
            gen = _gen(seed * 1000003 + 1000 * (l + 1) + i, device)
            if key.endswith("norm"):
                lw[key] = _gain(shapes[key][0], gen, device)
            else:
                lw[key] = _normal_bf16(shapes[key], std, gen, device)
        w["layers"].append(lw)
    return w


def make_selfcond_weights(cfg: ModelConfig, seed: int = SEED_WEIGHTS, device: str = "cpu",
                          std: float = 0.02) -> dict:
    """Random-init weights of the self-conditioning feed-forward network (a SwiGLU network
    d -> shared_ffn -> d): {"sc_gate_up": [2 Fs][d] (Fs gate rows, then Fs up rows),
    "sc_down": [d][Fs]}, bf16, each from its own seeded generator."""
    d, Fs = cfg.d_model, cfg.shared_ffn
    return {"sc_gate_up": _normal_bf16((2 * Fs, d), std, _gen(seed * 1000003 + 3, device), device),
            "sc_down": _normal_bf16((d, Fs), std, _gen(seed * 1000003 + 4, device), device)}


def make_prompt(cfg: ModelConfig, batch: int, length: int, seed: int = SEED_PROMPT,
                device: str = "cpu") -> torch.Tensor:
    """Uniform-random token ids in [0, V): int32 [batch][length]."""
    return torch.randint(0, cfg.vocab, (batch, length), generator=_gen(seed, device),
                         device=device, dtype=torch.int32)


def make_canvas(cfg: ModelConfig, batch: int, device: str = "cpu") -> torch.Tensor:
    """An all-[MASK] canvas: int32 [batch][C] filled with V."""
    return torch.full((batch, cfg.canvas), cfg.mask_id, dtype=torch.int32, device=device)


def make_sampler_logits(rows: int, vocab: int, seed: int = SEED_LOGITS, std: float = 4.0,
                        spike: float = 12.0, spike_frac: float = 0.6,
                        device: str = "cpu") -> torch.Tensor:
    """bf16 [rows][vocab] ~ N(0, std^2); for a seeded Bernoulli(spike_frac) subset of rows one
    seeded id per row gets +spike (the sampler-alone workload)."""
    gen = _gen(seed, device)
    x = torch.randn(rows, vocab, generator=gen, device=device, dtype=torch.float32) * std
    has = torch.rand(rows, generator=gen, device=device) < spike_frac
    ids = torch.randint(0, vocab, (rows,), generator=gen, device=device)
    r = torch.arange(rows, device=device)
    x[r[has], ids[has]] += spike
    return x.to(torch.bfloat16)


def make_masked_canvas(rows: int, vocab: int, n_masked: int, seed: int = SEED_MASKED,
                       device: str = "cpu") -> torch.Tensor:
    """int32 [rows]: a seeded subset of exactly n_masked positions holds [MASK] (= vocab); the
    others hold seeded committed ids in [0, vocab)."""
    gen = _gen(seed, device)
    canvas = torch.randint(0, vocab, (rows,), generator=gen, device=device, dtype=torch.int32)
    perm = torch.randperm(rows, generator=gen, device=device)
    canvas[perm[:n_masked]] = vocab
    return canvas


def make_uniforms(n: int, seed: int, device: str = "cpu") -> torch.Tensor:
    """fp64 U[0,1) draws, one per position (used by the absorbing forward process)."""
    return torch.rand(n, generator=_gen(seed, device), device=device, dtype=torch.float64)


def expected_unique_experts(n_experts: int, assignments: int) -> float:
    """E[#distinct experts] when `assignments` picks are uniform over n_experts (for reporting)."""
    return n_experts * (1.0 - (1.0 - 1.0 / n_experts) ** assignments)


__all__ = ["ModelConfig", "CONFIGS", "make_weights", "make_selfcond_weights", "make_prompt", "make_canvas",
           "make_sampler_logits", "make_masked_canvas", "make_uniforms", "layer_shapes",
           "LAYER_KEYS", "SEED_WEIGHTS", "SEED_PROMPT", "SEED_LOGITS", "SEED_MASKED",
           "expected_unique_experts"]
