"""Inference-efficiency metrics of block diffusion decoding.

DiffusionGemma Technical Report, §3.4: with K canvases, canvas k denoised in
N_k steps and holding C_k valid tokens, total tokens = sum C_k, total denoising
steps = sum N_k, effective steps = sum C_k N_k / sum C_k, and tokens per
forward (TPF) = total tokens / (total steps + K - 1), the K - 1 term counting
the causal passes that append each finished canvas to the KV cache.
§6 (eq. 12): throughput TPS = TPF / t_fwd.
"""
from typing import Sequence


def total_tokens(canvas_tokens: Sequence[int]) -> int:
    return int(sum(canvas_tokens))


def total_steps(steps: Sequence[int]) -> int:
    return int(sum(steps))


def effective_steps(canvas_tokens: Sequence[int], steps: Sequence[int]) -> float:
    return sum(c * n for c, n in zip(canvas_tokens, steps)) / float(sum(canvas_tokens))


def tokens_per_forward(canvas_tokens: Sequence[int], steps: Sequence[int]) -> float:
    return total_tokens(canvas_tokens) / float(total_steps(steps) + len(canvas_tokens) - 1)


def tokens_per_second(tpf: float, t_fwd_s: float) -> float:
    return tpf / t_fwd_s
