"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""
import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from discrete_diffusion_block_amd import dg
    dg.lib()     # fails loudly when the HIP library is missing


def to_np_bf16(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def eb_valid(H: np.ndarray, masked, committed, gamma: float, commit_all: bool) -> bool:
    """Property check: `committed` is the selection the rule makes on its own float32
    entropies H (running float64 sum in (H, position) order, at least one)."""
    if commit_all:
        return sorted(committed) == sorted(masked)
    if not masked:
        return not committed
    order = sorted(masked, key=lambda i: (float(H[i]), i))
    s, k = 0.0, 0
    for j, i in enumerate(order):
        s += float(np.float32(H[i]))
        if s <= float(np.float32(gamma)):
            k = j + 1
        else:
            break
    return sorted(committed) == sorted(order[:max(1, k)])


# Router logits of the engine and of the oracle differ by fp32-vs-fp64 accumulation and by
# rare one-ulp differences of the bf16-rounded normed input (~0.02 * 2^-8 per element);
# 1e-3 bounds that generously.  A token whose k-th and (k+1)-th router logits are closer
# than this is a routing near-tie: either expert set is correct under the precision contract.
ROUTER_DELTA = 1e-3


def routing_near_ties(trace_layers, k: int, delta: float = ROUTER_DELTA):
    """Per layer, the set of token rows whose top-k router decision is a near-tie."""
    out = []
    for t in trace_layers:
        r = -np.sort(-np.asarray(t["router"]), axis=1)
        gap = r[:, k - 1] - r[:, k] if r.shape[1] > k else np.full(r.shape[0], np.inf)
        out.append(set(np.nonzero(gap < delta)[0].tolist()))
    return out


def forced_ids(traces, n_layers, lo=0, hi=None):
    """int32 [n_layers][B * (hi - lo)][k]: the oracle's expert ids of tokens lo..hi-1 of
    every sequence (traces[b][l]["ids"], sequences in batch order), the layout the
    engine's forced-routing tap reads for one pass."""
    out = []
    for l in range(n_layers):
        rows = [np.asarray(tr[l]["ids"])[lo:hi] for tr in traces]
        out.append(np.concatenate(rows, axis=0))
    return np.ascontiguousarray(np.stack(out).astype(np.int32))


class forced_routing:
    """Within the block, every pass through eng uses the given expert ids (one pass)."""

    def __init__(self, eng, ids):
        self.eng = eng
        self.ids = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()

    def __enter__(self):
        from discrete_diffusion_block_amd import dg
        dg.dg_test_force_routing(self.eng.ctx, self.ids)
        return self

    def __exit__(self, *exc):
        from discrete_diffusion_block_amd import dg
        torch.cuda.synchronize()          # the ids stay alive until the pass has read them
        dg.dg_test_force_routing(self.eng.ctx, None)
        return False


def argmax_agreement(gpu_logits, ref_logits, margin):
    """(raw agreement, agreement on rows whose reference top-2 gap exceeds margin, number
    of such rows) of the row argmaxes."""
    a_g = np.argmax(gpu_logits, axis=1)
    a_r = np.argmax(ref_logits, axis=1)
    top2 = -np.sort(-ref_logits, axis=1)[:, :2]
    clear = (top2[:, 0] - top2[:, 1]) > margin
    raw = float(np.mean(a_g == a_r))
    cl = float(np.mean((a_g == a_r)[clear])) if clear.any() else 1.0
    return raw, cl, int(clear.sum())


def logit_error_split(lg, ref):
    """Where the max |engine - oracle| of stored bf16 logits comes from: the engine stores
    bf16, whose rounding alone moves a logit by up to half an ulp (1/64 in [4, 8)).  Returns
    a short text with the max difference, the max difference beyond the rounding of the
    oracle's own value to bf16 (|lg - ref| - |bf16(ref) - ref|, the computation's share),
    and the 99.99th percentile."""
    from oracle import dg_oracle as O
    d = np.abs(lg - ref)
    own = np.abs(O.bf16(ref) - ref)
    return (f"compute share {float((d - own).max()):.3e}, p99.99 {float(np.quantile(d, 0.9999)):.3e}, "
            f"largest |ref| {float(np.abs(ref).max()):.2f}")


def oracle_nudged_logits(cfg, w_np, prompt, canvas, t, prefill_ids, denoise_ids, eps=1e-7):
    """The oracle again with every normed state multiplied by (1 + eps N(0, 1)) -- a
    perturbation below an fp32 ulp for eps 1e-7 -- and the routing replayed from the given
    per-layer expert ids (prefill, then denoise), so no routing decision can differ:
    logits [C][V] of one denoising step after prefilling prompt [1][P].  Their distance
    from the plain oracle's logits is the model's own spread under sub-ulp rounding
    differences, the floor under any bf16-compute implementation's tolerance."""
    from oracle import dg_oracle as O
    replay = iter([np.asarray(x) for x in prefill_ids] + [np.asarray(x) for x in denoise_ids])
    orig_norm, orig_topk = O.rms_norm, O.router_topk
    O.rms_norm = lambda x, g, e: orig_norm(x, g, e) * (1 + eps * np.random.default_rng(0).standard_normal(np.shape(x)))

    def topk_replay(r, k):
        ids = next(replay)
        sel = np.take_along_axis(np.asarray(r, np.float64), ids, axis=1)
        wts = np.exp(sel - sel.max(axis=1, keepdims=True))
        return ids, wts / wts.sum(axis=1, keepdims=True)
    O.router_topk = topk_replay
    try:
        kv = O.KVCache(cfg, 1)
        O.prefill_kv(cfg, w_np, kv, np.asarray(prompt))
        return O.denoise_step(cfg, w_np, kv, np.asarray(canvas), t)[0]
    finally:
        O.rms_norm, O.router_topk = orig_norm, orig_topk
