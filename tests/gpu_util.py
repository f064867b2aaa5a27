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


def eb_decision_margin(H: np.ndarray, masked, gamma: float, commit_all: bool, eps: float) -> bool:
    """True when the entropy-bounded selection on H (float64) cannot change under any
    perturbation of each entropy by at most eps (the decision is certified)."""
    if commit_all or len(masked) == 0:
        return True
    order = sorted(masked, key=lambda i: (H[i], i))
    hs = [H[i] for i in order]
    s, k = 0.0, 0
    sums = []
    for j, h in enumerate(hs):
        s += h
        sums.append(s)
    for j, sj in enumerate(sums):
        if sj <= gamma:
            k = j + 1
        else:
            break
    k = max(1, k)
    # the k-th and (k+1)-th ranked rows must be separated, and the running sums at the
    # decision boundary must be farther from gamma than the accumulated uncertainty
    if k < len(hs) and hs[k] - hs[k - 1] <= 2 * eps:
        return False
    for j in (k - 1, k):
        if 0 <= j < len(sums) and abs(sums[j] - gamma) <= (j + 1) * eps:
            return False
    return True


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
