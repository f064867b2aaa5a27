"""The sampler entry point that allocates nothing (dg_sample_eb_noalloc, for callers
that cannot allocate) against the one that takes a workspace (dg_sample_eb), through the
C ABI: two calls in a row on the library's static scratch, the second smaller, each
bitwise equal to dg_sample_eb on the same inputs; and a request beyond the scratch is
refused before anything runs."""
import numpy as np
import pytest
import torch

from discrete_diffusion_block_amd import dg, synth
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _inputs(B, C, V, seed):
    logits = torch.stack([synth.make_sampler_logits(C, V, seed=seed + b) for b in range(B)])
    canvas = torch.stack([synth.make_masked_canvas(C, V, C // 2 + 7 * b, seed=seed + 10 + b) for b in range(B)])
    return logits.cuda(), canvas.cuda()


def _both(logits, canvas, gamma):
    B, C, V = logits.shape
    outs = []
    for noalloc in (True, False):
        cv = canvas.clone()
        H = torch.full((B, C), -7.0, device="cuda")
        am = torch.full((B, C), -7, dtype=torch.int32, device="cuda")
        nm = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        if noalloc:
            dg.dg_sample_eb_noalloc(logits, cv, gamma, False, nm, H, am)
        else:
            ws = torch.empty(dg.dg_sample_workspace_size(B, C, V), dtype=torch.uint8, device="cuda")
            dg.dg_sample_eb(logits, cv, gamma, False, nm, ws, H, am)
        torch.cuda.synchronize()
        outs.append((cv.cpu(), H.cpu(), am.cpu(), nm.cpu()))
    return outs


def test_noalloc_sampler_equals_workspace_sampler_twice():
    print("no-alloc sampler: 2 x 256 x 262144, then 1 x 64 x 40008", flush=True)
    for (B, C, V, gamma, seed) in ((2, 256, 262144, 2.0, 100), (1, 64, 40008, 60.0, 200)):
        logits, canvas = _inputs(B, C, V, seed)
        (c1, h1, a1, n1), (c2, h2, a2, n2) = _both(logits, canvas, gamma)
        assert torch.equal(c1, c2) and torch.equal(a1, a2) and torch.equal(n1, n2)
        assert np.array_equal(h1.numpy().view(np.uint32), h2.numpy().view(np.uint32))
        assert int((c1 != canvas.cpu()).sum()) >= 1


def test_noalloc_sampler_refuses_oversized_requests():
    logits = torch.empty(1, dtype=torch.bfloat16, device="cuda")
    canvas = torch.empty(1, dtype=torch.int32, device="cuda")
    nm = torch.empty(1, dtype=torch.int32, device="cuda")
    L = dg.lib()
    import ctypes as C
    # 64 x 1024 rows of 262144 logits need far more than the static scratch
    st = L.dg_sample_eb_noalloc(C.c_void_p(logits.data_ptr()), C.c_void_p(canvas.data_ptr()), 64, 1024, 262144,
                                C.c_float(2.0), 0, None, None, C.c_void_p(nm.data_ptr()), None)
    assert st == -3 and b"static" in L.dg_last_error()
