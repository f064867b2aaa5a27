"""The adaptive stop's saved work (Technical Report §3.3, adaptive stopping; Fig. 5: about
12 effective steps of a budget of 48).  With the stop on, the block generators skip the
denoising passes that follow the completion of every canvas: the host reads the completion
steps two steps behind the device, so the passes that run are the last completion step plus
at most one (and never fewer than two).  The results equal the same kernels driven step by
step over the whole budget, bit for bit: canvas, completion steps, open counts and KV cache."""
import numpy as np
import pytest
import torch

from discrete_diffusion_block_amd import dg, synth
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.CONFIGS["tiny"]
    w_cpu = synth.make_weights(cfg)
    w_gpu = {"embed": w_cpu["embed"].cuda(), "final_norm": w_cpu["final_norm"].cuda(),
             "layers": [{k: v.cuda() for k, v in lw.items()} for lw in w_cpu["layers"]]}
    prompt = synth.make_prompt(cfg, 2, 64)
    return cfg, w_gpu, prompt


@pytest.mark.parametrize("variant,gamma", [("absorbing", 1e9), ("absorbing", 1.0), ("uniform", 1e9)])
def test_stop_skips_passes(tiny, variant, gamma):
    cfg, w_gpu, prompt = tiny
    V, C, B, steps, seed = cfg.vocab, cfg.canvas, 2, 48, 2 ** 40 + 3
    tmax, tmin, e_stop = 0.8, 0.4, 1e30        # e_stop 1e30: the stop fires once the argmaxes repeat
    print(f"stop skips passes: {variant} gamma={gamma} budget {steps}", flush=True)
    logits = torch.empty(B, C, V, dtype=torch.bfloat16, device="cuda")
    n = torch.empty(B, dtype=torch.int32, device="cuda")
    done = torch.empty(B, dtype=torch.int32, device="cuda")
    eng = dg.Engine(cfg, w_gpu, max_batch=B, max_ctx=128)
    eng.prefill_kv(prompt.cuda())
    torch.cuda.synchronize()
    blk = torch.empty(B, C, dtype=torch.int32, device="cuda")
    dg.dg_profile_begin(eng.ctx, 512, kinds=["prep"])
    if variant == "uniform":
        eng.generate_block_uniform(blk, steps, gamma, tmax, tmin, e_stop, seed, True, logits, n, done)
    else:
        eng.generate_block_ex(blk, steps, gamma, tmax, tmin, e_stop, True, logits, n, done)
    passes = dg.dg_profile_end(eng.ctx)["prep"][1] - 1      # every pass has one prep; the append is the last
    torch.cuda.synchronize()
    d = int(done.max().item())
    print(f"  completion steps {done.tolist()}; denoising passes run {passes} of {steps}", flush=True)
    assert n.tolist() == [0, 0] and eng.lengths == [64 + C, 64 + C]
    assert passes == min(steps, max(2, d + 1))
    if gamma > 1e6:
        assert d + 1 < steps                    # these settings complete early: passes were skipped

    ref = dg.Engine(cfg, w_gpu, max_batch=B, max_ctx=128)
    ref.prefill_kv(prompt.cuda())
    canvas = torch.empty(B, C, dtype=torch.int32, device="cuda")
    if variant == "uniform":
        dg.dg_uniform_canvas(canvas, V, seed, 0)
    else:
        canvas.fill_(cfg.mask_id)
    prev = torch.full((B, C), -1, dtype=torch.int32, device="cuda")
    done_ref = torch.zeros(B, dtype=torch.int32, device="cuda")
    n_ref = torch.empty(B, dtype=torch.int32, device="cuda")
    for s in range(steps):
        t = np.float32(1) - np.float32(s) / np.float32(steps)
        tau = np.float32(tmin) + (np.float32(tmax) - np.float32(tmin)) * t
        ref.denoise_step(canvas, float(t), logits)
        if variant == "uniform":
            ref.sample_eb_uniform(logits, canvas, gamma, s == steps - 1, float(tau), e_stop, prev, s, done_ref,
                                  seed, s + 1, n_ref)
        else:
            ref.sample_eb_ex(logits, canvas, gamma, s == steps - 1, float(tau), e_stop, prev, s, done_ref, n_ref)
    ref.prefill_kv(canvas)
    torch.cuda.synchronize()
    assert torch.equal(blk, canvas)
    assert torch.equal(done, done_ref)
    assert torch.equal(n, n_ref)
    k1, v1 = eng.kv_view()
    k2, v2 = ref.kv_view()
    assert torch.equal(k1[:, :, :, :64 + C], k2[:, :, :, :64 + C])
    assert torch.equal(v1[:, :, :, :64 + C], v2[:, :, :, :64 + C])
    eng.close(); ref.close()


def test_stop_off_runs_every_pass(tiny):
    """With the stop off (e_stop < 0) every step of the budget runs, even after the first
    step has committed the whole canvas."""
    cfg, w_gpu, prompt = tiny
    V, C, B, steps = cfg.vocab, cfg.canvas, 2, 6
    print("stop off runs every pass", flush=True)
    logits = torch.empty(B, C, V, dtype=torch.bfloat16, device="cuda")
    n = torch.empty(B, dtype=torch.int32, device="cuda")
    done = torch.empty(B, dtype=torch.int32, device="cuda")
    eng = dg.Engine(cfg, w_gpu, max_batch=B, max_ctx=128)
    eng.prefill_kv(prompt.cuda())
    blk = torch.empty(B, C, dtype=torch.int32, device="cuda")
    dg.dg_profile_begin(eng.ctx, 128, kinds=["prep"])
    eng.generate_block_ex(blk, steps, 1e9, 1.0, 1.0, -1.0, False, logits, n, done)
    passes = dg.dg_profile_end(eng.ctx)["prep"][1]
    torch.cuda.synchronize()
    assert done.tolist() == [1, 1] and passes == steps
    eng.close()
