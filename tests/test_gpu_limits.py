"""The boundary's stated limits, each on a narrow model the oracle finishes quickly: a
canvas of 1024 (the largest), a batch of DG_MAX_BATCH = 64 sequences, 256 experts with
top-16 routing and head dim 64, head dim 64 on the long-key attention shape, and a
sequence with an empty prefix beside one with a prompt.  Each case prefills its prompts
and runs one teacher-forced denoising step against the oracle (routing forced to the oracle's expert
ids, as in the other model tests): logits within 3e-2, and the entropy-bounded selection
the engine makes on its own logits equal to the oracle's selection on the same logits."""
import dataclasses

import numpy as np
import pytest
import torch

from discrete_diffusion_block_amd import dg, synth
from oracle import dg_oracle as O
from gpu_util import forced_ids, forced_routing, require_gpu, to_np_bf16

pytestmark = pytest.mark.gpu

LOGIT_TOL = 3e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


CASES = {
    "canvas 1024": (dict(canvas=1024), 1, 64),
    "batch 64": (dict(canvas=32), 64, 16),
    "256 experts top-16, head dim 64": (dict(n_q_heads=4, n_kv_heads=2, head_dim=64, n_experts=256, top_k=16,
                                             expert_ffn=64, shared_ffn=64), 1, 64),
    # the long-key attention shape (over 4096 keys on the global layer) at head dim 64
    "head dim 64, global layer over 4200 keys": (dict(n_q_heads=4, n_kv_heads=2, head_dim=64, window=24,
                                                      global_every=2), 1, 4200),
}
PREFILL_PASS = 512   # the library's prefill pass length: forced ids are indexed per pass


@pytest.mark.parametrize("name", list(CASES))
def test_limits_teacher_forced_step(name):
    over, batch, prompt_len = CASES[name]
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], **over)
    C, V = cfg.canvas, cfg.vocab
    print(f"limits: {name} (batch {batch}, canvas {C}, {cfg.n_experts} experts top-{cfg.top_k}, "
          f"head dim {cfg.head_dim})", flush=True)
    w_cpu = synth.make_weights(cfg)
    w_np = O.to_numpy_weights(w_cpu)
    w_gpu = {"embed": w_cpu["embed"].cuda(), "final_norm": w_cpu["final_norm"].cuda(),
             "layers": [{k: v.cuda() for k, v in lw.items()} for lw in w_cpu["layers"]]}
    g = torch.Generator().manual_seed(len(name))
    prompt = torch.randint(0, V, (batch, prompt_len), generator=g, dtype=torch.int32)
    max_ctx = ((prompt_len + C) + 63) // 64 * 64
    eng = dg.Engine(cfg, w_gpu, max_batch=batch, max_ctx=max_ctx)
    kv = O.KVCache(cfg, batch)
    tr = [[] for _ in range(batch)]
    O.prefill_kv(cfg, w_np, kv, prompt.numpy(), trace=tr)
    if prompt_len <= PREFILL_PASS:
        with forced_routing(eng, forced_ids(tr, cfg.n_layers)):
            eng.prefill_kv(prompt.cuda())
    else:                                          # one call per pass, each forced with its own rows
        assert batch == 1
        for s0 in range(0, prompt_len, PREFILL_PASS):
            s1 = min(prompt_len, s0 + PREFILL_PASS)
            with forced_routing(eng, forced_ids(tr, cfg.n_layers, s0, s1)):
                eng.prefill_kv(prompt[:, s0:s1].contiguous().cuda())
    canvas = torch.full((batch, C), cfg.mask_id, dtype=torch.int32)
    keep = torch.rand(batch, C, generator=g) < 0.3                 # some committed tokens
    canvas[keep] = torch.randint(0, V, (int(keep.sum()),), generator=g, dtype=torch.int32)
    tr = [[] for _ in range(batch)]
    ref = O.denoise_step(cfg, w_np, kv, canvas.numpy(), 0.7, trace=tr)
    logits = torch.empty(batch, C, V, dtype=torch.bfloat16, device="cuda")
    d_canvas = canvas.cuda()
    with forced_routing(eng, forced_ids(tr, cfg.n_layers)):
        eng.denoise_step(d_canvas, 0.7, logits)
    torch.cuda.synchronize()
    lg = to_np_bf16(logits)
    masked = canvas.numpy() == cfg.mask_id
    err = np.abs(lg - ref)[masked].max()
    print(f"  max |logit delta| on [MASK] rows {err:.2e}", flush=True)
    assert err <= LOGIT_TOL, err
    # the selection on the engine's own logits equals the oracle's on the same logits
    nm = torch.empty(batch, dtype=torch.int32, device="cuda")
    eng.sample_eb(logits, d_canvas, 2.0, False, nm)
    torch.cuda.synchronize()
    want = O.sample_eb(lg, canvas.numpy(), 2.0, False, cfg.mask_id)
    np.testing.assert_array_equal(d_canvas.cpu().numpy(), want[0])
    np.testing.assert_array_equal(nm.cpu().numpy(), want[3])
    eng.close()


def test_empty_prefix_beside_a_prompt():
    """A sequence with nothing cached (length 0: its canvas attends to itself only) in one
    pass with a sequence holding a 40-token prompt."""
    cfg = synth.CONFIGS["tiny"]
    C, V = cfg.canvas, cfg.vocab
    print("limits: empty prefix beside a 40-token prompt (batch 2)", flush=True)
    w_cpu = synth.make_weights(cfg)
    w_np = O.to_numpy_weights(w_cpu)
    w_gpu = {"embed": w_cpu["embed"].cuda(), "final_norm": w_cpu["final_norm"].cuda(),
             "layers": [{k: v.cuda() for k, v in lw.items()} for lw in w_cpu["layers"]]}
    prompt = synth.make_prompt(cfg, 2, 40)
    eng = dg.Engine(cfg, w_gpu, max_batch=2, max_ctx=128)
    kvp = O.KVCache(cfg, 2)
    tr = [[], []]
    O.prefill_kv(cfg, w_np, kvp, prompt.numpy(), trace=tr)
    with forced_routing(eng, forced_ids(tr, cfg.n_layers)):
        eng.prefill_kv(prompt.cuda())
    eng.kv.len[0] = 0                              # sequence 0: nothing cached
    kv = O.KVCache(cfg, 2)
    for l in range(cfg.n_layers):
        kv.k[l] = [kvp.k[l][0][:0], kvp.k[l][1]]
        kv.v[l] = [kvp.v[l][0][:0], kvp.v[l][1]]
    kv.len = [0, 40]
    canvas = torch.full((2, C), cfg.mask_id, dtype=torch.int32)
    canvas[1, 5] = 11
    tr = [[], []]
    ref = O.denoise_step(cfg, w_np, kv, canvas.numpy(), 0.8, trace=tr)
    logits = torch.empty(2, C, V, dtype=torch.bfloat16, device="cuda")
    d_canvas = canvas.cuda()
    with forced_routing(eng, forced_ids(tr, cfg.n_layers)):
        eng.denoise_step(d_canvas, 0.8, logits)
    torch.cuda.synchronize()
    lg = to_np_bf16(logits)
    err = np.abs(lg - ref)[canvas.numpy() == cfg.mask_id].max()
    print(f"  max |logit delta| on [MASK] rows {err:.2e}", flush=True)
    assert err <= LOGIT_TOL, err
    nm = torch.empty(2, dtype=torch.int32, device="cuda")
    eng.sample_eb(logits, d_canvas, 1.0, False, nm)
    torch.cuda.synchronize()
    want = O.sample_eb(lg, canvas.numpy(), 1.0, False, cfg.mask_id)
    np.testing.assert_array_equal(d_canvas.cpu().numpy(), want[0])
    eng.close()
