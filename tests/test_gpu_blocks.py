"""Consecutive blocks with the KV append of each block fused into the next block's first
denoising pass (dg_generate_blocks), against the same number of dg_generate_block calls:
canvases, the last block's logits and masked counts, the KV cache and the lengths must be
equal bit for bit, since every row of the fused pass computes what it computes in its own
pass (the append's keys/values are written by each layer's projection before that
layer's attention reads them).  The launch profiler shows the saved passes."""
import dataclasses

import pytest
import torch

from discrete_diffusion_block_amd import dg, synth
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _weights(cfg):
    w_cpu = synth.make_weights(cfg)
    return {"embed": w_cpu["embed"].cuda(), "final_norm": w_cpu["final_norm"].cuda(),
            "layers": [{k: v.cuda() for k, v in lw.items()} for lw in w_cpu["layers"]]}


CASES = [
    ("tiny", dict(), 2, 64, 3, 4, 1.0),
    ("tiny window 24, global every 2", dict(window=24, global_every=2), 2, 64, 3, 3, 3.0),
    ("full width, 2 layers", "layer", 1, 1100, 3, 3, 2.0),
]


@pytest.mark.parametrize("name,over,batch,prompt_len,n_blocks,steps,gamma", CASES)
@pytest.mark.parametrize("append_last", [True, False])
def test_generate_blocks_equals_block_calls(name, over, batch, prompt_len, n_blocks, steps, gamma, append_last):
    if over == "layer":
        cfg = dataclasses.replace(synth.CONFIGS["layer"], n_layers=2)
    else:
        cfg = dataclasses.replace(synth.CONFIGS["tiny"], **over)
    print(f"generate_blocks: {name}, batch {batch}, prompt {prompt_len}, {n_blocks} blocks x {steps} steps, "
          f"append_last {append_last}", flush=True)
    C, V = cfg.canvas, cfg.vocab
    w = _weights(cfg)
    max_ctx = ((prompt_len + (n_blocks + 1) * C) + 63) // 64 * 64
    prompt = synth.make_prompt(cfg, batch, prompt_len).cuda()
    runs = []
    for fused in (True, False):
        eng = dg.Engine(cfg, w, max_batch=batch, max_ctx=max_ctx)
        eng.prefill_kv(prompt)
        canvas = torch.empty(n_blocks, batch, C, dtype=torch.int32, device="cuda")
        logits = torch.empty(batch, C, V, dtype=torch.bfloat16, device="cuda")
        nm = torch.empty(batch, dtype=torch.int32, device="cuda")
        dg.dg_profile_begin(eng.ctx, 1024, kinds=["prep"])
        if fused:
            eng.generate_blocks(canvas, steps, gamma, append_last, logits, nm)
        else:
            for j in range(n_blocks):
                eng.generate_block(canvas[j], steps, gamma, append_last or j + 1 < n_blocks, logits, nm)
        passes = dg.dg_profile_end(eng.ctx)["prep"][1]
        torch.cuda.synchronize()
        k, v = eng.kv_view()
        n = eng.lengths[0]
        runs.append(dict(canvas=canvas, logits=logits, nm=nm, k=k[:, :, :, :n].clone(), v=v[:, :, :, :n].clone(),
                         lengths=list(eng.lengths[:batch]), passes=passes))
        eng.close()
    a, b = runs
    assert a["lengths"] == b["lengths"] == [prompt_len + C * (n_blocks if append_last else n_blocks - 1)] * batch
    for key in ("canvas", "logits", "nm", "k", "v"):
        assert torch.equal(a[key], b[key]), key
    assert (a["canvas"] != cfg.mask_id).all() and a["nm"].tolist() == [0] * batch
    # each block boundary saves one pass
    assert b["passes"] - a["passes"] == n_blocks - 1, (a["passes"], b["passes"])
    print(f"  bitwise equal; passes {a['passes']} fused vs {b['passes']}", flush=True)
