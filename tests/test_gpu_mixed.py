"""GPU parity of mixed batches and continuous batching (Technical Report §6) through the C
ABI, on the tiny model.

A mixed pass runs denoising sequences and KV-updating (causal encoder) sequences in one
batch: against the oracle's mixed_step (teacher-forced routing; logits within the model's
bf16 tolerance, appended K/V per head vector within 1%), and bitwise against the
single-kind calls when every sequence is of one kind.  dg_serve is checked bitwise against
block generation in lockstep and against the same mixed passes and sampler calls driven
one by one, and every pass of a staggered schedule against the oracle's serving loop,
teacher-forced (the oracle's canvas and routing at every pass; the sampler's decisions on
the engine's own logits equal the oracle sampler's on those logits)."""
import numpy as np
import pytest
import torch

from discrete_diffusion_block_amd import dg, synth
from oracle import dg_oracle as O
from gpu_util import forced_ids, forced_routing, require_gpu, to_np_bf16

pytestmark = pytest.mark.gpu

LOGIT_TOL = 3e-2
KV_REL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.CONFIGS["tiny"]
    w_cpu = synth.make_weights(cfg)
    w_np = O.to_numpy_weights(w_cpu)
    w_gpu = {"embed": w_cpu["embed"].cuda(), "final_norm": w_cpu["final_norm"].cuda(),
             "layers": [{k: v.cuda() for k, v in lw.items()} for lw in w_cpu["layers"]]}
    prompt = synth.make_prompt(cfg, 3, 16)
    return cfg, w_np, w_gpu, prompt


def _prefill_both(cfg, w_np, eng, prompt):
    kv = O.KVCache(cfg, prompt.shape[0])
    tr = [[] for _ in range(prompt.shape[0])]
    O.prefill_kv(cfg, w_np, kv, prompt.numpy(), trace=tr)
    with forced_routing(eng, forced_ids(tr, cfg.n_layers)):
        eng.prefill_kv(prompt.cuda())
    return kv


def _kv_rel(eng, kv_ref, b, lo, hi):
    k, v = eng.kv_view()
    worst = 0.0
    for l in range(eng.cfg.n_layers):
        kg = k[l, b, :, lo:hi, :].float().cpu().numpy().transpose(1, 0, 2)
        vg = v[l, b, :, lo:hi, :].float().cpu().numpy().transpose(1, 0, 2)
        for got, ref in ((kg, kv_ref.k[l][b][lo:hi]), (vg, kv_ref.v[l][b][lo:hi])):
            rel = np.linalg.norm(got - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-6)
            worst = max(worst, float(rel.max()))
    return worst


def test_mixed_step_vs_oracle(tiny):
    cfg, w_np, w_gpu, prompt = tiny
    C, V = cfg.canvas, cfg.vocab
    print("mixed step: denoise t=0.7, encode, denoise t=0.2", flush=True)
    eng = dg.Engine(cfg, w_gpu, max_batch=3, max_ctx=128)
    kv = _prefill_both(cfg, w_np, eng, prompt)
    toks = np.stack([synth.make_masked_canvas(C, V, 12, seed=3).numpy(),
                     synth.make_prompt(cfg, 1, C, seed=4).numpy()[0],
                     synth.make_masked_canvas(C, V, 30, seed=5).numpy()])
    enc, t = [False, True, False], [0.7, 0.0, 0.2]
    tr = [[] for _ in range(3)]
    ref = O.mixed_step(cfg, w_np, kv, toks, enc, t, trace=tr)
    logits = torch.zeros(3, C, V, dtype=torch.bfloat16, device="cuda")
    with forced_routing(eng, forced_ids(tr, cfg.n_layers)):
        eng.mixed_step(torch.from_numpy(toks.astype(np.int32)).cuda(), enc, t, logits)
    torch.cuda.synchronize()
    lg = to_np_bf16(logits)
    err = max(float(np.abs(lg[b] - ref[b]).max()) for b in (0, 2))
    rel = _kv_rel(eng, kv, 1, 16, 16 + C)
    print(f"  max |logit delta| {err:.2e}; appended K/V max per-head relative error {rel:.2e}", flush=True)
    assert err <= LOGIT_TOL
    assert rel <= KV_REL
    assert eng.lengths == [16, 16 + C, 16]
    assert (lg[1] == 0).all()                  # the encoding sequence's logits rows are not written
    eng.close()


def test_mixed_step_of_one_kind_is_the_single_kind_call(tiny):
    cfg, w_np, w_gpu, prompt = tiny
    C, V = cfg.canvas, cfg.vocab
    print("mixed step, one kind: bitwise against denoise_step and prefill_kv", flush=True)
    canvas = torch.stack([synth.make_masked_canvas(C, V, 10, seed=s) for s in (1, 2, 3)]).cuda()
    a, b = (dg.Engine(cfg, w_gpu, max_batch=3, max_ctx=128) for _ in range(2))
    for e in (a, b):
        e.prefill_kv(prompt.cuda())
    la = torch.empty(3, C, V, dtype=torch.bfloat16, device="cuda")
    lb = torch.empty_like(la)
    a.mixed_step(canvas, [0, 0, 0], [0.6, 0.6, 0.6], la)
    b.denoise_step(canvas, 0.6, lb)
    torch.cuda.synchronize()
    assert torch.equal(la, lb)
    toks = synth.make_prompt(cfg, 3, C, seed=7).cuda()
    a.mixed_step(toks, [1, 1, 1], [0, 0, 0], None)
    b.prefill_kv(toks)
    torch.cuda.synchronize()
    assert a.lengths == b.lengths == [16 + C] * 3
    ka, va = a.kv_view()
    kb, vb = b.kv_view()
    assert torch.equal(ka[:, :, :, :16 + C], kb[:, :, :, :16 + C])
    assert torch.equal(va[:, :, :, :16 + C], vb[:, :, :, :16 + C])
    a.close(); b.close()


def test_serve_in_lockstep_is_block_generation(tiny):
    cfg, w_np, w_gpu, prompt = tiny
    C, V, B, steps, gamma = cfg.canvas, cfg.vocab, 2, 4, 20.0
    print("serve in lockstep vs generate_block (bitwise)", flush=True)
    a, b = (dg.Engine(cfg, w_gpu, max_batch=B, max_ctx=256) for _ in range(2))
    for e in (a, b):
        e.prefill_kv(prompt[:B].cuda())
    logits = torch.empty(B, C, V, dtype=torch.bfloat16, device="cuda")
    nm = torch.empty(B, dtype=torch.int32, device="cuda")
    canvas = torch.full((B, C), V, dtype=torch.int32, device="cuda")
    out = torch.full((B, 4, C), -1, dtype=torch.int32, device="cuda")
    phase, count = [0] * B, [0] * B
    a.serve(canvas, steps, gamma, 2 * (steps + 1), phase, logits, nm, out, count)
    blocks = []
    for _ in range(2):
        blk = torch.empty(B, C, dtype=torch.int32, device="cuda")
        b.generate_block(blk, steps, gamma, True, logits, nm)
        blocks.append(blk)
    torch.cuda.synchronize()
    assert phase == [0] * B and count == [2] * B
    for i in range(2):
        assert torch.equal(out[:, i], blocks[i])
    assert (canvas == V).all() and (out[:, 2:] == -1).all()
    assert a.lengths == b.lengths == [16 + 2 * C] * B
    ka, va = a.kv_view()
    kb, vb = b.kv_view()
    assert torch.equal(ka[:, :B, :, :16 + 2 * C], kb[:, :B, :, :16 + 2 * C])
    a.close(); b.close()


def test_serve_is_the_mixed_passes_one_by_one(tiny):
    """Staggered phases: dg_serve equals dg_mixed_step + dg_sample_eb_seq + the canvas refill
    driven one pass at a time (bitwise), including the ring of finished canvases, and a
    call split in two continues where the first stopped."""
    cfg, w_np, w_gpu, prompt = tiny
    C, V, B, steps, gamma, passes = cfg.canvas, cfg.vocab, 3, 4, 20.0, 12
    print("serve staggered vs one pass at a time (bitwise)", flush=True)
    a, b = (dg.Engine(cfg, w_gpu, max_batch=B, max_ctx=256) for _ in range(2))
    for e in (a, b):
        e.prefill_kv(prompt.cuda())
    logits = torch.empty(B, C, V, dtype=torch.bfloat16, device="cuda")
    nm = torch.empty(B, dtype=torch.int32, device="cuda")
    canvas = torch.full((B, C), V, dtype=torch.int32, device="cuda")
    out = torch.full((B, 2, C), -1, dtype=torch.int32, device="cuda")
    phase, count = [0, 2, 3], [0, 0, 0]
    a.serve(canvas, steps, gamma, 5, phase, logits, nm, out, count)
    a.serve(canvas, steps, gamma, passes - 5, phase, logits, nm, out, count)

    c2 = torch.full((B, C), V, dtype=torch.int32, device="cuda")
    ph, finished = [0, 2, 3], [[] for _ in range(B)]
    for _ in range(passes):
        enc = [p == steps for p in ph]
        t = [0.0 if e else np.float32(1) - np.float32(p) / np.float32(steps) for p, e in zip(ph, enc)]
        b.mixed_step(c2, enc, [float(x) for x in t], logits)
        if not all(enc):
            b.sample_eb_seq(logits, c2, gamma, [p == steps - 1 for p in ph], nm)
        for i in range(B):
            if enc[i]:
                finished[i].append(c2[i].clone())
                c2[i].fill_(V)
        ph = [(p + 1) % (steps + 1) for p in ph]
    torch.cuda.synchronize()
    assert phase == ph
    assert torch.equal(canvas, c2)
    for i in range(B):
        assert count[i] == len(finished[i]) >= 2
        for j, f in enumerate(finished[i]):
            if j >= count[i] - 2:            # the ring keeps the last two
                assert torch.equal(out[i, j % 2], f)
    assert a.lengths == b.lengths
    ka, _ = a.kv_view()
    kb, _ = b.kv_view()
    assert torch.equal(ka, kb)
    a.close(); b.close()


def test_serve_passes_vs_oracle(tiny):
    """Every pass of a staggered schedule against the oracle's serving loop, teacher-forced."""
    cfg, w_np, w_gpu, prompt = tiny
    C, V, B, steps, gamma, passes = cfg.canvas, cfg.vocab, 3, 4, 20.0, 10
    print("serve passes vs oracle, teacher-forced", flush=True)
    eng = dg.Engine(cfg, w_gpu, max_batch=B, max_ctx=256)
    kv = _prefill_both(cfg, w_np, eng, prompt)
    rec = []
    O.serve(cfg, w_np, kv, B, steps, gamma, passes, [0, 2, 3], record=rec)
    logits = torch.empty(B, C, V, dtype=torch.bfloat16, device="cuda")
    nm = torch.empty(B, dtype=torch.int32, device="cuda")
    worst = 0.0
    ref_kv = O.KVCache(cfg, B)
    O.prefill_kv(cfg, w_np, ref_kv, prompt.numpy())
    for r in rec:
        canvas = torch.from_numpy(r["canvas_in"].astype(np.int32)).cuda()
        enc = [bool(e) for e in r["encode"]]
        tr = [[] for _ in range(B)]
        ref = O.mixed_step(cfg, w_np, ref_kv, r["canvas_in"], enc, r["t"], trace=tr)
        with forced_routing(eng, forced_ids(tr, cfg.n_layers)):
            eng.mixed_step(canvas, enc, [float(x) for x in r["t"]], logits)
        lg = to_np_bf16(logits)
        den = [b for b in range(B) if not enc[b]]
        if den:
            worst = max(worst, max(float(np.abs(lg[b] - ref[b]).max()) for b in den))
            commit = [int(p == steps - 1) for p in r["phase"]]
            eng.sample_eb_seq(logits, canvas, gamma, commit, nm)
            torch.cuda.synchronize()
            got = canvas.cpu().numpy()
            for b in den:
                want = O.sample_eb(lg[b:b + 1], r["canvas_in"][b:b + 1], gamma, bool(commit[b]), cfg.mask_id)[0]
                np.testing.assert_array_equal(got[b], want[0])
            for b in range(B):
                if enc[b]:
                    np.testing.assert_array_equal(got[b], r["canvas_in"][b])
    rel = max(_kv_rel(eng, ref_kv, b, 16, ref_kv.len[b]) for b in range(B))
    print(f"  max |logit delta| over {passes} passes {worst:.2e}; appended K/V worst per-head relative {rel:.2e}",
          flush=True)
    assert worst <= LOGIT_TOL
    assert rel <= KV_REL
    assert eng.lengths == ref_kv.len
    eng.close()
