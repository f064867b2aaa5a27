"""End-to-end GPU parity through the C ABI on the tiny model (2 layers, d 256, 8q/4kv
heads of 32, 8 experts top-2 + shared, vocab 4096 + [MASK], 64-token prompt, canvas 32,
4 steps, gamma 1.0): prefill K/V, teacher-forced denoise steps (logits, argmax, entropy,
committed set), whole-block generation with the KV append.

Routing is teacher-forced too (dg_test_force_routing): each pass takes the oracle's
expert ids, so a router logit that the engine's fp32 sum and the oracle's float64 sum
put on different sides of a near-tie cannot send a row to another expert, and every row
is compared.  The engine's weights for those ids are still its own router softmax.

Decisions on identical inputs are exact: the entropy-bounded selection the engine makes
on its own logits equals the oracle's selection on those same logits (bf16 values, the
canonical entropy)."""
import dataclasses
import math

import numpy as np
import pytest
import torch

from discrete_diffusion_block_amd import dg, synth
from oracle import dg_oracle as O
from gpu_util import argmax_agreement, forced_ids, forced_routing, require_gpu, to_np_bf16

pytestmark = pytest.mark.gpu

LOGIT_TOL = 3e-2          # max |delta| of per-step logits (bf16 compute, fp32 accumulate)
AGREE = 0.995             # teacher-forced argmax agreement on masked rows
KV_REL, KV_ABS = 1e-2, 2e-2


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
    prompt = synth.make_prompt(cfg, 1, 64)
    return cfg, w_np, w_gpu, prompt


def _kv_compare(eng, kv_ref, lo, hi, b=0, bref=0):
    """K/V of positions lo..hi-1 agree up to bf16 rounding: each head vector by relative
    norm (the bf16-rounded attention probabilities alone move the tiny model's residual
    stream by ~1e-3 relative)."""
    k, v = eng.kv_view()
    for l in range(eng.cfg.n_layers):
        kg = k[l, b, :, lo:hi, :].float().cpu().numpy().transpose(1, 0, 2)   # [pos][h][hd]
        vg = v[l, b, :, lo:hi, :].float().cpu().numpy().transpose(1, 0, 2)
        for got, ref in ((kg, kv_ref.k[l][bref][lo:hi]), (vg, kv_ref.v[l][bref][lo:hi])):
            d = got - ref
            rel = np.linalg.norm(d, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-6)
            assert rel.max() <= KV_REL, float(rel.max())
            assert np.abs(d).max() <= KV_ABS, float(np.abs(d).max())


PREFILL_CHUNK = 512   # the library's prefill pass length: forced ids are indexed per pass


def _prefill_forced(eng, cfg, w_np, prompt):
    """Oracle prefill (with its trace), then the engine's prefill routed like it.  A
    single-sequence prompt longer than one prefill pass goes in pass-sized calls, each
    forced with its own tokens' expert ids."""
    kv = O.KVCache(cfg, prompt.shape[0])
    tr = [[] for _ in range(prompt.shape[0])]
    O.prefill_kv(cfg, w_np, kv, prompt.numpy(), trace=tr)
    n = prompt.shape[1]
    if prompt.shape[0] == 1 and n > PREFILL_CHUNK:
        for s0 in range(0, n, PREFILL_CHUNK):
            s1 = min(n, s0 + PREFILL_CHUNK)
            with forced_routing(eng, forced_ids(tr, cfg.n_layers, s0, s1)):
                eng.prefill_kv(prompt[:, s0:s1].contiguous().cuda())
        return kv
    assert n <= PREFILL_CHUNK, "one forced pass per call"
    with forced_routing(eng, forced_ids(tr, cfg.n_layers)):
        eng.prefill_kv(prompt.cuda())
    return kv


def test_prefill_kv_matches_oracle(tiny):
    cfg, w_np, w_gpu, prompt = tiny
    print("tiny prefill", flush=True)
    eng = dg.Engine(cfg, w_gpu, max_batch=1, max_ctx=128)
    kv = _prefill_forced(eng, cfg, w_np, prompt)
    assert eng.lengths[0] == 64
    _kv_compare(eng, kv, 0, 64)
    # chunked prefill (two calls) leaves a bitwise identical cache
    tr = [[]]
    O.prefill_kv(cfg, w_np, O.KVCache(cfg, 1), prompt.numpy(), trace=tr)
    eng2 = dg.Engine(cfg, w_gpu, max_batch=1, max_ctx=128)
    with forced_routing(eng2, forced_ids(tr, cfg.n_layers, 0, 23)):
        eng2.prefill_kv(prompt[:, :23].contiguous().cuda())
    with forced_routing(eng2, forced_ids(tr, cfg.n_layers, 23, 64)):
        eng2.prefill_kv(prompt[:, 23:].contiguous().cuda())
    torch.cuda.synchronize()
    k1, v1 = eng.kv_view()
    k2, v2 = eng2.kv_view()
    assert torch.equal(k1[:, :, :, :64], k2[:, :, :, :64]) and torch.equal(v1[:, :, :, :64], v2[:, :, :, :64])
    # and with the router's own choices it is the same cache wherever no near-tie decided
    eng3 = dg.Engine(cfg, w_gpu, max_batch=1, max_ctx=128)
    eng3.prefill_kv(prompt.cuda())
    torch.cuda.synchronize()
    k3, _ = eng3.kv_view()
    assert torch.equal(k1[0, :, :, :64], k3[0, :, :, :64])      # layer 0 K/V precede any routing
    eng.close(); eng2.close(); eng3.close()


def test_wide_tile_prefill_matches_oracle(tiny):
    """A prefill pass of 4 x 512 rows runs its dense GEMMs on the wide tile (passes of
    2048 rows or more): the QKV + RoPE epilogue writing K/V of every sequence, the
    residual adds and the shared expert's SwiGLU and store.  Its K/V match the oracle's
    as the small-tile passes do, routing teacher-forced."""
    cfg, w_np, w_gpu, _ = tiny
    print("tiny prefill of 4 x 512 tokens (wide-tile dense GEMMs)", flush=True)
    prompt = synth.make_prompt(cfg, 4, 512, seed=23)
    eng = dg.Engine(cfg, w_gpu, max_batch=4, max_ctx=576)
    kv = _prefill_forced(eng, cfg, w_np, prompt)
    assert eng.lengths[:4] == [512] * 4
    for b in range(4):
        _kv_compare(eng, kv, 0, 512, b=b, bref=b)
    eng.close()


def test_teacher_forced_steps(tiny):
    """Each step consumes the oracle's canvas and routing, so divergence cannot compound."""
    cfg, w_np, w_gpu, prompt = tiny
    V, C = cfg.vocab, cfg.canvas
    steps, gamma = 4, 1.0
    kv = O.KVCache(cfg, 1)
    O.prefill_kv(cfg, w_np, kv, prompt.numpy())
    rec = []
    O.generate_block(cfg, w_np, kv, 1, steps, gamma, append=False, record=rec)

    eng = dg.Engine(cfg, w_gpu, max_batch=1, max_ctx=128)
    _prefill_forced(eng, cfg, w_np, prompt)
    logits = torch.empty(1, C, V, dtype=torch.bfloat16, device="cuda")
    H = torch.empty(1, C, device="cuda")
    am = torch.empty(1, C, dtype=torch.int32, device="cuda")
    nm = torch.empty(1, dtype=torch.int32, device="cuda")
    agree, total, worst = 0, 0, 0.0
    for s, r in enumerate(rec):
        print(f"tiny step {s}", flush=True)
        tr = [[]]
        O.denoise_step(cfg, w_np, kv, r["canvas_in"], r["t"], trace=tr)
        canvas = torch.from_numpy(r["canvas_in"].astype(np.int32)).cuda()
        with forced_routing(eng, forced_ids(tr, cfg.n_layers)):
            eng.denoise_step(canvas, r["t"], logits)
        lg_gpu = logits.clone()
        eng.sample_eb(logits, canvas, gamma, s == steps - 1, nm, H, am)
        torch.cuda.synchronize()
        lg = to_np_bf16(lg_gpu)[0]
        err = np.abs(lg - r["logits"][0]).max()
        worst = max(worst, err)
        assert err <= LOGIT_TOL, err
        masked = [i for i in range(C) if r["canvas_in"][0, i] == cfg.mask_id]
        a_gpu = am.cpu().numpy()[0][masked]
        agree += int(np.sum(np.argmax(O.bf16(r["logits"][0][masked]), axis=1) == a_gpu))
        total += len(masked)
        # the engine's selection on its own logits == the oracle's on the same logits
        ref = O.sample_eb(lg[None], r["canvas_in"], gamma, s == steps - 1, cfg.mask_id)
        np.testing.assert_array_equal(canvas.cpu().numpy(), ref[0])
        assert nm.item() == ref[3][0]
        Hg = H.cpu().numpy()[0]
        assert np.max(np.abs(Hg[masked] - ref[1][0][masked])) <= 2e-5
        # and the entropies the engine reports stay close to the oracle's own
        assert np.max(np.abs(Hg[masked] - r["H"][0][masked])) <= 1e-3
    print(f"tiny: max |logit delta| {worst:.2e}; argmax agreement {agree}/{total}", flush=True)
    assert agree / total >= AGREE, agree / total
    eng.close()


def test_generate_block_equals_stepwise_and_appends(tiny):
    """dg_generate_block == the same kernels driven step by step (bitwise), then the append."""
    cfg, w_np, w_gpu, prompt = tiny
    V, C = cfg.vocab, cfg.canvas
    steps, gamma = 4, 1.0
    logits = torch.empty(1, C, V, dtype=torch.bfloat16, device="cuda")
    nm = torch.empty(1, dtype=torch.int32, device="cuda")
    eng = dg.Engine(cfg, w_gpu, max_batch=1, max_ctx=128)
    eng.prefill_kv(prompt.cuda())
    blk = torch.empty(1, C, dtype=torch.int32, device="cuda")
    eng.generate_block(blk, steps, gamma, True, logits, nm)
    torch.cuda.synchronize()
    assert nm.item() == 0 and eng.lengths[0] == 64 + C

    ref = dg.Engine(cfg, w_gpu, max_batch=1, max_ctx=128)
    ref.prefill_kv(prompt.cuda())
    canvas = torch.full((1, C), cfg.mask_id, dtype=torch.int32, device="cuda")
    counts = []
    for s in range(steps):
        ref.denoise_step(canvas, 1.0 - s / steps, logits)
        ref.sample_eb(logits, canvas, gamma, s == steps - 1, nm)
        torch.cuda.synchronize()
        counts.append(nm.item())
    ref.prefill_kv(canvas)
    torch.cuda.synchronize()
    assert torch.equal(blk, canvas)
    # near-uniform logits of a random-init model: H ~ log V >> gamma, one commit per step
    assert counts == [C - 1, C - 2, C - 3, 0]
    b = blk.cpu().numpy()[0]
    assert np.all(b >= 0) and np.all(b < V)
    k1, v1 = eng.kv_view()
    k2, v2 = ref.kv_view()
    assert torch.equal(k1[:, :, :, :64 + C], k2[:, :, :, :64 + C])
    assert torch.equal(v1[:, :, :, :64 + C], v2[:, :, :, :64 + C])
    eng.close(); ref.close()


def test_denoise_is_deterministic(tiny):
    cfg, w_np, w_gpu, prompt = tiny
    V, C = cfg.vocab, cfg.canvas
    eng = dg.Engine(cfg, w_gpu, max_batch=1, max_ctx=128)
    eng.prefill_kv(prompt.cuda())
    canvas = torch.full((1, C), cfg.mask_id, dtype=torch.int32, device="cuda")
    a = torch.empty(1, C, V, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    eng.denoise_step(canvas, 0.5, a)
    eng.denoise_step(canvas, 0.5, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    eng.close()


def test_batch_two_sequences_with_different_lengths(tiny):
    cfg, w_np, w_gpu, prompt = tiny
    V, C = cfg.vocab, cfg.canvas
    p2 = synth.make_prompt(cfg, 1, 40, seed=77)
    both = torch.stack([prompt[0, :40], p2[0]]).contiguous()
    print("tiny batch-2 denoise", flush=True)
    eng = dg.Engine(cfg, w_gpu, max_batch=2, max_ctx=128)
    kvp = _prefill_forced(eng, cfg, w_np, both)
    # causal encoding: the first 30 positions of sequence 1 do not depend on the rest,
    # so truncating its committed length leaves a valid 30-token cache
    eng.kv.len[1] = 30
    kv = O.KVCache(cfg, 2)
    for l in range(cfg.n_layers):
        kv.k[l] = [kvp.k[l][0], kvp.k[l][1][:30]]
        kv.v[l] = [kvp.v[l][0], kvp.v[l][1][:30]]
    kv.len = [40, 30]
    canvas = torch.full((2, C), cfg.mask_id, dtype=torch.int32)
    canvas[0, 3] = 17
    canvas[1, 0] = 5
    tr = [[], []]
    ref = O.denoise_step(cfg, w_np, kv, canvas.numpy(), 0.75, trace=tr)
    logits = torch.empty(2, C, V, dtype=torch.bfloat16, device="cuda")
    with forced_routing(eng, forced_ids(tr, cfg.n_layers)):
        eng.denoise_step(canvas.cuda(), 0.75, logits)
    err = np.abs(to_np_bf16(logits) - ref).max()
    assert err <= LOGIT_TOL, err
    eng.close()


@pytest.mark.parametrize("global_every", [0, 2])
def test_short_window_and_global_layers(tiny, global_every):
    """A 24-token sliding window on a 64-token prompt (every layer, or layer 0 only with
    layer 1 global): the encoder's causal window during prefill and, in the denoising
    pass, a truncated prefix on sliding layers and the whole prefix on the global one.
    K/V after prefill and the logits of one denoising step against the oracle."""
    cfg0, w_np, w_gpu, prompt = tiny
    cfg = dataclasses.replace(cfg0, window=24, global_every=global_every)
    V, C = cfg.vocab, cfg.canvas
    print(f"tiny window 24, global_every {global_every}", flush=True)
    eng = dg.Engine(cfg, w_gpu, max_batch=1, max_ctx=128)
    kv = _prefill_forced(eng, cfg, w_np, prompt)
    _kv_compare(eng, kv, 0, 64)
    canvas = synth.make_masked_canvas(C, V, 20, seed=3).reshape(1, C)
    tr = [[]]
    ref = O.denoise_step(cfg, w_np, kv, canvas.numpy(), 0.7, trace=tr)
    logits = torch.empty(1, C, V, dtype=torch.bfloat16, device="cuda")
    with forced_routing(eng, forced_ids(tr, cfg.n_layers)):
        eng.denoise_step(canvas.cuda(), 0.7, logits)
    err = np.abs(to_np_bf16(logits)[0] - ref[0]).max()
    assert err <= LOGIT_TOL, err
    eng.close()


def test_long_prefix_global_layer(tiny):
    """A 4200-token prompt with layer 1 global (layer 0: a 24-token window): the later
    prefill chunks (causal) and the denoising pass attend over more than 4096 keys on
    the global layer, which takes the long-range attention shape (8 waves sharing each
    K/V stage, the pipelined four-slot ring).  K/V after prefill and the logits of one denoising
    step against the oracle."""
    cfg0, w_np, w_gpu, _ = tiny
    cfg = dataclasses.replace(cfg0, window=24, global_every=2)
    V, C = cfg.vocab, cfg.canvas
    print("tiny, 4200-token prompt, layer 1 global", flush=True)
    prompt = synth.make_prompt(cfg, 1, 4200, seed=31)
    eng = dg.Engine(cfg, w_gpu, max_batch=1, max_ctx=4288)
    kv = _prefill_forced(eng, cfg, w_np, prompt)
    _kv_compare(eng, kv, 0, 4200)
    canvas = synth.make_masked_canvas(C, V, 20, seed=3).reshape(1, C)
    tr = [[]]
    ref = O.denoise_step(cfg, w_np, kv, canvas.numpy(), 0.7, trace=tr)
    logits = torch.empty(1, C, V, dtype=torch.bfloat16, device="cuda")
    with forced_routing(eng, forced_ids(tr, cfg.n_layers)):
        eng.denoise_step(canvas.cuda(), 0.7, logits)
    err = np.abs(to_np_bf16(logits)[0] - ref[0]).max()
    print(f"  max |logit delta| {err:.2e}", flush=True)
    assert err <= LOGIT_TOL, err
    eng.close()


@pytest.mark.parametrize("e_stop,gamma", [(0.005, 1.0), (1e30, 1.0), (0.005, math.inf)])
def test_generate_block_ex_equals_stepwise(tiny, e_stop, gamma):
    """dg_generate_block_ex == dg_denoise_step + dg_sample_eb_ex driven step by step (bitwise), with
    the temperature annealed 0.8 -> 0.4 and the adaptive stop (with e_stop 1e30 it fires at the
    first step whose masked argmaxes all repeat).  With gamma = inf the first step commits the
    whole canvas and the four later steps must change nothing."""
    cfg, w_np, w_gpu, prompt = tiny
    V, C = cfg.vocab, cfg.canvas
    steps, tmax, tmin = 5, 0.8, 0.4
    print(f"generate_block_ex e_stop={e_stop} gamma={gamma}", flush=True)
    logits = torch.empty(1, C, V, dtype=torch.bfloat16, device="cuda")
    nm = torch.empty(1, dtype=torch.int32, device="cuda")
    done = torch.empty(1, dtype=torch.int32, device="cuda")
    eng = dg.Engine(cfg, w_gpu, max_batch=1, max_ctx=128)
    eng.prefill_kv(prompt.cuda())
    blk = torch.empty(1, C, dtype=torch.int32, device="cuda")
    eng.generate_block_ex(blk, steps, gamma, tmax, tmin, e_stop, True, logits, nm, done)
    torch.cuda.synchronize()
    assert nm.item() == 0 and eng.lengths[0] == 64 + C

    ref = dg.Engine(cfg, w_gpu, max_batch=1, max_ctx=128)
    ref.prefill_kv(prompt.cuda())
    canvas = torch.full((1, C), cfg.mask_id, dtype=torch.int32, device="cuda")
    prev = torch.full((1, C), -1, dtype=torch.int32, device="cuda")
    done_ref = torch.zeros(1, dtype=torch.int32, device="cuda")
    for s in range(steps):
        t = np.float32(1) - np.float32(s) / np.float32(steps)
        tau = np.float32(tmin) + (np.float32(tmax) - np.float32(tmin)) * t
        ref.denoise_step(canvas, float(t), logits)
        ref.sample_eb_ex(logits, canvas, gamma, s == steps - 1, float(tau), e_stop, prev, s, done_ref, nm)
    ref.prefill_kv(canvas)
    torch.cuda.synchronize()
    assert torch.equal(blk, canvas)
    assert done.item() == done_ref.item()
    if e_stop == 0.005 and gamma == 1.0:
        assert done.item() == steps                 # random-init logits: H ~ log V, no early stop
    if gamma == math.inf:
        assert done.item() == 1
    assert 1 <= done.item() <= steps
    k1, v1 = eng.kv_view()
    k2, v2 = ref.kv_view()
    assert torch.equal(k1[:, :, :, :64 + C], k2[:, :, :, :64 + C])
    eng.close(); ref.close()


@pytest.mark.parametrize("e_stop,gamma,steps", [(1e30, 1.0, 48), (-1.0, 3.0 * 8.27, 6)])
def test_generate_block_ex_vs_annealed_oracle(tiny, e_stop, gamma, steps):
    """The annealed sampler with the adaptive stop against the oracle's generator
    (generate_block_annealed), teacher-forced: at every step the engine consumes the
    oracle's canvas, routing and previous argmaxes; its logits stay within LOGIT_TOL of the
    oracle's, and its selection and stop decision on its own logits equal the oracle's
    sampler on those logits.  The stop fires (e_stop 1e30, budget 48) or the budget commits
    several rows per step (tau 0.8 -> 0.4 either way)."""
    cfg, w_np, w_gpu, prompt = tiny
    V, C = cfg.vocab, cfg.canvas
    print(f"annealed vs oracle e_stop={e_stop} steps={steps}", flush=True)
    p16 = prompt[:, :16].contiguous()
    kv = O.KVCache(cfg, 1)
    O.prefill_kv(cfg, w_np, kv, p16.numpy())
    rec = []
    final, done_o = O.generate_block_annealed(cfg, w_np, kv, 1, steps, gamma, 0.8, 0.4, e_stop, append=False,
                                              record=rec)
    eng = dg.Engine(cfg, w_gpu, max_batch=1, max_ctx=128)
    _prefill_forced(eng, cfg, w_np, p16)
    logits = torch.empty(1, C, V, dtype=torch.bfloat16, device="cuda")
    nm = torch.empty(1, dtype=torch.int32, device="cuda")
    done = torch.zeros(1, dtype=torch.int32, device="cuda")
    H = torch.empty(1, C, device="cuda")
    prev_np = np.full((1, C), -1)
    worst = 0.0
    same_as_oracle = 0
    for s, r in enumerate(rec):
        tr = [[]]
        logits_o = O.denoise_step(cfg, w_np, kv, r["canvas_in"], r["t"], trace=tr)
        canvas = torch.from_numpy(r["canvas_in"].astype(np.int32)).cuda()
        prev = torch.from_numpy(prev_np.astype(np.int32)).cuda()
        with forced_routing(eng, forced_ids(tr, cfg.n_layers)):
            eng.denoise_step(canvas, r["t"], logits)
        lg = to_np_bf16(logits)[0]
        worst = max(worst, float(np.abs(lg - logits_o[0]).max()))
        eng.sample_eb_ex(logits, canvas, gamma, s == steps - 1, r["tau"], e_stop, prev, s, done, nm, H)
        torch.cuda.synchronize()
        ref = O.sample_eb(lg[None], r["canvas_in"], gamma, s == steps - 1, cfg.mask_id, r["tau"], e_stop,
                          prev_np)
        np.testing.assert_array_equal(canvas.cpu().numpy(), ref[0])
        assert nm.item() == ref[3][0]
        same_as_oracle += int(sorted(ref[4][0]) == sorted(r["committed"][0]))
        prev_np = r["argmax"]
        if ref[3][0] == 0:
            break
    n_steps = s + 1
    print(f"  max |logit delta| {worst:.2e}; steps whose commits equal the oracle's own "
          f"{same_as_oracle}/{n_steps}; oracle done after {done_o[0]} steps, engine {done.item()}", flush=True)
    assert worst <= LOGIT_TOL
    if same_as_oracle == n_steps:          # the same decisions at every step: the same end
        assert done.item() == done_o[0]
    if e_stop > 1:
        assert done_o[0] < steps
    eng.close()
