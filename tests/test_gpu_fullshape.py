"""GPU parity through the C ABI at the model's real layer shapes: two layers of d 2816,
16 query / 8 KV heads of 128, 128 experts of 704 top-8 + a 2112-wide shared expert,
vocab 262144 + [MASK], canvas 256, sliding window 1024.  These shapes take the kernel
variants the tiny model never reaches (head-dim-128 attention, the LDS-staged expert
gate/up and vocabulary head, multi-tile GEMMs) on a prefix longer than the window, and
a global layer over a 4096-token prefix (the long-context workload's layer type).

Routing is teacher-forced (dg_test_force_routing): every pass takes the oracle's expert
ids, so near-tied router logits (the engine's fp32 sums against the oracle's float64
ones move them by up to ~7e-3 at this width) cannot send a row to another expert, and
every row of every output is compared.

Tolerances.  The random-init model amplifies rounding differences far below fp32
resolution (tests/test_oracle_sensitivity.py): nudging the oracle's normed states by a
relative 1e-7 moves its own logits by up to ~2e-2 at this shape.  So the logits are held
to the bf16-compute bound 3e-2 on the 99.99th percentile of |delta| over all 67M values,
and the maximum to max(3e-2, 2 x that floor), the floor measured for each case (its own
prompt, canvas and routing, the oracle's routing replayed; both printed).  The factor 2:
the nudge perturbs the normed states only, while the engine differs from the float64
oracle at every fp32 operation; measured ratios are 1.2-1.55 at two layers and 1.0 at
thirty.  Logits stored as bf16 carry up to half an ulp (1/64 for values in [4, 8)) of
their own on top.  K/V: each head vector
within 1.5% relative.  Argmax: raw agreement is reported; rows whose oracle top-two logits
are more than 2 x 3e-2 apart must agree (closer ones are decided by bf16 noise)."""
import dataclasses

import numpy as np
import pytest
import torch

from discrete_diffusion_block_amd import dg, synth
from oracle import dg_oracle as O
from gpu_util import (argmax_agreement, forced_ids, forced_routing, logit_error_split, oracle_nudged_logits,
                      require_gpu, to_np_bf16)

pytestmark = pytest.mark.gpu

KV_REL = 1.5e-2           # per-head relative error of K/V vectors
KV_ABS = 6e-2
LOGIT_ABS = 3e-2          # |delta| of the logits: the 99.99th percentile over every row
FLOOR_FACTOR = 2.0        # the maximum's bound: max(LOGIT_ABS, FLOOR_FACTOR x the case's measured floor)
PROMPT = 1100             # > window: the canvas and the last prefill rows see a truncated prefix
CALLS = [(0, 512), (512, 700), (700, 1100)]   # prefill calls (one pass each); the last crosses the window edge


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _load(cfg):
    w_cpu = synth.make_weights(cfg)
    w_np = O.to_numpy_weights(w_cpu)
    w_gpu = {"embed": w_cpu["embed"].cuda(), "final_norm": w_cpu["final_norm"].cuda(),
             "layers": [{k: v.cuda() for k, v in lw.items()} for lw in w_cpu["layers"]]}
    return w_np, w_gpu


@pytest.fixture(scope="module")
def full():
    cfg = dataclasses.replace(synth.CONFIGS["layer"], n_layers=2)
    print("full-shape weights (2 layers, vocab 262144)", flush=True)
    w_np, w_gpu = _load(cfg)
    prompt = synth.make_prompt(cfg, 1, PROMPT)
    kv = O.KVCache(cfg, 1)
    tr = [[]]
    O.prefill_kv(cfg, w_np, kv, prompt.numpy(), trace=tr)
    eng = dg.Engine(cfg, w_gpu, max_batch=2, max_ctx=2048)
    yield cfg, w_np, w_gpu, prompt, kv, tr, eng
    eng.close()


def _prefill(eng, cfg, prompt, tr, calls):
    eng.reset()
    for lo, hi in calls:
        with forced_routing(eng, forced_ids(tr, cfg.n_layers, lo, hi)):
            eng.prefill_kv(prompt[:, lo:hi].contiguous().cuda())


def _rel_check(got, ref):
    d = got - ref
    rel = np.linalg.norm(d, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-6)
    assert rel.max() <= KV_REL, float(rel.max())
    assert np.abs(d).max() <= KV_ABS, float(np.abs(d).max())
    return float(rel.max())


def _logit_check(lg, ref, nudged, label):
    """Every row compared: the 99.99th percentile of |delta| within LOGIT_ABS, the maximum
    within max(LOGIT_ABS, FLOOR_FACTOR x the case's floor -- the nudged oracle's distance
    from the oracle); argmax agreement reported, and required on clear rows."""
    d = np.abs(lg - ref)
    err, p9999 = float(d.max()), float(np.quantile(d, 0.9999))
    floor = float(np.abs(nudged - ref).max())
    bound = max(LOGIT_ABS, FLOOR_FACTOR * floor)
    raw, clear, n_clear = argmax_agreement(lg, ref, 2 * LOGIT_ABS)
    print(f"  {label}: max |delta| {err:.3e} (the oracle's own spread {floor:.3e}: bound {bound:.3e}), p99.99 "
          f"{p9999:.3e} over {lg.shape[0]} rows ({logit_error_split(lg, ref)}); argmax agreement raw {raw:.4f}, "
          f"{clear:.4f} on the {n_clear} rows with a top-2 margin > {2 * LOGIT_ABS}", flush=True)
    assert p9999 <= LOGIT_ABS, p9999
    assert err <= bound, (err, bound)
    assert clear == 1.0
    return err, raw


def test_fullshape_prefill_kv(full):
    cfg, w_np, w_gpu, prompt, kv, tr, eng = full
    print(f"full-shape prefill in calls {CALLS}", flush=True)
    _prefill(eng, cfg, prompt, tr, CALLS)
    torch.cuda.synchronize()
    assert eng.lengths[0] == PROMPT
    k, v = eng.kv_view()
    for l in range(cfg.n_layers):
        kg = k[l, 0, :, :PROMPT, :].float().cpu().numpy().transpose(1, 0, 2)
        vg = v[l, 0, :, :PROMPT, :].float().cpu().numpy().transpose(1, 0, 2)
        rk, rv = _rel_check(kg, kv.k[l][0]), _rel_check(vg, kv.v[l][0])
        print(f"  layer {l}: K rel {rk:.2e}, V rel {rv:.2e}", flush=True)


@pytest.mark.parametrize("masked,t", [(256, 1.0), (128, 0.5)])
def test_fullshape_denoise_logits(full, masked, t):
    cfg, w_np, w_gpu, prompt, kv, tr, eng = full
    V, C = cfg.vocab, cfg.canvas
    print(f"full-shape denoise masked={masked} t={t}", flush=True)
    _prefill(eng, cfg, prompt, tr, CALLS)
    canvas = synth.make_masked_canvas(C, V, masked).view(1, C)
    trd = [[]]
    ref = O.denoise_step(cfg, w_np, kv, canvas.numpy(), t, trace=trd)[0]
    logits = torch.empty(1, C, V, dtype=torch.bfloat16, device="cuda")
    with forced_routing(eng, forced_ids(trd, cfg.n_layers)):
        eng.denoise_step(canvas.cuda(), t, logits)
    nudged = oracle_nudged_logits(cfg, w_np, prompt.numpy(), canvas.numpy(), t, [x["ids"] for x in tr[0]],
                                  [x["ids"] for x in trd[0]])
    _logit_check(to_np_bf16(logits)[0], ref, nudged, f"masked {masked}")


def test_fullshape_batch_two_ragged(full):
    """Two sequences (1100 and 300 committed tokens) denoised in one pass: M = 512 rows
    through every kernel, one prefix longer than the window and one shorter."""
    cfg, w_np, w_gpu, prompt, kv, tr, eng = full
    V, C = cfg.vocab, cfg.canvas
    p2 = synth.make_prompt(cfg, 1, PROMPT, seed=91)
    print("full-shape batch-2 denoise (1100 + 300)", flush=True)
    kv2 = O.KVCache(cfg, 1)
    tr2 = [[]]
    O.prefill_kv(cfg, w_np, kv2, p2[:, :300].numpy(), trace=tr2)
    # batch-2 prefill passes of n <= 256 tokens per sequence (M = 2n <= 512: one pass each);
    # sequence 1 only needs its first 300 tokens (causal: later ones do not change them)
    both = torch.cat([prompt, p2]).contiguous()
    eng.reset()
    for lo in range(0, PROMPT, 256):
        hi = min(PROMPT, lo + 256)
        ids0 = forced_ids(tr, cfg.n_layers, lo, hi)
        # sequence 1's tokens from 300 on are past its compared range: any valid routing
        ids1 = np.zeros_like(ids0)
        if lo < 300:
            part = forced_ids(tr2, cfg.n_layers, lo, min(hi, 300))
            ids1[:, :part.shape[1]] = part
        ids = np.ascontiguousarray(np.concatenate([ids0, ids1], axis=1))
        with forced_routing(eng, ids):
            eng.prefill_kv(both[:, lo:hi].contiguous().cuda())
    eng.kv.len[1] = 300
    canvas = torch.stack([synth.make_masked_canvas(C, V, 200, seed=5),
                          synth.make_masked_canvas(C, V, 256, seed=6)]).contiguous()
    bothkv = O.KVCache(cfg, 2)
    for l in range(cfg.n_layers):
        bothkv.k[l] = [kv.k[l][0], kv2.k[l][0]]
        bothkv.v[l] = [kv.v[l][0], kv2.v[l][0]]
    bothkv.len = [PROMPT, 300]
    trd = [[], []]
    ref = O.denoise_step(cfg, w_np, bothkv, canvas.numpy(), 0.8, trace=trd)
    logits = torch.empty(2, C, V, dtype=torch.bfloat16, device="cuda")
    with forced_routing(eng, forced_ids(trd, cfg.n_layers)):
        eng.denoise_step(canvas.cuda(), 0.8, logits)
    lg = to_np_bf16(logits)
    for b, (pr, trp) in enumerate(((prompt, tr), (p2[:, :300], tr2))):
        nudged = oracle_nudged_logits(cfg, w_np, pr.numpy(), canvas[b:b + 1].numpy(), 0.8,
                                      [x["ids"] for x in trp[0]], [x["ids"] for x in trd[b]])
        _logit_check(lg[b], ref[b], nudged, f"sequence {b}")


def test_fullshape_generate_block_masked_head(full):
    """dg_generate_block computes the head only for the rows still [MASK]; with gamma set
    to commit ~100 rows per step the head sees 256, ~156 and ~56 rows (16, 10 and 4 token
    blocks of its tile).  Its canvas must equal the same steps driven through
    dg_denoise_step (whole head) and dg_sample_eb, bit for bit, for two sequences."""
    cfg, w_np, w_gpu, prompt, kv, tr, eng = full
    V, C = cfg.vocab, cfg.canvas
    steps, gamma = 3, 100 * float(np.log(V))
    p2 = synth.make_prompt(cfg, 1, 600, seed=17)
    print("full-shape generate_block with the masked-row head (2 sequences)", flush=True)
    logits = torch.empty(2, C, V, dtype=torch.bfloat16, device="cuda")
    nm = torch.empty(2, dtype=torch.int32, device="cuda")

    def fresh():
        eng.reset()
        eng.prefill_kv(torch.cat([prompt[:, :600], p2]).contiguous().cuda())
        eng.kv.len[1] = 600

    fresh()
    blk = torch.empty(2, C, dtype=torch.int32, device="cuda")
    eng.generate_block(blk, steps, gamma, False, logits, nm)
    torch.cuda.synchronize()
    assert nm.tolist() == [0, 0]

    fresh()
    canvas = torch.full((2, C), cfg.mask_id, dtype=torch.int32, device="cuda")
    left = []
    for s in range(steps):
        # t exactly as dg_generate_block forms it, in fp32 (the EB ranking of the
        # near-uniform random-init rows turns a 1-ulp change of t into other commits)
        t = float(np.float32(1.0) - np.float32(s) / np.float32(steps))
        eng.denoise_step(canvas, t, logits)
        eng.sample_eb(logits, canvas, gamma, s == steps - 1, nm)
        torch.cuda.synchronize()
        left.append(nm.tolist())
    print(f"  masked rows left after each step: {left}", flush=True)
    assert 100 <= C - left[0][0] <= 110 and left[1][0] < left[0][0]   # the head saw shrinking row sets
    assert torch.equal(blk, canvas)


def test_fullshape_global_layer_long_prefix():
    """Layer 1 global (the long-context workload's every-6th-layer type, here global_every
    2) over a 4096-token prefix, layer 0 sliding (window 1024): the prefill's causal mask
    over thousands of keys in the global layer, and a denoising step whose canvas attends
    to all 4096 cached keys there and to the last 1024 in layer 0."""
    cfg = dataclasses.replace(synth.CONFIGS["layer"], n_layers=2, global_every=2)
    P = 4096
    print(f"full-shape global layer, {P}-token prefix", flush=True)
    w_np, w_gpu = _load(cfg)
    prompt = synth.make_prompt(cfg, 1, P, seed=23)
    kv = O.KVCache(cfg, 1)
    tr = [[]]
    O.prefill_kv(cfg, w_np, kv, prompt.numpy(), trace=tr)
    eng = dg.Engine(cfg, w_gpu, max_batch=1, max_ctx=P + cfg.canvas)
    _prefill(eng, cfg, prompt, tr, [(lo, lo + 512) for lo in range(0, P, 512)])
    torch.cuda.synchronize()
    k, v = eng.kv_view()
    for l in range(cfg.n_layers):
        rk = _rel_check(k[l, 0, :, :P, :].float().cpu().numpy().transpose(1, 0, 2), kv.k[l][0])
        rv = _rel_check(v[l, 0, :, :P, :].float().cpu().numpy().transpose(1, 0, 2), kv.v[l][0])
        print(f"  layer {l} ({'global' if cfg.is_global(l) else 'sliding'}): K rel {rk:.2e}, V rel {rv:.2e}",
              flush=True)
    C, V = cfg.canvas, cfg.vocab
    canvas = synth.make_masked_canvas(C, V, 192, seed=8).view(1, C)
    trd = [[]]
    ref = O.denoise_step(cfg, w_np, kv, canvas.numpy(), 0.9, trace=trd)[0]
    logits = torch.empty(1, C, V, dtype=torch.bfloat16, device="cuda")
    with forced_routing(eng, forced_ids(trd, cfg.n_layers)):
        eng.denoise_step(canvas.cuda(), 0.9, logits)
    nudged = oracle_nudged_logits(cfg, w_np, prompt.numpy(), canvas.numpy(), 0.9, [x["ids"] for x in tr[0]],
                                  [x["ids"] for x in trd[0]])
    _logit_check(to_np_bf16(logits)[0], ref, nudged, "global layer over 4096 keys")
    eng.close()
