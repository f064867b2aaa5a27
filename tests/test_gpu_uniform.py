"""GPU parity of the uniform ("multinomial") variant (Technical Report §3.2 canvas
initialisation and multinomial diffusion, §3.3 acceptance with uniform re-noising)
through the C ABI, against the oracle.

Random tokens are integer work: bit-exact.  The sampler's decisions are taken on the
canonical entropy, so with identical bf16 logits the whole new canvas -- accepted
argmaxes and re-noised tokens alike -- equals the oracle's bit for bit.  The generator is
compared with the same kernels driven step by step (bitwise) and, teacher-forced (the
oracle's canvas and routing at every step), with the oracle's generator."""
import math

import numpy as np
import pytest
import torch

from discrete_diffusion_block_amd import dg, synth
from oracle import dg_oracle as O
from gpu_util import forced_ids, forced_routing, require_gpu, to_np_bf16

pytestmark = pytest.mark.gpu

H_FAST = 2e-5          # |H_engine - Ĥ| on rows the fast pass decided
LOGIT_TOL = 3e-2       # max |delta| of the tiny model's per-step logits


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("B,C,V,seed,draw", [(3, 256, 262144, 2 ** 64 - 5, 0), (2, 256, 262144, 12345, 7),
                                             (1, 1000, 1000, 1, 3), (1, 37, 4096, 0, 2 ** 31 - 1)])
def test_uniform_canvas_bit_exact(B, C, V, seed, draw):
    print(f"uniform canvas {B}x{C} V={V} seed={seed} draw={draw}", flush=True)
    c = torch.empty(B, C, dtype=torch.int32, device="cuda")
    dg.dg_uniform_canvas(c, V, seed, draw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(c.cpu().numpy(), O.uniform_canvas(seed, draw, B, C, V))


def _run(logits, canvas, gamma, commit_all=False, tau=1.0, e_stop=-1.0, prev=None, done=None, seed=17, draw=1,
         step=0):
    B, C, V = logits.shape
    d_canvas = canvas.cuda()
    H = torch.empty(B, C, device="cuda")
    am = torch.empty(B, C, dtype=torch.int32, device="cuda")
    n_open = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(dg.dg_sample_workspace_size(B, C, V), dtype=torch.uint8, device="cuda")
    d_prev = None if prev is None else prev.cuda()
    d_done = None if done is None else done.cuda()
    dg.dg_sample_eb_uniform(logits.cuda(), d_canvas, gamma, commit_all, tau, e_stop, d_prev, step, d_done, seed,
                            draw, n_open, ws, H, am)
    torch.cuda.synchronize()
    return (d_canvas.cpu().numpy(), H.cpu().numpy(), am.cpu().numpy(), n_open.cpu().numpy(),
            None if d_done is None else d_done.cpu().numpy(), None if d_prev is None else d_prev.cpu().numpy())


def _check(logits, canvas, got, gamma, commit_all=False, tau=1.0, e_stop=None, prev=None, frozen=None, seed=17,
           draw=1):
    out, Hg, ag, n_open = got[:4]
    ref = O.sample_eb_uniform(logits.double().numpy(), canvas.numpy(), gamma, commit_all, seed, draw, tau, e_stop,
                              None if prev is None else prev.numpy(), frozen)
    np.testing.assert_array_equal(out, ref[0])
    np.testing.assert_array_equal(ag, ref[2])
    np.testing.assert_array_equal(n_open, ref[3])
    live = ~np.isnan(ref[1])
    assert np.array_equal(np.isnan(Hg), ~live)
    if live.any():
        assert float(np.abs(Hg[live].astype(np.float64) - ref[1][live]).max()) <= H_FAST / tau
    return ref


def _full_inputs():
    V, C = 262144, 256
    l1 = synth.make_sampler_logits(C, V)                          # N(0, 4^2) + 12 spike on 60% of rows
    l2 = synth.make_sampler_logits(C, V, seed=5).float()
    g = torch.Generator().manual_seed(9)
    sharp = torch.randperm(C, generator=g)[:40]
    l2[sharp, torch.randint(0, V, (40,), generator=g)] += 40.0    # H ~ 0
    l2[sharp[30:40]] = l2[sharp[20:30]].clone()                   # exact ties
    logits = torch.stack([l1, l2.to(torch.bfloat16)])
    canvas = torch.from_numpy(O.uniform_canvas(17, 0, 2, C, V).astype(np.int32))
    return logits, canvas


@pytest.mark.parametrize("gamma,commit_all", [(0.5, False), (2.0, False), (1e9, False), (2.0, True)])
def test_uniform_sampler_full_size_vs_oracle(gamma, commit_all):
    """2 x 256 x 262144 logits, every row a candidate: the new canvas (argmaxes of the
    accepted rows, Philox tokens elsewhere) equals the oracle's bit for bit."""
    print(f"uniform sampler 2x256x262144 gamma={gamma} commit_all={commit_all}", flush=True)
    logits, canvas = _full_inputs()
    got = _run(logits, canvas, gamma, commit_all)
    ref = _check(logits, canvas, got, gamma, commit_all)
    acc = ref[4]
    assert len(acc[1]) >= 40 if not commit_all else all(len(a) == 256 for a in acc)


def test_uniform_sampler_ambiguous_and_tempered():
    """A cluster of near-identical rows at the budget boundary (the order inside it is
    open to the fast pass and is taken on Ĥ), at tau 1 and at tau 0.6."""
    V, C = 262144, 64
    print(f"uniform sampler ambiguous 1x{C}x{V}", flush=True)
    rest = torch.randn(C, V, generator=torch.Generator().manual_seed(41)).to(torch.bfloat16)
    g = torch.Generator().manual_seed(42)
    base = (torch.randn(V, generator=g) * 4.0).to(torch.bfloat16)
    u = base.float().max() - base.float()
    cl = base.repeat(8, 1)
    bits = cl.view(torch.int16)
    for i in range(1, 8):
        lo = 8.5 + 0.6 * i
        cand = torch.nonzero((u >= lo) & (u <= lo + 0.5) & (base.float() > 0)).view(-1)
        bits[i, cand[0]] += 1
    pos = [3 + 7 * i for i in range(8)]
    lg = rest.clone()
    lg[pos] = cl
    canvas = torch.from_numpy(O.uniform_canvas(5, 0, 1, C, V).astype(np.int32))
    for tau in (1.0, 0.6):
        Hc = O.entropy_canonical(lg.double().numpy()[pos], tau)
        for gamma in (float(4.5 * Hc[0]), float(2.5 * Hc[0])):
            got = _run(lg.view(1, C, V), canvas, gamma, tau=tau, seed=5, draw=3)
            ref = _check(lg.view(1, C, V), canvas, got, gamma, tau=tau, seed=5, draw=3)
            assert 2 <= len(ref[4][0]) <= 5


def test_uniform_sampler_stop_and_frozen():
    """Sequence 0: every row sharp with its argmax repeated -- the stop fires, every row
    takes its argmax and the done step is set.  Sequence 1: one argmax moved -- the budget
    decides.  Sequence 2: complete before the call -- untouched."""
    V, C, B = 32768, 64, 3
    print(f"uniform sampler stop/frozen {B}x{C}x{V}", flush=True)
    g = torch.Generator().manual_seed(31)
    lf = torch.randn(B, C, V, generator=g)
    ids = torch.randint(0, V, (B, C), generator=g)
    lf.scatter_(2, ids.unsqueeze(2), 60.0)
    logits = lf.to(torch.bfloat16)
    canvas = torch.from_numpy(O.uniform_canvas(8, 0, B, C, V).astype(np.int32))
    prev = ids.to(torch.int32).clone()
    prev[1, 20] = (prev[1, 20] + 1) % V
    done = torch.tensor([0, 0, 3], dtype=torch.int32)
    got = _run(logits, canvas, -1.0, tau=0.6, e_stop=0.005, prev=prev, done=done, seed=8, draw=6, step=5)
    _check(logits, canvas, got, -1.0, tau=0.6, e_stop=0.005, prev=prev, frozen=np.array([False, False, True]),
           seed=8, draw=6)
    out, Hg, ag, n_open, done_out, prev_out = got
    assert done_out.tolist() == [6, 0, 3]
    assert n_open.tolist() == [0, C - 1, 0]
    np.testing.assert_array_equal(out[2], canvas[2].numpy())
    np.testing.assert_array_equal(prev_out, ag)          # this step's argmax, -1 where frozen
    assert (ag[2] == -1).all()


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.CONFIGS["tiny"]
    w_cpu = synth.make_weights(cfg)
    w_np = O.to_numpy_weights(w_cpu)
    w_gpu = {"embed": w_cpu["embed"].cuda(), "final_norm": w_cpu["final_norm"].cuda(),
             "layers": [{k: v.cuda() for k, v in lw.items()} for lw in w_cpu["layers"]]}
    prompt = synth.make_prompt(cfg, 2, 64)
    return cfg, w_np, w_gpu, prompt


@pytest.mark.parametrize("e_stop,gamma,tau", [(-1.0, 3.0 * 8.27, (1.0, 1.0)), (1e30, 1e9, (0.8, 0.4)),
                                              (0.005, 40.0, (0.8, 0.4))])
def test_generate_block_uniform_equals_stepwise(tiny, e_stop, gamma, tau):
    """dg_generate_block_uniform == dg_uniform_canvas + (dg_denoise_step + dg_sample_eb_uniform)
    per step, bitwise, for two sequences, then the append."""
    cfg, w_np, w_gpu, prompt = tiny
    V, C, B, steps, seed = cfg.vocab, cfg.canvas, 2, 6, 2 ** 40 + 3
    print(f"generate_block_uniform e_stop={e_stop} gamma={gamma} tau={tau}", flush=True)
    logits = torch.empty(B, C, V, dtype=torch.bfloat16, device="cuda")
    n_open = torch.empty(B, dtype=torch.int32, device="cuda")
    done = torch.empty(B, dtype=torch.int32, device="cuda")
    eng = dg.Engine(cfg, w_gpu, max_batch=B, max_ctx=128)
    eng.prefill_kv(prompt.cuda())
    blk = torch.empty(B, C, dtype=torch.int32, device="cuda")
    eng.generate_block_uniform(blk, steps, gamma, tau[0], tau[1], e_stop, seed, True, logits, n_open, done)
    torch.cuda.synchronize()
    assert n_open.tolist() == [0, 0] and eng.lengths == [64 + C, 64 + C]

    ref = dg.Engine(cfg, w_gpu, max_batch=B, max_ctx=128)
    ref.prefill_kv(prompt.cuda())
    canvas = torch.empty(B, C, dtype=torch.int32, device="cuda")
    dg.dg_uniform_canvas(canvas, V, seed, 0)
    prev = torch.full((B, C), -1, dtype=torch.int32, device="cuda")
    done_ref = torch.zeros(B, dtype=torch.int32, device="cuda")
    for s in range(steps):
        t = np.float32(1) - np.float32(s) / np.float32(steps)
        tt = np.float32(tau[1]) + (np.float32(tau[0]) - np.float32(tau[1])) * t
        ref.denoise_step(canvas, float(t), logits)
        ref.sample_eb_uniform(logits, canvas, gamma, s == steps - 1, float(tt), e_stop, prev, s, done_ref, seed,
                              s + 1, n_open)
    ref.prefill_kv(canvas)
    torch.cuda.synchronize()
    assert torch.equal(blk, canvas)
    assert torch.equal(done, done_ref)
    if e_stop > 1:
        assert (done < steps).all() and (done >= 2).all()     # gamma huge: the argmaxes settle, the stop fires
    else:
        assert (done == steps).all()
    k1, v1 = eng.kv_view()
    k2, v2 = ref.kv_view()
    assert torch.equal(k1[:, :, :, :64 + C], k2[:, :, :, :64 + C])
    assert torch.equal(v1[:, :, :, :64 + C], v2[:, :, :, :64 + C])
    eng.close(); ref.close()


@pytest.mark.parametrize("steps,gamma,tau,e_stop", [(6, 3.0 * 8.27, (1.0, 1.0), -1.0),
                                                    (24, 1e9, (1.0, 1.0), 1e30)])
def test_generate_block_uniform_vs_oracle(tiny, steps, gamma, tau, e_stop):
    """Teacher-forced against the oracle's generator: at every step the engine consumes the
    oracle's canvas, routing and previous argmaxes; its logits stay within LOGIT_TOL of the
    oracle's, and its new canvas on its own logits equals the oracle's sampler on those
    logits bit for bit (re-noised tokens included)."""
    cfg, w_np, w_gpu, prompt = tiny
    V, C, seed = cfg.vocab, cfg.canvas, 9
    print(f"generate_block_uniform vs oracle steps={steps} gamma={gamma} e_stop={e_stop}", flush=True)
    p16 = prompt[:1, :16].contiguous()
    kv = O.KVCache(cfg, 1)
    tr = [[]]
    O.prefill_kv(cfg, w_np, kv, p16.numpy(), trace=tr)
    rec = []
    final, done_o = O.generate_block_uniform(cfg, w_np, kv, 1, steps, gamma, seed, tau[0], tau[1], e_stop,
                                             append=False, record=rec)
    eng = dg.Engine(cfg, w_gpu, max_batch=1, max_ctx=128)
    with forced_routing(eng, forced_ids(tr, cfg.n_layers)):
        eng.prefill_kv(p16.cuda())
    d0 = torch.empty(1, C, dtype=torch.int32, device="cuda")
    dg.dg_uniform_canvas(d0, V, seed, 0)
    np.testing.assert_array_equal(d0.cpu().numpy(), rec[0]["canvas_in"])
    logits = torch.empty(1, C, V, dtype=torch.bfloat16, device="cuda")
    n_open = torch.empty(1, dtype=torch.int32, device="cuda")
    done = torch.zeros(1, dtype=torch.int32, device="cuda")
    prev_np = np.full((1, C), -1)
    worst, same, want_done = 0.0, 0, 0
    for s, r in enumerate(rec[:done_o[0]]):
        trd = [[]]
        logits_o = O.denoise_step(cfg, w_np, kv, r["canvas_in"], r["t"], trace=trd)
        canvas = torch.from_numpy(r["canvas_in"].astype(np.int32)).cuda()
        with forced_routing(eng, forced_ids(trd, cfg.n_layers)):
            eng.denoise_step(canvas, r["t"], logits)
        lg = to_np_bf16(logits)[0]
        worst = max(worst, float(np.abs(lg - logits_o[0]).max()))
        prev = torch.from_numpy(prev_np.astype(np.int32)).cuda()
        eng.sample_eb_uniform(logits, canvas, gamma, s == steps - 1, r["tau"], e_stop, prev, s, done, seed, s + 1,
                              n_open)
        torch.cuda.synchronize()
        ref = O.sample_eb_uniform(lg[None], r["canvas_in"], gamma, s == steps - 1, seed, s + 1, r["tau"], e_stop,
                                  prev_np, np.array([want_done > 0]))
        np.testing.assert_array_equal(canvas.cpu().numpy(), ref[0])
        assert n_open.item() == ref[3][0]
        if ref[5][0] and want_done == 0:
            want_done = s + 1
        same += int(sorted(ref[4][0]) == sorted(r["accepted"][0]) and
                    np.array_equal(ref[2][0], r["argmax"][0]))
        prev_np = r["argmax"]
    n = int(done_o[0])
    print(f"  max |logit delta| {worst:.2e}; steps whose accepted sets and argmaxes equal the oracle's own "
          f"{same}/{n}; oracle complete after {n} steps, engine {done.item()}", flush=True)
    assert worst <= LOGIT_TOL
    assert done.item() == want_done          # the stop on the engine's own logits, as the oracle takes it
    if same == n:
        assert want_done == n
    eng.close()
