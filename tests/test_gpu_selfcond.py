"""GPU parity of self-conditioning (Technical Report §3.2, eq. 5-6) through the C ABI,
against the oracle.

Tolerances come from the arithmetic.  u = p̂₀ E: the engine carries p = exp(x - max) to
2^-18 relative (two bf16 parts, 4e-6), its exp and 1/S to a few fp32 ulps, and adds at
most ~360 MFMA results (one per 32-wide k step of a slice, 262144 / 23 / 32) in fp32
before the slices are summed, each addition off by at most 2^-24 of a running sum no
larger than sum_v p_v |E_vn|: |u_engine - u| <= U_REL * sum_v p_v |E_vn|, U_REL = 4e-5.  z = FFW(bf16(u)): the engine and
the oracle round u and the activation to bf16 at the same points but from values that
differ by fp32 rounding, so an element can land one bf16 step (at most 2^-7 relative)
apart; z is checked against the oracle's FFW applied to the engine's own u, with
|delta z_n| <= 2^-7 * sum_f |W_d[n][f] a_f| + fp32 slack.
"""
import numpy as np
import pytest
import torch

from discrete_diffusion_block_amd import dg, synth
from oracle import dg_oracle as O
from gpu_util import forced_ids, forced_routing, require_gpu, to_np_bf16

pytestmark = pytest.mark.gpu

U_REL = 4e-5
LOGIT_TOL = 3e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_transpose_pack_layout():
    """Element (n, v) of the packed E^T sits at the fragment-major offset of row n,
    column v: 16 x 32 tiles, k tiles of a row block consecutive, lane l = 16 (c/8) + r."""
    V, d = 4096, 256
    print(f"transpose pack {V}x{d}", flush=True)
    E = (torch.randn(V, d, generator=torch.Generator().manual_seed(3)) * 0.02).to(torch.bfloat16).cuda()
    P = dg.pack(E, dg.PACK_TRANSPOSE)
    torch.cuda.synchronize()
    t = P.view(d // 16, V // 32, 4, 16, 8).permute(0, 3, 1, 2, 4).reshape(d, V)
    assert torch.equal(t.cpu(), E.t().contiguous().cpu())


def _sc_engine(cfg, std=1.0):
    w = synth.make_weights(cfg, device="cuda")
    sc = synth.make_selfcond_weights(cfg, device="cuda", std=std)
    return w, sc


def _u_bound(logits_np, E, u_ref):
    L = logits_np.astype(np.float64)
    e = np.exp(L - L.max(axis=-1, keepdims=True))
    p = e / e.sum(axis=-1, keepdims=True)
    return U_REL * (p @ np.abs(E.astype(np.float64))) + 1e-12


def _z_check(z_eng, u_eng, sc_np, z_ref_fn):
    """z against the oracle's FFW of the engine's own u (see the module note)."""
    z_ref, _ = z_ref_fn(u_eng)
    wgu = sc_np["sc_gate_up"].astype(np.float64)
    Fs = wgu.shape[0] // 2
    ub = O.bf16(u_eng)
    a = O.bf16(O.silu(ub @ wgu[:Fs].T) * (ub @ wgu[Fs:].T))
    bound = 2.0 ** -7 * (np.abs(a) @ np.abs(sc_np["sc_down"].astype(np.float64)).T) + 1e-6 * np.abs(z_ref).max()
    err = np.abs(z_eng - z_ref)
    assert (err <= bound).all(), float((err / bound).max())
    return float(err.max()), float(np.abs(z_ref).max())


def _ffw_only(sc_np):
    wgu = sc_np["sc_gate_up"].astype(np.float64)
    Fs = wgu.shape[0] // 2

    def f(u):
        return O.swiglu_ffn(O.bf16(u), wgu[:Fs], wgu[Fs:], sc_np["sc_down"], O.bf16), None
    return f


@pytest.mark.parametrize("kind", ["model", "spiky"])
def test_self_cond_tiny_vs_oracle(kind):
    cfg = synth.CONFIGS["tiny"]
    B, C, V, d = 2, cfg.canvas, cfg.vocab, cfg.d_model
    print(f"self-cond tiny {kind} {B}x{C}x{V}", flush=True)
    w, sc = _sc_engine(cfg)
    eng = dg.Engine(cfg, w, max_batch=B, max_ctx=128, selfcond=sc)
    if kind == "model":
        L = (torch.randn(B, C, V, generator=torch.Generator().manual_seed(5))).to(torch.bfloat16)
    else:
        L = synth.make_sampler_logits(B * C, V, seed=6).view(B, C, V)
    z = torch.empty(B, C, d, device="cuda")
    u = torch.empty(B, C, d, device="cuda")
    eng.self_cond(L.cuda(), z, u)
    torch.cuda.synchronize()
    E = w["embed"][:V].float().cpu().numpy()
    sc_np = {k: v.float().cpu().numpy() for k, v in sc.items()}
    Ln = L.float().numpy()
    for b in range(B):
        z_ref, u_ref = O.self_condition(Ln[b], E, sc_np)
        ue = u[b].cpu().numpy().astype(np.float64)
        bound = _u_bound(Ln[b], E, u_ref)
        assert (np.abs(ue - u_ref) <= bound).all(), float((np.abs(ue - u_ref) / bound).max())
        err, scale = _z_check(z[b].cpu().numpy().astype(np.float64), ue, sc_np, _ffw_only(sc_np))
        print(f"  seq {b}: max |u delta| {np.abs(ue - u_ref).max():.2e}; z max |delta| {err:.2e} of {scale:.2e}",
              flush=True)
    eng.close()


def test_self_cond_full_width_sampled_rows():
    """The production shape: 256 rows of 262144 logits against the 2816-wide embedding
    (11 feature tiles x 23 k slices); every row's u is checked on a sample of 12 rows,
    whose oracle product is computed in float64."""
    cfg = synth.CONFIGS["layer"]
    C, V, d = cfg.canvas, cfg.vocab, cfg.d_model
    print(f"self-cond full width 1x{C}x{V} d={d}", flush=True)
    w = synth.make_weights(cfg, device="cuda")
    sc = synth.make_selfcond_weights(cfg, device="cuda")
    eng = dg.Engine(cfg, w, max_batch=1, max_ctx=1280, selfcond=sc)
    L = synth.make_sampler_logits(C, V, seed=7).view(1, C, V)
    z = torch.empty(1, C, d, device="cuda")
    u = torch.empty(1, C, d, device="cuda")
    eng.self_cond(L.cuda(), z, u)
    torch.cuda.synchronize()
    rows = [0, 1, 17, 63, 64, 100, 127, 128, 191, 200, 254, 255]
    E = w["embed"][:V].float().cpu().numpy()
    sc_np = {k: v.float().cpu().numpy() for k, v in sc.items()}
    Ln = L[0, rows].float().numpy()
    z_ref, u_ref = O.self_condition(Ln, E, sc_np)
    ue = u[0, rows].cpu().numpy().astype(np.float64)
    bound = _u_bound(Ln, E, u_ref)
    print(f"  max |u delta| {np.abs(ue - u_ref).max():.2e}; worst / bound {(np.abs(ue - u_ref) / bound).max():.3f}",
          flush=True)
    assert (np.abs(ue - u_ref) <= bound).all()
    err, scale = _z_check(z[0, rows].cpu().numpy().astype(np.float64), ue, sc_np, _ffw_only(sc_np))
    print(f"  z max |delta| {err:.2e} of {scale:.2e}", flush=True)
    assert torch.isfinite(u).all() and torch.isfinite(z).all()
    eng.close()


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.CONFIGS["tiny"]
    w_cpu = synth.make_weights(cfg)
    sc_cpu = synth.make_selfcond_weights(cfg, std=1.0)
    w_np = O.to_numpy_weights(w_cpu)
    sc_np = {k: v.float().numpy() for k, v in sc_cpu.items()}
    w_gpu = {"embed": w_cpu["embed"].cuda(), "final_norm": w_cpu["final_norm"].cuda(),
             "layers": [{k: v.cuda() for k, v in lw.items()} for lw in w_cpu["layers"]]}
    sc_gpu = {k: v.cuda() for k, v in sc_cpu.items()}
    prompt = synth.make_prompt(cfg, 2, 64)
    return cfg, w_np, sc_np, w_gpu, sc_gpu, prompt


def test_denoise_step_with_signal_vs_oracle(tiny):
    """z added to the canvas input: teacher-forced routing, logits within LOGIT_TOL of the
    oracle's; z = NULL is bitwise the plain pass."""
    cfg, w_np, sc_np, w_gpu, sc_gpu, prompt = tiny
    C, V, d = cfg.canvas, cfg.vocab, cfg.d_model
    print("denoise_step_sc vs oracle", flush=True)
    p16 = prompt[:1, :16].contiguous()
    kv = O.KVCache(cfg, 1)
    tr = [[]]
    O.prefill_kv(cfg, w_np, kv, p16.numpy(), trace=tr)
    eng = dg.Engine(cfg, w_gpu, max_batch=1, max_ctx=128, selfcond=sc_gpu)
    with forced_routing(eng, forced_ids(tr, cfg.n_layers)):
        eng.prefill_kv(p16.cuda())
    canvas = synth.make_masked_canvas(C, V, 20, seed=4).view(1, C)
    zt = (torch.randn(1, C, d, generator=torch.Generator().manual_seed(8)) * 0.5).float()
    trd = [[]]
    ref = O.denoise_step(cfg, w_np, kv, canvas.numpy(), 0.6, trace=trd, z=zt.numpy().astype(np.float64))
    logits = torch.empty(1, C, V, dtype=torch.bfloat16, device="cuda")
    with forced_routing(eng, forced_ids(trd, cfg.n_layers)):
        eng.denoise_step_sc(canvas.cuda(), 0.6, zt.cuda(), logits)
    lg = to_np_bf16(logits)[0]
    err = float(np.abs(lg - ref[0]).max())
    plain = O.denoise_step(cfg, w_np, kv, canvas.numpy(), 0.6)
    print(f"  max |logit delta| {err:.2e}; the signal moves the oracle's logits by "
          f"{float(np.abs(plain - ref).max()):.2e}", flush=True)
    assert err <= LOGIT_TOL
    assert float(np.abs(plain - ref).max()) > 10 * LOGIT_TOL
    a = torch.empty_like(logits)
    b = torch.empty_like(logits)
    eng.denoise_step_sc(canvas.cuda(), 0.6, None, a)
    eng.denoise_step(canvas.cuda(), 0.6, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    eng.close()


@pytest.mark.parametrize("uniform", [False, True])
def test_generate_block_sc_equals_stepwise(tiny, uniform):
    """dg_generate_block_sc == denoise_step_sc + self_cond + the sampler driven step by step,
    bitwise, for two sequences, then the append."""
    cfg, w_np, sc_np, w_gpu, sc_gpu, prompt = tiny
    C, V, d, B, steps, seed = cfg.canvas, cfg.vocab, cfg.d_model, 2, 5, 77
    gamma, tmax, tmin, e_stop = 3.0 * 8.27, 0.8, 0.4, 0.005
    print(f"generate_block_sc uniform={uniform}", flush=True)
    logits = torch.empty(B, C, V, dtype=torch.bfloat16, device="cuda")
    n = torch.empty(B, dtype=torch.int32, device="cuda")
    done = torch.empty(B, dtype=torch.int32, device="cuda")
    eng = dg.Engine(cfg, w_gpu, max_batch=B, max_ctx=128, selfcond=sc_gpu)
    eng.prefill_kv(prompt.cuda())
    blk = torch.empty(B, C, dtype=torch.int32, device="cuda")
    eng.generate_block_sc(blk, steps, gamma, tmax, tmin, e_stop, uniform, seed, True, logits, n, done)
    torch.cuda.synchronize()
    assert n.tolist() == [0, 0] and done.tolist() == [steps, steps]

    ref = dg.Engine(cfg, w_gpu, max_batch=B, max_ctx=128, selfcond=sc_gpu)
    ref.prefill_kv(prompt.cuda())
    canvas = torch.empty(B, C, dtype=torch.int32, device="cuda")
    if uniform:
        dg.dg_uniform_canvas(canvas, V, seed, 0)
    else:
        canvas.fill_(V)
    prev = torch.full((B, C), -1, dtype=torch.int32, device="cuda")
    done_ref = torch.zeros(B, dtype=torch.int32, device="cuda")
    z = torch.zeros(B, C, d, device="cuda")
    for s in range(steps):
        t = np.float32(1) - np.float32(s) / np.float32(steps)
        tau = np.float32(tmin) + (np.float32(tmax) - np.float32(tmin)) * t
        ref.denoise_step_sc(canvas, float(t), z if s > 0 else None, logits)
        if s + 1 < steps:
            ref.self_cond(logits, z)
        if uniform:
            ref.sample_eb_uniform(logits, canvas, gamma, s == steps - 1, float(tau), e_stop, prev, s, done_ref, seed,
                                  s + 1, n)
        else:
            ref.sample_eb_ex(logits, canvas, gamma, s == steps - 1, float(tau), e_stop, prev, s, done_ref, n)
    ref.prefill_kv(canvas)
    torch.cuda.synchronize()
    assert torch.equal(blk, canvas)
    assert torch.equal(done, done_ref)
    k1, v1 = eng.kv_view()
    k2, v2 = ref.kv_view()
    assert torch.equal(k1[:, :, :, :64 + C], k2[:, :, :, :64 + C])
    eng.close(); ref.close()


@pytest.mark.parametrize("uniform", [False, True])
def test_generate_block_sc_vs_oracle(tiny, uniform):
    """Teacher-forced against the oracle's self-conditioned generator: at every step the
    engine consumes the oracle's canvas, signal z, routing and previous argmaxes; its
    logits stay within LOGIT_TOL, its signal from its own logits matches the oracle's on
    those logits (the bounds above), and its sampler decisions on its own logits are the
    oracle's."""
    cfg, w_np, sc_np, w_gpu, sc_gpu, prompt = tiny
    C, V, d, steps, gamma, seed = cfg.canvas, cfg.vocab, cfg.d_model, 5, 3.0 * 8.27, 5
    print(f"generate_block_sc vs oracle uniform={uniform}", flush=True)
    p16 = prompt[:1, :16].contiguous()
    kv = O.KVCache(cfg, 1)
    tr = [[]]
    O.prefill_kv(cfg, w_np, kv, p16.numpy(), trace=tr)
    rec = []
    if uniform:
        O.generate_block_uniform(cfg, w_np, kv, 1, steps, gamma, seed, 0.8, 0.4, -1.0, append=False, record=rec,
                                 self_cond=sc_np)
    else:
        O.generate_block_annealed(cfg, w_np, kv, 1, steps, gamma, 0.8, 0.4, -1.0, append=False, record=rec,
                                  self_cond=sc_np)
    eng = dg.Engine(cfg, w_gpu, max_batch=1, max_ctx=128, selfcond=sc_gpu)
    with forced_routing(eng, forced_ids(tr, cfg.n_layers)):
        eng.prefill_kv(p16.cuda())
    logits = torch.empty(1, C, V, dtype=torch.bfloat16, device="cuda")
    n = torch.empty(1, dtype=torch.int32, device="cuda")
    done = torch.zeros(1, dtype=torch.int32, device="cuda")
    z = torch.empty(1, C, d, device="cuda")
    u = torch.empty(1, C, d, device="cuda")
    E = w_np["embed"][:V]
    prev_np = np.full((1, C), -1)
    worst = 0.0
    for s, r in enumerate(rec):
        trd = [[]]
        z_in = r["z_in"]
        logits_o = O.denoise_step(cfg, w_np, kv, r["canvas_in"], r["t"], trace=trd, z=z_in)
        canvas = torch.from_numpy(r["canvas_in"].astype(np.int32)).cuda()
        zt = None if z_in is None or not z_in.any() else torch.from_numpy(z_in.astype(np.float32)).cuda()
        with forced_routing(eng, forced_ids(trd, cfg.n_layers)):
            eng.denoise_step_sc(canvas, r["t"], zt, logits)
        lg = to_np_bf16(logits)[0]
        worst = max(worst, float(np.abs(lg - logits_o[0]).max()))
        eng.self_cond(logits, z, u)
        prev = torch.from_numpy(prev_np.astype(np.int32)).cuda()
        if uniform:
            eng.sample_eb_uniform(logits, canvas, gamma, s == steps - 1, r["tau"], -1.0, prev, s, done, seed, s + 1, n)
        else:
            eng.sample_eb_ex(logits, canvas, gamma, s == steps - 1, r["tau"], -1.0, prev, s, done, n)
        torch.cuda.synchronize()
        z_ref, u_ref = O.self_condition(lg, E, sc_np)
        ue = u[0].cpu().numpy().astype(np.float64)
        assert (np.abs(ue - u_ref) <= _u_bound(lg, E, u_ref)).all()
        _z_check(z[0].cpu().numpy().astype(np.float64), ue, sc_np, _ffw_only(sc_np))
        if uniform:
            ref = O.sample_eb_uniform(lg[None], r["canvas_in"], gamma, s == steps - 1, seed, s + 1, r["tau"], -1.0,
                                      prev_np)
        else:
            ref = O.sample_eb(lg[None], r["canvas_in"], gamma, s == steps - 1, cfg.mask_id, r["tau"], -1.0, prev_np)
        np.testing.assert_array_equal(canvas.cpu().numpy(), ref[0])
        prev_np = r["argmax"]
    print(f"  max |logit delta| over {steps} steps {worst:.2e}", flush=True)
    assert worst <= LOGIT_TOL
    eng.close()
