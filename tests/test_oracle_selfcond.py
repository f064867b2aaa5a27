"""Pins of the oracle's self-conditioning (Technical Report §3.2, eq. 5-6) (CPU only).

The signal z = FFW(softmax(L) E) is checked against closed forms (a one-hot row gives its
own embedding row, flat logits the mean embedding, two live logits a two-term mixture),
against torch's float64 softmax and product, and its place in the decoder against the
embedding it is added to: z = 0 is the plain pass, and a z shared by every [MASK] row is
the same as moving the [MASK] embedding row (which the tied head never reads).  The
generators' use of z (from the previous step's logits, 0 at the first step) is checked
against a loop written out here with torch arithmetic.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import dg_oracle as O
from discrete_diffusion_block_amd import synth


def _setup(std=0.02):
    cfg = synth.CONFIGS["tiny"]
    w = O.to_numpy_weights(synth.make_weights(cfg))
    sc = {k: v.float().numpy() for k, v in synth.make_selfcond_weights(cfg, std=std).items()}
    return cfg, w, sc


def _torch_ffw(u_bf16: torch.Tensor, sc) -> torch.Tensor:
    """SwiGLU written with torch ops on float64 (activation rounded to bf16 like the
    model's other feed-forward networks)."""
    wgu = torch.from_numpy(sc["sc_gate_up"]).double()
    Fs = wgu.shape[0] // 2
    a = F.silu(u_bf16 @ wgu[:Fs].T) * (u_bf16 @ wgu[Fs:].T)
    a = a.float().to(torch.bfloat16).double()
    return a @ torch.from_numpy(sc["sc_down"]).double().T


def test_one_hot_row_gives_its_embedding_row():
    cfg, w, sc = _setup()
    V = cfg.vocab
    L = np.random.default_rng(0).standard_normal((3, V))
    ids = [5, 4000, 123]
    for i, a in enumerate(ids):
        L[i, a] = 2000.0                      # e^-2000 underflows to 0: p is exactly one-hot
    z, u = O.self_condition(L, w["embed"], sc)
    np.testing.assert_array_equal(u, w["embed"][ids].astype(np.float64))
    ref = _torch_ffw(torch.from_numpy(w["embed"][ids]).double(), sc).numpy()
    np.testing.assert_allclose(z, ref, rtol=1e-12, atol=1e-15)


def test_flat_logits_give_the_mean_embedding():
    cfg, w, sc = _setup()
    L = np.full((2, cfg.vocab), 3.25)
    _, u = O.self_condition(L, w["embed"], sc)
    mean = np.mean(w["embed"][:cfg.vocab].astype(np.float64), axis=0)
    np.testing.assert_allclose(u, np.stack([mean, mean]), rtol=1e-11, atol=1e-15)


def test_two_live_logits_give_the_two_term_mixture():
    cfg, w, sc = _setup()
    L = np.full((1, cfg.vocab), -1.0e4)
    L[0, 17], L[0, 99] = 2.0, 0.5
    _, u = O.self_condition(L, w["embed"], sc)
    pa = 1.0 / (1.0 + np.exp(0.5 - 2.0))
    want = pa * w["embed"][17].astype(np.float64) + (1 - pa) * w["embed"][99].astype(np.float64)
    np.testing.assert_allclose(u[0], want, rtol=1e-13, atol=1e-17)


def test_matches_torch_softmax_and_product():
    cfg, w, sc = _setup()
    L = O.bf16(synth.make_sampler_logits(8, cfg.vocab).float().numpy())
    z, u = O.self_condition(L, w["embed"], sc)
    Lt = torch.from_numpy(L).double()
    Et = torch.from_numpy(w["embed"][:cfg.vocab]).double()
    ut = torch.softmax(Lt, dim=-1) @ Et
    np.testing.assert_allclose(u, ut.numpy(), rtol=1e-12, atol=1e-16)
    zt = _torch_ffw(ut.float().to(torch.bfloat16).double(), sc)
    np.testing.assert_allclose(z, zt.numpy(), rtol=1e-10, atol=1e-16)
    # the temperature plays no part: z depends on the logits alone
    assert np.abs(z).max() > 0


def test_zero_signal_is_the_plain_pass():
    cfg, w, sc = _setup()
    prompt = synth.make_prompt(cfg, 1, 16).numpy()
    kv = O.KVCache(cfg, 1)
    O.prefill_kv(cfg, w, kv, prompt)
    canvas = np.full((1, cfg.canvas), cfg.mask_id)
    a = O.denoise_step(cfg, w, kv, canvas, 0.7)
    b = O.denoise_step(cfg, w, kv, canvas, 0.7, z=np.zeros((1, cfg.canvas, cfg.d_model)))
    np.testing.assert_array_equal(a, b)


def test_signal_enters_with_the_input_embedding():
    """A z shared by every [MASK] row equals moving the [MASK] embedding row by z."""
    cfg, w, sc = _setup()
    prompt = synth.make_prompt(cfg, 1, 16).numpy()
    kv = O.KVCache(cfg, 1)
    O.prefill_kv(cfg, w, kv, prompt)
    canvas = np.full((1, cfg.canvas), cfg.mask_id)
    r = np.random.default_rng(3).standard_normal(cfg.d_model) * 0.5
    a = O.denoise_step(cfg, w, kv, canvas, 0.4, z=np.broadcast_to(r, (1, cfg.canvas, cfg.d_model)))
    w2 = dict(w)
    w2["embed"] = w["embed"].astype(np.float64).copy()
    w2["embed"][cfg.mask_id] += r
    b = O.denoise_step(cfg, w2, kv, canvas, 0.4)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-9)
    assert np.abs(a - O.denoise_step(cfg, w, kv, canvas, 0.4)).max() > 1e-3    # and it moves the logits


def _selfcond_loop(cfg, w, sc, kv, steps, gamma, tau_max, tau_min):
    """The annealed absorbing sampler with self-conditioning, written out: z = 0 at the first
    step; after each step z = FFW(softmax(L) E) from that step's stored logits (torch)."""
    V, C = cfg.vocab, cfg.canvas
    canvas = np.full(C, V)
    z = np.zeros((C, cfg.d_model))
    zs = []
    Et = torch.from_numpy(w["embed"][:V]).double()
    for s in range(steps):
        t = 1.0 - s / steps
        tau = tau_min + (tau_max - tau_min) * t
        zs.append(z)
        logits = O.bf16(O.denoise_step(cfg, w, kv, canvas[None], t, z=z[None]))[0]
        u = torch.softmax(torch.from_numpy(logits).double(), dim=-1) @ Et
        z = _torch_ffw(u.float().to(torch.bfloat16).double(), sc).numpy()
        masked = [i for i in range(C) if canvas[i] == V]
        H = O.entropy_canonical(logits[masked], tau)
        a = np.argmax(logits[masked], axis=1)
        order = sorted(range(len(masked)), key=lambda j: (float(H[j]), masked[j]))
        if s == steps - 1:
            chosen = order
        else:
            run, chosen = 0.0, []
            for j in order:
                run += float(H[j])
                if run > float(np.float32(gamma)):
                    break
                chosen.append(j)
            chosen = chosen or order[:1]
        for j in chosen:
            canvas[masked[j]] = a[j]
    return canvas, zs


def test_annealed_generator_with_selfcond_vs_independent_loop():
    cfg, w, sc = _setup(std=1.0)
    prompt = synth.make_prompt(cfg, 1, 16).numpy()
    kv1, kv2, kv3 = O.KVCache(cfg, 1), O.KVCache(cfg, 1), O.KVCache(cfg, 1)
    for kv in (kv1, kv2, kv3):
        O.prefill_kv(cfg, w, kv, prompt)
    steps, gamma = 5, 3.0 * 8.27
    rec = []
    got, done = O.generate_block_annealed(cfg, w, kv1, 1, steps, gamma, 0.8, 0.4, -1.0, append=False,
                                          record=rec, self_cond=sc)
    want, zs = _selfcond_loop(cfg, w, sc, kv2, steps, gamma, 0.8, 0.4)
    np.testing.assert_array_equal(got[0], want)
    assert done[0] == steps
    assert not rec[0]["z_in"].any()
    for r, z in zip(rec[1:], zs[1:]):
        np.testing.assert_allclose(r["z_in"][0], z, rtol=1e-10, atol=1e-18)
    # the signal reaches the decoder: with these weights it moves the second step's logits
    # by ~2e-3 against the same step without it
    with_z = O.denoise_step(cfg, w, kv3, rec[1]["canvas_in"], rec[1]["t"], z=rec[1]["z_in"])
    without = O.denoise_step(cfg, w, kv3, rec[1]["canvas_in"], rec[1]["t"])
    assert np.abs(with_z - without).max() > 5e-4


def test_uniform_generator_with_selfcond_uses_previous_logits():
    cfg, w, sc = _setup(std=1.0)
    prompt = synth.make_prompt(cfg, 1, 16).numpy()
    kv = O.KVCache(cfg, 1)
    O.prefill_kv(cfg, w, kv, prompt)
    rec = []
    O.generate_block_uniform(cfg, w, kv, 1, 4, 3.0 * 8.27, seed=2, append=False, record=rec, self_cond=sc)
    assert not rec[0]["z_in"].any()
    for s in range(1, 4):
        logits = O.bf16(O.denoise_step(cfg, w, kv, rec[s - 1]["canvas_in"], rec[s - 1]["t"],
                                       z=rec[s - 1]["z_in"]))[0]
        z, _ = O.self_condition(logits, w["embed"], sc)
        np.testing.assert_array_equal(rec[s]["z_in"][0], z)
