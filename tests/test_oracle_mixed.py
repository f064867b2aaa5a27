"""Pins of the oracle's mixed batches and serving loop (Technical Report §6) (CPU only).

A mixed batch is pinned to its plain definition -- each sequence's own pass, through the
already pinned denoise_step and prefill_kv -- and to the independence of rows across
sequences; the serving loop is pinned to block generation when every sequence runs in
lockstep, and to each sequence served alone when they are staggered.
"""
import numpy as np

from oracle import dg_oracle as O
from discrete_diffusion_block_amd import synth


def _setup(batch, plen=16):
    cfg = synth.CONFIGS["tiny"]
    w = O.to_numpy_weights(synth.make_weights(cfg))
    prompt = synth.make_prompt(cfg, batch, plen).numpy()
    return cfg, w, prompt


def _kv(cfg, w, prompt):
    kv = O.KVCache(cfg, prompt.shape[0])
    O.prefill_kv(cfg, w, kv, prompt)
    return kv


def test_all_denoise_is_the_denoising_pass():
    cfg, w, prompt = _setup(2)
    canvas = np.stack([synth.make_masked_canvas(cfg.canvas, cfg.vocab, 10, seed=s).numpy() for s in (1, 2)])
    a = O.mixed_step(cfg, w, _kv(cfg, w, prompt), canvas, [False, False], [0.6, 0.6])
    b = O.denoise_step(cfg, w, _kv(cfg, w, prompt), canvas, 0.6)
    np.testing.assert_array_equal(a, b)


def test_all_encode_is_the_kv_append():
    cfg, w, prompt = _setup(2)
    toks = synth.make_prompt(cfg, 2, cfg.canvas, seed=9).numpy()
    kv1, kv2 = _kv(cfg, w, prompt), _kv(cfg, w, prompt)
    out = O.mixed_step(cfg, w, kv1, toks, [True, True], [0.0, 0.0])
    O.prefill_kv(cfg, w, kv2, toks)
    assert np.isnan(out).all()
    assert kv1.len == kv2.len == [16 + cfg.canvas] * 2
    for l in range(cfg.n_layers):
        for b in range(2):
            np.testing.assert_array_equal(kv1.k[l][b], kv2.k[l][b])
            np.testing.assert_array_equal(kv1.v[l][b], kv2.v[l][b])


def test_mixed_batch_is_each_sequence_alone():
    cfg, w, prompt = _setup(3)
    C, V = cfg.canvas, cfg.vocab
    toks = np.stack([synth.make_masked_canvas(C, V, 12, seed=3).numpy(),
                     synth.make_prompt(cfg, 1, C, seed=4).numpy()[0],
                     synth.make_masked_canvas(C, V, 30, seed=5).numpy()])
    kv = _kv(cfg, w, prompt)
    out = O.mixed_step(cfg, w, kv, toks, [False, True, False], [0.7, 0.0, 0.2])
    for b, t in ((0, 0.7), (2, 0.2)):
        alone = _kv(cfg, w, prompt[b:b + 1])
        np.testing.assert_array_equal(out[b], O.denoise_step(cfg, w, alone, toks[b:b + 1], t)[0])
    assert np.isnan(out[1]).all()
    alone = _kv(cfg, w, prompt[1:2])
    O.prefill_kv(cfg, w, alone, toks[1:2])
    assert kv.len == [16, 16 + C, 16]
    for l in range(cfg.n_layers):
        np.testing.assert_array_equal(kv.k[l][1], alone.k[l][0])
        np.testing.assert_array_equal(kv.v[l][1], alone.v[l][0])
    # another sequence's tokens change nothing in a denoising sequence's logits
    toks2 = toks.copy()
    toks2[1] = synth.make_prompt(cfg, 1, C, seed=6).numpy()[0]
    out2 = O.mixed_step(cfg, w, _kv(cfg, w, prompt), toks2, [False, True, False], [0.7, 0.0, 0.2])
    np.testing.assert_array_equal(out2[0], out[0])
    np.testing.assert_array_equal(out2[2], out[2])


def test_serve_in_lockstep_is_block_generation():
    cfg, w, prompt = _setup(2)
    steps, gamma = 4, 20.0
    kv1, kv2 = _kv(cfg, w, prompt), _kv(cfg, w, prompt)
    canvas, finished, phase = O.serve(cfg, w, kv1, 2, steps, gamma, 2 * (steps + 1), [0, 0])
    blocks = [O.generate_block(cfg, w, kv2, 2, steps, gamma) for _ in range(2)]
    for b in range(2):
        assert len(finished[b]) == 2
        for i in range(2):
            np.testing.assert_array_equal(finished[b][i], blocks[i][b])
    assert (canvas == cfg.mask_id).all() and phase.tolist() == [0, 0]
    assert kv1.len == kv2.len
    for l in range(cfg.n_layers):
        for b in range(2):
            np.testing.assert_array_equal(kv1.k[l][b], kv2.k[l][b])


def test_serve_staggered_is_each_sequence_alone():
    cfg, w, prompt = _setup(3)
    steps, gamma, passes, phase0 = 4, 20.0, 12, [0, 2, 3]
    kv = _kv(cfg, w, prompt)
    canvas, finished, phase = O.serve(cfg, w, kv, 3, steps, gamma, passes, phase0)
    assert phase.tolist() == [(p + passes) % (steps + 1) for p in phase0]
    for b in range(3):
        one = _kv(cfg, w, prompt[b:b + 1])
        c1, f1, _ = O.serve(cfg, w, one, 1, steps, gamma, passes, [phase0[b]])
        np.testing.assert_array_equal(canvas[b], c1[0])
        assert len(finished[b]) == len(f1[0]) >= 2
        for x, y in zip(finished[b], f1[0]):
            np.testing.assert_array_equal(x, y)
        assert kv.len[b] == one.len[0]
    # a later start shortens the first canvas only: it is still complete when appended
    assert all((f != cfg.mask_id).all() for fb in finished for f in fb)
