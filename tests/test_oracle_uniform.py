"""Pins of the oracle's uniform ("multinomial") variant (CPU only).

The random tokens are checked against numpy's own Philox4x64-10 generator (a library
implementation of the same published generator, reached through its own counter
convention), the sampler against the absorbing sampler it reduces to when every
position is a candidate, and the generator against a loop written out here from the
Technical Report's description (§3.2 canvas initialisation and multinomial diffusion,
§3.3 entropy-bounded acceptance with uniform re-noising), drawing its tokens from numpy.
"""
import numpy as np
import pytest

from oracle import dg_oracle as O
from discrete_diffusion_block_amd import synth

U64 = (1 << 64) - 1


def numpy_philox_words(counter, key):
    """The four output words of the Philox4x64-10 block at `counter`, from numpy's
    bit generator (which advances its 256-bit counter by one before each block)."""
    n = sum(int(c) << (64 * i) for i, c in enumerate(counter))
    n = (n - 1) % (1 << 256)
    start = np.array([(n >> (64 * i)) & U64 for i in range(4)], dtype=np.uint64)
    g = np.random.Philox(counter=start, key=np.array([int(k) & U64 for k in key], dtype=np.uint64))
    return [int(v) for v in g.random_raw(4)]


def numpy_token(seed, draw, seq, pos, vocab):
    x = numpy_philox_words((pos, seq, draw, 0), (seed, 0))[0]
    return (x * vocab) >> 64


@pytest.mark.parametrize("counter,key", [((0, 0, 0, 0), (0, 0)), ((1, 0, 0, 0), (0, 0)),
                                         ((5, 7, 11, 13), (123, 456)), ((0, 1, 0, 0), (2 ** 63, 1)),
                                         ((U64, U64, 3, 0), (U64, U64)), ((255, 1, 12, 0), (20260101, 0))])
def test_philox_matches_numpy(counter, key):
    assert list(O.philox4x64(counter, key)) == numpy_philox_words(counter, key)


def test_philox_round_count_matters():
    # 10 rounds is the generator's definition; a different count gives other words
    assert O.philox4x64((3, 0, 0, 0), (9, 0), rounds=7) != O.philox4x64((3, 0, 0, 0), (9, 0))


def test_uniform_token_is_the_top_bits_for_power_of_two_vocab():
    for pos in range(40):
        x = numpy_philox_words((pos, 1, 2, 0), (77, 0))[0]
        assert O.uniform_token(77, 2, 1, pos, 4096) == x >> 52
        assert O.uniform_token(77, 2, 1, pos, 262144) == x >> 46


def test_uniform_token_is_uniform_for_other_vocab():
    V, n = 1000, 100000
    counts = np.zeros(V)
    for i in range(n):
        t = O.uniform_token(5, i // 256, 0, i % 256, V)
        assert 0 <= t < V
        counts[t] += 1
    chi2 = float(((counts - n / V) ** 2 / (n / V)).sum())
    assert chi2 < (V - 1) + 6 * np.sqrt(2 * (V - 1)), chi2


def test_uniform_canvas_coordinates():
    c = O.uniform_canvas(11, 0, 2, 16, 4096)
    assert c.shape == (2, 16) and c.min() >= 0 and c.max() < 4096
    for b in range(2):
        for i in range(16):
            assert c[b, i] == numpy_token(11, 0, b, i, 4096)
    # every coordinate of the counter and the key changes the tokens
    assert not np.array_equal(c[0], c[1])
    assert not np.array_equal(c, O.uniform_canvas(11, 1, 2, 16, 4096))
    assert not np.array_equal(c, O.uniform_canvas(12, 0, 2, 16, 4096))


def _logits(B, C, V, seed):
    return O.bf16(synth.make_sampler_logits(B * C, V, seed=seed).float().numpy()).reshape(B, C, V)


@pytest.mark.parametrize("gamma,commit_all", [(0.5, False), (2.0, False), (1e9, False), (0.5, True)])
def test_uniform_sampler_reduces_to_absorbing_on_every_position(gamma, commit_all):
    """With every position a candidate, the accepted set and its tokens are the absorbing
    sampler's on an all-[MASK] canvas of the same logits; every other position holds the
    generator's token for this draw."""
    B, C, V = 2, 64, 4096
    L = _logits(B, C, V, 21)
    canvas = O.uniform_canvas(3, 0, B, C, V)
    got, H, a, n_open, acc, complete = O.sample_eb_uniform(L, canvas, gamma, commit_all, seed=3, draw=4)
    ref, H_ref, a_ref, n_ref, committed = O.sample_eb(L, np.full((B, C), V), gamma, commit_all, V)
    np.testing.assert_array_equal(H, H_ref)
    np.testing.assert_array_equal(a, a_ref)
    for b in range(B):
        assert acc[b] == committed[b]
        assert n_open[b] == C - len(acc[b]) == n_ref[b]
        assert complete[b] == commit_all
        for i in range(C):
            want = ref[b, i] if i in committed[b] else numpy_token(3, 4, b, i, V)
            assert got[b, i] == want, (b, i)
    if gamma == 1e9 or commit_all:
        assert all(len(x) == C for x in acc)
    else:
        assert all(1 <= len(x) < C for x in acc)


def test_uniform_sampler_revises_earlier_acceptances():
    """An accepted token is not frozen: on the next step a position that is no longer
    among the accepted ones is re-noised (the absorbing sampler would keep it)."""
    C, V = 32, 4096
    L1 = np.zeros((1, C, V))
    L2 = np.zeros((1, C, V))
    L1[0, 3, 17] = 60.0           # only row 3 is sharp at the first step
    L2[0, 5, 99] = 60.0           # only row 5 at the second
    c0 = O.uniform_canvas(1, 0, 1, C, V)
    c1, *_ , acc1, _ = O.sample_eb_uniform(L1, c0, 0.5, False, seed=1, draw=1)
    assert acc1 == [[3]] and c1[0, 3] == 17
    c2, *_ , acc2, _ = O.sample_eb_uniform(L2, c1, 0.5, False, seed=1, draw=2)
    assert acc2 == [[5]] and c2[0, 5] == 99
    assert c2[0, 3] == numpy_token(1, 2, 0, 3, V)
    # the absorbing sampler keeps its committed token
    a1, *_ = O.sample_eb(L1, np.full((1, C), V), 0.5, False, V)
    a2, *_ = O.sample_eb(L2, a1, 0.5, False, V)
    assert a2[0, 3] == 17


def test_uniform_sampler_stop_and_frozen():
    B, C, V = 2, 32, 4096
    L = np.zeros((B, C, V))
    for b in range(B):
        for i in range(C):
            L[b, i, (7 * i + b) % V] = 80.0        # every row sharp: H ~ 0
    prev = np.argmax(L, axis=-1)
    canvas = O.uniform_canvas(2, 0, B, C, V)
    frozen = np.array([False, True])
    got, H, a, n_open, acc, complete = O.sample_eb_uniform(L, canvas, 0.0, False, 2, 1, e_stop=0.005,
                                                           prev_amax=prev, frozen=frozen)
    assert complete.tolist() == [True, False]
    np.testing.assert_array_equal(got[0], prev[0])          # stop: every position accepted
    np.testing.assert_array_equal(got[1], canvas[1])        # frozen: untouched
    assert np.isnan(H[1]).all() and (a[1] == -1).all() and n_open.tolist() == [0, 0]
    # one argmax different from the previous step: no stop, the budget decides
    prev2 = prev.copy()
    prev2[0, 4] += 1
    got2, *_ , acc2, complete2 = O.sample_eb_uniform(L, canvas, 0.0, False, 2, 1, e_stop=0.005,
                                                     prev_amax=prev2)
    assert not complete2[0] and len(acc2[0]) == C          # H = 0 exactly: every running sum <= 0


def _uniform_loop(cfg, w, kv, steps, gamma, seed, tau_max, tau_min, e_stop):
    """The uniform variant written out step by step: a canvas of numpy-Philox tokens
    (draw 0); at step s the decoder at t_s = 1 - s/N over the whole canvas, canonical
    entropies at tau_s (linear in t_s), every position ranked by (entropy, position), the
    running sum within gamma (at least one; all at the last step or when the stop fires),
    accepted positions take their argmax and the others numpy-Philox tokens of draw s + 1."""
    V, C = cfg.vocab, cfg.canvas
    canvas = np.array([numpy_token(seed, 0, 0, i, V) for i in range(C)])
    prev = np.full(C, -1)
    done, history = 0, []
    for s in range(steps):
        t = 1.0 - s / steps
        tau = tau_min + (tau_max - tau_min) * t
        logits = O.bf16(O.denoise_step(cfg, w, kv, canvas[None], t))[0]
        H = O.entropy_canonical(logits, tau)
        a = np.argmax(logits, axis=1)
        mean = sum(float(h) for h in H) / C
        stop = mean < float(np.float32(e_stop)) and bool(np.all(a == prev))
        order = sorted(range(C), key=lambda i: (float(H[i]), i))
        if s == steps - 1 or stop:
            chosen = order
        else:
            run, chosen = 0.0, []
            for i in order:
                run += float(H[i])
                if run > float(np.float32(gamma)):
                    break
                chosen.append(i)
            chosen = chosen or order[:1]
        nxt = np.array([numpy_token(seed, s + 1, 0, i, V) for i in range(C)])
        nxt[chosen] = a[chosen]
        history.append((sorted(chosen), a))
        canvas = nxt
        prev = a
        if s == steps - 1 or stop:
            done = s + 1
            break
    return canvas, done, history


@pytest.mark.parametrize("steps,gamma,tau,e_stop", [(6, 3.0 * 8.27, (1.0, 1.0), -1.0),
                                                    (8, 40.0, (0.8, 0.4), -1.0)])
def test_uniform_generator_vs_independent_loop(steps, gamma, tau, e_stop):
    cfg = synth.CONFIGS["tiny"]
    w = O.to_numpy_weights(synth.make_weights(cfg))
    prompt = synth.make_prompt(cfg, 1, 16).numpy()
    kv1, kv2 = O.KVCache(cfg, 1), O.KVCache(cfg, 1)
    O.prefill_kv(cfg, w, kv1, prompt)
    O.prefill_kv(cfg, w, kv2, prompt)
    rec = []
    got, done = O.generate_block_uniform(cfg, w, kv1, 1, steps, gamma, seed=9, tau_max=tau[0], tau_min=tau[1],
                                         e_stop=e_stop, append=False, record=rec)
    want, want_done, history = _uniform_loop(cfg, w, kv2, steps, gamma, 9, tau[0], tau[1], e_stop)
    np.testing.assert_array_equal(got[0], want)
    assert done[0] == want_done == steps
    assert [sorted(r["accepted"][0]) for r in rec] == [h[0] for h in history]
    # the input canvas never holds [MASK]; the last step accepts every position
    assert all((r["canvas_in"] < cfg.vocab).all() for r in rec)
    np.testing.assert_array_equal(got[0], history[-1][1])
    # more than one position accepted per step, and at least one acceptance revised later
    assert all(len(h[0]) >= 2 for h in history[:-1])
    revised = any(set(history[s][0]) - set(history[s + 1][0]) for s in range(steps - 2))
    assert revised


def test_uniform_generator_stop_fires_and_freezes():
    """With e_stop huge the stop fires at the first step whose argmaxes all repeat the
    previous step's; the canvas is complete there and later steps leave it alone."""
    cfg = synth.CONFIGS["tiny"]
    w = O.to_numpy_weights(synth.make_weights(cfg))
    prompt = synth.make_prompt(cfg, 1, 16).numpy()
    kv1, kv2 = O.KVCache(cfg, 1), O.KVCache(cfg, 1)
    O.prefill_kv(cfg, w, kv1, prompt)
    O.prefill_kv(cfg, w, kv2, prompt)
    steps, gamma = 24, 1e9          # gamma huge: every position accepted at every step
    rec = []
    got, done = O.generate_block_uniform(cfg, w, kv1, 1, steps, gamma, seed=4, e_stop=1e30, append=False,
                                         record=rec)
    want, want_done, history = _uniform_loop(cfg, w, kv2, steps, gamma, 4, 1.0, 1.0, 1e30)
    np.testing.assert_array_equal(got[0], want)
    assert done[0] == want_done
    assert 1 < want_done < steps
    # after completion: nothing read (H NaN) and the canvas unchanged
    for r in rec[want_done:]:
        assert np.isnan(r["H"][0]).all()
        np.testing.assert_array_equal(r["canvas_in"][0], got[0])
