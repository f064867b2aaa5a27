"""Pins of the oracle's canonical decision entropy Ĥ (CPU only).

Ĥ is the value on which the entropy-bounded sampler (DiffusionGemma Technical
Report §3.3) takes its decisions: a fixed sequence of IEEE float64 operations and
exact integer sums, so that an independent implementation can reproduce it bit for
bit.  Here it is checked against things other than itself: high-precision decimal
arithmetic for its constants, the platform's exp/log for its two kernels, the plain
entropy -sum p log p (and torch's Categorical) for the result, closed forms, and the
exact integer arithmetic of Python for its sums.
"""
import math
from decimal import Context, Decimal
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import dg_oracle as O


def rng(seed):
    return np.random.default_rng(seed)


def test_constants_from_high_precision_decimals():
    ctx = Context(prec=60)
    ln2 = Decimal(2).ln(ctx)
    assert O._LN2 == float(ln2)
    # the two-part split: hi has >= 21 trailing zero significand bits, hi + lo == ln 2
    # to far below a double's precision
    mant = Fraction(O._LN2_HI) / Fraction(2) ** math.frexp(O._LN2_HI)[1]
    assert (mant * 2 ** 32).denominator == 1
    err = abs(Decimal(O._LN2_HI) + Decimal(O._LN2_LO) - ln2)
    assert err < Decimal("1e-25")
    for k in (1, 17, 44, (1 << 21) - 1):       # k * ln2_hi exact
        assert Fraction(k * O._LN2_HI) == k * Fraction(O._LN2_HI)
    assert O._INV_LN2 == float(ctx.divide(Decimal(1), ln2))
    assert O._SQRT_HALF == float(Decimal("0.5").sqrt(ctx))
    for i, c in enumerate(O._EXP_C):
        assert c == float(Fraction(1, math.factorial(i)))
    for i, c in enumerate(O._LOG_C):
        assert c == float(Fraction(1, 2 * i + 1))


def test_canonical_exp_against_platform_exp():
    u = np.concatenate([np.linspace(0.0, 29.999, 200001), [0.0, 1e-300, 0.34657359, 0.34657360, 29.99999]])
    e = O.canon_exp_neg(u)
    ref = np.exp(-u)
    assert np.max(np.abs(e - ref) / ref) < 2e-15
    assert O.canon_exp_neg(np.array([0.0]))[0] == 1.0
    assert np.all(O.canon_exp_neg(np.array([30.0, 31.5, 1e6])) == 0.0)


def test_canonical_log_against_platform_log():
    a = np.concatenate([np.exp(np.linspace(0.0, 41.0, 100001)), [1.0, 2.0 ** 40, 2.0 ** 58 - 1, 1.4142135623730951]])
    assert np.max(np.abs(O.canon_log(a) - np.log(a))) < 2e-14
    assert O.canon_log(np.array([1.0]))[0] == 0.0


@pytest.mark.parametrize("V", [4096, 40008, 262144])
@pytest.mark.parametrize("std", [0.05, 1.0, 4.0, 10.0])
def test_canonical_entropy_close_to_plain_entropy(V, std):
    x = O.bf16(rng(V + int(std * 10)).standard_normal((4, V)) * std)
    H, _ = O.entropy_argmax(x)
    Hc = O.entropy_canonical(x)
    assert Hc.dtype == np.float32
    assert np.max(np.abs(Hc.astype(np.float64) - H)) <= 1e-6


@pytest.mark.parametrize("tau", [0.4, 0.6, 0.8, 2.5])
def test_canonical_entropy_tempered_vs_torch(tau):
    x = O.bf16(rng(int(tau * 100)).standard_normal((3, 50000)) * 4)
    tau32 = float(np.float32(tau))
    ref = torch.distributions.Categorical(logits=torch.from_numpy(x / tau32)).entropy().numpy()
    Hc = O.entropy_canonical(x, tau)
    assert np.max(np.abs(Hc.astype(np.float64) - ref)) <= 1e-6


def test_canonical_entropy_closed_forms():
    V = 262144
    # uniform row: log V
    assert abs(float(O.entropy_canonical(np.zeros((1, V)))[0]) - math.log(V)) <= 1e-6
    # a spike far above the rest: every other term is dropped (u >= 30), H = 0 exactly
    sp = np.zeros((1, V)); sp[0, 5] = 40.0
    assert O.entropy_canonical(sp)[0] == 0.0
    # two-point row (a, b): binary entropy of p = sigmoid(a - b)
    for a, b in ((1.0, 0.0), (3.5, -2.0), (0.25, 0.0)):
        q = 1.0 / (1.0 + math.exp(-(a - b)))
        Hb = -(q * math.log(q) + (1 - q) * math.log(1 - q))
        assert abs(float(O.entropy_canonical(np.array([[a, b]]))[0]) - Hb) <= 1e-6
    # k equal maxima and the rest far below: log k
    r = np.full((1, 1000), -50.0); r[0, [3, 99, 500]] = 7.0
    assert abs(float(O.entropy_canonical(r)[0]) - math.log(3)) <= 1e-6


def test_canonical_sums_exact_and_order_independent():
    x = O.bf16(rng(3).standard_normal(5000) * 3)
    S, T = O.entropy_canonical_sums(x[None])
    # the same terms summed as Python integers (exact)
    m = x.max()
    u = (m - x) * (1.0 / float(np.float32(1.0)))
    e = O.canon_exp_neg(u)
    qs = [int(v) for v in np.rint(e * 2.0 ** 40)]
    qt = [int(v) for v in np.rint((e * u) * 2.0 ** 40)]
    assert int(S[0]) == sum(qs) and int(T[0]) == sum(qt)
    # any permutation of the row: bitwise the same Ĥ
    h0 = O.entropy_canonical(x[None])
    for seed in range(3):
        assert O.entropy_canonical(rng(seed).permutation(x)[None]).tobytes() == h0.tobytes()


def test_u64_to_f64_is_correctly_rounded():
    vals = np.array([0, 1, (1 << 53) + 1, (1 << 58) - 1, 0x3ABCDEF123456789 & ((1 << 58) - 1)], dtype=np.uint64)
    got = O._u64_to_f64(vals)
    for v, g in zip(vals.tolist(), got.tolist()):
        assert g == float(Fraction(int(v)))      # Fraction -> float rounds to nearest even


def test_sampler_decides_on_canonical_entropy():
    # sample_eb reports Ĥ and takes its order and budget on it
    V, C = 3000, 12
    x = O.bf16(rng(11).standard_normal((1, C, V)) * 2.5)
    canvas = np.full((1, C), V)
    _, H32, amax, _, sel = O.sample_eb(x, canvas, 30.0, False, V)
    Hc = O.entropy_canonical(x[0])
    assert H32[0].tobytes() == Hc.tobytes()
    assert sel[0] == O.eb_select(Hc, list(range(C)), 30.0, False)
    np.testing.assert_array_equal(amax[0], np.argmax(x[0], axis=1))
