"""Metric formulas and constants pinned to the values printed on the pages (tests/golden)."""
import json
import os

import numpy as np
import pytest

from discrete_diffusion_block_amd import metrics, synth
from oracle import dg_oracle as O

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))


def test_tps_equals_tpf_over_step_time():
    g = G["tps_from_tpf"]
    assert round(metrics.tokens_per_second(g["tpf"], g["t_fwd_ms"] / 1000.0)) == g["tps"]


def test_tpf_counts_append_passes():
    for c in G["tpf_definition"]["cases"]:
        assert metrics.tokens_per_forward(c["canvas_tokens"], c["steps"]) == pytest.approx(c["tpf"])


def test_effective_steps_equal_budget_without_adaptive_stop():
    n = G["effective_steps_without_adaptive_stop"]["budget"]
    assert metrics.effective_steps([256, 256, 37], [n, n, n]) == n


def test_absorbing_forward_page_example():
    g = G["absorbing_forward"]
    x = np.array([10, 20, 30, 40, 50])
    u = synth.make_uniforms(5, seed=7).numpy()
    out0, m0 = O.absorbing_forward(x, 0, g["T"], u, g["mask_id"])
    outT, mT = O.absorbing_forward(x, g["T"], g["T"], u, g["mask_id"])
    assert m0.mean() == g["rate_at_t0"] and mT.mean() == g["rate_at_T"]
    assert np.all(outT == g["vocab_size"])


def test_architecture_constants_in_full_config():
    a = G["architecture"]
    c = synth.CONFIGS["full"]
    assert (c.n_layers, c.window, c.canvas, c.n_experts, c.top_k) == (
        a["layers"], a["sliding_window"], a["canvas"], a["experts"], a["active_experts"])
    assert abs(c.vocab - a["vocab_approx"]) / a["vocab_approx"] < 0.01
