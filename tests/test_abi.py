"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments before anything is enqueued."""
import ctypes as C
import os

import pytest

from discrete_diffusion_block_amd import build, dg, synth


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dg.LIB_PATH):
        build.build()
    return dg.lib()


def test_exports_every_header_function(L):
    names = dg.header_functions()
    assert {"dg_prefill_kv", "dg_denoise_step", "dg_sample_eb", "dg_generate_block"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    assert L.dg_status_string(0) == b"ok"
    assert L.dg_status_string(-4) == b"KV cache capacity exceeded"


def _fake_weights(cfg):
    n = cfg.n_layers
    layers = (dg.LayerWeights * n)()
    for l in range(n):
        for k in synth.LAYER_KEYS:
            setattr(layers[l], k, 0x1000)
    return dg.Weights(0x1000, 0x1000, C.cast(layers, C.POINTER(dg.LayerWeights))), layers


def test_create_and_sizes_without_gpu(L):
    cfg = synth.CONFIGS["full"]
    w, keep = _fake_weights(cfg)
    ctx = dg.dg_create(dg.make_config(cfg, 1, 2048), w)
    try:
        ws = dg.dg_workspace_size(ctx, 1)
        assert 50e6 < ws < 2e9
        kvb = dg.dg_kv_size(dg.make_config(cfg, 1, 2048))
        assert kvb == 30 * 1 * 8 * 2048 * 128 * 2
        with pytest.raises(dg.DgError) as e:
            dg.dg_workspace_size(ctx, 2)                     # above max_batch
        assert e.value.status == -1
    finally:
        dg.dg_destroy(ctx)


@pytest.mark.parametrize("field,value", [("d_model", 100), ("head_dim", 48), ("n_kv_heads", 3),
                                         ("n_experts", 6), ("top_k", 17), ("expert_ffn", 96),
                                         ("vocab", 1001), ("canvas", 2000), ("max_ctx", 1000),
                                         ("max_batch", 65)])
def test_create_rejects_unsupported_shapes(L, field, value):
    cfg = synth.CONFIGS["tiny"]
    w, keep = _fake_weights(cfg)
    cc = dg.make_config(cfg, 1, 2048)
    setattr(cc, field, value)
    with pytest.raises(dg.DgError) as e:
        dg.dg_create(cc, w)
    assert e.value.status == -2
    assert len(L.dg_last_error()) > 0


def test_create_rejects_null_weights(L):
    cfg = synth.CONFIGS["tiny"]
    w, keep = _fake_weights(cfg)
    keep[1].w_down = None
    with pytest.raises(dg.DgError) as e:
        dg.dg_create(dg.make_config(cfg, 1, 2048), w)
    assert e.value.status == -1 and b"layer 1" in L.dg_last_error()


def test_calls_validate_before_launch(L):
    cfg = synth.CONFIGS["tiny"]
    w, keep = _fake_weights(cfg)
    ctx = dg.dg_create(dg.make_config(cfg, 2, 128), w)
    try:
        kv = dg.KV(0x1000, 0x1000)
        kv.len[0] = 100
        need = dg.dg_workspace_size(ctx, 1)
        # canvas (32) does not fit after 100 committed positions in a 128-slot cache
        st = L.dg_denoise_step(ctx, C.byref(kv), C.c_void_p(0x1000), 1, 0.5, C.c_void_p(0x1000),
                               C.c_void_p(0x1000), need, None)
        assert st == -4
        kv.len[0] = 0
        st = L.dg_denoise_step(ctx, C.byref(kv), C.c_void_p(0x1000), 1, 0.5, C.c_void_p(0x1000),
                               C.c_void_p(0x1000), need - 1, None)
        assert st == -3                                       # workspace too small
        st = L.dg_denoise_step(ctx, C.byref(kv), C.c_void_p(0x1000), 1, 1.5, C.c_void_p(0x1000),
                               C.c_void_p(0x1000), need, None)
        assert st == -1                                       # t outside [0, 1]
        st = L.dg_prefill_kv(ctx, C.byref(kv), C.c_void_p(0x1000), 3, 4, C.c_void_p(0x1000), need, None)
        assert st == -1                                       # batch above max_batch
        st = L.dg_prefill_kv(ctx, C.byref(kv), C.c_void_p(0x1000), 1, 129, C.c_void_p(0x1000), need, None)
        assert st == -4
        assert kv.len[0] == 0                                 # nothing advanced on error
        st = L.dg_generate_block(ctx, C.byref(kv), C.c_void_p(0x1000), 1, 0, 1.0, 1, C.c_void_p(0x1000),
                                 C.c_void_p(0x1000), C.c_void_p(0x1000), need, None)
        assert st == -1                                       # zero steps
    finally:
        dg.dg_destroy(ctx)


def test_sampler_validates(L):
    with pytest.raises(dg.DgError):
        dg.dg_sample_workspace_size(1, 256, 1001)
    need = dg.dg_sample_workspace_size(1, 256, 262144)
    assert need >= 256 * (262144 // 16384) * 20     # a 20-byte partial per row and chunk
    st = L.dg_sample_eb(C.c_void_p(0x1000), C.c_void_p(0x1000), 1, 256, 262144, 1.0, 0, None, None,
                        C.c_void_p(0x1000), C.c_void_p(0x1000), need - 1, None)
    assert st == -3
    st = L.dg_sample_eb(C.c_void_p(0x1000), C.c_void_p(0x1000), 1, 256, 262144, float("nan"), 0, None,
                        None, C.c_void_p(0x1000), C.c_void_p(0x1000), need, None)
    assert st == -1


def test_copy_tap_validates(L):
    for n in (0, 24, 17):                                     # empty, not a multiple of 16
        assert L.dg_test_copy(C.c_void_p(0x1000), C.c_void_p(0x2000), n, None) == -1
    assert L.dg_test_copy(None, C.c_void_p(0x2000), 32, None) == -1


def test_sampler_ex_validates(L):
    need = dg.dg_sample_workspace_size(1, 256, 262144)
    p = C.c_void_p(0x1000)
    ok = dict(temperature=0.6, e_stop=0.005, step=0)
    def call(temperature, e_stop, step, ws_bytes=need):
        return L.dg_sample_eb_ex(p, p, 1, 256, 262144, 1.0, 0, temperature, e_stop, None, step, None, None,
                                 None, p, p, ws_bytes, None)
    assert call(0.0, 0.005, 0) == -1                      # temperature must be > 0
    assert call(-1.0, 0.005, 0) == -1
    assert call(float("inf"), 0.005, 0) == -1
    assert call(float("nan"), 0.005, 0) == -1
    assert call(0.6, float("nan"), 0) == -1
    assert call(0.6, 0.005, -1) == -1
    assert call(**ok, ws_bytes=need - 1) == -3


def test_generate_ex_validates_before_launching(L):
    cfg = synth.CONFIGS["tiny"]
    w, keep = _fake_weights(cfg)
    ctx = dg.dg_create(dg.make_config(cfg, 1, 128), w)
    try:
        kv = dg.KV(0x1000, 0x1000)
        need = dg.dg_workspace_size(ctx, 1)
        p = C.c_void_p(0x1000)
        for max_steps, tau_max, tau_min, e_stop in ((0, 0.8, 0.4, 0.005), (4, 0.0, 0.4, 0.005),
                                                    (4, 0.8, -0.4, 0.005), (4, 0.8, 0.4, float("nan")),
                                                    (4, float("inf"), 0.4, 0.005)):
            st = L.dg_generate_block_ex(ctx, C.byref(kv), p, 1, max_steps, 1.0, tau_max, tau_min, e_stop, 1,
                                        p, p, p, p, need, None)
            assert st == -1
        st = L.dg_generate_block_ex(ctx, C.byref(kv), p, 1, 4, 1.0, 0.8, 0.4, 0.005, 1, p, p, None, p,
                                    need, None)
        assert st == -1                                   # d_done_step is required
        st = L.dg_generate_block_ex(ctx, C.byref(kv), p, 1, 4, 1.0, 0.8, 0.4, 0.005, 1, p, p, p, p,
                                    need - 1, None)
        assert st == -3
        assert kv.len[0] == 0
    finally:
        dg.dg_destroy(ctx)
