"""Thin ctypes binding of libdg.so (include/dg.h).

Argument marshalling only: every computation runs in the library's HIP
kernels.  torch tensors supply device memory and the current HIP stream.
Functions keep the C names (dg_prefill_kv, dg_denoise_step, dg_sample_eb,
dg_generate_block, ...) and raise DgError on a non-zero status.  If the
library has not been built, loading fails loudly — there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import re
from typing import Optional

import torch

from .build import source_digest
from .synth import ModelConfig, LAYER_KEYS

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdg.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dg.h")
MAX_BATCH = 64

KERNEL_KINDS = ["prep", "embed", "qkv", "attention", "o_proj", "norm", "router", "topk", "route",
                "moe_gate_up", "moe_down", "shared_gate_up", "shared_down", "combine", "head",
                "sample_pass1", "sample_select", "fill", "sample_canon", "sample_select_canon",
                "attention_global", "sc_stats", "sc_embed", "sc_reduce", "sc_ffw"]
PACK_PLAIN, PACK_QKV, PACK_GATE_UP, PACK_TRANSPOSE = 0, 1, 2, 3
MOE_GROUP = 64   # tokens per grouped-GEMM work item in the routing tap's item list

STATUS = {0: "DG_OK", -1: "DG_ERR_INVALID_ARG", -2: "DG_ERR_SHAPE", -3: "DG_ERR_WORKSPACE",
          -4: "DG_ERR_KV_CAPACITY", -5: "DG_ERR_HIP", -6: "DG_ERR_UNSUPPORTED"}


class DgError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class Config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim",
                                         "n_experts", "top_k", "expert_ffn", "shared_ffn", "vocab",
                                         "canvas", "window", "global_every", "max_batch", "max_ctx")] + \
              [("rms_eps", C.c_float), ("rope_theta", C.c_float)]


class LayerWeights(C.Structure):
    _fields_ = [(k, C.c_void_p) for k in LAYER_KEYS]


class Weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p), ("layers", C.POINTER(LayerWeights)),
                ("embed_t", C.c_void_p), ("sc_gate_up", C.c_void_p), ("sc_down", C.c_void_p)]


class KV(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("len", C.c_int64 * MAX_BATCH)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with discrete_diffusion_block_amd.build")
        L = C.CDLL(LIB_PATH)
        vp, i32, f32, sz, u64 = C.c_void_p, C.c_int, C.c_float, C.c_size_t, C.c_uint64
        sig = {
            "dg_create": [C.POINTER(Config), C.POINTER(Weights), C.POINTER(vp)],
            "dg_destroy": [vp],
            "dg_workspace_size": [vp, i32, C.POINTER(sz)],
            "dg_kv_size": [C.POINTER(Config), C.POINTER(sz)],
            "dg_prefill_kv": [vp, C.POINTER(KV), vp, i32, i32, vp, sz, vp],
            "dg_denoise_step": [vp, C.POINTER(KV), vp, i32, f32, vp, vp, sz, vp],
            "dg_sample_workspace_size": [i32, i32, i32, C.POINTER(sz)],
            "dg_sample_eb": [vp, vp, i32, i32, i32, f32, i32, vp, vp, vp, vp, sz, vp],
            "dg_sample_eb_noalloc": [vp, vp, i32, i32, i32, f32, i32, vp, vp, vp, vp],
            "dg_generate_block": [vp, C.POINTER(KV), vp, i32, i32, f32, i32, vp, vp, vp, sz, vp],
            "dg_generate_blocks": [vp, C.POINTER(KV), vp, i32, i32, i32, f32, i32, vp, vp, vp, sz, vp],
            "dg_sample_eb_ex": [vp, vp, i32, i32, i32, f32, i32, f32, f32, vp, i32, vp, vp, vp, vp, vp, sz,
                                vp],
            "dg_generate_block_ex": [vp, C.POINTER(KV), vp, i32, i32, f32, f32, f32, f32, i32, vp, vp, vp,
                                     vp, sz, vp],
            "dg_uniform_canvas": [vp, i32, i32, i32, u64, i32, vp],
            "dg_sample_eb_uniform": [vp, vp, i32, i32, i32, f32, i32, f32, f32, vp, i32, vp, u64, i32, vp, vp,
                                     vp, vp, sz, vp],
            "dg_generate_block_uniform": [vp, C.POINTER(KV), vp, i32, i32, f32, f32, f32, f32, u64, i32, vp, vp,
                                          vp, vp, sz, vp],
            "dg_self_cond": [vp, vp, i32, vp, vp, vp, sz, vp],
            "dg_denoise_step_sc": [vp, C.POINTER(KV), vp, i32, f32, vp, vp, vp, sz, vp],
            "dg_generate_block_sc": [vp, C.POINTER(KV), vp, i32, i32, f32, f32, f32, f32, i32, u64, i32, vp, vp,
                                     vp, vp, sz, vp],
            "dg_mixed_step": [vp, C.POINTER(KV), vp, i32, vp, vp, vp, vp, sz, vp],
            "dg_sample_eb_seq": [vp, vp, i32, i32, i32, f32, vp, vp, vp, vp, vp, sz, vp],
            "dg_serve": [vp, C.POINTER(KV), vp, i32, i32, f32, i32, vp, vp, vp, vp, i32, vp, vp, sz, vp],
            "dg_packed_elems": [i32, i32, C.POINTER(sz)],
            "dg_pack_weight": [i32, vp, vp, i32, i32, i32, i32, vp],
            "dg_profile_begin": [vp, i32, C.c_uint32],
            "dg_profile_end": [vp, C.POINTER(C.c_double), C.POINTER(C.c_int32)],
            "dg_workspace_moe_counts": [vp, i32, C.POINTER(sz)],
            "dg_test_router_topk": [vp, i32, i32, i32, vp, vp, vp],
            "dg_test_force_routing": [vp, vp],
            "dg_test_sample_eb_profiled": [vp, vp, vp, i32, i32, i32, f32, i32, vp, vp, sz, vp],
            "dg_test_eb_select": [vp, vp, vp, i32, i32, i32, f32, i32, vp, vp],
            "dg_test_route": [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
            "dg_test_gemm": [vp, vp, vp, i32, i32, i32, vp],
            "dg_test_copy": [vp, vp, C.c_size_t, vp],
            "dg_test_mfma_rate": [i32, i32, vp, vp],
            "dg_test_read_rate": [vp, C.c_size_t, i32, vp, vp],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = None if name == "dg_destroy" else C.c_int
        L.dg_status_string.argtypes = [C.c_int]
        L.dg_status_string.restype = C.c_char_p
        L.dg_last_error.argtypes = []
        L.dg_last_error.restype = C.c_char_p
        L.dg_source_digest.argtypes = []
        L.dg_source_digest.restype = C.c_char_p
        built, here = L.dg_source_digest().decode(), source_digest()
        if built != here:
            raise RuntimeError(f"{LIB_PATH} was built from other sources (digest {built}, tree {here}): "
                               "rebuild it with discrete_diffusion_block_amd.build")
        _lib = L
    return _lib


def header_functions():
    """Names of every function declared in include/dg.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:dg_status|void|const char\*)\s+(dg_\w+)\s*\(", text, re.M)))


def _check(status: int):
    if status != 0:
        raise DgError(status, lib().dg_last_error().decode())


def _p(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def make_config(cfg: ModelConfig, max_batch: int = 1, max_ctx: int = 2048) -> Config:
    return Config(cfg.n_layers, cfg.d_model, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                  cfg.n_experts, cfg.top_k, cfg.expert_ffn, cfg.shared_ffn, cfg.vocab, cfg.canvas,
                  cfg.window, cfg.global_every, max_batch, max_ctx, cfg.rms_eps, cfg.rope_theta)


# ------------------------------------------------------------------ raw C-named wrappers


def dg_create(cfg: Config, weights: Weights):
    ctx = C.c_void_p()
    _check(lib().dg_create(C.byref(cfg), C.byref(weights), C.byref(ctx)))
    return ctx


def dg_destroy(ctx):
    lib().dg_destroy(ctx)


def dg_workspace_size(ctx, batch: int) -> int:
    n = C.c_size_t()
    _check(lib().dg_workspace_size(ctx, batch, C.byref(n)))
    return n.value


def dg_kv_size(cfg: Config) -> int:
    n = C.c_size_t()
    _check(lib().dg_kv_size(C.byref(cfg), C.byref(n)))
    return n.value


def dg_prefill_kv(ctx, kv: KV, tokens: torch.Tensor, ws: torch.Tensor, stream=None):
    b, n = tokens.shape
    _check(lib().dg_prefill_kv(ctx, C.byref(kv), _p(tokens), b, n, _p(ws), ws.numel(), _stream(stream)))


def dg_denoise_step(ctx, kv: KV, canvas: torch.Tensor, t: float, logits: torch.Tensor,
                    ws: torch.Tensor, stream=None):
    _check(lib().dg_denoise_step(ctx, C.byref(kv), _p(canvas), canvas.shape[0], float(t), _p(logits),
                                 _p(ws), ws.numel(), _stream(stream)))


def dg_sample_workspace_size(batch: int, canvas: int, vocab: int) -> int:
    n = C.c_size_t()
    _check(lib().dg_sample_workspace_size(batch, canvas, vocab, C.byref(n)))
    return n.value


def dg_sample_eb(logits: torch.Tensor, canvas: torch.Tensor, gamma: float, commit_all: bool,
                 n_masked: torch.Tensor, ws: torch.Tensor, entropy: Optional[torch.Tensor] = None,
                 argmax: Optional[torch.Tensor] = None, stream=None):
    b, c, v = logits.shape
    _check(lib().dg_sample_eb(_p(logits), _p(canvas), b, c, v, float(gamma), int(bool(commit_all)),
                              _p(entropy), _p(argmax), _p(n_masked), _p(ws), ws.numel(), _stream(stream)))


def dg_sample_eb_noalloc(logits: torch.Tensor, canvas: torch.Tensor, gamma: float, commit_all: bool,
                         n_masked: torch.Tensor, entropy: Optional[torch.Tensor] = None,
                         argmax: Optional[torch.Tensor] = None, stream=None):
    """dg_sample_eb with the library's static scratch in place of a workspace."""
    b, c, v = logits.shape
    _check(lib().dg_sample_eb_noalloc(_p(logits), _p(canvas), b, c, v, float(gamma), int(bool(commit_all)),
                                      _p(entropy), _p(argmax), _p(n_masked), _stream(stream)))


def dg_sample_eb_ex(logits: torch.Tensor, canvas: torch.Tensor, gamma: float, commit_all: bool,
                    temperature: float, e_stop: float, prev_argmax: Optional[torch.Tensor], step: int,
                    done_step: Optional[torch.Tensor], n_masked: torch.Tensor, ws: torch.Tensor,
                    entropy: Optional[torch.Tensor] = None, argmax: Optional[torch.Tensor] = None,
                    stream=None):
    b, c, v = logits.shape
    _check(lib().dg_sample_eb_ex(_p(logits), _p(canvas), b, c, v, float(gamma), int(bool(commit_all)),
                                 float(temperature), float(e_stop), _p(prev_argmax), int(step),
                                 _p(done_step), _p(entropy), _p(argmax), _p(n_masked), _p(ws), ws.numel(),
                                 _stream(stream)))


def dg_generate_block_ex(ctx, kv: KV, canvas: torch.Tensor, max_steps: int, gamma: float, tau_max: float,
                         tau_min: float, e_stop: float, append_kv: bool, logits: torch.Tensor,
                         n_masked: torch.Tensor, done_step: torch.Tensor, ws: torch.Tensor, stream=None):
    _check(lib().dg_generate_block_ex(ctx, C.byref(kv), _p(canvas), canvas.shape[0], max_steps, float(gamma),
                                      float(tau_max), float(tau_min), float(e_stop), int(bool(append_kv)),
                                      _p(logits), _p(n_masked), _p(done_step), _p(ws), ws.numel(),
                                      _stream(stream)))


def dg_uniform_canvas(canvas: torch.Tensor, vocab: int, seed: int, draw: int, stream=None):
    b, c = canvas.shape
    _check(lib().dg_uniform_canvas(_p(canvas), b, c, int(vocab), int(seed) & (2 ** 64 - 1), int(draw),
                                   _stream(stream)))


def dg_sample_eb_uniform(logits: torch.Tensor, canvas: torch.Tensor, gamma: float, commit_all: bool,
                         temperature: float, e_stop: float, prev_argmax: Optional[torch.Tensor], step: int,
                         done_step: Optional[torch.Tensor], seed: int, draw: int, n_open: torch.Tensor,
                         ws: torch.Tensor, entropy: Optional[torch.Tensor] = None,
                         argmax: Optional[torch.Tensor] = None, stream=None):
    b, c, v = logits.shape
    _check(lib().dg_sample_eb_uniform(_p(logits), _p(canvas), b, c, v, float(gamma), int(bool(commit_all)),
                                      float(temperature), float(e_stop), _p(prev_argmax), int(step),
                                      _p(done_step), int(seed) & (2 ** 64 - 1), int(draw), _p(entropy),
                                      _p(argmax), _p(n_open), _p(ws), ws.numel(), _stream(stream)))


def dg_generate_block_uniform(ctx, kv: KV, canvas: torch.Tensor, max_steps: int, gamma: float, tau_max: float,
                              tau_min: float, e_stop: float, seed: int, append_kv: bool, logits: torch.Tensor,
                              n_open: torch.Tensor, done_step: torch.Tensor, ws: torch.Tensor, stream=None):
    _check(lib().dg_generate_block_uniform(ctx, C.byref(kv), _p(canvas), canvas.shape[0], max_steps,
                                           float(gamma), float(tau_max), float(tau_min), float(e_stop),
                                           int(seed) & (2 ** 64 - 1), int(bool(append_kv)), _p(logits),
                                           _p(n_open), _p(done_step), _p(ws), ws.numel(), _stream(stream)))


def dg_self_cond(ctx, logits: torch.Tensor, z: torch.Tensor, ws: torch.Tensor, u: Optional[torch.Tensor] = None,
                 stream=None):
    _check(lib().dg_self_cond(ctx, _p(logits), logits.shape[0], _p(z), _p(u), _p(ws), ws.numel(), _stream(stream)))


def dg_denoise_step_sc(ctx, kv: KV, canvas: torch.Tensor, t: float, z: Optional[torch.Tensor], logits: torch.Tensor,
                       ws: torch.Tensor, stream=None):
    _check(lib().dg_denoise_step_sc(ctx, C.byref(kv), _p(canvas), canvas.shape[0], float(t), _p(z), _p(logits),
                                    _p(ws), ws.numel(), _stream(stream)))


def dg_generate_block_sc(ctx, kv: KV, canvas: torch.Tensor, max_steps: int, gamma: float, tau_max: float,
                         tau_min: float, e_stop: float, uniform: bool, seed: int, append_kv: bool,
                         logits: torch.Tensor, n: torch.Tensor, done_step: torch.Tensor, ws: torch.Tensor,
                         stream=None):
    _check(lib().dg_generate_block_sc(ctx, C.byref(kv), _p(canvas), canvas.shape[0], max_steps, float(gamma),
                                      float(tau_max), float(tau_min), float(e_stop), int(bool(uniform)),
                                      int(seed) & (2 ** 64 - 1), int(bool(append_kv)), _p(logits), _p(n),
                                      _p(done_step), _p(ws), ws.numel(), _stream(stream)))


def _i32_array(values):
    vals = [int(v) for v in values]
    return (C.c_int32 * len(vals))(*vals)


def dg_mixed_step(ctx, kv: KV, tokens: torch.Tensor, encode, t, logits: Optional[torch.Tensor], ws: torch.Tensor,
                  stream=None):
    b = tokens.shape[0]
    enc = _i32_array(encode)
    tt = (C.c_float * b)(*[float(x) for x in t])
    _check(lib().dg_mixed_step(ctx, C.byref(kv), _p(tokens), b, enc, tt, _p(logits), _p(ws), ws.numel(),
                               _stream(stream)))


def dg_sample_eb_seq(logits: torch.Tensor, canvas: torch.Tensor, gamma: float, commit_all, n_masked: torch.Tensor,
                     ws: torch.Tensor, entropy: Optional[torch.Tensor] = None, argmax: Optional[torch.Tensor] = None,
                     stream=None):
    b, c, v = logits.shape
    _check(lib().dg_sample_eb_seq(_p(logits), _p(canvas), b, c, v, float(gamma), _i32_array(commit_all), _p(entropy),
                                  _p(argmax), _p(n_masked), _p(ws), ws.numel(), _stream(stream)))


def dg_serve(ctx, kv: KV, canvas: torch.Tensor, steps: int, gamma: float, n_passes: int, phase: list,
             logits: torch.Tensor, n_masked: torch.Tensor, ws: torch.Tensor, out: Optional[torch.Tensor] = None,
             out_count: Optional[list] = None, stream=None):
    """phase (and out_count, with out [batch][out_blocks][C]) are lists updated in place."""
    b = canvas.shape[0]
    ph = _i32_array(phase)
    cnt = _i32_array(out_count) if out_count is not None else None
    _check(lib().dg_serve(ctx, C.byref(kv), _p(canvas), b, steps, float(gamma), n_passes, ph, _p(logits),
                          _p(n_masked), _p(out), out.shape[1] if out is not None else 0, cnt, _p(ws), ws.numel(),
                          _stream(stream)))
    phase[:] = list(ph)
    if out_count is not None:
        out_count[:] = list(cnt)


def dg_generate_block(ctx, kv: KV, canvas: torch.Tensor, steps: int, gamma: float, append_kv: bool,
                      logits: torch.Tensor, n_masked: torch.Tensor, ws: torch.Tensor, stream=None):
    _check(lib().dg_generate_block(ctx, C.byref(kv), _p(canvas), canvas.shape[0], steps, float(gamma),
                                   int(bool(append_kv)), _p(logits), _p(n_masked), _p(ws), ws.numel(),
                                   _stream(stream)))


def dg_generate_blocks(ctx, kv: KV, canvas: torch.Tensor, steps: int, gamma: float, append_last: bool,
                       logits: torch.Tensor, n_masked: torch.Tensor, ws: torch.Tensor, stream=None):
    """canvas: int32 [n_blocks][batch][C] (out)."""
    _check(lib().dg_generate_blocks(ctx, C.byref(kv), _p(canvas), canvas.shape[1], canvas.shape[0], steps,
                                    float(gamma), int(bool(append_last)), _p(logits), _p(n_masked), _p(ws),
                                    ws.numel(), _stream(stream)))


def dg_packed_elems(rows: int, cols: int) -> int:
    n = C.c_size_t()
    _check(lib().dg_packed_elems(rows, cols, C.byref(n)))
    return n.value


def dg_pack_weight(kind: int, src: torch.Tensor, dst: torch.Tensor, n_mats: int, rows: int, cols: int,
                   param: int = 0, stream=None):
    _check(lib().dg_pack_weight(kind, _p(src), _p(dst), n_mats, rows, cols, param, _stream(stream)))


def pack(t: torch.Tensor, kind: int = PACK_PLAIN, param: int = 0) -> torch.Tensor:
    """Fragment-major copy of the bf16 matrices in t (shape [..., rows, cols]); with
    PACK_TRANSPOSE, of the transpose of the single matrix t."""
    rows, cols = t.shape[-2], t.shape[-1]
    n_mats = t.numel() // (rows * cols)
    elems = dg_packed_elems(cols, rows) if kind == PACK_TRANSPOSE else n_mats * dg_packed_elems(rows, cols)
    dst = torch.empty(elems, dtype=torch.bfloat16, device=t.device)
    dg_pack_weight(kind, t.contiguous(), dst, n_mats, rows, cols, param)
    return dst


def pack_layer(cfg: ModelConfig, lw: dict) -> dict:
    """Engine-layout copy of one layer of synth.make_weights output (device tensors)."""
    return {
        "attn_norm": lw["attn_norm"], "ffn_norm": lw["ffn_norm"],
        "w_qkv": pack(lw["w_qkv"], PACK_QKV, cfg.head_dim),
        "w_o": pack(lw["w_o"]),
        "w_router": pack(lw["w_router"]),
        "w_gate_up": pack(lw["w_gate_up"], PACK_GATE_UP, cfg.expert_ffn),
        "w_down": pack(lw["w_down"]),
        "ws_gate_up": pack(lw["ws_gate_up"], PACK_GATE_UP, cfg.shared_ffn),
        "ws_down": pack(lw["ws_down"]),
    }


def pack_selfcond(cfg: ModelConfig, embed: torch.Tensor, sc: dict) -> dict:
    """Engine-layout self-conditioning weights: the transposed embedding rows 0..V-1 and
    the FFW of synth.make_selfcond_weights (device tensors)."""
    return {"embed_t": pack(embed[:cfg.vocab], PACK_TRANSPOSE),
            "sc_gate_up": pack(sc["sc_gate_up"], PACK_GATE_UP, cfg.shared_ffn),
            "sc_down": pack(sc["sc_down"])}


def pack_weights(cfg: ModelConfig, w: dict, free_source: bool = False, selfcond: Optional[dict] = None) -> dict:
    """Engine-layout copy of synth.make_weights output (device tensors); with selfcond
    (synth.make_selfcond_weights output), also the self-conditioning weights."""
    out = {"embed": pack(w["embed"]), "final_norm": w["final_norm"], "layers": []}
    if selfcond is not None:
        out["selfcond"] = pack_selfcond(cfg, w["embed"], selfcond)
    if free_source:
        w["embed"] = None
    for l, lw in enumerate(w["layers"]):
        out["layers"].append(pack_layer(cfg, lw))
        if free_source:
            w["layers"][l] = None
    return out


def _k_index(p: torch.Tensor, c: torch.Tensor, hd: int) -> torch.Tensor:
    pp = p & 31
    bb = (pp >> 2) & 1
    r = ((pp >> 3) << 2) | (pp & 3)
    return ((((p >> 5) * 2 + bb) * (hd >> 5) + (c >> 5)) << 9) + (((((c & 31) >> 3) << 4) + r) << 3) + (c & 7)


def _v_index(p: torch.Tensor, c: torch.Tensor, hd: int) -> torch.Tensor:
    return ((((p >> 5) * (hd >> 4)) + (c >> 4)) << 9) + (((((p & 31) >> 3) << 4) + (c & 15)) << 3) + (p & 7)


def dg_profile_begin(ctx, capacity: int, kinds=None):
    """kinds: iterable of names from KERNEL_KINDS to time (None: every kind)."""
    mask = 0 if kinds is None else sum(1 << KERNEL_KINDS.index(k) for k in kinds)
    _check(lib().dg_profile_begin(ctx, capacity, mask))


def dg_profile_end(ctx):
    """{kind: (total_ms, launches)} for the launches bracketed since dg_profile_begin."""
    n = len(KERNEL_KINDS)
    ms = (C.c_double * n)()
    cnt = (C.c_int32 * n)()
    _check(lib().dg_profile_end(ctx, ms, cnt))
    return {KERNEL_KINDS[i]: (ms[i], cnt[i]) for i in range(n)}


def dg_workspace_moe_counts(ctx, batch: int) -> int:
    off = C.c_size_t()
    _check(lib().dg_workspace_moe_counts(ctx, batch, C.byref(off)))
    return off.value


def dg_test_force_routing(ctx, ids: Optional[torch.Tensor]):
    """ids: int32 device tensor [n_layers][M][top_k] (the expert ids each layer of the
    following passes uses), or None to restore the router."""
    _check(lib().dg_test_force_routing(ctx, _p(ids)))


def dg_test_sample_eb_profiled(ctx, logits: torch.Tensor, canvas: torch.Tensor, gamma: float,
                               commit_all: bool, n_masked: torch.Tensor, ws: torch.Tensor, stream=None):
    """dg_sample_eb with its launches timed by ctx's profiler."""
    b, c, v = logits.shape
    _check(lib().dg_test_sample_eb_profiled(ctx, _p(logits), _p(canvas), b, c, v, float(gamma),
                                            int(bool(commit_all)), _p(n_masked), _p(ws), ws.numel(),
                                            _stream(stream)))


def dg_test_router_topk(r: torch.Tensor, k: int, ids: torch.Tensor, w: torch.Tensor, stream=None):
    M, E = r.shape
    _check(lib().dg_test_router_topk(_p(r), M, E, k, _p(ids), _p(w), _stream(stream)))


def dg_test_route(r: torch.Tensor, k: int, stream=None) -> dict:
    """Runs the routing kernels on router logits r [M][E]; returns their outputs."""
    M, E = r.shape
    A = M * k
    dev = r.device
    out = {"ids": torch.empty(M, k, dtype=torch.int32, device=dev),
           "w": torch.empty(M, k, device=dev),
           "cnt": torch.empty(E, dtype=torch.int32, device=dev),
           "poff": torch.empty(E + 1, dtype=torch.int32, device=dev),
           "perm": torch.empty(A + 15 * E, dtype=torch.int32, device=dev),
           "inv": torch.empty(A, dtype=torch.int32, device=dev),
           "items": torch.empty((A + 31) // 32 + E, 2, dtype=torch.int32, device=dev),
           "n_items": torch.empty(1, dtype=torch.int32, device=dev),
           "items2": torch.empty((A + 127) // 128 + E, 2, dtype=torch.int32, device=dev),
           "n_items2": torch.empty(1, dtype=torch.int32, device=dev)}
    _check(lib().dg_test_route(_p(r), M, E, k, _p(out["ids"]), _p(out["w"]), _p(out["cnt"]),
                               _p(out["poff"]), _p(out["perm"]), _p(out["inv"]), _p(out["items"]),
                               _p(out["n_items"]), _p(out["items2"]), _p(out["n_items2"]), _stream(stream)))
    return out


def dg_test_eb_select(entropy: torch.Tensor, argmax: torch.Tensor, canvas: torch.Tensor, vocab: int,
                      gamma: float, commit_all: bool, n_masked: torch.Tensor, stream=None):
    b, c = canvas.shape
    _check(lib().dg_test_eb_select(_p(entropy), _p(argmax), _p(canvas), b, c, vocab, float(gamma),
                                   int(bool(commit_all)), _p(n_masked), _stream(stream)))


def dg_test_copy(src: torch.Tensor, dst: torch.Tensor, n_bytes: int, stream=None) -> None:
    """Plain 16-byte-vector device copy (hardware byte-counter calibration)."""
    _check(lib().dg_test_copy(_p(src), _p(dst), n_bytes, _stream(stream)))


def dg_test_mfma_rate(blocks: int, iters: int, out: torch.Tensor, stream=None) -> None:
    """Register-only bf16 MFMA chains (achievable matrix-core rate); out: float32 [blocks * 256]."""
    assert out.dtype == torch.float32 and out.numel() >= blocks * 256 and out.is_cuda
    _check(lib().dg_test_mfma_rate(blocks, iters, _p(out), _stream(stream)))


def dg_test_read_rate(src: torch.Tensor, n_bytes: int, blocks: int, out: torch.Tensor, stream=None) -> None:
    """Streaming read of src (achievable HBM read rate); out: int32 [blocks * 256] (XOR words)."""
    assert src.is_cuda and src.numel() * src.element_size() >= n_bytes
    assert out.is_cuda and out.element_size() == 4 and out.numel() >= blocks * 256
    _check(lib().dg_test_read_rate(_p(src), n_bytes, blocks, _p(out), _stream(stream)))


def dg_test_gemm(x_packed: torch.Tensor, w_packed: torch.Tensor, y: torch.Tensor, M: int, N: int,
                 K: int, stream=None):
    _check(lib().dg_test_gemm(_p(x_packed), _p(w_packed), _p(y), M, N, K, _stream(stream)))


# ------------------------------------------------------------------ convenience engine


class Engine:
    """Owns the ctx, the KV cache and the workspace for one model on one GPU.

    `weights` is the dict produced by synth.make_weights on a CUDA device; the
    engine keeps a reference so the borrowed device pointers stay valid.
    """

    def __init__(self, cfg: ModelConfig, weights: dict, max_batch: int = 1, max_ctx: int = 2048,
                 device: str = "cuda", packed: bool = False, free_source: bool = False,
                 selfcond: Optional[dict] = None):
        """selfcond: self-conditioning weights (synth.make_selfcond_weights) for unpacked
        `weights`; packed weights carry them packed under "selfcond" (pack_weights)."""
        self.cfg = cfg
        self.weights = weights if packed else pack_weights(cfg, weights, free_source, selfcond)
        weights = self.weights
        self.ccfg = make_config(cfg, max_batch, max_ctx)
        n = cfg.n_layers
        self._layers = (LayerWeights * n)()
        for l in range(n):
            lw = weights["layers"][l]
            for key in LAYER_KEYS:
                setattr(self._layers[l], key, lw[key].data_ptr())
        sc = weights.get("selfcond")
        self._w = Weights(weights["embed"].data_ptr(), weights["final_norm"].data_ptr(),
                          C.cast(self._layers, C.POINTER(LayerWeights)),
                          sc["embed_t"].data_ptr() if sc else None, sc["sc_gate_up"].data_ptr() if sc else None,
                          sc["sc_down"].data_ptr() if sc else None)
        self.ctx = dg_create(self.ccfg, self._w)
        kv_bytes = dg_kv_size(self.ccfg)
        self.k_cache = torch.zeros(kv_bytes // 2, dtype=torch.int16, device=device)
        self.v_cache = torch.zeros(kv_bytes // 2, dtype=torch.int16, device=device)
        self.kv = KV(self.k_cache.data_ptr(), self.v_cache.data_ptr())
        self.max_batch = max_batch
        self.ws = torch.empty(dg_workspace_size(self.ctx, max_batch), dtype=torch.uint8, device=device)

    def close(self):
        if self.ctx is not None:
            dg_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def lengths(self):
        return [int(self.kv.len[b]) for b in range(self.max_batch)]

    def reset(self):
        for b in range(MAX_BATCH):
            self.kv.len[b] = 0

    def kv_view(self):
        """(k, v) decoded from the cache layout to bf16 [L][B][Hkv][max_ctx][hd] each."""
        c = self.cfg
        T, hd = self.ccfg.max_ctx, c.head_dim
        p = torch.arange(T, device=self.k_cache.device).view(T, 1)
        d = torch.arange(hd, device=self.k_cache.device).view(1, hd)
        blocks = (c.n_layers, self.max_batch, c.n_kv_heads, T * hd)
        k = self.k_cache.view(torch.bfloat16).view(blocks)[..., _k_index(p, d, hd).reshape(-1)]
        v = self.v_cache.view(torch.bfloat16).view(blocks)[..., _v_index(p, d, hd).reshape(-1)]
        shp = (c.n_layers, self.max_batch, c.n_kv_heads, T, hd)
        return k.view(shp), v.view(shp)

    def prefill_kv(self, tokens: torch.Tensor, stream=None):
        dg_prefill_kv(self.ctx, self.kv, tokens, self.ws, stream)

    def denoise_step(self, canvas: torch.Tensor, t: float, logits: torch.Tensor, stream=None):
        dg_denoise_step(self.ctx, self.kv, canvas, t, logits, self.ws, stream)

    def sample_eb(self, logits, canvas, gamma, commit_all, n_masked, entropy=None, argmax=None,
                  stream=None):
        dg_sample_eb(logits, canvas, gamma, commit_all, n_masked, self.ws, entropy, argmax, stream)

    def sample_eb_ex(self, logits, canvas, gamma, commit_all, temperature, e_stop, prev_argmax, step,
                     done_step, n_masked, entropy=None, argmax=None, stream=None):
        dg_sample_eb_ex(logits, canvas, gamma, commit_all, temperature, e_stop, prev_argmax, step, done_step,
                        n_masked, self.ws, entropy, argmax, stream)

    def moe_counts(self):
        """Per-layer per-expert token counts of the latest pass (int32 [L][E], device)."""
        off = dg_workspace_moe_counts(self.ctx, self.max_batch)
        n = self.cfg.n_layers * self.cfg.n_experts
        return self.ws[off:off + 4 * n].view(torch.int32).view(self.cfg.n_layers, self.cfg.n_experts)

    def generate_blocks(self, canvas, steps, gamma, append_last, logits, n_masked, stream=None):
        dg_generate_blocks(self.ctx, self.kv, canvas, steps, gamma, append_last, logits, n_masked, self.ws, stream)

    def generate_block(self, canvas, steps, gamma, append_kv, logits, n_masked, stream=None):
        dg_generate_block(self.ctx, self.kv, canvas, steps, gamma, append_kv, logits, n_masked,
                          self.ws, stream)

    def generate_block_ex(self, canvas, max_steps, gamma, tau_max, tau_min, e_stop, append_kv, logits,
                          n_masked, done_step, stream=None):
        dg_generate_block_ex(self.ctx, self.kv, canvas, max_steps, gamma, tau_max, tau_min, e_stop,
                             append_kv, logits, n_masked, done_step, self.ws, stream)

    def sample_eb_uniform(self, logits, canvas, gamma, commit_all, temperature, e_stop, prev_argmax, step,
                          done_step, seed, draw, n_open, entropy=None, argmax=None, stream=None):
        dg_sample_eb_uniform(logits, canvas, gamma, commit_all, temperature, e_stop, prev_argmax, step, done_step,
                             seed, draw, n_open, self.ws, entropy, argmax, stream)

    def mixed_step(self, tokens, encode, t, logits, stream=None):
        dg_mixed_step(self.ctx, self.kv, tokens, encode, t, logits, self.ws, stream)

    def sample_eb_seq(self, logits, canvas, gamma, commit_all, n_masked, entropy=None, argmax=None, stream=None):
        dg_sample_eb_seq(logits, canvas, gamma, commit_all, n_masked, self.ws, entropy, argmax, stream)

    def serve(self, canvas, steps, gamma, n_passes, phase, logits, n_masked, out=None, out_count=None, stream=None):
        dg_serve(self.ctx, self.kv, canvas, steps, gamma, n_passes, phase, logits, n_masked, self.ws, out, out_count,
                 stream)

    def self_cond(self, logits, z, u=None, stream=None):
        dg_self_cond(self.ctx, logits, z, self.ws, u, stream)

    def denoise_step_sc(self, canvas, t, z, logits, stream=None):
        dg_denoise_step_sc(self.ctx, self.kv, canvas, t, z, logits, self.ws, stream)

    def generate_block_sc(self, canvas, max_steps, gamma, tau_max, tau_min, e_stop, uniform, seed, append_kv, logits,
                          n, done_step, stream=None):
        dg_generate_block_sc(self.ctx, self.kv, canvas, max_steps, gamma, tau_max, tau_min, e_stop, uniform, seed,
                             append_kv, logits, n, done_step, self.ws, stream)

    def generate_block_uniform(self, canvas, max_steps, gamma, tau_max, tau_min, e_stop, seed, append_kv,
                               logits, n_open, done_step, stream=None):
        dg_generate_block_uniform(self.ctx, self.kv, canvas, max_steps, gamma, tau_max, tau_min, e_stop, seed,
                                  append_kv, logits, n_open, done_step, self.ws, stream)
