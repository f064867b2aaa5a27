"""Benchmark: block-parallel diffusion decoding on one MI355X.

One bench step = one 256-token block on the full 30-layer model (d 2816,
16q/8kv heads of 128, 128 experts top-8 + shared, vocab 262144, canvas 256): 12
denoising steps with entropy-bounded unmasking (gamma 2.0) and the causal append
of the finished canvas to the KV cache.  The timed steps are consecutive blocks
of one dg_generate_blocks call (each append shares a pass with the next block's
first denoising step); the same blocks as one dg_generate_block call each are
timed beside them.  The 1024-token random prompt is prefilled once before timing
(the pages exclude prefill from latency).  Weights are random-init N(0, 0.02)
bf16 and inputs are synthetic.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the translation unit of each counted kernel kind (its launcher included) and the
# headers every kernel source includes
KIND_SOURCES = {"moe_gate_up": "k_moe.hip", "moe_down": "k_moe.hip", "head": "k_gemm.hip",
                "sample_pass1": "k_sampler.hip", "attention": "k_attention.hip"}


def kernel_source_digest(kind: str = "moe_gate_up") -> str:
    """Digest of the sources that define one kernel kind: a traffic measurement stays
    valid while they are unchanged (host-side runtime changes do not touch it)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "discrete_diffusion_block_amd", "csrc")
    for f in ("dg_common.h", "dg_internal.h", KIND_SOURCES[kind]):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def algorithmic_work(kind, cfg, M, counts_per_layer):
    """(bound, unit, amount per launch) for a kernel kind at M canvas rows.

    MoE kinds use the per-layer expert token counts of the latest denoising pass:
    every expert with at least one token streams its weights once; every
    assignment reads its activation row and writes its output row."""
    d, F, Fs, E, V = cfg.d_model, cfg.expert_ffn, cfg.shared_ffn, cfg.n_experts, cfg.vocab
    hq, hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    if kind in ("moe_gate_up", "moe_down"):
        if counts_per_layer is None:
            return "hbm", "GB/s", None
        per = []
        for cnt in counts_per_layer:
            used = sum(1 for c in cnt if c > 0)
            A = sum(cnt)
            if kind == "moe_gate_up":
                per.append(used * 2 * F * d * 2 + A * d * 2 + A * F * 2)
            else:
                per.append(used * d * F * 2 + A * F * 2 + A * d * 4)
        return "hbm", "GB/s", sum(per) / len(per)
    if kind == "head":
        return "hbm", "GB/s", V * d * 2 + M * d * 2 + M * V * 2
    if kind == "qkv":
        R = (hq + 2 * hkv) * hd
        return "mfma", "TFLOP/s", 2.0 * M * R * d
    if kind == "o_proj":
        return "mfma", "TFLOP/s", 2.0 * M * d * hq * hd
    if kind == "shared_gate_up":
        return "mfma", "TFLOP/s", 2.0 * M * 2 * Fs * d
    if kind == "shared_down":
        return "mfma", "TFLOP/s", 2.0 * M * d * Fs
    if kind == "attention":
        keys = cfg.window + cfg.canvas
        return "mfma", "TFLOP/s", 4.0 * M * hq * keys * hd
    if kind == "attention_global":
        return "mfma", "TFLOP/s", None     # depends on the prefix length: computed by the caller
    if kind == "sample_pass1":
        return "hbm", "GB/s", M * V * 2
    return None, None, None


def cpu_baseline(budget_note: str):
    """The oracle, as it stands, on a bounded sample of the same workload.

    Sample: one full-shape MoE layer (d 2816, 128 experts) plus the 262144-row
    tied head, on a 256-token canvas over a 1024-token prefix.  Timed: one
    denoising step of that 1-layer model (layer + head), the same step with the
    head cut to 8 rows (layer alone), and one sampler call.  Extrapolated to the
    benchmark unit (tokens/s of 256-token blocks, 12 steps + append, 30 layers):
    block = 12 * (30 * t_layer + t_head + t_sample) + 30 * t_layer."""
    import dataclasses
    import numpy as np
    import torch
    from discrete_diffusion_block_amd import synth
    from oracle import dg_oracle as O

    cfg = dataclasses.replace(synth.CONFIGS["full"], n_layers=1)
    w = O.to_numpy_weights(synth.make_weights(cfg, device="cpu"))
    prompt = synth.make_prompt(cfg, 1, 1024).numpy()
    kv = O.KVCache(cfg, 1)
    t0 = time.perf_counter()
    O.prefill_kv(cfg, w, kv, prompt)
    t_prefill = time.perf_counter() - t0
    canvas = np.full((1, cfg.canvas), cfg.mask_id)
    t0 = time.perf_counter()
    logits = O.denoise_step(cfg, w, kv, canvas, 1.0)
    t_a = time.perf_counter() - t0
    cfg8 = dataclasses.replace(cfg, vocab=8)
    w8 = dict(w)
    w8["embed"] = np.concatenate([w["embed"][:8], w["embed"][cfg.vocab:cfg.vocab + 1]])
    t0 = time.perf_counter()
    O.denoise_step(cfg8, w8, kv, np.full((1, cfg.canvas), 8), 1.0)
    t_layer = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.sample_eb(O.bf16(logits), canvas, 2.0, False, cfg.mask_id)
    t_sample = time.perf_counter() - t0
    t_head = max(t_a - t_layer, 0.0)
    L = synth.CONFIGS["full"].n_layers
    block = 12 * (L * t_layer + t_head + t_sample) + L * t_layer
    cores = len(os.sched_getaffinity(0))
    # the same sample on one core (BLAS and OpenMP pools limited to one thread)
    one_core = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            O.denoise_step(cfg8, w8, kv, np.full((1, cfg.canvas), 8), 1.0)
            t_layer1 = time.perf_counter() - t0
            t0 = time.perf_counter()
            O.denoise_step(cfg, w, kv, canvas, 1.0)
            t_a1 = time.perf_counter() - t0
        block1 = 12 * (L * t_layer1 + max(t_a1 - t_layer1, 0.0) + t_sample) + L * t_layer1
        one_core = {"value": 256.0 / block1, "cores": 1,
                    "sample": f"layer alone {t_layer1:.2f}s, layer + head {t_a1:.2f}s on one core, same extrapolation"}
    except Exception as exc:  # threadpoolctl missing or a pool it cannot limit
        one_core = {"error": repr(exc)}
    return {
        "value": 256.0 / block,
        "unit": "tok/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"numpy float64 oracle: one full-shape MoE layer + 262144-row head denoising step "
                   f"{t_a:.2f}s, layer alone {t_layer:.2f}s, sampler {t_sample:.2f}s (prefix prefill "
                   f"{t_prefill:.1f}s untimed); extrapolated to 30 layers x (12 steps + append) per "
                   f"256-token block; {budget_note}"),
        "block_s_extrapolated": block,
        "one_core": one_core,
    }


def moe_bytes(kind, cfg, counts):
    """Algorithmic bytes of one launch of an expert GEMM kind, from one layer's expert
    token counts (see algorithmic_work)."""
    return algorithmic_work(kind, cfg, cfg.canvas, [counts])[2]


def pmc_workload(n_steps: int = 2, counts_out: str = None) -> None:
    """Workload for hardware-counter passes (rocprofv3 --pmc): first the library's
    plain 256 MiB copy kernel (a known byte count that calibrates the traffic
    counters), then n_steps denoising steps of the full model over a 1024-token
    prefix.  Nothing is timed.  counts_out: a JSON file that receives this run's own
    per-layer expert token counts of every denoising pass and the gate/up and down
    GEMMs' algorithmic bytes per launch they imply."""
    import torch
    from discrete_diffusion_block_amd import dg, synth

    cfg = synth.CONFIGS["full"]
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dg.dg_test_copy(src, dst, src.numel())      # dg::copy16_kernel: reads and writes 256 MiB
    torch.cuda.synchronize()
    del src, dst
    w = synth.make_weights(cfg, device="cuda")
    eng = dg.Engine(cfg, w, max_batch=1, max_ctx=1024 + cfg.canvas, free_source=True)
    eng.prefill_kv(synth.make_prompt(cfg, 1, 1024, device="cuda"))
    logits = torch.empty(1, cfg.canvas, cfg.vocab, dtype=torch.bfloat16, device="cuda")
    canvas = torch.full((1, cfg.canvas), cfg.vocab, dtype=torch.int32, device="cuda")
    passes = []
    for s in range(n_steps):
        eng.denoise_step(canvas, 1.0 - s / n_steps, logits)
        passes.append(eng.moe_counts().cpu().tolist())
    torch.cuda.synchronize()
    flat = [c for p in passes for c in p]
    rec = {"workload": "python3 bench.py --pmc-workload: 2 denoising steps of the 30-layer model, 1024-token prefix",
           "experts_used_per_layer_mean": sum(sum(1 for x in c if x) for c in flat) / len(flat),
           "moe_gate_up_bytes_per_launch": sum(moe_bytes("moe_gate_up", cfg, c) for c in flat) / len(flat),
           "moe_down_bytes_per_launch": sum(moe_bytes("moe_down", cfg, c) for c in flat) / len(flat),
           "counts": passes}
    if counts_out:
        with open(counts_out, "w") as fh:
            json.dump(rec, fh)
    log(f"pmc workload done ({n_steps} denoising steps, {rec['experts_used_per_layer_mean']:.1f} experts/layer)")


def summarize_pmc(root: str) -> str:
    """Per-kernel mean of every counter in the rocprofv3 counter CSVs under root,
    over the denoising passes of the counter workload only: dispatches from the
    third embedding kernel on (the 1024-token prefill runs as two 512-token passes
    before it)."""
    import csv
    import glob
    import collections
    rows = []
    for f in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    embeds = sorted({int(r["Dispatch_Id"]) for r in rows if "embed_norm_kernel" in r["Kernel_Name"]})
    start = embeds[2] if len(embeds) > 2 else 0
    agg = collections.defaultdict(list)
    for r in rows:
        if int(r["Dispatch_Id"]) >= start or "copy16_kernel" in r["Kernel_Name"]:
            agg[(r["Kernel_Name"].split("(")[0][:60], r["Counter_Name"])].append(float(r["Counter_Value"]))
    lines = [f"{k:62s} {c:14s} dispatches {len(v):5d} mean {sum(v) / len(v):14.1f}"
             for (k, c), v in sorted(agg.items())]
    return "\n".join(lines)


def summarize_trace(root: str, warmup: int, steps: int, denoise_steps: int, prompt: int,
                    bench_json: str = None) -> str:
    """Per-kernel launch statistics from the rocprofv3 kernel-trace CSV under root of a
    `bench.py --steps S --warmup W` run: the denoising passes of the S timed blocks.
    Passes start at the engine's prep kernel.  The run's passes, in order: the prompt
    prefill (ceil(prompt / 512) passes); W warm-up blocks of denoise_steps denoising
    passes (the ones that end in the vocabulary head) and one append pass each; a
    2-block dg_generate_blocks call (2 * denoise_steps passes, the first block's append
    inside the second block's first pass, then the last append); the timed S-block
    call (S * denoise_steps passes + one append); S blocks as one call each; the
    profiled block; then the roofline passes.  bench_json: that same
    run's JSON line, whose roofline figure (the dominant kind's algorithmic bytes per
    launch over the run's last denoise_steps passes, from their own expert counts) is
    divided by the trace's average duration of the same launches."""
    import csv
    import glob
    import collections
    rows = []
    for f in glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            rows.extend(r for r in csv.DictReader(fh) if r["Kernel_Name"].startswith(("dg::", "void dg::")))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    starts = [i for i, r in enumerate(rows) if "prep_kernel" in r["Kernel_Name"]] + [len(rows)]
    passes = [rows[a:b] for a, b in zip(starts[:-1], starts[1:])]
    per_block = denoise_steps + 1
    first = -(-prompt // 512) + warmup * per_block + (2 * denoise_steps + 1)
    timed = passes[first:first + steps * denoise_steps + 1]
    denoise = [p for p in timed if any("head_gemm" in r["Kernel_Name"] for r in p)]
    agg = collections.defaultdict(list)
    for p in denoise:
        for r in p:
            name = r["Kernel_Name"].replace("void ", "").split("(")[0]
            agg[name].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    span = sum((int(p[-1]["End_Timestamp"]) - int(p[0]["Start_Timestamp"])) / 1e3 for p in denoise)
    total = sum(sum(v) for v in agg.values())
    lines = [f"denoising passes of the timed blocks: {len(denoise)} (of {len(timed)} passes in "
             f"{steps} blocks); mean pass span {span / max(1, len(denoise)) / 1e3:.3f} ms",
             f"{'kernel':58s} {'calls':>6s} {'total ms':>9s} {'avg us':>8s} {'min us':>8s} "
             f"{'max us':>8s} {'share':>6s}"]
    for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{k[:58]:58s} {len(v):6d} {sum(v) / 1e3:9.2f} {sum(v) / len(v):8.2f} "
                     f"{min(v):8.2f} {max(v):8.2f} {100 * sum(v) / total:5.1f}%")
    # the run's last denoise_steps denoising passes of the 30-layer model are the ones in
    # which bench.py times the dominant kind with HIP events (the roofline figure of its
    # JSON line); they precede the sampler and the secondary workloads' passes
    heads = [p for p in passes if sum("head_gemm" in r["Kernel_Name"] for r in p) == 1 and len(p) > 300]
    roof = heads[(warmup + 2 + 2 * steps + 1) * denoise_steps:][:denoise_steps]
    ragg = collections.defaultdict(list)
    for p in roof:
        for r in p:
            name = r["Kernel_Name"].replace("void ", "").split("(")[0]
            ragg[name].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines.append("")
    lines.append(f"roofline passes ({len(roof)} denoising passes after the profiled block, in which bench.py "
                 f"times the dominant kind with HIP events on its launches):")
    for k, v in sorted(ragg.items(), key=lambda kv: -sum(kv[1]))[:8]:
        lines.append(f"{k[:58]:58s} {len(v):6d} launches, avg {sum(v) / len(v):8.2f} us")
    if bench_json:
        js = json.loads(open(bench_json).read().strip().splitlines()[-1])
        rf = js["roofline"]
        name = f"dg::{rf['kernel']}_kernel"
        v = ragg.get(name)
        if v:
            avg = sum(v) / len(v)
            ach = rf["algorithmic_per_launch"] / (avg * 1e-6) / 1e9
            lines.append(f"{name}: this run's algorithmic {rf['algorithmic_per_launch'] / 1e6:.1f} MB per launch "
                         f"(its own expert counts, {js.get('experts_used_per_layer_mean')} experts/layer) / trace "
                         f"average {avg:.2f} us = {ach:.0f} GB/s = {ach / HBM_PEAK_GBS:.3f} of HBM peak; the "
                         f"HIP-event average of the same launches {rf['avg_launch_ms'] * 1e3:.2f} us -> frac "
                         f"{rf['frac']}")
    return "\n".join(lines)


def write_traffic(fetch_txt: str, write_txt: str, kind: str, counts_json: str) -> dict:
    """Calibrated HBM bytes per launch of one kernel kind from the two counter summaries
    (FETCH_SIZE and WRITE_SIZE passes of --pmc-workload, printed by --summarize-pmc), set
    against that workload's own algorithmic bytes (its counts file).  Each counter is
    scaled by the ratio of the copy kernel's true byte count (256 MiB read, 256 MiB
    written) to what the same counter reads for it."""
    def means(path):
        out = {}
        for line in open(path):
            parts = line.split()
            if len(parts) >= 6:
                out[parts[0]] = float(parts[-1])
        return out
    fe, wr = means(fetch_txt), means(write_txt)
    cj = json.load(open(counts_json))
    copy_kib = float(256 << 10)
    fs, ws = copy_kib / fe["dg::copy16_kernel"], copy_kib / wr["dg::copy16_kernel"]
    name = f"dg::{kind}_kernel"
    hw = int(round((fe[name] * fs + wr[name] * ws) * 1024))
    alg = cj.get(f"{kind}_bytes_per_launch")
    t = {"kernel": kind, "source_digest": kernel_source_digest(kind),
         "bytes_per_launch": hw,
         "algorithmic_bytes_per_launch": alg,
         "traffic_over_algorithmic": round(hw / alg, 3) if alg else None,
         "experts_used_per_layer_mean": cj.get("experts_used_per_layer_mean"),
         "fetch_kib_per_launch_raw": fe[name], "write_kib_per_launch_raw": wr[name],
         "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
         "calibration": f"dg::copy16_kernel copying 256 MiB reads FETCH_SIZE {fe['dg::copy16_kernel']:.1f} KiB "
                        f"and WRITE_SIZE {wr['dg::copy16_kernel']:.1f} KiB",
         "workload": cj.get("workload")}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as fh:
        json.dump(t, fh, indent=1)
    return t


def spread_canvas(cfg, n_distinct: int, seed: int = 4):
    """int32 [1][C]: committed tokens drawn from n_distinct seeded random ids."""
    import torch
    g = torch.Generator().manual_seed(seed)
    ids = torch.randint(0, cfg.vocab, (n_distinct,), generator=g, dtype=torch.int32)
    return ids[torch.randint(0, n_distinct, (1, cfg.canvas), generator=g)].contiguous()


def kind_roofline(eng, cfg, kind, run_pass, reps, counts_fn=None, flops_fn=None):
    """HIP-event timing of one kind's launches over `reps` passes (run_pass(s) enqueues
    pass s); the algorithmic amount of every pass from its own expert counts
    (counts_fn) or flops_fn(s).  Returns (avg launch ms, amount per launch, launches,
    per-pass extras)."""
    from discrete_diffusion_block_amd import dg
    import torch
    tot_ms, launches, amount_sum, used = 0.0, 0, 0.0, []
    for s in range(reps):
        dg.dg_profile_begin(eng.ctx, 8 * cfg.n_layers, kinds=[kind])
        run_pass(s)
        p1 = dg.dg_profile_end(eng.ctx)[kind]
        if counts_fn is not None:
            counts = counts_fn()
            amount = algorithmic_work(kind, cfg, cfg.canvas, counts)[2]
            used += [sum(1 for c in row if c > 0) for row in counts]
        else:
            amount = flops_fn(s)
        tot_ms += p1[0]
        launches += p1[1]
        amount_sum += amount * p1[1]
    torch.cuda.synchronize()
    return tot_ms / launches, amount_sum / launches, launches, used


def roofline_obj(bound, unit, avg_ms, amount, launches, kind, traffic=None, **extra):
    if unit == "GB/s":
        achieved, peak = amount / (avg_ms * 1e-3) / 1e9, HBM_PEAK_GBS
    else:
        achieved, peak = amount / (avg_ms * 1e-3) / 1e12, MFMA_BF16_PEAK_TFLOPS
    out = {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
           "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": kind,
           "avg_launch_ms": round(avg_ms, 4), "launches": launches, "algorithmic_per_launch": round(amount)}
    out.update(extra)
    return out


def achievable_peaks():
    """The chip's measured peaks beside the vendor figures: HBM by a streaming read and by
    the library's copy kernel over 2 GiB (8x the 256 MB Infinity Cache; the copy counts
    read + write bytes), bf16 MFMA by register-only matrix-core pairs (no memory
    traffic).  Medians of 5 timed runs."""
    import torch
    from discrete_diffusion_block_amd import dg
    stream = torch.cuda.current_stream()

    def timed(fn, reps=5):
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]

    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    copy_ms = timed(lambda: dg.dg_test_copy(src, dst, n))
    words = torch.empty(8192 * 256, dtype=torch.int32, device="cuda")
    read_ms, read_blocks = min((timed(lambda: dg.dg_test_read_rate(src, n, b, words)), b)
                               for b in (1024, 2048, 4096, 8192))
    del src, dst, words
    blocks, iters = 4096, 4096
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    mfma_ms = timed(lambda: dg.dg_test_mfma_rate(blocks, iters, out))
    flops = blocks * 4 * 8 * iters * 16384.0
    hbm = 2 * n / (copy_ms * 1e-3) / 1e9
    rd = n / (read_ms * 1e-3) / 1e9
    tf = flops / (mfma_ms * 1e-3) / 1e12
    return {"hbm_read_gbs": round(rd, 1), "hbm_read_frac_of_vendor": round(rd / HBM_PEAK_GBS, 4),
            "hbm_copy_gbs": round(hbm, 1), "hbm_frac_of_vendor": round(hbm / HBM_PEAK_GBS, 4),
            "mfma_bf16_tflops": round(tf, 1), "mfma_frac_of_vendor": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "read_blocks": read_blocks,
            "method": "streaming read of 2 GiB, four 16-byte loads in flight per thread, the fastest of "
                      "1024/2048/4096/8192 x 256 threads (dg_test_read_rate); copy of 2 GiB (read + write bytes; dg_test_copy); 4096 x 256 threads "
                      "of register-only bf16 MFMA pairs (dg_test_mfma_rate); HIP-event medians of 5 runs"}


def sampler_roofline(eng, cfg, gamma):
    """The sampler on four distinct 128 MiB logits buffers in rotation (512 MiB: more than
    the 256 MB Infinity Cache, so every call reads its logits from HBM), each a fully
    masked 256 x 262144 canvas of the sampler workload (N(0, 4^2) + a +12 spike on 60% of
    rows).  The whole call is timed with HIP events on the stream; the pass alone with
    the profiler's events on its launches (dg_test_sample_eb_profiled)."""
    import torch
    from discrete_diffusion_block_amd import dg, synth
    C, V = cfg.canvas, cfg.vocab
    bufs = [synth.make_sampler_logits(C, V, seed=70 + i, device="cuda").view(1, C, V) for i in range(4)]
    canv = [torch.full((1, C), V, dtype=torch.int32, device="cuda") for _ in range(4)]
    nm = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(dg.dg_sample_workspace_size(1, C, V), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    n = 24
    for c in canv:
        c.fill_(V)
    for i in range(4):                                     # warm-up
        dg.dg_sample_eb(bufs[i], canv[i], gamma, False, nm, ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fill_ms = 0.0
    for c in canv:
        c.fill_(V)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(n):
        dg.dg_sample_eb(bufs[i % 4], canv[i % 4], gamma, False, nm, ws)
        if i % 4 == 3:
            for c in canv:
                c.fill_(V)
    e1.record(stream)
    torch.cuda.synchronize()
    call_ms = e0.elapsed_time(e1) / n
    # the pass alone (and the selection kernels), timed on their own launches
    for c in canv:
        c.fill_(V)
    dg.dg_profile_begin(eng.ctx, 16 * n)
    for i in range(n):
        dg.dg_test_sample_eb_profiled(eng.ctx, bufs[i % 4], canv[i % 4], gamma, False, nm, ws)
        if i % 4 == 3:
            for c in canv:
                c.fill_(V)
    prof = dg.dg_profile_end(eng.ctx)
    pass_ms = prof["sample_pass1"][0] / prof["sample_pass1"][1]
    nbytes = C * V * 2
    return {"bound": "hbm", "achieved": round(nbytes / (pass_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(nbytes / (pass_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel": "sample_partials (entropy/argmax pass) on 4 rotating 128 MiB buffers",
            "avg_launch_ms": round(pass_ms, 4), "bytes_per_launch": nbytes,
            "call": {"avg_call_ms": round(call_ms, 4),
                     "achieved": round(nbytes / (call_ms * 1e-3) / 1e9, 1),
                     "frac": round(nbytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "note": "whole dg_sample_eb call: pass, selection, the canonical-entropy passes "
                             "(they return at once for certified decisions), launch gaps; the canvas "
                             "refill every 4 calls is inside the span"},
            "select_ms": round(prof["sample_select"][0] / max(1, prof["sample_select"][1]), 4),
            "canonical_passes_ms": round((prof["sample_canon"][0] + prof["sample_select_canon"][0]) /
                                         max(1, prof["sample_canon"][1]), 4)}


def spread_line(eng, cfg, n_distinct, reps, prompt_len):
    """The expert GEMMs at a routing spread like the Technical Report's (~84 unique experts
    per layer on a real 256-token canvas, §6 GPU time breakdown, MoE).  With random-init
    weights a denoising pass cannot show it: the timestep embedding (norm ~37 against ~1 for
    a token embedding) makes every canvas row alike, and the whole canvas goes to ~15
    experts.  The causal encoder pass that appends a finished canvas adds no timestep
    embedding, and its causal contexts differ from row to row: its 2048 assignments reach
    93-99 of the 128 experts per layer (measured: 92.8 over a canvas of 6 distinct token
    ids, 99 over 256 random ones), about 21 tokens each -- the regime of a trained model.
    Timed: that append pass over a canvas of n_distinct ids, repeated over the same cache
    slots, with HIP events on the expert GEMMs' launches (layers 0-28: the encoder's last
    layer feeds no K/V and has no FFN)."""
    import torch
    canvas = spread_canvas(cfg, n_distinct).cuda()
    # the pass runs right after the prompt (its window: the 1024 random prompt tokens),
    # as the append of the first block does
    L_saved = eng.lengths[0]
    L0 = prompt_len
    L = cfg.n_layers

    def append(s):
        eng.kv.len[0] = L0
        eng.prefill_kv(canvas)

    append(0)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(reps):
        append(s)
    e1.record(stream)
    torch.cuda.synchronize()
    pass_ms = e0.elapsed_time(e1) / reps
    out = {}
    for kind in ("moe_gate_up", "moe_down"):
        avg, amount, launches, used = kind_roofline(
            eng, cfg, kind, append, reps, counts_fn=lambda: eng.moe_counts()[:L - 1].cpu().tolist())
        out[kind] = roofline_obj("hbm", "GB/s", avg, amount, launches, kind,
                                 experts_used_per_layer_mean=round(sum(used) / len(used), 1),
                                 tokens_per_used_expert=round(2048 * (L - 1) / sum(used), 1))
    eng.kv.len[0] = L_saved
    return {"workload": f"causal append pass of the 30-layer model over a 256-token canvas of {n_distinct} "
                        f"distinct token ids: the random-init router spreads its 2048 assignments to "
                        f"{out['moe_gate_up']['experts_used_per_layer_mean']} of 128 experts per layer (the "
                        f"Technical Report's ~84 on a real canvas)",
            "append_pass_ms": round(pass_ms, 3), "roofline": out["moe_gate_up"], "moe_down": out["moe_down"]}


UNIFORM_BLOCKS, UNIFORM_WARMUP = 3, 1


def uniform_line(eng, cfg, args, logits):
    """The uniform ("multinomial") variant of the Technical Report (§3.2, multinomial
    diffusion; §3.3): the same model, context and sampler settings as the headline, but the
    canvas starts as uniformly random tokens, every position stays a candidate at every
    step (so the head computes all 256 rows of every step, where the absorbing canvas
    needs only its [MASK] rows) and the rest are re-noised from the counter-based
    generator.  Whole blocks with the KV append, timed on the host clock."""
    import torch
    C = cfg.canvas
    canvas = torch.empty(1, C, dtype=torch.int32, device="cuda")
    n_open = torch.empty(1, dtype=torch.int32, device="cuda")
    done = torch.empty(1, dtype=torch.int32, device="cuda")

    def block(i):
        eng.generate_block_uniform(canvas, args.denoise_steps, args.gamma, 1.0, 1.0, -1.0, 1000 + i, True, logits,
                                   n_open, done)
    for i in range(UNIFORM_WARMUP):
        block(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(UNIFORM_BLOCKS):
        block(UNIFORM_WARMUP + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert n_open.item() == 0 and done.item() == args.denoise_steps
    return {"workload": f"uniform-noise variant of the headline workload: a canvas of uniformly random tokens, "
                        f"{args.denoise_steps} steps, gamma {args.gamma}, tau 1, every position revisable and "
                        f"re-noised unless accepted, head over all {C} rows each step, KV append, batch 1",
            "value": round(C * UNIFORM_BLOCKS / wall, 1), "unit": "tok/s",
            "ms_per_block": round(wall * 1e3 / UNIFORM_BLOCKS, 2), "blocks": UNIFORM_BLOCKS,
            "warmup": UNIFORM_WARMUP}


STOP_BUDGET, STOP_BLOCKS, STOP_WARMUP, STOP_GAMMA = 48, 2, 1, 128.0


def stop_line(eng, cfg, args, logits):
    """Adaptive stopping (Technical Report §3.3, Fig. 5: about 12 effective steps of a
    budget of 48): blocks of the headline model with a budget of 48 steps and the stop on,
    e_stop 1e30 (a sequence stops at the first step whose [MASK] rows all keep their
    argmax; the random-init model's entropies, ~log V, never pass a realistic threshold),
    and gamma 128 (about ten rows per step at those entropies).  On random-init weights
    the argmaxes keep moving, so the canvas completes through the entropy budget rather
    than the stop; either way the generator skips the passes after completion, and a
    block costs its completion step plus at most one pass.  Every run starts its blocks right after the prompt (the cache
    rewound to the prompt's length), so the blocks, and where the stop fires, are the
    same from run to run.  The warm-up block counts the passes that ran with the
    library's launch profiler; the timed blocks run without it."""
    import torch
    from discrete_diffusion_block_amd import dg
    C = cfg.canvas
    canvas = torch.empty(1, C, dtype=torch.int32, device="cuda")
    nm = torch.empty(1, dtype=torch.int32, device="cuda")
    done = torch.empty(1, dtype=torch.int32, device="cuda")
    L_saved = eng.lengths[0]

    def block():
        eng.generate_block_ex(canvas, STOP_BUDGET, STOP_GAMMA, 1.0, 1.0, 1e30, True, logits, nm, done)
    eng.kv.len[0] = args.prompt
    dg.dg_profile_begin(eng.ctx, 256, kinds=["prep"])
    block()
    passes = dg.dg_profile_end(eng.ctx)["prep"][1] - 1
    for _ in range(STOP_WARMUP - 1):
        block()
    torch.cuda.synchronize()
    eng.kv.len[0] = args.prompt
    steps_seen = []
    t0 = time.perf_counter()
    for _ in range(STOP_BLOCKS):
        block()
        steps_seen.append(done)         # read after the clock stops
        done = torch.empty_like(done)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert nm.item() == 0
    eng.kv.len[0] = max(L_saved, eng.lengths[0])
    return {"workload": f"headline model with the adaptive stop: budget {STOP_BUDGET} steps, gamma {STOP_GAMMA}, "
                        f"tau 1, e_stop 1e30 (stop at the first step whose [MASK] argmaxes all repeat), passes "
                        f"after completion skipped, KV append, batch 1; {STOP_BLOCKS} consecutive blocks right after "
                        f"the {args.prompt}-token prompt",
            "value": round(C * STOP_BLOCKS / wall, 1), "unit": "tok/s",
            "ms_per_block": round(wall * 1e3 / STOP_BLOCKS, 2),
            "completion_steps": [int(d.item()) for d in steps_seen],
            "passes_run_first_block": passes, "budget": STOP_BUDGET, "blocks": STOP_BLOCKS,
            "warmup": STOP_WARMUP}


SC_REPS, SC_BLOCKS, SC_WARMUP = 10, 3, 1
FP32_MFMA_PEAK_TFLOPS = 157.3


def selfcond_line(eng, cfg, args, logits):
    """Self-conditioning (Technical Report §3.2, eq. 5-6; §6, sampling): the signal
    z = FFW(softmax(L) E) of a 256-row step, its kernels timed alone with HIP events over
    SC_REPS calls on the logits of a denoising pass, and whole blocks of the absorbing
    sampler with self-conditioning on (the head then computes every row at every step).
    The embedding product is 2 * 256 * 2816 * 262144 = 378 GFLOP at the pages' full
    precision; the engine runs it as two bf16 MFMA products (p in two bf16 parts), so
    its rate is reported against the fp32 MFMA peak (the product's own precision) and,
    for the MFMA work it issues, against the bf16 peak."""
    import torch
    from discrete_diffusion_block_amd import dg
    C, V, d = cfg.canvas, cfg.vocab, cfg.d_model
    c2 = torch.full((1, C), V, dtype=torch.int32, device="cuda")
    eng.denoise_step(c2, 1.0, logits)
    z = torch.empty(1, C, d, device="cuda")
    eng.self_cond(logits, z)
    torch.cuda.synchronize()
    kinds = ["sc_stats", "sc_embed", "sc_reduce", "sc_ffw"]
    dg.dg_profile_begin(eng.ctx, 8 * SC_REPS, kinds=kinds)
    for _ in range(SC_REPS):
        eng.self_cond(logits, z)
    prof = dg.dg_profile_end(eng.ctx)
    per = {k: prof[k][0] / SC_REPS for k in kinds}
    emb_ms = prof["sc_embed"][0] / prof["sc_embed"][1]
    flops = 2.0 * C * d * V
    achieved = flops / (emb_ms * 1e-3) / 1e12
    n = torch.empty(1, dtype=torch.int32, device="cuda")
    done = torch.empty(1, dtype=torch.int32, device="cuda")
    canvas = torch.empty(1, C, dtype=torch.int32, device="cuda")

    def block():
        eng.generate_block_sc(canvas, args.denoise_steps, args.gamma, 1.0, 1.0, -1.0, False, 0, True, logits, n,
                              done)
    for _ in range(SC_WARMUP):
        block()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(SC_BLOCKS):
        block()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert n.item() == 0
    return {"workload": f"self-conditioning signal of a {C}-row step (V {V}, d {d}, FFW width {cfg.shared_ffn}); "
                        f"blocks: the headline workload with self-conditioning on ({args.denoise_steps} steps, gamma "
                        f"{args.gamma}, z from each step's logits into the next, head over all rows)",
            "ms_per_step": round(sum(per.values()), 4),
            "kernel_ms": {k: round(v, 4) for k, v in per.items()},
            "embed_product": {"bound": "mfma", "algorithmic_gflop": round(flops / 1e9, 1),
                              "achieved": round(achieved, 1), "unit": "TFLOP/s",
                              "peak_fp32": FP32_MFMA_PEAK_TFLOPS,
                              "frac_of_fp32_peak": round(achieved / FP32_MFMA_PEAK_TFLOPS, 3),
                              "bf16_mfma_issued_tflops": round(2 * achieved, 1),
                              "frac_of_bf16_peak": round(2 * achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                              "avg_launch_ms": round(emb_ms, 4)},
            "blocks_tok_s": round(C * SC_BLOCKS / wall, 1), "ms_per_block": round(wall * 1e3 / SC_BLOCKS, 2),
            "blocks": SC_BLOCKS, "warmup": SC_WARMUP}


def long_context_line(packed, args):
    """The long-context batched workload: the same 30-layer model with every 6th layer
    attending globally (layers 5, 11, ..., 29; the rest a 1024-token window), 8 sequences
    with 32768-token random prompts prefilled once, then whole blocks (12 steps + append)
    for all 8 canvases at once."""
    import torch
    from discrete_diffusion_block_amd import dg, synth
    cfg = synth.CONFIGS["long"]
    B, P, C, V = args.lc_batch, args.lc_prompt, cfg.canvas, cfg.vocab
    blocks = args.lc_warmup + args.lc_steps + 1
    max_ctx = int(math.ceil((P + C * (blocks + 1)) / 64.0) * 64)
    eng = dg.Engine(cfg, packed, max_batch=B, max_ctx=max_ctx, packed=True)
    prompt = synth.make_prompt(cfg, B, P, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    eng.prefill_kv(prompt)
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - t0
    log(f"long context: prefill {B} x {P} tokens {prefill_s:.1f}s")
    logits = torch.empty(B, C, V, dtype=torch.bfloat16, device="cuda")
    nm = torch.empty(B, dtype=torch.int32, device="cuda")
    canvas = torch.empty(B, C, dtype=torch.int32, device="cuda")
    for _ in range(args.lc_warmup):
        eng.generate_block(canvas, args.denoise_steps, args.gamma, True, logits, nm)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.lc_steps):
        eng.generate_block(canvas, args.denoise_steps, args.gamma, True, logits, nm)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    value = B * C * args.lc_steps / wall
    # global-layer attention: HIP events on its launches over one block's denoising passes
    hq, hd = cfg.n_q_heads, cfg.head_dim
    c2 = torch.full((B, C), V, dtype=torch.int32, device="cuda")
    lens = [int(x) for x in eng.lengths[:B]]
    flops = sum(4.0 * C * hq * (L + C) * hd for L in lens)
    reps = args.denoise_steps
    avg, amount, launches, _ = kind_roofline(
        eng, cfg, "attention_global", lambda s: eng.denoise_step(c2, 1.0 - s / reps, logits), reps,
        flops_fn=lambda s: flops)
    dg.dg_profile_begin(eng.ctx, 20000)
    eng.generate_block(canvas, args.denoise_steps, args.gamma, True, logits, nm)
    torch.cuda.synchronize()
    prof = dg.dg_profile_end(eng.ctx)
    eng.close()
    return {"metric": "output tok/s (8 canvases of 256 tokens, 12 denoise steps + KV append per block)",
            "value": round(value, 1), "unit": "tok/s", "ms_per_block": round(wall * 1e3 / args.lc_steps, 2),
            "workload": f"long-context batched block generation: 30 MoE layers (every 6th global, the rest "
                        f"window 1024), batch {B}, {P}-token random prompts prefilled once ({prefill_s:.1f}s), "
                        f"12 steps, gamma {args.gamma}",
            "blocks": args.lc_steps, "warmup": args.lc_warmup,
            "roofline": roofline_obj("mfma", "TFLOP/s", avg, amount, launches, "attention_global",
                                     keys_per_query=[L + C for L in lens]),
            "kernel_ms_per_block": {k: round(v[0], 3) for k, v in prof.items() if v[1]}}


CONC_BATCHES = (1, 2, 4, 8, 16)
CONC_BLOCKS = 2


def concurrency_line(packed, args):
    """Multi-user throughput against the number of concurrent sequences (Technical Report
    §6, multi-user throughput): the 30-layer model, each sequence with its own 1024-token
    random prompt, whole blocks of 12 steps + the KV append.  Two schedules per batch size:
    lockstep (every sequence in the same step; the append is a pass of its own) and
    staggered continuous batching (dg_serve: sequences spread over the 13 phases, every
    pass mixing denoising sequences with one or more sequences appending their finished
    canvas, with the per-sequence causal flag).  tok/s = committed canvas tokens / wall."""
    import torch
    from discrete_diffusion_block_amd import dg, synth
    cfg = synth.CONFIGS["full"]
    C, V, P, N = cfg.canvas, cfg.vocab, args.prompt, args.denoise_steps
    Bmax = max(CONC_BATCHES)
    max_ctx = int(math.ceil((P + C * (2 * CONC_BLOCKS + 4)) / 64.0) * 64)
    eng = dg.Engine(cfg, packed, max_batch=Bmax, max_ctx=max_ctx, packed=True)
    logits = torch.empty(Bmax, C, V, dtype=torch.bfloat16, device="cuda")
    nm = torch.empty(Bmax, dtype=torch.int32, device="cuda")
    rows = []
    for B in CONC_BATCHES:
        eng.reset()
        eng.prefill_kv(synth.make_prompt(cfg, B, P, device="cuda"))
        canvas = torch.empty(B, C, dtype=torch.int32, device="cuda")
        lg, n = logits[:B], nm[:B]
        eng.generate_block(canvas, N, args.gamma, True, lg, n)          # warm-up
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(CONC_BLOCKS):
            eng.generate_block(canvas, N, args.gamma, True, lg, n)
        torch.cuda.synchronize()
        lock = B * C * CONC_BLOCKS / (time.perf_counter() - t0)
        eng.reset()
        eng.prefill_kv(synth.make_prompt(cfg, B, P, device="cuda"))
        canvas.fill_(V)
        phase = [(b * N) // B for b in range(B)]
        dg.dg_serve(eng.ctx, eng.kv, canvas, N, args.gamma, N + 1, phase, lg, n, eng.ws)   # warm-up cycle
        count = [0] * B
        out = torch.empty(B, 1, C, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        dg.dg_serve(eng.ctx, eng.kv, canvas, N, args.gamma, CONC_BLOCKS * (N + 1), phase, lg, n, eng.ws, out, count)
        torch.cuda.synchronize()
        stag = sum(count) * C / (time.perf_counter() - t0)
        rows.append({"batch": B, "lockstep_tok_s": round(lock, 1), "staggered_tok_s": round(stag, 1)})
        log(f"concurrency {B}: lockstep {lock:.0f}, staggered {stag:.0f} tok/s")
    eng.close()
    return {"workload": f"multi-user throughput of the 30-layer model: batch B of independent sequences, "
                        f"{P}-token prompts, {N} steps + append per {C}-token block, gamma {args.gamma}; lockstep "
                        f"blocks vs staggered continuous batching with mixed denoise/append passes",
            "unit": "tok/s", "blocks_per_sequence": CONC_BLOCKS, "rows": rows}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10, help="timed blocks")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--denoise-steps", type=int, default=12)
    ap.add_argument("--gamma", type=float, default=2.0)
    ap.add_argument("--prompt", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline only: skip the sampler, spread-routing and long-context lines")
    ap.add_argument("--spread-distinct", type=int, default=6,
                    help="distinct token ids of the spread-routing canvas")
    ap.add_argument("--lc-batch", type=int, default=8)
    ap.add_argument("--lc-prompt", type=int, default=32768)
    ap.add_argument("--lc-steps", type=int, default=2, help="timed blocks of the long-context line")
    ap.add_argument("--lc-warmup", type=int, default=1)
    ap.add_argument("--pmc-workload", action="store_true",
                    help="run the hardware-counter workload (copy calibration + 2 denoising steps) and exit")
    ap.add_argument("--counts-out", metavar="JSON", help="with --pmc-workload: where its expert counts go")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="print per-kernel counter means from rocprofv3 CSV output under DIR and exit")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print per-kernel launch statistics from rocprofv3 kernel-trace CSVs under DIR and exit")
    ap.add_argument("--bench-json", metavar="FILE", help="with --summarize-trace: the profiled run's JSON line")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_TXT", "WRITE_TXT", "KIND", "COUNTS_JSON"),
                    help="write profiles/traffic.json for KIND from two --summarize-pmc outputs and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc))
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.warmup, args.steps, args.denoise_steps,
                              args.prompt, args.bench_json))
        return
    if args.write_traffic:
        print(json.dumps(write_traffic(*args.write_traffic)))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the engine runs one process on one MI355X; see the design notes on sharding).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from discrete_diffusion_block_amd import dg, synth

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    dg.lib()
    if args.pmc_workload:
        pmc_workload(counts_out=args.counts_out)
        return
    cfg = synth.CONFIGS["full"]
    C, V = cfg.canvas, cfg.vocab
    n_blocks = (args.warmup + 2 * args.steps + 2 + 4 + UNIFORM_BLOCKS + UNIFORM_WARMUP + SC_BLOCKS + SC_WARMUP
                + STOP_BLOCKS + STOP_WARMUP)
    max_ctx = int(math.ceil((args.prompt + C * n_blocks) / 64.0) * 64)
    t0 = time.time()
    w = synth.make_weights(cfg, device="cuda")
    torch.cuda.synchronize()
    log(f"weights {time.time() - t0:.1f}s ({torch.cuda.memory_allocated() / 1e9:.1f} GB)")
    eng = dg.Engine(cfg, w, max_batch=1, max_ctx=max_ctx, free_source=True,
                    selfcond=synth.make_selfcond_weights(cfg, device="cuda"))
    prompt = synth.make_prompt(cfg, 1, args.prompt, device="cuda")
    eng.prefill_kv(prompt)
    torch.cuda.synchronize()
    logits = torch.empty(1, C, V, dtype=torch.bfloat16, device="cuda")
    nm = torch.empty(1, dtype=torch.int32, device="cuda")
    canvas = torch.empty(1, C, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        eng.generate_block(canvas, args.denoise_steps, args.gamma, True, logits, nm)
    torch.cuda.synchronize()

    # ---- timed region: K whole blocks, each generated and appended to the cache, in
    # one dg_generate_blocks call (each block's append shares a pass with the next
    # block's first denoising step; the last block's append runs on its own)
    blocks = torch.empty(args.steps, 1, C, dtype=torch.int32, device="cuda")
    eng.generate_blocks(blocks[:2], args.denoise_steps, args.gamma, True, logits, nm)   # warm-up of the call
    L0 = eng.lengths[0]
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    eng.generate_blocks(blocks, args.denoise_steps, args.gamma, True, logits, nm)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    assert nm.item() == 0 and (blocks != V).all()
    ms_per_block = wall * 1000.0 / args.steps
    value = C * args.steps / wall
    log(f"{args.steps} blocks: {wall * 1e3:.1f} ms wall, {gpu_ms:.1f} ms GPU -> {value:.0f} tok/s")
    # the same blocks (the cache rewound to the same length: generation is deterministic)
    # as one dg_generate_block call each, the append as its own pass
    eng.kv.len[0] = L0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        eng.generate_block(canvas, args.denoise_steps, args.gamma, True, logits, nm)
        same = torch.equal(canvas[0], blocks[j, 0]) if j == 0 else same
    torch.cuda.synchronize()
    per_call_tok_s = C * args.steps / (time.perf_counter() - t0)
    assert eng.lengths[0] == L0 + C * args.steps and torch.equal(canvas[0], blocks[-1, 0]) and same
    log(f"  the same blocks, one dg_generate_block call each: {per_call_tok_s:.0f} tok/s")

    # ---- one more block with per-launch HIP events (same stream, same work)
    dg.dg_profile_begin(eng.ctx, 20000)
    t0 = time.perf_counter()
    eng.generate_block(canvas, args.denoise_steps, args.gamma, True, logits, nm)
    torch.cuda.synchronize()
    prof_block_ms = (time.perf_counter() - t0) * 1e3
    prof = dg.dg_profile_end(eng.ctx)
    log("per-kind kernel ms in one block: " +
        ", ".join(f"{k} {v[0]:.2f}/{v[1]}" for k, v in sorted(prof.items(), key=lambda kv: -kv[1][0]) if v[1]))

    # ---- roofline of the dominant kernel kind: among the kinds bound by HBM or MFMA
    # (the row kernels are latency-bound), the one with the most time in the profiled
    # block.  Its launches are timed alone (HIP events on the engine's stream around
    # that kind only) over the denoising passes of one block's worth of steps on a fresh
    # all-[MASK] canvas; the algorithmic amount of each pass uses that pass's own
    # per-layer expert counts.
    dom = max((k for k in prof if prof[k][1] and algorithmic_work(k, cfg, C, None)[0] and k != "attention_global"),
              key=lambda k: prof[k][0])
    c2 = torch.full((1, C), V, dtype=torch.int32, device="cuda")
    reps = args.denoise_steps

    def dom_pass(s):
        eng.denoise_step(c2, 1.0 - s / reps, logits)

    bound, unit, _ = algorithmic_work(dom, cfg, C, None)
    counts_fn = (lambda: eng.moe_counts().cpu().tolist()) if dom.startswith("moe") else None
    flops_fn = None if counts_fn else (lambda s: algorithmic_work(dom, cfg, C, None)[2])
    avg_ms, amount, dom_launches, used = kind_roofline(eng, cfg, dom, dom_pass, reps, counts_fn, flops_fn)
    log(f"{dom}: {dom_launches} launches, {avg_ms * 1e3:.2f} us average")
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        t = json.load(open(tfile))
        if (t.get("kernel") == dom and dom in KIND_SOURCES
                and t.get("source_digest") == kernel_source_digest(dom)):
            traffic = t.get("bytes_per_launch")
    log("achievable peaks (streaming read, copy, register-only MFMA)...")
    peaks = achievable_peaks()
    ceiling = peaks["hbm_read_gbs"] if unit == "GB/s" else peaks["mfma_bf16_tflops"]
    roofline = roofline_obj(bound, unit, avg_ms, amount, dom_launches, dom, traffic)
    roofline["measured_ceiling"] = ceiling
    roofline["frac_of_measured_ceiling"] = round(roofline["achieved"] / ceiling, 4)
    if not used:
        used = [sum(1 for c in row if c > 0) for row in eng.moe_counts().cpu().tolist()]
    experts = round(sum(used) / len(used), 1)

    # ---- denoise step alone (denoise + sampler)
    c2.fill_(V)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(reps):
        eng.denoise_step(c2, 1.0 - s / reps, logits)
        eng.sample_eb(logits, c2, args.gamma, s == reps - 1, nm)
    e1.record(stream)
    torch.cuda.synchronize()
    denoise_ms = e0.elapsed_time(e1) / reps

    out = {
        "metric": "output tok/s (256-tok canvas, 12 denoise steps + KV append per block)",
        "value": round(value, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_block, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (random-init N(0,0.02) bf16 weights, uniform-random 1024-token prompt)",
        "config": {"workload": "full 256-token block generation: 30 MoE layers d2816, 16q/8kv x128, "
                               "128 experts top-8 (F 704) + shared (F 2112), vocab 262144 tied, "
                               f"1024-token prompt, {args.steps} consecutive blocks of 12 steps, gamma 2.0, batch 1, "
                               "every block generated and appended to the KV cache (dg_generate_blocks: each "
                               "append shares a pass with the next block's first denoising step, bit-identical "
                               "to separate passes); the random-init router sends "
                               f"the all-[MASK] canvas to ~{experts} of the 128 experts per layer, so the MoE "
                               "streams that many experts' weights (a trained model spreads to ~84: see "
                               "spread_routing)",
                   "global_batch": 1, "seq_len": args.prompt, "canvas": C,
                   "denoise_steps": args.denoise_steps, "parallelism": "single GPU"},
        "per_block_call_tok_s": round(per_call_tok_s, 1),
        "denoise_step_ms": round(denoise_ms, 3),
        "gpu_ms_per_step": round(gpu_ms / args.steps, 3),
        "tokens_per_forward": round(C * args.steps / (args.denoise_steps * args.steps + 1), 3),
        "experts_used_per_layer_mean": experts,
        "profiled_block_ms": round(prof_block_ms, 3),
        "kernel_ms_per_block": {k: round(v[0], 3) for k, v in prof.items() if v[1]},
        "roofline": roofline,
        "sampler_roofline": None,
        "spread_routing": None,
        "long_context_batch8": None,
        "uniform_variant": None,
        "adaptive_stop": None,
        "self_conditioning": None,
        "concurrency": None,
        "cpu_baseline": None,
        "achievable_peaks": None,
    }
    out["achievable_peaks"] = peaks
    if not args.no_extras:
        log("sampler on rotating buffers...")
        out["sampler_roofline"] = sampler_roofline(eng, cfg, args.gamma)
        log("spread routing...")
        out["spread_routing"] = spread_line(eng, cfg, args.spread_distinct, reps, args.prompt)
        log("uniform-noise variant...")
        out["uniform_variant"] = uniform_line(eng, cfg, args, logits)
        log("adaptive stop...")
        out["adaptive_stop"] = stop_line(eng, cfg, args, logits)
        log(f"adaptive stop: completion steps {out['adaptive_stop']['completion_steps']}, "
            f"{out['adaptive_stop']['value']} tok/s")
        log("self-conditioning...")
        out["self_conditioning"] = selfcond_line(eng, cfg, args, logits)
        packed = eng.weights
        eng.close()
        del logits
        torch.cuda.empty_cache()
        log("long-context batched workload...")
        try:
            out["long_context_batch8"] = long_context_line(packed, args)
        except Exception as exc:  # report, but never lose the headline
            out["long_context_batch8"] = {"error": repr(exc)}
        torch.cuda.empty_cache()
        log("concurrency sweep...")
        try:
            out["concurrency"] = concurrency_line(packed, args)
        except Exception as exc:  # report, but never lose the headline
            out["concurrency"] = {"error": repr(exc)}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)...")
        try:
            out["cpu_baseline"] = cpu_baseline("rank 0, N=1")
        except Exception as exc:  # a host-side failure must not hide the GPU result
            out["cpu_baseline"] = {"error": repr(exc)}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
