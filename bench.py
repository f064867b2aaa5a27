"""Benchmark: block-parallel diffusion decoding on one MI355X.

One bench step = one call of dg_generate_block on the full 30-layer model
(d 2816, 16q/8kv heads of 128, 128 experts top-8 + shared, vocab 262144,
canvas 256): 12 denoising steps with entropy-bounded unmasking (gamma 2.0),
then the causal append of the finished canvas to the KV cache.  The 1024-token
random prompt is prefilled once before timing (the pages exclude prefill from
latency).  Weights are random-init N(0, 0.02) bf16 and inputs are synthetic.

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


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "discrete_diffusion_block_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
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
    }


def pmc_workload(n_steps: int = 2) -> None:
    """Workload for hardware-counter passes (rocprofv3 --pmc): first the library's
    plain 256 MiB copy kernel (a known byte count that calibrates the traffic
    counters), then n_steps denoising steps of the full model over a 1024-token
    prefix.  Nothing is timed."""
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
    for s in range(n_steps):
        eng.denoise_step(canvas, 1.0 - s / n_steps, logits)
    torch.cuda.synchronize()
    log(f"pmc workload done ({n_steps} denoising steps)")


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


def summarize_trace(root: str, warmup: int, steps: int, denoise_steps: int, prompt: int) -> str:
    """Per-kernel launch statistics from the rocprofv3 kernel-trace CSV under root of a
    `bench.py --steps S --warmup W` run: the denoising passes of the S timed blocks.
    Passes start at the engine's prep kernel; the prompt prefill takes the first
    ceil(prompt / 512) passes, then each block runs denoise_steps denoising passes (the
    ones that end in the vocabulary head) and one append pass."""
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
    first = -(-prompt // 512) + warmup * per_block
    timed = passes[first:first + steps * per_block]
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
    # the run's last denoise_steps denoising passes are the ones in which bench.py times
    # the dominant kind with HIP events (the roofline figure of its JSON line)
    roof = [p for p in passes if any("head_gemm" in r["Kernel_Name"] for r in p)][-denoise_steps:]
    ragg = collections.defaultdict(list)
    for p in roof:
        for r in p:
            name = r["Kernel_Name"].replace("void ", "").split("(")[0]
            ragg[name].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines.append("")
    lines.append(f"roofline passes (the run's last {len(roof)} denoising passes, in which bench.py times "
                 f"the dominant kind with HIP events on its launches):")
    for k, v in sorted(ragg.items(), key=lambda kv: -sum(kv[1]))[:6]:
        lines.append(f"{k[:58]:58s} {len(v):6d} launches, avg {sum(v) / len(v):8.2f} us")
    return "\n".join(lines)


def write_traffic(fetch_txt: str, write_txt: str, kind: str) -> dict:
    """Calibrated HBM bytes per launch of one kernel kind from the two counter summaries
    (FETCH_SIZE and WRITE_SIZE passes of --pmc-workload, printed by --summarize-pmc).
    Each counter is scaled by the ratio of the copy kernel's true byte count (256 MiB
    read, 256 MiB written) to what the same counter reads for it."""
    def means(path):
        out = {}
        for line in open(path):
            parts = line.split()
            if len(parts) >= 6:
                out[parts[0]] = float(parts[-1])
        return out
    fe, wr = means(fetch_txt), means(write_txt)
    copy_kib = float(256 << 10)
    fs, ws = copy_kib / fe["dg::copy16_kernel"], copy_kib / wr["dg::copy16_kernel"]
    name = f"dg::{kind}_kernel"
    t = {"kernel": kind, "source_digest": kernel_source_digest(),
         "bytes_per_launch": int(round((fe[name] * fs + wr[name] * ws) * 1024)),
         "fetch_kib_per_launch_raw": fe[name], "write_kib_per_launch_raw": wr[name],
         "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
         "calibration": f"dg::copy16_kernel copying 256 MiB reads FETCH_SIZE {fe['dg::copy16_kernel']:.1f} KiB "
                        f"and WRITE_SIZE {wr['dg::copy16_kernel']:.1f} KiB",
         "workload": "python3 bench.py --pmc-workload (denoising passes only: 2 steps, 30 layers)"}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as fh:
        json.dump(t, fh, indent=1)
    return t


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10, help="timed blocks")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--denoise-steps", type=int, default=12)
    ap.add_argument("--gamma", type=float, default=2.0)
    ap.add_argument("--prompt", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-workload", action="store_true",
                    help="run the hardware-counter workload (copy calibration + 2 denoising steps) and exit")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="print per-kernel counter means from rocprofv3 CSV output under DIR and exit")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print per-kernel launch statistics from rocprofv3 kernel-trace CSVs under DIR and exit")
    ap.add_argument("--write-traffic", nargs=3, metavar=("FETCH_TXT", "WRITE_TXT", "KIND"),
                    help="write profiles/traffic.json for KIND from two --summarize-pmc outputs and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc))
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.warmup, args.steps, args.denoise_steps,
                              args.prompt))
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
        pmc_workload()
        return
    cfg = synth.CONFIGS["full"]
    C, V = cfg.canvas, cfg.vocab
    n_blocks = args.warmup + args.steps + 3
    max_ctx = int(math.ceil((args.prompt + C * n_blocks) / 64.0) * 64)
    t0 = time.time()
    w = synth.make_weights(cfg, device="cuda")
    torch.cuda.synchronize()
    log(f"weights {time.time() - t0:.1f}s ({torch.cuda.memory_allocated() / 1e9:.1f} GB)")
    eng = dg.Engine(cfg, w, max_batch=1, max_ctx=max_ctx, free_source=True)
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

    # ---- timed region: K whole blocks
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        eng.generate_block(canvas, args.denoise_steps, args.gamma, True, logits, nm)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    assert nm.item() == 0
    ms_per_block = wall * 1000.0 / args.steps
    value = C * args.steps / wall
    log(f"{args.steps} blocks: {wall * 1e3:.1f} ms wall, {gpu_ms:.1f} ms GPU -> {value:.0f} tok/s")

    # ---- one more block with per-launch HIP events (same stream, same work)
    dg.dg_profile_begin(eng.ctx, 20000)
    t0 = time.perf_counter()
    eng.generate_block(canvas, args.denoise_steps, args.gamma, True, logits, nm)
    torch.cuda.synchronize()
    prof_block_ms = (time.perf_counter() - t0) * 1e3
    prof = dg.dg_profile_end(eng.ctx)
    log("per-kind kernel ms in one block: " +
        ", ".join(f"{k} {v[0]:.2f}/{v[1]}" for k, v in sorted(prof.items(), key=lambda kv: -kv[1][0]) if v[1]))

    # ---- denoise step alone (denoise + sampler)
    c2 = torch.full((1, C), V, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    reps = args.denoise_steps
    for s in range(reps):
        eng.denoise_step(c2, 1.0 - s / reps, logits)
        eng.sample_eb(logits, c2, args.gamma, s == reps - 1, nm)
    e1.record(stream)
    torch.cuda.synchronize()
    denoise_ms = e0.elapsed_time(e1) / reps

    # ---- roofline of the dominant kernel kind: among the kinds bound by HBM or MFMA
    # (the row kernels are latency-bound), the one with the most time in the profiled
    # block.  Its launches are timed alone (HIP events on the engine's stream around
    # that kind only) over the denoising passes of one block's worth of steps; the
    # algorithmic amount of each pass uses that pass's own per-layer expert counts.
    dom = max((k for k in prof if prof[k][1] and algorithmic_work(k, cfg, C, None)[0]),
              key=lambda k: prof[k][0])
    c2.fill_(V)
    dom_ms, dom_launches, amount_sum, used = 0.0, 0, 0.0, []
    for s in range(reps):
        dg.dg_profile_begin(eng.ctx, 4 * cfg.n_layers, kinds=[dom])
        eng.denoise_step(c2, 1.0 - s / reps, logits)
        p1 = dg.dg_profile_end(eng.ctx)[dom]
        counts = eng.moe_counts().cpu().tolist()
        eng.sample_eb(logits, c2, args.gamma, s == reps - 1, nm)
        bound, unit, amount = algorithmic_work(dom, cfg, C, counts)
        dom_ms += p1[0]
        dom_launches += p1[1]
        amount_sum += amount * p1[1]
        used += [sum(1 for c in row if c > 0) for row in counts]
    torch.cuda.synchronize()
    avg_ms = dom_ms / dom_launches
    amount = amount_sum / dom_launches
    log(f"{dom}: {dom_launches} launches, {avg_ms * 1e3:.2f} us average")
    roofline = None
    if bound is not None:
        if unit == "GB/s":
            achieved, peak = amount / (avg_ms * 1e-3) / 1e9, HBM_PEAK_GBS
        else:
            achieved, peak = amount / (avg_ms * 1e-3) / 1e12, MFMA_BF16_PEAK_TFLOPS
        traffic = None
        tfile = os.path.join(ROOT, "profiles", "traffic.json")
        if os.path.exists(tfile):
            t = json.load(open(tfile))
            if t.get("kernel") == dom and t.get("source_digest") == kernel_source_digest():
                traffic = t.get("bytes_per_launch")
        roofline = {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                    "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": dom,
                    "avg_launch_ms": round(avg_ms, 4), "launches": dom_launches,
                    "algorithmic_per_launch": round(amount)}

    # the whole sampler call (entropy/argmax pass over all 256 rows' logits + selection) on a
    # fully masked canvas, 10 calls back to back; the canvas reset between calls (a fill
    # kernel) is inside the timed span, so the rate is slightly understated
    n_s = 10
    es0, es1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    es0.record(stream)
    for _ in range(n_s):
        c2.fill_(V)
        eng.sample_eb(logits, c2, args.gamma, False, nm)
    es1.record(stream)
    torch.cuda.synchronize()
    samp_ms = es0.elapsed_time(es1) / n_s
    samp_bytes = C * V * 2
    sampler = {"bound": "hbm", "achieved": round(samp_bytes / (samp_ms * 1e-3) / 1e9, 1),
               "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(samp_bytes / (samp_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "kernel": "dg_sample_eb call (entropy/argmax pass + selection)",
               "avg_call_ms": round(samp_ms, 4), "bytes_per_call": samp_bytes}
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
                               "1024-token prompt, 12 steps, gamma 2.0, batch 1",
                   "global_batch": 1, "seq_len": args.prompt, "canvas": C,
                   "denoise_steps": args.denoise_steps, "parallelism": "single GPU"},
        "denoise_step_ms": round(denoise_ms, 3),
        "gpu_ms_per_step": round(gpu_ms / args.steps, 3),
        "tokens_per_forward": round(C / (args.denoise_steps + 1), 3),
        "experts_used_per_layer_mean": round(sum(used) / len(used), 1),
        "profiled_block_ms": round(prof_block_ms, 3),
        "kernel_ms_per_block": {k: round(v[0], 3) for k, v in prof.items() if v[1]},
        "roofline": roofline,
        "sampler_roofline": sampler,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)...")
        try:
            out["cpu_baseline"] = cpu_baseline("rank 0, N=1")
        except Exception as exc:  # a host-side failure must not hide the GPU result
            out["cpu_baseline"] = {"error": repr(exc)}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
