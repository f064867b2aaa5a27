"""One dg_ctx shared by host threads: two threads, each with its own stream, workspace, KV
cache and canvas/logits buffers, generate blocks through the same ctx at the same time
(each call forks the shared expert onto the ctx's one side stream with a fork/join event
pair of its own).  Every thread's canvases, logits and cache must equal those of the same
work run alone, bit for bit."""
import threading

import pytest
import torch

from discrete_diffusion_block_amd import dg, synth
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _weights(cfg):
    w_cpu = synth.make_weights(cfg)
    return {"embed": w_cpu["embed"].cuda(), "final_norm": w_cpu["final_norm"].cuda(),
            "layers": [{k: v.cuda() for k, v in lw.items()} for lw in w_cpu["layers"]]}


BLOCKS, STEPS, GAMMA = 3, 4, 1.0


def _state(eng, cfg, prompt_len, seed):
    kv_bytes = dg.dg_kv_size(eng.ccfg)
    st = {"k": torch.zeros(kv_bytes // 2, dtype=torch.int16, device="cuda"),
          "v": torch.zeros(kv_bytes // 2, dtype=torch.int16, device="cuda"),
          "ws": torch.empty(dg.dg_workspace_size(eng.ctx, 1), dtype=torch.uint8, device="cuda"),
          "canvas": torch.empty(BLOCKS, 1, cfg.canvas, dtype=torch.int32, device="cuda"),
          "logits": torch.empty(1, cfg.canvas, cfg.vocab, dtype=torch.bfloat16, device="cuda"),
          "nm": torch.empty(1, dtype=torch.int32, device="cuda"),
          "stream": torch.cuda.Stream()}
    g = torch.Generator().manual_seed(seed)
    st["prompt"] = torch.randint(0, cfg.vocab, (1, prompt_len), generator=g, dtype=torch.int32).cuda()
    st["kv"] = dg.KV(st["k"].data_ptr(), st["v"].data_ptr())
    return st


def _work(eng, st, errors):
    try:
        s = st["stream"]
        dg.dg_prefill_kv(eng.ctx, st["kv"], st["prompt"], st["ws"], s)
        for j in range(BLOCKS):
            dg.dg_generate_block(eng.ctx, st["kv"], st["canvas"][j], STEPS, GAMMA, True, st["logits"], st["nm"],
                                 st["ws"], s)
        s.synchronize()
    except Exception as e:                                   # reported by the main thread
        errors.append(e)


def test_two_threads_on_one_ctx_match_runs_alone():
    cfg = synth.CONFIGS["tiny"]
    print(f"two threads on one ctx: tiny model, {BLOCKS} blocks x {STEPS} steps each", flush=True)
    w = _weights(cfg)
    max_ctx = ((64 + (BLOCKS + 1) * cfg.canvas) + 63) // 64 * 64
    eng = dg.Engine(cfg, w, max_batch=1, max_ctx=max_ctx)
    lens = (40, 53)
    alone = []
    for i, n in enumerate(lens):                             # each thread's work run alone
        st = _state(eng, cfg, n, 7 + i)
        errors = []
        _work(eng, st, errors)
        assert not errors, errors
        alone.append(st)
    torch.cuda.synchronize()
    for rnd in range(3):
        sts = [_state(eng, cfg, n, 7 + i) for i, n in enumerate(lens)]
        torch.cuda.synchronize()
        errors = []
        threads = [threading.Thread(target=_work, args=(eng, st, errors)) for st in sts]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        assert not errors, errors
        torch.cuda.synchronize()
        for a, b in zip(alone, sts):
            assert [int(x) for x in b["kv"].len[:1]] == [int(x) for x in a["kv"].len[:1]]
            for key in ("canvas", "logits", "nm", "k", "v"):
                assert torch.equal(a[key], b[key]), (rnd, key)
        print(f"  round {rnd}: both threads bitwise equal to their runs alone", flush=True)
    eng.close()
