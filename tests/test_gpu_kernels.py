"""GPU parity of single kernels through the C ABI: GEMM, router top-k, entropy-bounded
selection, and the full sampler on the 256 x 262144 sampler workload."""
import math

import numpy as np
import pytest
import torch

from discrete_diffusion_block_amd import dg, synth
from oracle import dg_oracle as O
from gpu_util import require_gpu, to_np_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16)


@pytest.mark.parametrize("M,N,K", [(1, 4, 64), (37, 100, 128), (256, 4096, 2816), (300, 132, 704),
                                   (16, 2816, 2112), (1024, 512, 256),
                                   # passes of >= 2048 rows take the wide tile (256 weight rows x 128 tokens)
                                   (2048, 4096, 2816), (2100, 4224, 2816), (2200, 300, 192)])
def test_gemm_matches_fp64(M, N, K):
    print(f"gemm M={M} N={N} K={K}", flush=True)
    x, w = _bf16((M, K), 1), _bf16((N, K), 2, 0.05)
    y = torch.full((M, N), float("nan"), device="cuda")
    dg.dg_test_gemm(dg.pack(x.cuda()), dg.pack(w.cuda()), y, M, N, K)
    torch.cuda.synchronize()
    xd, wd = to_np_bf16(x), to_np_bf16(w)
    ref = xd @ wd.T
    bound = 1.01 * K * 2.0 ** -24 * (np.abs(xd) @ np.abs(wd).T) + 1e-30
    err = np.abs(y.cpu().numpy() - ref)
    assert np.all(err <= bound), float((err / bound).max())


@pytest.mark.parametrize("n_bytes", [16, 4096 + 48, 64 << 20])
def test_copy_tap_bit_exact(n_bytes):
    print(f"copy {n_bytes} bytes", flush=True)
    g = torch.Generator().manual_seed(n_bytes % 1000)
    src = torch.randint(0, 256, (n_bytes,), generator=g, dtype=torch.uint8).cuda()
    dst = torch.zeros(n_bytes + 64, dtype=torch.uint8, device="cuda")
    dg.dg_test_copy(src, dst, n_bytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n_bytes], src)
    assert int(dst[n_bytes:].count_nonzero()) == 0            # nothing written past the end


@pytest.mark.parametrize("M,E,k", [(300, 128, 8), (64, 8, 2), (5, 256, 16), (33, 4, 4), (70, 100, 5),
                                   (40, 48, 6), (17, 32, 16)])
def test_router_topk_bit_exact(M, E, k):
    print(f"topk M={M} E={E} k={k}", flush=True)
    g = torch.Generator().manual_seed(M * 7 + E)
    r = torch.randn(M, E, generator=g)
    r[::3] = torch.round(r[::3] * 4) / 4            # exact ties (and -0 vs +0) in every third row
    r[1] = 0.0                                       # a row of all-equal logits
    r[2, ::2] = -0.0                                 # signed zeros tie with +0
    r[4, :5] = float("nan")                          # NaN ranks as -inf
    if M > 7:
        r[7, 3:9] = float("-inf")
    ids = torch.empty(M, k, dtype=torch.int32, device="cuda")
    w = torch.empty(M, k, device="cuda")
    dg.dg_test_router_topk(r.cuda(), k, ids, w)
    torch.cuda.synchronize()
    ref_ids, ref_w = O.router_topk(r.double().numpy(), k)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=2e-6, atol=1e-7)


def _eb_case(batch, C, seed, quant=0.25, pmask=0.6):
    g = torch.Generator().manual_seed(seed)
    H = (torch.randint(0, 12, (batch, C), generator=g).float() * quant)
    H += (torch.rand(batch, C, generator=g) < 0.3).float() * torch.rand(batch, C, generator=g)
    amax = torch.randint(0, 1000, (batch, C), generator=g, dtype=torch.int32)
    canvas = torch.randint(0, 1000, (batch, C), generator=g, dtype=torch.int32)
    canvas[torch.rand(batch, C, generator=g) < pmask] = 1000
    return H, amax, canvas


@pytest.mark.parametrize("batch,C,gamma,commit_all,pmask", [
    (3, 256, 2.0, False, 0.6), (1, 256, 0.0, False, 0.6), (2, 64, 1.5, False, 1.0),
    (1, 1024, 7.25, False, 0.5), (1, 1, 0.5, False, 1.0), (2, 100, float("inf"), False, 0.7),
    (2, 256, 0.5, True, 0.6), (1, 256, 3.0, False, 0.0)])
def test_eb_select_bit_exact(batch, C, gamma, commit_all, pmask):
    print(f"eb_select batch={batch} C={C} gamma={gamma} all={commit_all}", flush=True)
    H, amax, canvas = _eb_case(batch, C, seed=C + batch, pmask=pmask)
    d_canvas = canvas.cuda()
    nm = torch.empty(batch, dtype=torch.int32, device="cuda")
    dg.dg_test_eb_select(H.cuda(), amax.cuda(), d_canvas, 1000, gamma, commit_all, nm)
    torch.cuda.synchronize()
    out = d_canvas.cpu().numpy()
    for b in range(batch):
        masked = [i for i in range(C) if canvas[b, i] == 1000]
        sel = O.eb_select(H[b].numpy(), masked, gamma, commit_all)
        ref = canvas[b].numpy().copy()
        ref[sel] = amax[b].numpy()[sel]
        np.testing.assert_array_equal(out[b], ref)
        assert nm[b].item() == len(masked) - len(sel)


def test_eb_select_gamma_exactly_on_running_sum():
    # entropies 0.5 each: S_4 == 2.0 exactly, so gamma = 2.0 commits 4 and 1.9999999 commits 3
    C = 16
    H = torch.full((1, C), 0.5)
    amax = torch.arange(C, dtype=torch.int32).view(1, C) + 7
    for gamma, want in ((2.0, 4), (1.9999999, 3), (0.49, 1)):
        canvas = torch.full((1, C), 50, dtype=torch.int32).cuda()
        nm = torch.empty(1, dtype=torch.int32, device="cuda")
        dg.dg_test_eb_select(H.cuda(), amax.cuda(), canvas, 50, gamma, False, nm)
        torch.cuda.synchronize()
        c = canvas.cpu().numpy()[0]
        assert list(c[:want]) == list(range(7, 7 + want)) and np.all(c[want:] == 50)
        assert nm.item() == C - want


def _sampler_inputs():
    V, C = 262144, 256
    logits = synth.make_sampler_logits(C, V)                     # N(0, 4^2) + 12 spike on 60% rows
    canvas = synth.make_masked_canvas(C, V, 128)
    # a second sequence exercising multi-commit, exact ties and near-zero entropies
    l2 = synth.make_sampler_logits(C, V, seed=5)
    l2f = l2.float()
    g = torch.Generator().manual_seed(9)
    sharp = torch.randperm(C, generator=g)[:40]
    ids = torch.randint(0, V, (40,), generator=g)
    l2f[sharp, ids] += 40.0                                       # H ~ 0
    l2f[sharp[30:40]] = l2f[sharp[20:30]].clone()                 # 10 duplicated rows: exact ties
    l2 = l2f.to(torch.bfloat16)
    c2 = synth.make_masked_canvas(C, V, 200, seed=11)
    c2[sharp] = V
    return torch.stack([logits, l2]), torch.stack([canvas, c2])


H_FAST = 2e-5        # |H_engine - Ĥ| on rows the fast pass decided (fp32 entropy error)


def _check_sampler_call(logits, canvas, out, Hg, ag, nm, gamma, tau=1.0):
    """The committed set, argmaxes and masked counts equal the oracle's (decisions on the
    canonical entropy Ĥ, identical bf16 logits); every reported entropy is within H_FAST of
    Ĥ, or bitwise Ĥ on the rows whose Ĥ the engine computed to decide.  Returns, per
    sequence, a boolean array over the positions: entropy bitwise equal to the oracle's Ĥ."""
    B, C, V = logits.shape
    ref_canvas, ref_H, ref_a, ref_nm, _ = O.sample_eb(logits.double().numpy(), canvas.numpy(), gamma, False, V,
                                                      tau)
    exact = []
    for b in range(B):
        masked = [i for i in range(C) if canvas[b, i] == V]
        np.testing.assert_array_equal(ag[b][masked], ref_a[b][masked])
        assert np.all(ag[b][[i for i in range(C) if i not in masked]] == -1)
        np.testing.assert_array_equal(out[b], ref_canvas[b])
        assert nm[b] == ref_nm[b]
        d = np.abs(Hg[b][masked].astype(np.float64) - ref_H[b][masked].astype(np.float64))
        assert d.max() <= H_FAST / tau, float(d.max())
        exact.append(Hg[b].view(np.uint32) == ref_H[b].astype(np.float32).view(np.uint32))
        assert np.all(Hg[b][masked] >= 0) and np.all(Hg[b][masked] <= math.log(V) + 1e-5)
    return exact


def _run_sampler(logits, canvas, gamma, tau=None, e_stop=-1.0, prev=None):
    B, C, V = logits.shape
    d_canvas = canvas.cuda()
    H = torch.empty(B, C, device="cuda")
    am = torch.empty(B, C, dtype=torch.int32, device="cuda")
    nm = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(dg.dg_sample_workspace_size(B, C, V), dtype=torch.uint8, device="cuda")
    if tau is None and prev is None:
        dg.dg_sample_eb(logits.cuda(), d_canvas, gamma, False, nm, ws, H, am)
    else:
        d_prev = None if prev is None else prev.cuda()
        dg.dg_sample_eb_ex(logits.cuda(), d_canvas, gamma, False, 1.0 if tau is None else tau, e_stop, d_prev, 0,
                           None, nm, ws, H, am)
    torch.cuda.synchronize()
    return d_canvas.cpu().numpy(), H.cpu().numpy(), am.cpu().numpy(), nm.cpu().numpy()


@pytest.mark.parametrize("gamma", [0.5, 2.0])
def test_sampler_full_size_vs_oracle(gamma):
    """Sampler workload (256 x 262144 bf16 logits ~ N(0, 4^2), +12 spikes on 60% of rows,
    half the rows masked) plus a sequence with +40 spikes (H ~ 0), exact duplicate rows and
    200 masked rows: committed sets identical to the oracle's on the same logits."""
    print(f"sampler 2x256x262144 gamma={gamma}", flush=True)
    logits, canvas = _sampler_inputs()
    out, Hg, ag, nm = _run_sampler(logits, canvas, gamma)
    _check_sampler_call(logits, canvas, out, Hg, ag, nm, gamma)
    V = logits.shape[2]
    # committed tokens never change; the sharp rows commit together
    for b in range(2):
        keep = canvas[b].numpy() != V
        assert np.array_equal(out[b][keep], canvas[b].numpy()[keep])
    assert len([i for i in range(256) if out[1, i] != V and canvas[1, i] == V]) >= 40


def _near_tie_rows(V, n, seed):
    """n copies of one N(0, 4^2) row; copy i > 0 has one logit 8.5 + 0.6 i nats below the
    row's maximum moved up by one bf16 ulp, which moves its entropy by ~1e-7 to ~1e-6 --
    about one float32 step, so the copies' entropies tie or differ by an ulp or two and
    the fast pass's order of them is arbitrary."""
    g = torch.Generator().manual_seed(seed)
    base = (torch.randn(V, generator=g) * 4.0).to(torch.bfloat16)
    u = base.float().max() - base.float()
    rows = base.repeat(n, 1)
    bits = rows.view(torch.int16)
    for i in range(1, n):
        lo = 8.5 + 0.6 * i
        cand = torch.nonzero((u >= lo) & (u <= lo + 0.5) & (base.float() > 0)).view(-1)
        bits[i, cand[0]] += 1
    return rows


def test_sampler_ambiguous_decisions_vs_oracle():
    """Decisions that fall inside the fast entropies' error bound are deferred to the
    canonical entropy and must still equal the oracle's: (a) eight near-identical rows at the
    budget boundary; (b) gamma on a running sum (the nearest float32 below and above);
    (c) the adaptive stop's mean entropy on the threshold."""
    V, C = 262144, 64
    print(f"sampler ambiguous cases 1x{C}x{V}", flush=True)
    rest = (torch.randn(C, V, generator=torch.Generator().manual_seed(41))).to(torch.bfloat16)
    # (a): rows 3, 10, 17, ... hold the cluster; its entropy (~5) is the lowest of the
    # canvas (the other rows are N(0, 1): ~12)
    cl = _near_tie_rows(V, 8, seed=42)
    pos = [3 + 7 * i for i in range(8)]
    lg = rest.clone()
    lg[pos] = cl
    canvas = torch.full((1, C), V, dtype=torch.int32)
    Hc = O.entropy_canonical(lg.double().numpy()[pos])
    for gamma in (float(4.5 * Hc[0]), float(2.5 * Hc[0])):
        out, Hg, ag, nm = _run_sampler(lg.view(1, C, V), canvas, gamma)
        exact = _check_sampler_call(lg.view(1, C, V), canvas, out, Hg, ag, nm, gamma)
        # only the order inside the cluster is open: the engine computes Ĥ for its rows alone
        assert exact[0][pos].all(), "the cluster at the boundary is decided on the canonical entropy"
        assert 2 <= C - nm[0] <= 5
    # (b): gamma within a float32 step of the running sum S_5 in (Ĥ, position) order
    lb = synth.make_sampler_logits(C, V, seed=43).float()
    g = torch.Generator().manual_seed(44)
    idx = torch.randperm(C, generator=g)[:12]
    lb[idx, torch.randint(0, V, (12,), generator=g)] += torch.linspace(9.0, 16.0, 12)
    lb = lb.to(torch.bfloat16)
    Hb = O.entropy_canonical(lb.double().numpy())
    order = sorted(range(C), key=lambda i: (float(Hb[i]), i))
    S5 = sum(float(Hb[i]) for i in order[:5])          # the oracle's float64 running sum
    for gamma in (float(np.nextafter(np.float32(S5), np.float32(0))),
                  float(np.nextafter(np.float32(S5), np.float32(100)))):
        out, Hg, ag, nm = _run_sampler(lb.view(1, C, V), canvas, gamma)
        exact = _check_sampler_call(lb.view(1, C, V), canvas, out, Hg, ag, nm, gamma)
        assert exact[0].all() and C - nm[0] in (4, 5)      # a sum on gamma: every row's Ĥ
    # (c): stop threshold on the mean Ĥ of sharp rows whose argmaxes all repeat
    lc = synth.make_sampler_logits(C, V, seed=45, spike=22.0, spike_frac=1.0)
    Hcn = O.entropy_canonical(lc.double().numpy())
    acc = 0.0
    for i in range(C):
        acc += float(Hcn[i])
    mean = acc / C
    prev = torch.from_numpy(np.argmax(lc.float().numpy(), axis=1).astype(np.int32)).view(1, C)
    for e_stop in (float(np.nextafter(np.float32(mean), np.float32(0))),
                   float(np.nextafter(np.float32(mean), np.float32(1e9)))):
        out, Hg, ag, nm = _run_sampler(lc.view(1, C, V), canvas, 0.0, tau=1.0, e_stop=e_stop, prev=prev)
        ref = O.sample_eb(lc.view(1, C, V).double().numpy(), canvas.numpy(), 0.0, False, V, 1.0, e_stop,
                          prev.numpy())
        np.testing.assert_array_equal(out[0], ref[0][0])
        assert nm[0] == ref[3][0] and nm[0] in (0, C - 1)
        assert Hg[0].tobytes() == ref[1][0].tobytes()


@pytest.mark.parametrize("V,tau", [(262144, 1.0), (40008, 0.55), (4096, 2.5)])
def test_canonical_entropy_bitwise_vs_oracle(V, tau):
    """A sequence whose two lowest-entropy rows are exact duplicates (an exact tie at the
    boundary with gamma 0) is always decided on the canonical entropy: the engine then
    reports Ĥ for every masked row, which must equal the oracle's bit for bit -- on rows
    of every kind: N(0, s^2) for s from 0.05 to 10, spikes, uniform rows, exact ties."""
    C = 48
    print(f"canonical entropy bitwise V={V} tau={tau}", flush=True)
    g = torch.Generator().manual_seed(V + int(10 * tau))
    sd = torch.tensor([0.05, 0.3, 1.0, 4.0, 10.0])[torch.arange(C) % 5].view(C, 1)
    lf = torch.randn(C, V, generator=g) * sd
    lf[5] = 0.0                                            # uniform
    lf[6, 17] = 10.0                                       # a moderate spike
    lf[7, :3] = 3.0                                        # three-way tie at the max
    lf[8, torch.randint(0, V, (1,), generator=g)] += 7.0
    lf[9, 2] = 20.0                                        # a sharp row
    lf[0, 11] += 100.0                                     # every other term dropped: Ĥ = 0
    lf[1] = lf[0]                                          # rows 0 and 1: duplicates, the only Ĥ = 0
    logits = lf.to(torch.bfloat16).view(1, C, V)
    canvas = torch.full((1, C), V, dtype=torch.int32)
    canvas[0, 40:] = 3                                     # a few committed rows
    out, Hg, ag, nm = _run_sampler(logits, canvas, 0.0, tau=tau)
    exact = _check_sampler_call(logits, canvas, out, Hg, ag, nm, 0.0, tau)
    assert exact[0][:40].all()                             # a running sum on gamma: every masked row
    # the two Ĥ = 0 rows commit together (their running sum 0 stays within gamma = 0);
    # every other row has Ĥ > 0
    committed = [i for i in range(C) if canvas[0, i] == V and out[0, i] != V]
    assert committed == [0, 1] and out[0, 0] == ag[0, 0]


def test_sampler_ragged_vocab_and_cross_chunk_ties():
    """A vocabulary that is not a whole number of the first pass's chunks (40008 logits:
    two full chunks and a ragged third), with the maximum planted at chunk edges, twice
    across chunks (the lower index must win) and twice inside one chunk."""
    V, C = 40008, 64
    print(f"sampler 1x{C}x{V} ragged", flush=True)
    g = torch.Generator().manual_seed(21)
    lf = torch.randn(C, V, generator=g) * 4.0
    big = 30.0
    lf[0, V - 1] = big                       # last logit of the ragged chunk
    lf[1, 0] = big                           # first logit
    lf[2, 16383] = big                       # last of chunk 0 ...
    lf[2, 16384] = big                       # ... and first of chunk 1: 16383 wins
    lf[3, 5] = big
    lf[3, 39000] = big                       # tie across the first and the ragged chunk
    lf[4, 100] = big
    lf[4, 101] = big                         # adjacent tie inside a chunk
    lf[5, 20000] = big
    lf[5, 20000 + 2048] = big                # tie inside chunk 1, different threads
    lf[6] = 0.0                              # uniform row: every index ties, H = log V
    logits = lf.to(torch.bfloat16).view(1, C, V)
    canvas = torch.full((1, C), V, dtype=torch.int32)
    d_canvas = canvas.cuda()
    H = torch.empty(1, C, device="cuda")
    am = torch.empty(1, C, dtype=torch.int32, device="cuda")
    nm = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(dg.dg_sample_workspace_size(1, C, V), dtype=torch.uint8, device="cuda")
    dg.dg_sample_eb(logits.cuda(), d_canvas, 1.0, False, nm, ws, H, am)
    torch.cuda.synchronize()
    Ho, ao = O.entropy_argmax(logits[0].double().numpy())
    ag = am.cpu().numpy()[0]
    np.testing.assert_array_equal(ag, ao)
    assert list(ag[:7]) == [V - 1, 0, 16383, 5, 100, 20000, 0]
    Hg = H.cpu().numpy()[0].astype(np.float64)
    assert np.max(np.abs(Hg - Ho)) <= 2e-5
    assert abs(Hg[6] - math.log(V)) <= 2e-5
    out = d_canvas.cpu().numpy()[0]
    np.testing.assert_array_equal(out, O.sample_eb(logits.double().numpy(), canvas.numpy(), 1.0, False, V)[0][0])


@pytest.mark.parametrize("M,E,k", [(256, 128, 8), (512, 128, 8), (33, 8, 2), (1000, 16, 3), (7, 4, 4),
                                   (4096, 256, 16), (300, 100, 5), (257, 128, 16),
                                   (2048, 128, 8), (1100, 128, 16)])   # ids: up to 4096 staged in LDS; 4112, 16384, 17600, 65536 read from memory
def test_routing_sort_bit_exact(M, E, k):
    """Top-k ids bit-exact vs the oracle (ties, signed zeros, -inf and NaN rows among
    them); the counting sort is a stable, padded grouping."""
    print(f"route M={M} E={E} k={k}", flush=True)
    g = torch.Generator().manual_seed(M + E)
    r = torch.randn(M, E, generator=g)
    r[::2] = torch.round(r[::2] * 2) / 2                    # exact ties
    r[5:40] = r[5]                                           # identical rows: all route alike
    r[1] = 0.0                                               # a row of all-equal logits
    r[2, ::2] = -0.0                                         # signed zeros tie with +0
    r[3, : E // 2] = float("-inf")
    r[4, :5] = float("nan")                                  # NaN ranks as -inf
    out = {k2: v.cpu() for k2, v in dg.dg_test_route(r.cuda(), k).items()}
    ref_ids, ref_w = O.router_topk(r.double().numpy(), k)
    np.testing.assert_array_equal(out["ids"].numpy(), ref_ids)
    np.testing.assert_allclose(out["w"].numpy(), ref_w, rtol=2e-6, atol=1e-7)
    ids = ref_ids.reshape(-1)
    cnt = np.bincount(ids, minlength=E)
    np.testing.assert_array_equal(out["cnt"].numpy(), cnt)
    poff = out["poff"].numpy()
    assert poff[0] == 0 and np.all(poff % 16 == 0)
    np.testing.assert_array_equal(np.diff(poff), (cnt + 15) // 16 * 16)
    perm, inv = out["perm"].numpy(), out["inv"].numpy()
    for e in range(E):
        assign = np.nonzero(ids == e)[0]                    # assignment order within the expert
        np.testing.assert_array_equal(inv[assign], poff[e] + np.arange(len(assign)))
        np.testing.assert_array_equal(perm[poff[e]:poff[e] + len(assign)], assign // k)
        assert np.all(perm[poff[e] + len(assign):poff[e + 1]] == -1)
    items = out["items"].numpy()[:out["n_items"].item()]
    want = [(e, t0) for e in range(E) for t0 in range(0, cnt[e], dg.MOE_GROUP)]
    assert [tuple(x) for x in items] == want
    # expert GEMM items: each expert's 16-token blocks dealt evenly into ceil(c / 128) items
    want2 = []
    for e in range(E):
        n, b = -(-cnt[e] // 128), -(-cnt[e] // 16)
        for i in range(n):
            t0, t1 = 16 * (i * b // n), min(cnt[e], 16 * ((i + 1) * b // n))
            assert 0 < t1 - t0 <= 128
            want2.append((e, t0 | t1 << 16))
    items2 = out["items2"].numpy()[:out["n_items2"].item()]
    assert [tuple(x) for x in items2] == want2


@pytest.mark.parametrize("tau", [0.5, 0.8])
def test_sampler_tempered_full_size_vs_oracle(tau):
    """Entropies at temperature tau (Technical Report §3.3) on the full-size workload."""
    print(f"sampler tempered 2x256x262144 tau={tau}", flush=True)
    logits, canvas = _sampler_inputs()
    out, Hg, ag, nm = _run_sampler(logits, canvas, 2.0, tau=tau)
    _check_sampler_call(logits, canvas, out, Hg, ag, nm, 2.0, tau)


def test_sampler_adaptive_stop_vs_oracle():
    """Adaptive stop (Technical Report §3.3): sharp rows with unchanged argmaxes commit at once;
    one moved argmax falls back to the entropy bound.  The rows' entropies are exactly 0 in
    the canonical entropy (every term but the spike is dropped), so any gamma >= 0 would
    commit them all; gamma -1 leaves the bound's minimum of one commit."""
    V, C, B = 32768, 64, 2
    print(f"sampler adaptive stop {B}x{C}x{V}", flush=True)
    g = torch.Generator().manual_seed(31)
    lf = torch.randn(B, C, V, generator=g)
    ids = torch.randint(0, V, (B, C), generator=g)
    lf.scatter_(2, ids.unsqueeze(2), 60.0)
    logits = lf.to(torch.bfloat16)
    canvas = torch.full((B, C), V, dtype=torch.int32)
    canvas[:, :5] = torch.arange(5, dtype=torch.int32)           # committed positions stay
    prev = torch.where(canvas == V, ids.to(torch.int32), torch.full_like(canvas, -1))
    prev[1, 20] = (prev[1, 20] + 1) % V                           # sequence 1: one mode moved
    d_canvas, d_prev = canvas.cuda(), prev.cuda()
    done = torch.zeros(B, dtype=torch.int32, device="cuda")
    H = torch.empty(B, C, device="cuda")
    am = torch.empty(B, C, dtype=torch.int32, device="cuda")
    nm = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(dg.dg_sample_workspace_size(B, C, V), dtype=torch.uint8, device="cuda")
    dg.dg_sample_eb_ex(logits.cuda(), d_canvas, -1.0, False, 0.6, 0.005, d_prev, 6, done, nm, ws, H, am)
    torch.cuda.synchronize()
    ref_canvas, _, ref_a, ref_nm, _ = O.sample_eb(logits.double().numpy(), canvas.numpy(), -1.0, False, V, 0.6,
                                                  0.005, prev.numpy())
    out, Hg = d_canvas.cpu().numpy(), H.cpu().numpy()
    # sequence 0 stops: every masked row takes its argmax at once
    np.testing.assert_array_equal(out[0], ref_canvas[0])
    assert nm[0].item() == ref_nm[0] == 0 and done[0].item() == 7
    # sequence 1 does not (one mode moved): the bound commits exactly one row, the first in
    # (Ĥ, position) order -- its entropies tie at 0, so the position decides
    masked1 = [i for i in range(C) if canvas[1, i] == V]
    committed1 = [i for i in masked1 if out[1, i] != V]
    np.testing.assert_array_equal(out[1], ref_canvas[1])
    assert committed1 == [5]
    assert nm[1].item() == ref_nm[1] == C - 5 - 1 and done[1].item() == 0
    Ho, _ = O.entropy_argmax(logits[1, masked1].double().numpy(), 0.6)
    assert np.max(np.abs(Hg[1][masked1] - Ho)) <= 2e-5
    np.testing.assert_array_equal(d_prev.cpu().numpy(), am.cpu().numpy())   # this step's argmax, -1 elsewhere
    np.testing.assert_array_equal(am.cpu().numpy(), ref_a)


def test_mfma_rate_tap_counts_its_work():
    """The matrix-core rate tap runs every MFMA it is asked for: all-ones operands add 32
    per MFMA to each accumulator element, two MFMAs per accumulator per round, so each
    lane's checksum is 4 accumulators x 4 elements x 64 x rounds, exactly."""
    print("mfma rate tap", flush=True)
    for blocks, iters in ((3, 1), (37, 1000)):
        out = torch.full((blocks * 256,), -1.0, device="cuda")
        dg.dg_test_mfma_rate(blocks, iters, out)
        torch.cuda.synchronize()
        assert torch.all(out == 4 * 4 * 64 * iters), (blocks, iters, out.unique()[:4].tolist())


def test_read_rate_tap_reads_every_word():
    """The streaming-read tap visits every 16-byte word once: with src one repeated
    word, thread t's XOR is that word when it read an odd number of words (t, t + S,
    ... below n), else zero."""
    print("read rate tap", flush=True)
    for blocks, nwords in ((2, 3000), (5, 1280), (3, 7)):
        w = 0x5A17C3E1
        src = torch.full((nwords * 4,), w, dtype=torch.int32, device="cuda")
        out = torch.full((blocks * 256,), -1, dtype=torch.int32, device="cuda")
        dg.dg_test_read_rate(src, nwords * 16, blocks, out)
        torch.cuda.synchronize()
        S = blocks * 256
        t = np.arange(S)
        reads = np.maximum(0, (nwords - t + S - 1) // S)
        want = np.where(reads % 2 == 1, w, 0).astype(np.int32)
        np.testing.assert_array_equal(out.cpu().numpy(), want)
