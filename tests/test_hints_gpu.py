"""GPU tests of the hint-guided guess: the previous step's top-K positions
steer the bracket, and the selection stays exact whatever the hints hold.

The oracle takes no hints: every case below must give the oracle's result.
The hint recipes are the degenerate buffers the pages' hint-robustness tests
name (all-zero, all-same, all-max, half-duplicated, -1) plus stale, past-the-
window and adversarial ones; row_stats pins which guess each row used.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import assert_parity, log, to_dev

pytestmark = pytest.mark.gpu

I32_MIN, I32_MAX = np.iinfo(np.int32).min, np.iinfo(np.int32).max


@pytest.fixture(scope="module")
def ert():
    import torch
    import exact_row_top_amd as m
    assert torch.cuda.is_available()
    m.load_library()
    return m


def _case(k, rows=10, stride=32768, cfg=61):
    forced = {3: k - 1, 4: k, 5: k + 1, 9: 0}
    return workloads.decode_step(rows=rows, stride=stride, k=k, lo=k // 2, hi=stride, cfg=cfg,
                                 forced=forced)


def _sample_starts(nv, k):
    """Where the block64 sample reads a window of nv > k scores: k/64 blocks
    of 64, block j from floor(j * (nv - 64) / (k/64 - 1)) (PR 20998, "What
    changes": K distinct scores spread over the whole valid length)."""
    nsb = k // 64
    return [(j * (nv - 64)) // (nsb - 1) for j in range(nsb)]


def _recipes(w, good, want):
    """name -> int32 [rows, k] hint buffer."""
    rows, k = good.shape
    nv = w.n_valid.astype(np.int64)
    rng = np.random.default_rng(5)
    r = {"good": good}
    r["all_zero"] = np.zeros_like(good)
    r["all_same"] = np.repeat((nv // 2).astype(np.int32)[:, None], k, axis=1)
    r["all_max"] = np.repeat(np.maximum(nv - 1, 0).astype(np.int32)[:, None], k, axis=1)
    past = np.repeat(nv.astype(np.int32)[:, None], k, axis=1)
    past[:, 1::3] = w.row_stride
    past[:, 2::3] = I32_MAX
    r["past_end"] = past
    r["all_neg1"] = np.full_like(good, -1)
    mixed = good.copy()
    sel = rng.random(good.shape) < 0.3
    mixed[sel] = rng.choice(np.array([-1, -5, I32_MIN], dtype=np.int32), size=int(sel.sum()))
    r["neg_mixed"] = mixed
    half = good.copy()
    half[:, k // 2:] = good[:, :k - k // 2]
    r["half_dup"] = half
    r["stale_other_row"] = np.roll(good, 1, axis=0)
    # the row's lowest scores: the floor lands at the bottom of the row
    low = np.full_like(good, -1)
    for i in range(rows):
        n = int(nv[i])
        if n > 0:
            o = np.argsort(w.logits[i, :n], kind="stable")[:k]
            low[i, :o.size] = o
    r["lowest"] = low
    # the top half of the true top-K, duplicated: the floor lies above the
    # K-th value, so the counts fall short and the row takes the rescue
    top = np.full_like(good, -1)
    for i in range(rows):
        if int(nv[i]) > k:
            vals = w.logits[i, want[i]]
            o = want[i][np.argsort(-vals, kind="stable")][:k // 2]
            top[i] = np.concatenate([o, o])[:k]
    r["top_half_dup"] = top
    return r


TIERS = ({}, {"force_wgs_per_row": 1}, {"force_wgs_per_row": 5}, {"force_rescue": True})


def _run(ert, w, dev, k, hd, **kw):
    import torch
    st = torch.full((w.num_rows, ert.STATS_WORDS), -7, dtype=torch.int32, device="cuda")
    if hd is not None:
        kw["pre_idx"] = hd
    got = ert.topk_decode(dev["logits"], dev["n_valid"], k, row_stats=st, **kw)
    torch.cuda.synchronize()
    return got.cpu().numpy(), st.cpu().numpy()


@pytest.mark.parametrize("k", [512, 1024, 2048])
def test_hint_recipes_exact_on_every_tier(ert, k):
    """Every hint buffer gives the oracle's result on every tier; hints never
    raise a split row's floor, and degenerate ones change nothing at all."""
    import torch
    w, good = _case(k)
    want = oracle.topk_workload(w)
    dev = to_dev(w)
    recipes = _recipes(w, good, want)
    long_rows = [r for r in range(w.num_rows) if int(w.n_valid[r]) > k]
    # rows where the sample's vote is active (lam + 8 sqrt(lam) + 16 < k)
    roomy = [r for r in long_rows if int(w.n_valid[r]) >= 4 * k]
    base = {}
    for kw in TIERS:
        got, st = _run(ert, w, dev, k, None, **kw)
        assert_parity(w, got, want)
        base[str(kw)] = st
    for name, hints in recipes.items():
        hd = torch.from_numpy(np.ascontiguousarray(hints)).cuda()
        for kw in TIERS:
            log(f"[hints] k={k} {name} {kw}")
            got, s = _run(ert, w, dev, k, hd, **kw)
            assert_parity(w, got, want)
            b = base[str(kw)]
            if kw.get("force_rescue"):
                assert all(s[r, 0] == 2 for r in long_rows), (name, s[:, 0])
                continue
            if s[0, 6] > 1:
                # split rows: the hint can only lower the floor bin
                assert all(s[r, 8] <= b[r, 8] for r in long_rows), (name, kw, s[:, 8], b[:, 8])
            if name in ("all_zero", "all_same", "all_max", "past_end", "all_neg1"):
                # one score or none: the guess is the sample's, word for word
                assert np.array_equal(s, b), (name, kw)
            if name == "lowest":
                # a floor at the row's bottom: the sample outvotes it where
                # its vote is active, and the bracket's top stays the sample's
                assert np.array_equal(s[roomy], b[roomy]), (name, kw)
            if name in ("good", "half_dup", "neg_mixed", "top_half_dup"):
                assert all(s[r, 0] in (1, 5) for r in long_rows), (name, kw, s[:, 0])


@pytest.mark.parametrize("k", [512, 2048])
@pytest.mark.parametrize("g", [1, 4])
def test_peaks_between_sample_blocks_need_the_hints(ert, k, g):
    """A cluster of high scores placed only between the sample's blocks: the
    sample's maximum lies below all of it, so the whole cluster piles into
    the top bin, over the candidate cap.  Without hints both tiers count
    that bin again up to the row's own maximum (row_stats path 5); split rows
    with hints on the cluster raise the bracket's top to its maximum at once
    and finish on the first pass (path 1)."""
    import torch
    rows, n = 3, 32768
    cluster = 3000 if k == 512 else 6000
    w = workloads.random_decode(rows, n, [n, n - 7, n - 1000], k, seed=k + g)
    hints = np.full((rows, k), -1, dtype=np.int32)
    rng = np.random.default_rng(k)
    for r in range(rows):
        nv = int(w.n_valid[r])
        taken = np.zeros(nv, dtype=bool)
        for a in _sample_starts(nv, k):
            taken[a:a + 64] = True
        free = np.flatnonzero(~taken)
        pos = rng.choice(free, size=cluster, replace=False)
        w.logits[r, pos] = (10.0 + rng.random(cluster)).astype(np.float32)
        order = pos[np.argsort(-w.logits[r, pos], kind="stable")]
        hints[r] = order[:k]  # the previous top-K, its maximum first
    want = oracle.topk_workload(w)
    dev = to_dev(w)
    log(f"[peaks] k={k} g={g}")
    got, b = _run(ert, w, dev, k, None, force_wgs_per_row=g)
    assert_parity(w, got, want)
    assert all(b[r, 0] == 5 for r in range(rows)), b[:, 0]
    got, s = _run(ert, w, dev, k, torch.from_numpy(hints).cuda(), force_wgs_per_row=g)
    assert_parity(w, got, want)
    for r in range(rows):
        top = int(w.logits[r, hints[r, 0]].view(np.int32))
        assert s[r, 5] == top and s[r, 0] == (5 if g == 1 else 1), (r, s[r])


@pytest.mark.parametrize("k", [512, 2048])
def test_peaks_at_the_sample_blocks_take_the_rescue(ert, k):
    """Peaks planted exactly where the sample reads: the sample's floor lies
    above the K-th value, the split row's counts fall short of K, the
    recount without a floor finds the crossing bin over the cap and the row
    finishes exactly through the rescue (path 3), hints or not."""
    import torch
    rows, n = 3, 32768
    w = workloads.random_decode(rows, n, [n, n - 5, 20000], k, seed=k)
    hints = np.full((rows, k), -1, dtype=np.int32)
    for r in range(rows):
        nv = int(w.n_valid[r])
        pos = np.concatenate([np.arange(a, a + 64) for a in _sample_starts(nv, k)])
        w.logits[r, pos] = (10.0 + np.linspace(0.0, 1.0, pos.size)).astype(np.float32)
        hints[r] = pos[np.argsort(-w.logits[r, pos], kind="stable")][:k]
    want = oracle.topk_workload(w)
    dev = to_dev(w)
    for hd in (None, torch.from_numpy(hints).cuda()):
        log(f"[sample peaks] k={k} hints={hd is not None}")
        got, s = _run(ert, w, dev, k, hd, force_wgs_per_row=4)
        assert_parity(w, got, want)
        if hd is None:
            assert all(s[r, 0] == 3 and s[r, 8] == 0 for r in range(rows)), s[:, [0, 8]]


def test_hinted_decode_step_parity_and_options(ert):
    """Workload 2's shape with hints of about 0.77 overlap: exact, and the
    canonical output with sorted + deterministic."""
    import torch
    w, hints = workloads.decode_step()
    want = oracle.topk_workload(w)
    dev = to_dev(w)
    hd = torch.from_numpy(hints).cuda()
    got = ert.topk_decode(dev["logits"], dev["n_valid"], w.k, pre_idx=hd)
    torch.cuda.synchronize()
    assert_parity(w, got.cpu().numpy(), want)
    idx, vals = ert.topk_decode(dev["logits"], dev["n_valid"], w.k, pre_idx=hd,
                                return_values=True, sorted=True, deterministic=True)
    torch.cuda.synchronize()
    idx, vals = idx.cpu().numpy(), vals.cpu().numpy()
    assert np.array_equal(idx, want)
    for r in range(w.num_rows):
        n = int(w.n_valid[r])
        if n > w.k:
            assert np.array_equal(vals[r].view(np.uint32), w.logits[r, idx[r]].view(np.uint32))
    # the generator's hints overlap the true top-K the way the pages report
    ov = [np.intersect1d(want[r], hints[r]).size / w.k
          for r in range(w.num_rows) if int(w.n_valid[r]) > w.k]
    assert 0.65 < float(np.mean(ov)) < 0.9


@pytest.mark.parametrize("next_n,cr", [(1, 1), (2, 4), (3, 1), (4, 4)])
def test_varlen_request_level_hints(ert, next_n, cr):
    """Hints are per request (row // next_n), in compressed positions."""
    import torch
    k, stride = 1024, 16384
    kv = np.array([0, 3, 4096, 4100, 20000, 40000, 65536, 70000], dtype=np.int32)
    kv = np.minimum(kv, stride * cr)
    rows = len(kv) * next_n
    w = workloads.random_decode(rows, stride, [stride] * rows, k, seed=7 * next_n + cr)
    nv = oracle.varlen_n_valid(kv, rows, next_n, cr, stride)
    poison = np.array(workloads.POISON_DECODE, dtype=np.float32)
    for r in range(rows):
        cols = np.arange(int(nv[r]), stride)
        w.logits[r, cols] = poison[cols % 3]
    w.n_valid = nv.astype(np.int32)
    want = oracle.topk_workload(w)
    # request q's hints: the top-K of its first row plus noise positions
    rng = np.random.default_rng(next_n)
    hints = np.full((len(kv), k), -1, dtype=np.int32)
    for q in range(len(kv)):
        n = int(nv[q * next_n])
        if n > 0:
            hints[q] = want[q * next_n]
            noise = rng.random(k) < 0.2
            hints[q][noise] = rng.integers(0, n, size=int(noise.sum()))
    x = torch.from_numpy(w.logits).cuda()
    kvd = torch.from_numpy(kv).cuda()
    hd = torch.from_numpy(hints).cuda()
    for kw in ({}, {"force_wgs_per_row": 1}, {"force_wgs_per_row": 3}):
        log(f"[varlen hints] next_n={next_n} cr={cr} {kw}")
        got = ert.topk_decode_varlen(x, kvd, k, next_n=next_n, compress_ratio=cr, pre_idx=hd,
                                     **kw)
        torch.cuda.synchronize()
        assert_parity(w, got.cpu().numpy(), want)


def test_hints_in_a_replayed_graph(ert):
    """A captured launch reads the hint buffer at replay: new hints each step."""
    import torch
    k = 512
    w, good = _case(k, rows=8, stride=16384, cfg=62)
    want = oracle.topk_workload(w)
    dev = to_dev(w)
    hd = torch.from_numpy(good).cuda()
    out = torch.empty((w.num_rows, k), dtype=torch.int32, device="cuda")
    ws = ert.new_workspace(w.num_rows, w.row_stride, k)
    ert.topk_decode(dev["logits"], dev["n_valid"], k, out, pre_idx=hd, workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            ert.topk_decode(dev["logits"], dev["n_valid"], k, out, pre_idx=hd, workspace=ws)
    torch.cuda.synchronize()
    recipes = _recipes(w, good, want)
    for name in ("good", "all_zero", "top_half_dup", "lowest", "good"):
        hd.copy_(torch.from_numpy(recipes[name]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_parity(w, out.cpu().numpy(), want)


def test_hint_argument_errors(ert):
    import torch
    w, good = _case(512, rows=4, stride=4096)
    dev = to_dev(w)
    with pytest.raises(TypeError):
        ert.topk_decode(dev["logits"], dev["n_valid"], 512,
                        pre_idx=torch.from_numpy(good.astype(np.int64)).cuda())
    with pytest.raises(ValueError):
        ert.topk_decode(dev["logits"], dev["n_valid"], 512,
                        pre_idx=torch.from_numpy(good[:, :100].copy()).cuda())
    with pytest.raises(ValueError):
        ert.topk_decode(dev["logits"], dev["n_valid"], 512,
                        pre_idx=torch.from_numpy(good[:2].copy()).cuda())
