"""GPU tests of the block-skip pass: per-32-score block maxima let a row visit
only the blocks that can reach the sampled floor; the result must be the
oracle's exact selection whatever the pass skips, on every rung of its retry
ladder (row_stats word 0: 1 survivors only, 5 recount without a floor, 3
crowded crossing bin, 2 whole-row radix select; word 8: blocks visited)."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import assert_parity, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ert():
    import torch
    import exact_row_top_amd as m
    assert torch.cuda.is_available()
    m.load_library()
    return m


def _bmax_np(w):
    """Per-32 block maxima of every row's full stride (NaN ignored unless the
    whole block is NaN), as the producer defines them."""
    x = w.logits
    nb = (w.row_stride + 31) // 32
    pad = np.full((w.num_rows, nb * 32), np.nan, dtype=np.float32)
    pad[:, :w.row_stride] = x
    with np.errstate(invalid="ignore"), __import__("warnings").catch_warnings():
        __import__("warnings").simplefilter("ignore", RuntimeWarning)
        return np.nanmax(pad.reshape(w.num_rows, nb, 32), axis=2)


def _run(ert, w, dev, bm, **kw):
    import torch
    st = torch.full((w.num_rows, ert.STATS_WORDS), -7, dtype=torch.int32, device="cuda")
    got = ert.topk_decode(dev["logits"], dev["n_valid"], w.k, bmax=bm, blockskip=1, row_stats=st,
                          **kw)
    torch.cuda.synchronize()
    if isinstance(got, tuple):
        return (got[0].cpu().numpy(), got[1].cpu().numpy()), st.cpu().numpy()
    return got.cpu().numpy(), st.cpu().numpy()


@pytest.mark.parametrize("stride", [1000, 1001, 4096])
def test_block_max_producer(ert, stride):
    # stride % 4 == 0 takes the coalesced producer, 1001 the per-block one;
    # 1000 and 1001 end on a partial block
    import torch
    w = workloads.random_decode(5, stride, [stride, 999, 37, 0, 640], 512, seed=3)
    w.logits[1, 64:96] = np.nan  # a whole NaN block
    w.logits[2, 100] = np.inf
    x = torch.from_numpy(w.logits).cuda()
    got = ert.block_max(x).cpu().numpy()
    with np.errstate(all="ignore"):
        want = _bmax_np(w)
    assert got.shape == want.shape
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok].view(np.uint32), want[ok].view(np.uint32))


@pytest.mark.parametrize("k", [512, 1024, 2048])
@pytest.mark.parametrize("smooth", [2.0, 0.0])
def test_blockskip_parity(ert, k, smooth):
    # rows with locality and i.i.d. rows; short rows and rows with fewer
    # than K blocks (no floor: every block walked)
    w = workloads.decode_blockskip(rows=12, stride=max(65536, 80 * k), k=k, lo=k // 2,
                                   hi=max(65536, 80 * k), smooth=smooth, cfg=70 + k)
    w.n_valid[:4] = [0, k, k + 1, k + 31]
    want = oracle.topk_workload(w)
    dev = to_dev(w)
    bm = ert.block_max(dev["logits"])
    log(f"[bsk] k={k} smooth={smooth}")
    got, st = _run(ert, w, dev, bm)
    assert_parity(w, got, want)
    long_rows = [r for r in range(w.num_rows) if int(w.n_valid[r]) > k]
    assert all(st[r, 0] in (1, 5) for r in long_rows), st[:, 0]
    # the floor is the K-th largest block maximum (a bin edge at or below
    # it): a row with at least K blocks visits about K of them, one with
    # fewer visits them all
    nb = (w.n_valid.astype(np.int64) + 31) // 32
    for r in long_rows:
        if nb[r] >= k:
            assert k <= st[r, 8] <= 1.25 * k + 64, (r, st[r], nb[r])
        else:
            assert st[r, 8] == nb[r], (r, st[r], nb[r])


def test_blockskip_retry_ladder(ert):
    import torch
    k, n = 512, 40000
    rows = 6
    w = workloads.random_decode(rows, n, [n] * rows, k, seed=11)
    g = np.random.default_rng(5)
    # rows 1-4: tie-heavy (one distinct maximum: the sample brackets, and the
    # crossing bin is crowded, path 3; a crowded crossing bin, path 3), all
    # equal (no bracket at all, path 2), a -inf class with signed zeros on
    # top (path 2)
    w.logits[1] = (np.floor(4.0 * g.random(n)) - 1.5).astype(np.float32)
    w.logits[2] = np.where(g.random(n) < 0.1, 3.0, -1.0).astype(np.float32)
    w.logits[3] = np.float32(1.25)
    v = np.full(n, -np.inf)
    hi = g.random(n) < 0.01
    v[hi] = np.where(g.random(int(hi.sum())) < 0.5, -0.0, 0.0)
    w.logits[4] = v.astype(np.float32)
    want = oracle.topk_workload(w)
    dev = to_dev(w)
    bm = ert.block_max(dev["logits"])
    # row 0: loose bounds -- +inf on K + 10 blocks of low scores -- put the
    # floor above the K-th value: the counts fall short and every block is
    # recounted without a floor, in the sample's bracket (path 5)
    low = np.argsort(bm[0].cpu().numpy()[: (n + 31) // 32], kind="stable")[: k + 10]
    bm[0, torch.from_numpy(low).cuda()] = float("inf")
    for kw in ({}, {"deterministic": True}, {"force_rescue": True}):
        log(f"[bsk ladder] {kw}")
        got, st = _run(ert, w, dev, bm, **kw)
        assert_parity(w, got, want)
        if kw.get("force_rescue"):
            assert all(st[r, 0] == 2 for r in range(rows)), st[:, 0]
        else:
            assert list(st[:, 0]) == [5, 3, 3, 2, 2, 1], st[:, 0]
        if kw.get("deterministic"):
            idx, _ = _run(ert, w, dev, bm, deterministic=True, sorted=True)
            assert np.array_equal(idx, want)


def test_blockskip_overflow_and_loose_maxima(ert):
    """Upper bounds instead of maxima: +inf everywhere makes every block
    survive (over the list's capacity on long rows: the walk covers every
    block); NaN maxima survive too."""
    import torch
    k, n = 1024, 300000
    w = workloads.random_decode(3, n, [n, n - 3, 150000], k, seed=21)
    want = oracle.topk_workload(w)
    dev = to_dev(w)
    nb = (n + 31) // 32
    for fill in (np.inf, np.nan):
        bm = torch.full((3, nb), float(fill), dtype=torch.float32, device="cuda")
        got, st = _run(ert, w, dev, bm)
        assert_parity(w, got, want)
        nbr = (w.n_valid.astype(np.int64) + 31) // 32
        assert all(st[r, 8] == nbr[r] for r in range(3)), (st[:, 8], nbr)
    # a looser bound on part of the row only changes the work
    bm = ert.block_max(dev["logits"])
    bm[:, ::7] = float("inf")
    got, st = _run(ert, w, dev, bm)
    assert_parity(w, got, want)


def test_blockskip_output_options(ert):
    w = workloads.decode_blockskip(rows=8, stride=65536, k=1024, lo=2000, hi=65536, cfg=75)
    want = oracle.topk_workload(w)
    dev = to_dev(w)
    bm = ert.block_max(dev["logits"])
    (idx, vals), _ = _run(ert, w, dev, bm, return_values=True, sorted=True, deterministic=True)
    assert np.array_equal(idx, want)
    for r in range(w.num_rows):
        n = int(w.n_valid[r])
        if n > w.k:
            assert np.array_equal(vals[r].view(np.uint32), w.logits[r, idx[r]].view(np.uint32))


def test_blockskip_varlen_form(ert):
    import torch
    k, next_n, cr, stride = 512, 2, 4, 40960
    kv = np.array([0, 3, 2100, 4096, 60000, 120000, 163840, 170000], dtype=np.int32)
    rows = len(kv) * next_n
    w = workloads.random_decode(rows, stride, [stride] * rows, k, seed=31)
    nv = oracle.varlen_n_valid(kv, rows, next_n, cr, stride)
    poison = np.array(workloads.POISON_DECODE, dtype=np.float32)
    for r in range(rows):
        cols = np.arange(int(nv[r]), stride)
        w.logits[r, cols] = poison[cols % 3]
    w.n_valid = nv.astype(np.int32)
    want = oracle.topk_workload(w)
    x = torch.from_numpy(w.logits).cuda()
    bm = ert.block_max(x)
    st = torch.full((rows, ert.STATS_WORDS), -7, dtype=torch.int32, device="cuda")
    got = ert.topk_decode_varlen(x, torch.from_numpy(kv).cuda(), k, next_n=next_n,
                                 compress_ratio=cr, bmax=bm, blockskip=1, row_stats=st)
    torch.cuda.synchronize()
    assert_parity(w, got.cpu().numpy(), want)
    s = st.cpu().numpy()
    assert all(s[r, 0] in (1, 5) for r in range(rows) if int(nv[r]) > k), s[:, 0]


def test_blockskip_gate(ert):
    """Below the gate the ordinary decode path runs (row_stats word 8 is not
    a block count there); blockskip=1 forces the pass, -1 refuses it."""
    import torch
    w = workloads.decode_blockskip(rows=4, stride=65536, k=512, cfg=77)
    want = oracle.topk_workload(w)
    dev = to_dev(w)
    bm = ert.block_max(dev["logits"])
    for mode, bsk in ((0, False), (-1, False), (1, True)):
        st = torch.full((w.num_rows, ert.STATS_WORDS), -7, dtype=torch.int32, device="cuda")
        got = ert.topk_decode(dev["logits"], dev["n_valid"], w.k, bmax=bm, blockskip=mode,
                              row_stats=st)
        torch.cuda.synchronize()
        assert_parity(w, got.cpu().numpy(), want)
        s = st.cpu().numpy()
        # the block-skip pass runs one workgroup per row; the ordinary path
        # takes G > 1 workgroups per row at this batch size
        if bsk:
            assert all(s[r, 6] == 1 and s[r, 8] > 0 for r in range(w.num_rows)), s
        else:
            assert all(s[r, 6] > 1 for r in range(w.num_rows)), s


@pytest.mark.parametrize("k", [512, 2048])
def test_streaming_pass_with_its_own_maxima(ert, k):
    """blockskip=2: the pass streams every block once, keeps its maxima in LDS
    and continues as with given maxima (no producer needed)."""
    import torch
    w = workloads.decode_blockskip(rows=10, stride=max(65536, 80 * k), k=k, lo=k // 2,
                                   hi=max(65536, 80 * k), cfg=90 + k)
    g = np.random.default_rng(k)
    w.logits[1, : int(w.n_valid[1])] = np.floor(4.0 * g.random(int(w.n_valid[1]))) - 1.5
    w.logits[2, : int(w.n_valid[2])] = np.float32(0.5)
    want = oracle.topk_workload(w)
    dev = to_dev(w)
    for kw in ({}, {"deterministic": True, "sorted": True}):
        log(f"[stream] k={k} {kw}")
        st = torch.full((w.num_rows, ert.STATS_WORDS), -7, dtype=torch.int32, device="cuda")
        got = ert.topk_decode(dev["logits"], dev["n_valid"], k, blockskip=2, row_stats=st, **kw)
        torch.cuda.synchronize()
        got = got.cpu().numpy()
        assert_parity(w, got, want)
        if kw:
            assert np.array_equal(got, want)
        s = st.cpu().numpy()
        assert all(s[r, 6] == 1 for r in range(w.num_rows)), s


def test_many_long_rows_take_the_streaming_tier(ert):
    """128+ decode rows longer than one resident workgroup holds, with at
    least 4 K blocks per row: the plan streams them (one workgroup per row,
    maxima made in the kernel) -- exact, rows with locality included."""
    import torch
    k = 512
    w = workloads.decode_blockskip(rows=128, stride=65536, k=k, lo=700, hi=65536, cfg=95)
    want = oracle.topk_workload(w)
    dev = to_dev(w)
    # the plain entry point (no options at all) plans the streaming tier too
    got = ert.topk_decode(dev["logits"], dev["n_valid"], k)
    torch.cuda.synchronize()
    assert_parity(w, got.cpu().numpy(), want)
    st = torch.full((w.num_rows, ert.STATS_WORDS), -7, dtype=torch.int32, device="cuda")
    got = ert.topk_decode(dev["logits"], dev["n_valid"], k, row_stats=st)
    torch.cuda.synchronize()
    assert_parity(w, got.cpu().numpy(), want)
    s = st.cpu().numpy()
    long_rows = [r for r in range(w.num_rows) if int(w.n_valid[r]) > k]
    assert all(s[r, 6] == 1 and s[r, 8] > 0 for r in long_rows), s[:4]
    # blockskip=-1 keeps the resident tiers
    st2 = torch.full((w.num_rows, ert.STATS_WORDS), -7, dtype=torch.int32, device="cuda")
    got = ert.topk_decode(dev["logits"], dev["n_valid"], k, row_stats=st2, blockskip=-1)
    torch.cuda.synchronize()
    assert_parity(w, got.cpu().numpy(), want)
    assert all(st2.cpu().numpy()[r, 6] > 1 for r in long_rows)


@pytest.mark.parametrize("dist", ["all_equal", "two_valued", "levels4", "signed_zero"])
def test_streaming_tier_tie_heavy_rows(ert, dist):
    """Tie-heavy rows in a batch the plan streams (128 x 65536, K = 512): the
    maxima give a floor equal to the row's top value class, so the pass ends
    in its radix ladder; exact, and deterministic ties are the smallest
    positions."""
    import torch
    k, rows, stride = 512, 128, 65536
    nv = [stride - (r % 5) for r in range(rows)]
    w = workloads.random_decode(rows, stride, nv, k, seed=len(dist) + 11, dist=dist)
    want = oracle.topk_workload(w)
    dev = to_dev(w)
    log(f"[stream ties] {dist}")
    st = torch.full((rows, ert.STATS_WORDS), -7, dtype=torch.int32, device="cuda")
    got = ert.topk_decode(dev["logits"], dev["n_valid"], k, row_stats=st)
    torch.cuda.synchronize()
    assert_parity(w, got.cpu().numpy(), want)
    assert all(st.cpu().numpy()[:, 6] == 1)  # one workgroup per row: the streaming tier
    got = ert.topk_decode(dev["logits"], dev["n_valid"], k, deterministic=True, sorted=True)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), want)
