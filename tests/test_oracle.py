"""Pins of the CPU oracle against things other than itself (no GPU).

Each check is chosen so a plausible slip in the oracle -- a reversed order, a
wrong tie-break, a dropped clamp, a frame offset, -0/+0 treated as distinct,
-inf treated as padding -- fails at least one of them:

- hand-worked contract cases (tests/golden/contract_cases.txt);
- an independent pure-Python brute force on small rows;
- exhaustive enumeration of tiny rows over an alphabet with every special value;
- numpy's sort as a library special case for the selected value multiset;
- closed forms for degenerate rows (all equal, two-valued, -inf and +-0 classes,
  a unique-answer row);
- invariants (distinct, in range, min selected >= max unselected);
- metamorphic relations (poison immunity, prefill window == decode of the window).
"""
import itertools
import math

import numpy as np
import pytest

import oracle
import workloads
from conftest import load_golden


def _parse_row(s):
    return np.array([float(t) for t in s.split()], dtype=np.float32)


@pytest.mark.parametrize("case", load_golden("contract_cases.txt"), ids=lambda c: c["case"])
def test_golden_contract_cases(case):
    row = _parse_row(case["row"])
    k = int(case["k"])
    ks, ke = int(case["ks"]), int(case["ke"])
    want = [int(t) for t in case["expect"].split()]
    x = row[None, :]
    got_p = oracle.topk_prefill(x, np.array([ks], np.int32), np.array([ke], np.int32), k)
    assert got_p[0].tolist() == want
    if ks == 0:
        got_d = oracle.topk_decode(x, np.array([ke], np.int32), k)
        assert got_d[0].tolist() == want


def test_brute_force_random_small_rows():
    rng = np.random.default_rng(1234)
    for trial in range(400):
        n = int(rng.integers(1, 80))
        k = int(rng.integers(1, 90))
        alphabet = rng.choice([2, 3, 5, 1000])
        vals = (rng.integers(0, alphabet, n) - alphabet // 2).astype(np.float32) * np.float32(0.5)
        if trial % 3 == 0:
            vals[rng.random(n) < 0.2] = -np.inf
        if trial % 5 == 0:
            z = vals == 0
            vals[z & (rng.random(n) < 0.5)] = -0.0
        want = oracle.brute_force_row(vals.tolist(), k)
        got = oracle.topk_window(vals, k).tolist()
        assert got == want, (n, k, vals.tolist())


def test_brute_force_just_above_k():
    # nv = K+1 .. K+64 at the library's K values, brute force by full Python sort.
    rng = np.random.default_rng(7)
    for k in (512, 1024, 2048):
        for extra in (1, 2, 3, 17, 63, 64):
            n = k + extra
            vals = rng.standard_normal(n).astype(np.float32)
            vals[rng.random(n) < 0.05] = vals[0]  # a tie class
            want = oracle.brute_force_row(vals.tolist(), k)
            got = oracle.topk_decode(vals[None, :], np.array([n], np.int32), k)[0].tolist()
            assert got == want


ALPHABET = [-math.inf, -1.5, -0.0, 0.0, 1.5, math.inf]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_exhaustive_tiny_rows(n):
    rows = list(itertools.product(ALPHABET, repeat=n))
    mat = np.array(rows, dtype=np.float32).reshape(len(rows), n)
    for k in range(1, n + 2):
        got = oracle.topk_decode(mat, np.full(len(rows), n, np.int32), k)
        for i, r in enumerate(rows):
            assert got[i].tolist() == oracle.brute_force_row(list(r), k), (r, k)


def test_exhaustive_len6_sampled_k():
    rows = list(itertools.product(ALPHABET, repeat=6))
    mat = np.array(rows, dtype=np.float32)
    for k in (1, 3, 5):
        got = oracle.topk_decode(mat, np.full(len(rows), 6, np.int32), k)
        for i in range(0, len(rows), 7):
            assert got[i].tolist() == oracle.brute_force_row(list(rows[i]), k)


@pytest.mark.parametrize("dist", workloads.DISTS)
@pytest.mark.parametrize("k", [512, 2048])
def test_value_multiset_matches_numpy_sort(dist, k):
    w = workloads.random_decode(3, 9000, [9000, 5000, k + 5], k, seed=11, dist=dist)
    out = oracle.topk_workload(w)
    for r in range(w.num_rows):
        nv = int(w.n_valid[r])
        win = w.logits[r, :nv]
        sel = win[out[r]]
        ref = np.sort(win)[-k:]
        assert np.array_equal(np.sort(sel), ref)  # numeric equality: -0 == +0
        assert np.unique(out[r]).shape[0] == k
        assert out[r].min() >= 0 and out[r].max() < nv
        mask = np.ones(nv, bool)
        mask[out[r]] = False
        if mask.any():
            assert sel.min() >= win[mask].max()


def test_canonical_order_and_tie_pick():
    rng = np.random.default_rng(3)
    v = np.floor(rng.random(5000) * 8).astype(np.float32)
    out = oracle.topk_window(v, 700)
    sel = v[out]
    assert np.all(np.diff(sel) <= 0)  # values non-increasing
    for a, b in zip(out[:-1], out[1:]):
        if v[a] == v[b]:
            assert a < b  # equal values by smaller position
    tau = sel[-1]
    # every strictly larger value is in; the tie class contributes its smallest positions
    assert set(np.nonzero(v > tau)[0]) <= set(out.tolist())
    ties = np.nonzero(v == tau)[0]
    need = 700 - int((v > tau).sum())
    assert set(out.tolist()) - set(np.nonzero(v > tau)[0]) == set(ties[:need].tolist())


def test_closed_form_all_equal():
    for k in (512, 1024, 2048):
        v = np.full(10000, 0.5, np.float32)
        assert oracle.topk_window(v, k).tolist() == list(range(k))


def test_closed_form_two_valued():
    rng = np.random.default_rng(5)
    v = np.where(rng.random(20000) < 0.01, 2.0, 1.0).astype(np.float32)
    hi = np.nonzero(v == 2.0)[0]
    lo = np.nonzero(v == 1.0)[0]
    k = 1024
    assert hi.shape[0] < k
    want = hi.tolist() + lo[: k - hi.shape[0]].tolist()
    assert oracle.topk_window(v, k).tolist() == want


def test_closed_form_neg_inf_class():
    rng = np.random.default_rng(6)
    v = np.full(30000, -np.inf, np.float32)
    pos = rng.permutation(30000)
    v[pos[:300]] = rng.standard_normal(300)
    k = 512
    fin = np.nonzero(np.isfinite(v))[0]
    fin_sorted = sorted(fin.tolist(), key=lambda i: (-float(v[i]), i))
    neg = np.nonzero(np.isinf(v))[0]
    want = fin_sorted + neg[: k - 300].tolist()
    got = oracle.topk_window(v, k).tolist()
    assert got == want
    assert all(0 <= i < 30000 for i in got)


def test_closed_form_signed_zero_class():
    rng = np.random.default_rng(8)
    n = 40000
    v = (-5.0 + rng.standard_normal(n)).astype(np.float32)
    pos = rng.permutation(n)
    v[pos[:100]] = 5.0 + rng.standard_normal(100)
    zpos = pos[100:5100]
    v[zpos] = np.where(rng.random(5000) < 0.5, -0.0, 0.0)
    k = 1024
    pos_sorted = sorted(pos[:100].tolist(), key=lambda i: (-float(v[i]), i))
    zeros = np.sort(zpos)
    want = pos_sorted + zeros[: k - 100].tolist()
    assert oracle.topk_window(v, k).tolist() == want


def test_closed_form_unique_answer_row():
    # Tie-heavy workload row 6: 1500 scores in [100, 200), 40000 distinct floats
    # just above 1.0, the rest below 0.5.  The top 2048 are the 1500 plus the 548
    # largest distinct floats: a unique set.
    n, k = 262144, 2048
    v = workloads.tie_row("dense_bin40k", n, workloads.row_rng(5, 6))
    big = np.nonzero(v >= 100.0)[0]
    assert big.shape[0] == 1500
    near1 = np.nonzero((v >= 1.0) & (v < 2.0))[0]
    assert near1.shape[0] == 40000
    bits = v[near1].view(np.uint32)
    top548 = near1[np.argsort(bits)[-548:]]
    got = oracle.topk_window(v, k)
    assert set(got.tolist()) == set(big.tolist()) | set(top548.tolist())


def test_decode_clamps():
    x = np.arange(40, dtype=np.float32).reshape(2, 20)
    # n_valid < 0 -> empty row; n_valid > stride -> whole row
    out = oracle.topk_decode(x, np.array([-5, 99], np.int32), 4)
    assert out[0].tolist() == [-1, -1, -1, -1]
    assert out[1].tolist() == [19, 18, 17, 16]


def test_prefill_clamps():
    x = np.arange(60, dtype=np.float32).reshape(3, 20)
    ks = np.array([5, -3, 18], np.int32)
    ke = np.array([2, 4, 99], np.int32)  # ke < ks -> empty; ks < 0 -> 0; ke > stride -> stride
    out = oracle.topk_prefill(x, ks, ke, 3)
    assert out[0].tolist() == [-1, -1, -1]
    assert out[1].tolist() == [3, 2, 1]
    assert out[2].tolist() == [0, 1, -1]


def test_prefill_window_equals_decode_of_window():
    rng = np.random.default_rng(9)
    k = 512
    for s in (0, 1, 2, 3, 4, 65, 130, 195):
        n = 3000
        base = rng.standard_normal(n).astype(np.float32)
        stride = 3400
        row = workloads.poison_fill(stride, workloads.POISON_PREFILL).copy()
        row[s:s + n] = base
        p = oracle.topk_prefill(row[None], np.array([s], np.int32), np.array([s + n], np.int32), k)
        d = oracle.topk_decode(base[None], np.array([n], np.int32), k)
        assert np.array_equal(p, d)


def test_poison_immunity():
    rng = np.random.default_rng(10)
    k = 1024
    n, stride = 5000, 6000
    base = rng.standard_normal(n).astype(np.float32)
    outs = []
    for pat in (workloads.POISON_DECODE, workloads.POISON_PREFILL, (0.0,), (-np.inf,), (1e30,)):
        row = workloads.poison_fill(stride, pat).copy()
        row[:n] = base
        outs.append(oracle.topk_decode(row[None], np.array([n], np.int32), k))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_nan_row_is_rejected():
    v = np.ones((1, 3000), np.float32)
    v[0, 7] = np.nan
    out, rej = oracle.topk_decode(v, np.array([3000], np.int32), 512, return_rejected=True)
    assert rej == 1
    # NaN outside the window does not matter
    out, rej = oracle.topk_decode(v, np.array([7], np.int32), 512, return_rejected=True)
    assert rej == 0


def test_threads_do_not_change_results():
    w = workloads.random_decode(16, 4096, np.arange(16) * 256 + 100, 512, seed=12)
    a = oracle.topk_decode(w.logits, w.n_valid, 512, nthreads=1)
    b = oracle.topk_decode(w.logits, w.n_valid, 512, nthreads=8)
    assert np.array_equal(a, b)


# --- the checker itself -------------------------------------------------------

def test_checker_accepts_tie_interchange_and_rejects_mistakes():
    v = np.array([1, 5, 5, -0.0, 0, 5, 2, 3], np.float32)
    k = 6
    want = oracle.topk_window(v, k)
    assert want.tolist() == [1, 2, 5, 7, 6, 0]
    # any order, and the zero class is not reached: fine
    assert oracle.check_row(v, np.array([0, 6, 7, 5, 2, 1]), want, k) is None
    # planted mistakes
    assert oracle.check_row(v, np.array([1, 2, 5, 7, 6, 3]), want, k) is not None  # 0 instead of 1
    assert oracle.check_row(v, np.array([1, 2, 5, 7, 6, 6]), want, k) is not None  # duplicate
    assert oracle.check_row(v, np.array([1, 2, 5, 7, 6, 8]), want, k) is not None  # out of range
    assert oracle.check_row(v, np.array([1, 2, 5, 7, 6, -1]), want, k) is not None  # pad in long row
    # tie class at -0/+0: either zero is acceptable
    k = 7
    want = oracle.topk_window(v, k)
    assert oracle.check_row(v, np.array([1, 2, 5, 7, 6, 0, 4]), want, k) is None
    # short rows must be index-exact
    s = v[:3]
    want = oracle.topk_window(s, 4)
    assert oracle.check_row(s, np.array([0, 1, 2, -1]), want, 4) is None
    assert oracle.check_row(s, np.array([1, 0, 2, -1]), want, 4) is not None


def test_workload_shapes_and_bytes():
    w1 = workloads.config(1)
    assert w1.logits.shape == (4, 4096) and w1.k == 512
    assert w1.algorithmic_bytes() == 65536 + 8192 + 16
    w3 = workloads.prefill_causal()
    ks, ke = w3.windows()
    assert set((ks % 4).tolist()) == {0, 1, 2, 3}
    nv = ke - ks
    assert nv.min() == 1 and nv.max() == 16384
    assert int((nv <= 1024).sum()) == 256
    assert int(4 * nv[nv > 1024].sum()) == 133700640
    assert w3.row_stride * 4 % 1024 == 0 and w3.row_stride - int(ke.max()) >= 0
    w2 = workloads.decode_varlen()
    assert [int(w2.n_valid[r]) for r in (7, 23, 40, 63)] == [2047, 2048, 2049, 0]
    n0 = int(w2.n_valid[0])
    pad = w2.logits[0, n0:]
    cols = np.arange(n0, w2.row_stride)
    assert np.all(np.isposinf(pad[cols % 3 == 0]))
    assert np.all(np.isnan(pad[cols % 3 == 1]))
    assert np.all(pad[cols % 3 == 2] == np.float32(3e38))
    w4 = workloads.long_skewed(bs=1)
    assert w4.logits.shape == (1, 131072)
    hot = w4.logits[0, :114963] > 120
    assert 1100 < int(hot.sum()) <= 1150
    assert int(hot[: int(0.8 * 114963)].sum()) == 0


# ---- varlen / MTP decode form ---------------------------------------------------

@pytest.mark.parametrize("case", load_golden("varlen_windows.txt"), ids=lambda c: c["case"])
def test_varlen_windows_golden(case):
    kv = [int(t) for t in case["kv_lens"].split()]
    got = oracle.varlen_n_valid(kv, int(case["rows"]), int(case["next_n"]), int(case["cr"]),
                                int(case["stride"]))
    assert got.tolist() == [int(t) for t in case["expect"].split()]


def test_varlen_window_properties():
    rng = np.random.default_rng(5)
    for next_n in (1, 2, 3, 4):
        for cr in (1, 4):
            kv = rng.integers(0, 5000, size=17)
            rows = 17 * next_n
            n = oracle.varlen_n_valid(kv, rows, next_n, cr, 1 << 20)
            for q in range(17):
                seg = n[q * next_n:(q + 1) * next_n]
                if kv[q] < next_n:
                    assert np.all(seg == 0)
                    continue
                # the last MTP row sees the whole (compressed) cache
                assert seg[-1] == kv[q] // cr
                # later MTP rows never see less, and with cr = 1 one more each
                assert np.all(np.diff(seg) >= 0)
                if cr == 1:
                    assert np.all(np.diff(seg) == 1)
            if next_n == 1 and cr == 1:
                assert np.array_equal(n, kv)  # the plain decode form


def test_varlen_oracle_is_decode_on_its_windows():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((8, 3000)).astype(np.float32)
    kv = np.array([2999, 1200, 1, 2400], dtype=np.int32)
    got = oracle.topk_varlen(x, kv, 2, 1, 512)
    nv = np.array([2998, 2999, 1199, 1200, 0, 0, 2399, 2400], dtype=np.int32)
    assert np.array_equal(got, oracle.topk_decode(x, nv, 512))
    assert got[4].tolist() == [-1] * 512
