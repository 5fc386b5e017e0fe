"""GPU tests of the output options: the values output, sorted output and
deterministic smallest-index ties.

With both sorted and deterministic, every row must equal the oracle's
canonical output index for index (positions by value descending, equal values
by position ascending; short rows identity + -1).
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import assert_parity, log, to_dev

pytestmark = pytest.mark.gpu

FLT_LOWEST = np.float32(-np.finfo(np.float32).max)


@pytest.fixture(scope="module")
def ert():
    import torch
    import exact_row_top_amd as m
    assert torch.cuda.is_available()
    m.load_library()
    return m


def _call(ert, w, dev=None, **kw):
    import torch
    dev = dev or to_dev(w)
    if w.mode == "decode":
        res = ert.topk_decode(dev["logits"], dev["n_valid"], w.k, **kw)
    else:
        res = ert.topk_prefill(dev["logits"], dev["row_starts"], dev["row_ends"], w.k, **kw)
    torch.cuda.synchronize()
    if isinstance(res, tuple):
        return res[0].cpu().numpy(), res[1].cpu().numpy()
    return res.cpu().numpy(), None


def _rows(w):
    ks, ke = w.windows()
    return [(int(a), int(b)) for a, b in zip(ks, ke)]


def _check_values(w, idx, vals):
    for r, ((ks, ke), row) in enumerate(zip(_rows(w), w.logits)):
        nv = ke - ks
        got = vals[r]
        if nv <= w.k:
            want = np.concatenate([row[ks:ke], np.full(w.k - nv, FLT_LOWEST, np.float32)])
        else:
            want = row[ks + idx[r]]
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"row {r}"


def _check_sorted(w, idx, vals):
    for r, (ks, ke) in enumerate(_rows(w)):
        if ke - ks <= w.k:
            continue
        v = w.logits[r, ks + idx[r]]
        assert np.all(v[:-1] >= v[1:]), f"row {r}: not value-descending"
        same = v[:-1] == v[1:]
        assert np.all(idx[r][:-1][same] < idx[r][1:][same]), f"row {r}: ties not by index"


WORKLOADS = {
    "decode_uniform": lambda: workloads.config(1),
    "decode_varlen": lambda: workloads.config(2),
    "prefill_subset": lambda: workloads.prefill_causal(requests=1),
    "tie_heavy": lambda: workloads.config(5),
    "long_skewed_bs8": lambda: workloads.long_skewed(bs=8),
}


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_values_output(ert, name):
    w = WORKLOADS[name]()
    log(f"[values] {name}")
    want = oracle.topk_workload(w)
    idx, vals = _call(ert, w, return_values=True)
    assert_parity(w, idx, want)
    _check_values(w, idx, vals)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_sorted_output(ert, name):
    w = WORKLOADS[name]()
    log(f"[sorted] {name}")
    want = oracle.topk_workload(w)
    idx, vals = _call(ert, w, return_values=True, sorted=True)
    assert_parity(w, idx, want)
    _check_sorted(w, idx, vals)
    _check_values(w, idx, vals)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_deterministic_sorted_equals_canonical(ert, name):
    w = WORKLOADS[name]()
    log(f"[canonical] {name}")
    want = oracle.topk_workload(w)
    dev = to_dev(w)
    for kw in ({}, {"force_rescue": True}):
        idx, _ = _call(ert, w, dev=dev, sorted=True, deterministic=True, **kw)
        bad = [r for r in range(w.num_rows) if not np.array_equal(idx[r], want[r])]
        assert not bad, f"{kw}: rows {bad[:8]} differ from the canonical output"


@pytest.mark.parametrize("k", [512, 2048])
@pytest.mark.parametrize("dist", ["levels4", "two_valued", "signed_zero", "neg_inf", "normal"])
def test_deterministic_ties_every_tier(ert, k, dist):
    # tie-heavy rows on every path: one workgroup, split, forced rescue
    rows, stride = 6, 16384
    nv = [16384, 16383, 9001, k + 1, k + 5, 12345]
    w = workloads.random_decode(rows, stride, nv, k, seed=k + 3 * len(dist), dist=dist)
    want = oracle.topk_workload(w)
    dev = to_dev(w)
    for kw in ({}, {"force_wgs_per_row": 1}, {"force_wgs_per_row": 5},
               {"force_rescue": True}, {"force_rescue": True, "force_wgs_per_row": 3}):
        log(f"[det] k={k} dist={dist} {kw}")
        idx, _ = _call(ert, w, dev=dev, deterministic=True, **kw)
        for r in range(rows):
            assert np.array_equal(np.sort(idx[r]), np.sort(want[r])), f"row {r} {kw}"
        idx2, _ = _call(ert, w, dev=dev, deterministic=True, sorted=True, **kw)
        assert np.array_equal(idx2, want), kw


def test_deterministic_calls_repeat_exactly(ert):
    w = workloads.config(5)
    dev = to_dev(w)
    first, _ = _call(ert, w, dev=dev, deterministic=True)
    for _ in range(3):
        again, _ = _call(ert, w, dev=dev, deterministic=True)
        assert np.array_equal(np.sort(first, axis=1), np.sort(again, axis=1))


def test_output_option_errors(ert):
    import torch
    w = workloads.config(1)
    dev = to_dev(w)
    with pytest.raises(TypeError):
        ert.topk_decode(dev["logits"], dev["n_valid"], w.k,
                        values=torch.empty((w.num_rows, w.k), dtype=torch.float64, device="cuda"))
    with pytest.raises(ValueError):
        ert.topk_decode(dev["logits"], dev["n_valid"], w.k,
                        values=torch.empty((w.num_rows, w.k + 1), dtype=torch.float32,
                                           device="cuda"))
