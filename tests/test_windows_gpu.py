"""GPU parity on window geometry: every lead (a window starting 0-3 scores
past a 16-byte boundary) against lengths at the edges of a thread's float4
group, of a wave's 64 groups, of a workgroup's 256 groups and of the
resident row's capacity, in both one-workgroup shapes (256 threads x 8 and
x 17 groups) and in the split tier.  These are the rows whose first or last
group holds NaN markers -- the lanes the one-workgroup histogram counts with
everything else and then takes out of the NaN bin -- and the rows where a
wave visits one group fewer than its neighbours."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import assert_parity, log, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ert():
    import torch
    import exact_row_top_amd as m
    assert torch.cuda.is_available()
    m.load_library()
    return m


def _lengths(k, cap):
    base = [k + 1, k + 2, k + 3, k + 4, k + 5, 1023, 1024, 1025, 1029, 4093, 4096, 4097,
            4099, 8185, 8187, 8188, 16381, 16383, 16384, 17397, 17400, 17401, 17404]
    return sorted({n for n in base if k < n <= cap})


# Largest row strides the one-workgroup shapes take: a window of the whole
# stride plus up to three lead scores must fit 256 threads x 8 (17) float4
# groups.
STRIDE = {"g8": 8188, "g17": 17404}


@pytest.mark.parametrize("k", [512, 1024, 2048])
@pytest.mark.parametrize("shape", ["g8", "g17"])
@pytest.mark.parametrize("dist", ["normal", "levels4", "neg_inf", "signed_zero", "all_equal"])
def test_leads_and_lengths(ert, k, shape, dist):
    stride = STRIDE[shape]
    starts, ends = [], []
    for lead in range(4):
        for base in (0, 64):
            s = base + lead
            for n in _lengths(k, stride - s):
                starts.append(s)
                ends.append(s + n)
    w = workloads.random_prefill(starts, ends, stride, k, seed=11, dist=dist)
    plan = ert.plan_query(w.num_rows, stride, k, force_wgs_per_row=1)
    assert plan["block"] * plan["quads_per_thread"] == (2048 if shape == "g8" else 4352), plan
    for kw in ({"force_wgs_per_row": 1}, {"force_wgs_per_row": 4}):
        log(f"[windows] k={k} {shape} {dist} rows={w.num_rows} {kw}")
        got = run_gpu(w, **kw)
        assert_parity(w, got)


@pytest.mark.parametrize("k", [512, 1024])
def test_leads_with_many_rows(ert, k):
    # enough rows that the default plan takes one workgroup per row on its own
    rng = np.random.default_rng(5)
    rows = 1024
    stride = 16640
    lead = rng.integers(0, 4, rows)
    n = rng.integers(k + 1, 16385, rows)
    starts = (16 + lead).astype(np.int32)
    ends = np.minimum(starts + n, stride - 4).astype(np.int32)
    w = workloads.random_prefill(starts, ends, stride, k, seed=13, dist="normal")
    log(f"[windows] many rows k={k}")
    got = run_gpu(w)
    assert_parity(w, got)


@pytest.mark.parametrize("dist", ["signed_zero", "two_valued"])
def test_split_rescue_repeated_calls(ert, dist):
    # Tie-heavy windows whose tie class barely exceeds what is needed (a
    # wrong count anywhere in the row's merged digit counts moves the
    # threshold) through the split rescue, many calls in a row on the same
    # workspace: every call must match the oracle and leave the slots at rest.
    import torch
    k, stride = 2048, STRIDE["g17"]
    starts, ends = [], []
    for lead in range(4):
        for base in (0, 64):
            s = base + lead
            for n in _lengths(k, stride - s):
                starts.append(s)
                ends.append(s + n)
    w = workloads.random_prefill(starts, ends, stride, k, seed=11, dist=dist)
    dev = {"logits": torch.from_numpy(np.ascontiguousarray(w.logits)).cuda(),
           "row_starts": torch.from_numpy(np.ascontiguousarray(w.row_starts)).cuda(),
           "row_ends": torch.from_numpy(np.ascontiguousarray(w.row_ends)).cuda()}
    want = oracle.topk_workload(w)
    log(f"[windows] repeated split rescue {dist} rows={w.num_rows}")
    for rep in range(24):
        out = torch.full((w.num_rows, k), -7, dtype=torch.int32, device="cuda")
        ert.topk_prefill(dev["logits"], dev["row_starts"], dev["row_ends"], k, indices=out,
                         force_wgs_per_row=4)
        torch.cuda.synchronize()
        bad = oracle.check_rows(w, out.cpu().numpy(), want)
        assert not bad, f"call {rep}: {len(bad)} bad rows, first {bad[:3]}"
