"""GPU parity on seeded random shapes: decode and prefill batches of random
row counts, strides, K, valid lengths and score distributions, on the default
plan, forced split counts and the forced rescue, with and without the
canonical (deterministic, sorted) output."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import log, run_gpu

pytestmark = pytest.mark.gpu

DISTS = ("normal", "uniform", "levels4", "two_valued", "signed_zero", "hidden_peak", "ramp_up",
         "ramp_down", "neg_inf", "pos_inf", "all_equal", "huge", "tiny")


@pytest.fixture(scope="module")
def ert():
    import torch
    import exact_row_top_amd as m
    assert torch.cuda.is_available()
    m.load_library()
    return m


def _case(g):
    k = int(g.choice([512, 1024, 2048]))
    stride = int(g.choice([8192, 16640, 32768, 65536, 131072, 262144]))
    rows = int(g.integers(1, 33 if stride <= 131072 else 9))
    dist = str(g.choice(DISTS))
    seed = int(g.integers(1 << 30))
    if g.random() < 0.5:
        nv = g.integers(0, stride + 1, rows)
        nv[g.random(rows) < 0.15] = k + int(g.integers(-2, 3))
        w = workloads.random_decode(rows, stride, nv, k, seed=seed, dist=dist)
    else:
        ks = g.integers(0, stride // 2, rows)
        ke = ks + g.integers(0, stride // 2 + 1, rows)
        exact = g.random(rows) < 0.15
        ke[exact] = ks[exact] + k
        w = workloads.random_prefill(ks, ke, stride, k, seed=seed, dist=dist)
    kw = {}
    if g.random() < 0.25:
        kw["force_wgs_per_row"] = int(g.choice([3, 8, 16, 40, 64]))
    if g.random() < 0.25:
        kw["force_rescue"] = True
    if g.random() < 0.5:
        kw["deterministic"] = True
        kw["sorted"] = True
    return w, kw


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes(ert, seed):
    g = np.random.default_rng([seed, 2718])
    w, kw = _case(g)
    if kw.get("force_wgs_per_row"):
        try:
            ert.plan_query(w.num_rows, w.logits.shape[1], w.k,
                           force_wgs_per_row=kw["force_wgs_per_row"])
        except ert.TopKError:
            kw.pop("force_wgs_per_row")  # too few parts for this stride
    log(f"[random] seed={seed} {w.name} {kw}")
    got = run_gpu(w, **kw)
    bad = oracle.check_rows(w, got)
    assert not bad, f"{w.name} {kw}: {bad[:3]}"
    if kw.get("deterministic"):
        want = oracle.topk_workload(w)
        diff = [r for r in range(w.num_rows) if not np.array_equal(got[r], want[r])]
        assert not diff, f"{w.name} {kw}: rows {diff[:8]} differ from the canonical output"
