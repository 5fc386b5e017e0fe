"""GPU tests of the split tier's bounded row-barrier waits and topk_status.

The waits are made to give up from the host (barrier_spins=1: one poll, then
the workgroup moves on), so every kernel still exits normally; the count
topk_status hands back must then be non-zero, and the library-owned slab or a
re-zeroed caller workspace must serve the next call exactly again.
"""
import numpy as np
import pytest

import workloads
from gpu_helpers import assert_parity, log, run_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ert():
    import torch
    import exact_row_top_amd as m
    assert torch.cuda.is_available()
    m.load_library()
    return m


def _batch():
    # 16 rows of up to 65536 scores, K=2048: the planner splits every long row
    # over several workgroups (the tier with row barriers)
    return workloads.random_decode(16, 65536, [65536 - 97 * r for r in range(16)], 2048, seed=31)


def _count(ert):
    import torch
    c = ert.status()
    torch.cuda.synchronize()
    return int(c.item())


def test_quiet_calls_report_no_timeouts(ert):
    w = _batch()
    _count(ert)  # start from a clean count
    got, st = run_gpu(w, stats=True)
    assert np.all(st[:, 6] > 1), "the batch must take the split tier"
    assert_parity(w, got)
    assert _count(ert) == 0


def test_forced_timeouts_are_counted_and_the_slab_recovers(ert):
    w = _batch()
    dev = to_dev(w)
    _count(ert)
    log("[status] NULL slab, waits forced to give up")
    run_gpu(w, dev=dev, barrier_spins=1)  # results undefined by design
    assert _count(ert) > 0
    assert _count(ert) == 0  # the query reset it
    # status re-zeroed the slab: the same call is exact again
    assert_parity(w, run_gpu(w, dev=dev))
    assert _count(ert) == 0


def test_forced_timeouts_with_a_caller_workspace(ert):
    import torch
    w = _batch()
    dev = to_dev(w)
    ws = ert.new_workspace(w.num_rows, w.row_stride, w.k)
    assert ws is not None
    _count(ert)
    log("[status] caller workspace, waits forced to give up")
    run_gpu(w, dev=dev, workspace=ws, barrier_spins=1)
    assert _count(ert) > 0
    # the caller re-zeroes its own workspace, then it serves exactly again
    ert.load_library().topk_workspace_init(ws.data_ptr(), ws.numel(), None)
    torch.cuda.synchronize()
    for _ in range(2):
        assert_parity(w, run_gpu(w, dev=dev, workspace=ws))
    assert _count(ert) == 0
