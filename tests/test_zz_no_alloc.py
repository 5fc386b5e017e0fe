"""GPU test of topk_decode_noalloc, the decode entry point that allocates
nothing (its split tier keeps its state in the library's fixed per-GPU
scratch array), called through the C ABI.

Its output must match topk_decode's (the existing entry point, here with a
caller workspace) to the parity bar: short rows index for index, long rows
the same value multiset bit for bit (indices interchange only inside the k-th
value's tie class), and both must pass the oracle.  Two calls in a row, the
second on a smaller input, so the second call finds the array as the first
left it.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import log, run_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ert():
    import torch
    import exact_row_top_amd as m
    assert torch.cuda.is_available()
    m.load_library()
    return m


def _noalloc(ert, w, dev):
    import torch
    out = torch.full((w.num_rows, w.k), -9, dtype=torch.int32, device="cuda")
    rc = ert.load_library().topk_decode_noalloc(
        dev["logits"].data_ptr(), w.row_stride, dev["n_valid"].data_ptr(), w.num_rows, w.k,
        out.data_ptr(), None)
    assert rc == ert.TOPK_OK, ert.strerror(rc)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check_against_decode(ert, w):
    dev = to_dev(w)
    ws = ert.new_workspace(w.num_rows, w.row_stride, w.k)
    ref = run_gpu(w, dev=dev, workspace=ws)
    bad = oracle.check_rows(w, ref)
    assert not bad, f"topk_decode: {bad[:3]}"
    got = _noalloc(ert, w, dev)
    bad = oracle.check_rows(w, got, want=ref)
    assert not bad, f"noalloc vs topk_decode: {bad[:3]}"
    return got


def test_noalloc_matches_decode_twice_second_smaller(ert):
    # 1: the decode varlen batch (64 x 131072, K=2048: split rows, boundary
    # rows 2047/2048/2049/0); 2: a smaller split batch on the same scratch
    w1 = workloads.decode_varlen()
    log(f"[noalloc] call 1: {w1.name}")
    _check_against_decode(ert, w1)
    w2 = workloads.random_decode(8, 65536, [65536, 40000, 2048, 70, 65535, 3000, 52001, 0],
                                 1024, seed=77, dist="levels4")
    log(f"[noalloc] call 2: {w2.name}")
    _check_against_decode(ert, w2)


def test_noalloc_tie_heavy_and_one_workgroup_rows(ert):
    # rescue paths through the scratch (tie-heavy rows), then one-workgroup rows
    w = workloads.tie_heavy()
    log(f"[noalloc] {w.name}")
    _check_against_decode(ert, w)
    w = workloads.decode_uniform()
    log(f"[noalloc] {w.name}")
    _check_against_decode(ert, w)


def test_noalloc_empty_and_invalid_calls(ert):
    # num_rows == 0 is a no-op; k outside {512, 1024, 2048} is rejected on the
    # host before any launch
    import torch
    x = torch.zeros(16, dtype=torch.float32, device="cuda")
    n = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib = ert.load_library()
    assert lib.topk_decode_noalloc(x.data_ptr(), 16, n.data_ptr(), 0, 512, out.data_ptr(),
                                   None) == ert.TOPK_OK
    assert lib.topk_decode_noalloc(x.data_ptr(), 16, n.data_ptr(), 1, 100, out.data_ptr(),
                                   None) == ert.TOPK_EINVAL
