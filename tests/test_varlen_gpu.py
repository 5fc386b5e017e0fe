"""GPU parity of the varlen / MTP decode form: per-request device kv_lens, the
row window computed on the device, against the oracle on the windows the
oracle's own reading of the contract gives."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import assert_parity, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ert():
    import torch
    import exact_row_top_amd as m
    assert torch.cuda.is_available()
    m.load_library()
    return m


def _varlen_case(kv, next_n, cr, stride, k, seed):
    """Rows of N(0,1) scores; every cell at or beyond the row's window (from
    the oracle's reading) is poisoned; plus the decode-form view of it."""
    rows = len(kv) * next_n
    w = workloads.random_decode(rows, stride, [stride] * rows, k, seed=seed, dist="normal")
    nv = oracle.varlen_n_valid(kv, rows, next_n, cr, stride)
    poison = np.array(workloads.POISON_DECODE, dtype=np.float32)
    for r in range(rows):
        cols = np.arange(int(nv[r]), stride)
        w.logits[r, cols] = poison[cols % 3]
    w.n_valid = nv.astype(np.int32)
    return w


def _kv_mix(k, cr, stride, next_n, rng):
    # below next_n, around the short-row boundary, mid, and the stride edge
    # (all in uncompressed token space)
    kv = [0, next_n - 1, next_n, k * cr - 1, k * cr, k * cr + next_n, (k + 1) * cr + 3,
          int(rng.integers(k * cr, stride * cr)), stride * cr, stride * cr + 7 * cr]
    return np.array([max(0, v) for v in kv], dtype=np.int32)


@pytest.mark.parametrize("cr", [1, 4])
@pytest.mark.parametrize("next_n", [1, 2, 3, 4])
@pytest.mark.parametrize("k", [512, 2048])
def test_varlen_parity(ert, k, next_n, cr):
    import torch
    stride = 8 * k + 64
    rng = np.random.default_rng(k + 10 * next_n + cr)
    kv = _kv_mix(k, cr, stride, next_n, rng)
    w = _varlen_case(kv, next_n, cr, stride, k, seed=next_n * 7 + cr)
    want = oracle.topk_workload(w)
    x = torch.from_numpy(w.logits).cuda()
    kvd = torch.from_numpy(kv).cuda()
    for kw in ({}, {"force_wgs_per_row": 1}, {"force_wgs_per_row": 4}, {"force_rescue": True}):
        log(f"[varlen] k={k} next_n={next_n} cr={cr} {kw}")
        got = ert.topk_decode_varlen(x, kvd, k, next_n=next_n, compress_ratio=cr, **kw)
        torch.cuda.synchronize()
        assert_parity(w, got.cpu().numpy(), want)


def test_varlen_values_and_canonical(ert):
    import torch
    k, next_n, cr, stride = 1024, 2, 4, 16384
    kv = np.array([0, 3, 4096, 4097, 5000, 40000, 65536, 70000], dtype=np.int32)
    w = _varlen_case(kv, next_n, cr, stride, k, seed=91)
    want = oracle.topk_workload(w)
    x = torch.from_numpy(w.logits).cuda()
    kvd = torch.from_numpy(kv).cuda()
    idx, vals = ert.topk_decode_varlen(x, kvd, k, next_n=next_n, compress_ratio=cr,
                                       return_values=True, sorted=True, deterministic=True)
    torch.cuda.synchronize()
    idx, vals = idx.cpu().numpy(), vals.cpu().numpy()
    assert np.array_equal(idx, want)
    for r in range(w.num_rows):
        n = int(w.n_valid[r])
        if n <= k:
            wantv = np.concatenate([w.logits[r, :n],
                                    np.full(k - n, -np.finfo(np.float32).max, np.float32)])
        else:
            wantv = w.logits[r, idx[r]]
        assert np.array_equal(vals[r].view(np.uint32), wantv.view(np.uint32)), r


def test_varlen_graph_replay_with_growing_cache(ert):
    # One captured launch, replayed while kv_lens grows in place: rows cross
    # the short-row boundary and the stride edge inside the graph.
    import torch
    k, next_n, cr, stride = 512, 2, 1, 8192
    kv0 = np.array([100, 500, 511, 6000, 8100], dtype=np.int32)
    rows = len(kv0) * next_n
    w = workloads.random_decode(rows, stride, [stride] * rows, k, seed=17, dist="normal")
    x = torch.from_numpy(w.logits).cuda()
    kvd = torch.from_numpy(kv0.copy()).cuda()
    out = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    ws = ert.new_workspace(rows, stride, k)
    ert.topk_decode_varlen(x, kvd, k, next_n=next_n, compress_ratio=cr, indices=out,
                           workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            ert.topk_decode_varlen(x, kvd, k, next_n=next_n, compress_ratio=cr, indices=out,
                                   workspace=ws)
    torch.cuda.synchronize()
    for step in range(6):
        kv = np.minimum(kv0 + 7 * step, 8300).astype(np.int32)
        kvd.copy_(torch.from_numpy(kv))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = oracle.topk_varlen(w.logits, kv, next_n, cr, k)
        view = workloads.Workload("varlen_graph", "decode", w.logits, k,
                                  n_valid=oracle.varlen_n_valid(kv, rows, next_n, cr,
                                                                stride).astype(np.int32))
        assert_parity(view, out.cpu().numpy(), want)
