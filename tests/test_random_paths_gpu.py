"""GPU parity on seeded random cases of the optional paths: the block-skip
pass with block maxima (forced), the streaming pass (forced), hint-guided
decode with hints of every quality, and the varlen / MTP form -- every
score distribution of the generators, checked against the oracle, and the
canonical output index for index where deterministic + sorted is asked."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import log, to_dev

pytestmark = pytest.mark.gpu

DISTS = workloads.DISTS


@pytest.fixture(scope="module")
def ert():
    import torch
    import exact_row_top_amd as m
    assert torch.cuda.is_available()
    m.load_library()
    return m


def _opts(g):
    return {"deterministic": True, "sorted": True} if g.random() < 0.5 else {}


def _check(w, got, kw):
    bad = oracle.check_rows(w, got)
    assert not bad, f"{w.name} {kw}: {bad[:3]}"
    if kw.get("deterministic"):
        want = oracle.topk_workload(w)
        diff = [r for r in range(w.num_rows) if not np.array_equal(got[r], want[r])]
        assert not diff, f"{w.name} {kw}: rows {diff[:8]} differ from the canonical output"


def _decode(g, rows_hi, strides, long_frac=0.8):
    k = int(g.choice([512, 1024, 2048]))
    stride = int(g.choice([s for s in strides if s >= 4 * k]))
    rows = int(g.integers(1, rows_hi + 1))
    dist = str(g.choice(DISTS))
    nv = np.where(g.random(rows) < long_frac, g.integers(k + 1, stride + 1, rows),
                  g.integers(0, k + 1, rows))
    return workloads.random_decode(rows, stride, nv, k, seed=int(g.integers(1 << 30)), dist=dist)


@pytest.mark.parametrize("seed", range(6))
def test_random_blockskip_with_block_maxima(ert, seed):
    import torch
    g = np.random.default_rng([seed, 31])
    w = _decode(g, 12, (32768, 65536, 131072, 262144))
    kw = _opts(g)
    dev = to_dev(w)
    bm = ert.block_max(dev["logits"])
    log(f"[random block-skip] seed={seed} {w.name} {kw}")
    got = ert.topk_decode(dev["logits"], dev["n_valid"], w.k, bmax=bm, blockskip=1, **kw)
    torch.cuda.synchronize()
    _check(w, got.cpu().numpy(), kw)


@pytest.mark.parametrize("seed", range(6))
def test_random_streaming_pass(ert, seed):
    import torch
    g = np.random.default_rng([seed, 37])
    w = _decode(g, 12, (32768, 65536, 131072, 262144))
    kw = _opts(g)
    dev = to_dev(w)
    log(f"[random streaming] seed={seed} {w.name} {kw}")
    got = ert.topk_decode(dev["logits"], dev["n_valid"], w.k, blockskip=2, **kw)
    torch.cuda.synchronize()
    _check(w, got.cpu().numpy(), kw)


def _hints(g, w, want):
    """Hints of a random quality: the true top-K, a partial overlap, random
    positions, duplicates, -1 pads or positions past the window."""
    rows, k = w.num_rows, w.k
    h = np.full((rows, k), -1, dtype=np.int32)
    kind = str(g.choice(["exact", "overlap", "random", "dup", "pad", "past"]))
    for r in range(rows):
        nv = int(w.n_valid[r])
        if kind == "exact":
            h[r] = want[r]
        elif kind == "overlap":
            keep = want[r][g.random(k) < 0.7]
            fill = g.integers(0, max(nv, 1), k - keep.size)
            h[r] = np.concatenate([keep, fill]).astype(np.int32)
        elif kind == "random":
            h[r] = g.integers(0, max(nv, 1), k)
        elif kind == "dup":
            h[r] = int(g.integers(0, max(nv, 1)))
        elif kind == "past":
            h[r] = nv + g.integers(0, 1000, k)
    return h, kind


@pytest.mark.parametrize("seed", range(8))
def test_random_hinted_decode(ert, seed):
    import torch
    g = np.random.default_rng([seed, 41])
    w = _decode(g, 16, (8192, 16640, 65536, 131072))
    want = oracle.topk_workload(w)
    h, kind = _hints(g, w, want)
    kw = _opts(g)
    if g.random() < 0.3:
        kw["force_wgs_per_row"] = int(g.choice([1, 4]))
    dev = to_dev(w)
    log(f"[random hints] seed={seed} {w.name} {kind} {kw}")
    try:
        got = ert.topk_decode(dev["logits"], dev["n_valid"], w.k,
                              pre_idx=torch.from_numpy(h).cuda(), **kw)
    except ert.TopKError:
        assert kw.pop("force_wgs_per_row", None) is not None  # a forced shape that does not fit
        got = ert.topk_decode(dev["logits"], dev["n_valid"], w.k,
                              pre_idx=torch.from_numpy(h).cuda(), **kw)
    torch.cuda.synchronize()
    _check(w, got.cpu().numpy(), kw)


@pytest.mark.parametrize("seed", range(8))
def test_random_varlen(ert, seed):
    import torch
    g = np.random.default_rng([seed, 43])
    k = int(g.choice([512, 1024, 2048]))
    next_n = int(g.integers(1, 5))
    cr = int(g.choice([1, 2, 4]))
    stride = int(g.choice([4 * k + 64, 8192, 65536]))
    reqs = int(g.integers(1, 9))
    kv = g.integers(0, stride * cr + 8 * cr, reqs).astype(np.int32)
    kv[g.random(reqs) < 0.2] = int(g.integers(0, next_n + 1))
    rows = reqs * next_n
    dist = str(g.choice(DISTS))
    w = workloads.random_decode(rows, stride, [stride] * rows, k, seed=int(g.integers(1 << 30)),
                                dist=dist)
    w.n_valid = oracle.varlen_n_valid(kv, rows, next_n, cr, stride).astype(np.int32)
    kw = _opts(g)
    x = torch.from_numpy(np.ascontiguousarray(w.logits)).cuda()
    log(f"[random varlen] seed={seed} k={k} next_n={next_n} cr={cr} stride={stride} {dist} {kw}")
    got = ert.topk_decode_varlen(x, torch.from_numpy(kv).cuda(), k, next_n=next_n,
                                 compress_ratio=cr, **kw)
    torch.cuda.synchronize()
    _check(w, got.cpu().numpy(), kw)
