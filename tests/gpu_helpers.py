"""Shared helpers for the GPU parity tests (run the HIP path, compare with the oracle)."""
import sys

import numpy as np

import oracle


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(w):
    import torch
    d = {"logits": torch.from_numpy(np.ascontiguousarray(w.logits)).cuda()}
    if w.mode == "decode":
        d["n_valid"] = torch.from_numpy(np.ascontiguousarray(w.n_valid, dtype=np.int32)).cuda()
    else:
        d["row_starts"] = torch.from_numpy(np.ascontiguousarray(w.row_starts, dtype=np.int32)).cuda()
        d["row_ends"] = torch.from_numpy(np.ascontiguousarray(w.row_ends, dtype=np.int32)).cuda()
    return d


def run_gpu(w, dev=None, stats=False, **kw):
    """Run the HIP path on a Workload; returns host int32 [rows, k] (and stats)."""
    import torch
    import exact_row_top_amd as ert
    if dev is None:
        dev = to_dev(w)
    st = None
    if stats:
        st = torch.full((w.num_rows, ert.STATS_WORDS), -7, dtype=torch.int32, device="cuda")
        kw["row_stats"] = st
    if w.mode == "decode":
        out = ert.topk_decode(dev["logits"], dev["n_valid"], w.k, **kw)
    else:
        out = ert.topk_prefill(dev["logits"], dev["row_starts"], dev["row_ends"], w.k, **kw)
    torch.cuda.synchronize()
    res = out.cpu().numpy()
    if stats:
        return res, st.cpu().numpy()
    return res


def assert_parity(w, got, want=None, rows=None):
    bad = oracle.check_rows(w, got, want, rows=rows)
    assert not bad, f"{w.name}: {len(bad)} bad rows, first: {bad[:3]}"
