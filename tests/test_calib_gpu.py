"""GPU check of the read-floor measurement aid: it runs in the selection's
launch shapes (one workgroup per row, and split rows) without error and
leaves the output untouched; it is timed by bench.py --read-floor."""
import pytest

import workloads
from gpu_helpers import log, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_read_floor_runs_in_the_plan_shapes(cfg):
    import torch
    import exact_row_top_amd as ert
    w = workloads.config(cfg)
    log(f"[calib] read floor {w.name}")
    d = to_dev(w)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    if w.mode == "decode":
        ert.read_floor(d["logits"], d["n_valid"], w.k, sink=sink)
    else:
        ert.read_floor(d["logits"], d["row_starts"], w.k, extents2=d["row_ends"], sink=sink)
    torch.cuda.synchronize()
    assert sink.numel() == 1
