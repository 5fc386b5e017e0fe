import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available() -> bool:
    try:
        import torch
        return bool(torch.cuda.is_available())
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def load_golden(name: str):
    """Parse a tests/golden/*.txt block file into a list of dicts."""
    path = os.path.join(ROOT, "tests", "golden", name)
    cases, cur = [], {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("#"):
                continue
            if not line:
                if cur:
                    cases.append(cur)
                    cur = {}
                continue
            key, _, val = line.partition(":")
            cur[key.strip()] = val.strip()
    if cur:
        cases.append(cur)
    return cases
