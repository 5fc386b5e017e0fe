"""Host-side checks of bench.py (no GPU): the one-GPU rule, the kernel source
hash, and when the committed counter traffic is reported."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_kernel_hash_is_stable_hex():
    b = _bench()
    h = b.kernel_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert h == b.kernel_hash()


def test_traffic_is_reported_only_for_the_sources_it_was_taken_on():
    # profiles/traffic.json is written from rocprofv3 counter runs; bench.py
    # reports an entry only while the kernel sources still hash to its value
    b = _bench()
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        tab = json.load(f)
    for name in ("decode_varlen_64x131072_k2048", "prefill_causal_4096x16640_k1024"):
        ent = tab[name]
        got = b.traffic_for(name)
        if ent["kernel_hash"] == b.kernel_hash():
            assert got == ent["hbm_bytes_per_launch"]
            assert got > ent["algorithmic_bytes_per_launch"] // 2
        else:
            assert got is None
    assert b.traffic_for("no_such_workload") is None


def test_headline_is_the_prefill_tile_and_every_workload_is_in_the_line():
    b = _bench()
    assert b.HEADLINE == 3
    import workloads
    assert workloads.config(b.HEADLINE).name == "prefill_causal_4096x16640_k1024"
    cfgs = sorted({c for c, _ in b.EXTRA} | {b.HEADLINE})
    assert cfgs == [1, 2, 3, 4, 5]
    assert {kw.get("bs") for c, kw in b.EXTRA if c == 4} == {1, 8}


def test_latency_samples_do_not_depend_on_steps():
    b = _bench()
    for steps in (1, 5, 20, 50, 199):
        assert b.latency_samples(steps) >= 200
    assert b.latency_samples(1000) == 1000


def test_rotation_reads_a_gib_between_reuses():
    b = _bench()
    for read in (65536, 459852, 15339924 - 4 * 2048 * 64 - 256, 133700640, 8388608):
        n = b.rotation(read)
        assert (n - 1) * read >= b.ROTATE_BYTES
