"""bench.py's command line on the CPU: more than one GPU is refused with a
message (this path runs on one GPU), the workload list matches the workload
table, and the router workload's algorithmic counts are the plain ones."""
import os
import subprocess
import sys

import datagen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_workload_choices_cover_the_table():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for name in datagen.WORKLOADS:
        assert name in r.stdout, name


def test_router_counts():
    w = datagen.workload("router")
    assert w.flops == 2 * 4096 * 4096 * 8
    assert w.bytes == 2 * 4096 * 4096 + 2 * 8 * 4096 + 4096 * 2 * 8


def test_default_headline_is_the_largest_config():
    """With no flags the headline is the 8192/28672 GeGLU at 4096 tokens (the
    largest single-GPU workload, bound by the matrix cores), and the configs
    table names every other workload."""
    import importlib.util

    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'ap.add_argument("--workload", default="large4096"' in src
    big = max(datagen.WORKLOADS.values(), key=lambda w: w.flops if w.op == "geglu" else 0)
    assert big.name == datagen.workload("large4096").name
    assert set(bench.CONFIG_ROWS) == set(datagen.WORKLOADS)
    assert set(bench.EST_US) == set(datagen.WORKLOADS)
