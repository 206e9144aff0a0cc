"""bench.py's command line on a GPU-less host: the one-GPU contract and the workload list.

Nothing here touches a GPU: --gpus above 1 is refused before torch is imported, and the
workload table is read from the seeded generators.
"""
import os
import subprocess
import sys

from conftest import ROOT


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_every_bench_workload_is_defined_and_seeded():
    from workloads import CONFIG_NAMES, make_config

    for idx, name in CONFIG_NAMES.items():
        a, b = make_config(idx), make_config(idx)
        assert a.name == name
        assert (a.context_lens == b.context_lens).all() and (a.block_tables == b.block_tables).all()
        assert make_config(idx, replica=1).seed != a.seed
