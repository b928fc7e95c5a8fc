"""The benchmark's command-line contract, checked without a GPU: one GPU only
(a multi-GPU request exits with a message and status 2 before touching the
device), and the workload choices it documents."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_help_lists_the_workloads():
    r = _run("--help")
    assert r.returncode == 0
    for w in ("b8_1m_full_reindex_reuse4", "b32_128k_full_reuse5", "ragged64_paged_20layer",
              "prefill_4096q_128k", "b8_1m_spec6"):
        assert w in r.stdout
