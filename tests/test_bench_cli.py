"""bench.py's command-line contract, on the CPU: one GPU only (any other
--gpus exits with status 2 and says why), and the help text lists every
workload."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = run("--gpus", n)
        assert r.returncode == 2
        assert "one GPU only" in r.stderr and f"--gpus {n}" in r.stderr
        assert r.stdout == ""


def test_help_lists_the_workloads():
    r = run("--help")
    assert r.returncode == 0
    for w in ("kv_chunk", "kv_store", "gather_steady", "gemm_attn", "ffn", "ring64s",
              "quant_act", "wgrad", "lora", "attn"):
        assert w in r.stdout
