"""bench.py's contract on the host: one GPU only, and the committed HBM-traffic summary
of the nvfp4 GEMM still belongs to the GEMM sources (otherwise the bench reports
traffic as null)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8", "--steps", "1"], None),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = run_bench(args, env)
    assert r.returncode == 2, (r.returncode, r.stdout, r.stderr)
    assert "one GPU" in r.stderr
    assert not r.stdout.strip(), "no JSON line for a refused run"


def test_traffic_summary_matches_gemm_sources():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.measured_traffic() is not None, (
        "profiles/ traffic summary was taken on other GEMM sources: re-take the FETCH_SIZE / WRITE_SIZE passes")
