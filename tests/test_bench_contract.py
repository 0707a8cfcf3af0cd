"""bench.py's command-line contract that holds without a GPU: the decode path
is not sharded, so more than one GPU is refused with a JSON message before
anything touches a device."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2
    assert "--gpus must be 1" in line["error"]


def test_default_run_is_a_launcher_that_never_imports_torch(tmp_path):
    # a torch that cannot be imported: the launcher must still run and
    # report its first child's failure as a JSON line (the child, which does
    # import torch, fails)
    fake = tmp_path / "torch"
    fake.mkdir()
    (fake / "__init__.py").write_text("raise ImportError('no torch in the launcher')\n")
    env = dict(os.environ, PYTHONPATH=str(tmp_path))
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "1",
                        "--warmup", "0", "--no-sweep"],
                       capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 1
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["error"].startswith("child --workload llama13b --bs 16")
    assert "[bench] child: --workload llama13b" in r.stderr
