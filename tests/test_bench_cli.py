"""bench.py's argument checks, which run before any device work.  No GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_json_line():
    r = run("--gpus", "2")
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_config_list_is_checked():
    for bad in ("5", "0", "x", "1,7"):
        r = run("--config", bad, "--gpus", "2")
        assert r.returncode == 2 and "--config" in r.stderr, bad
