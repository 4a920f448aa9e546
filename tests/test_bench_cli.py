"""bench.py's command-line contract, on the host: one GPU only, and a clear exit without a GPU."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_exits_with_a_message():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line for a run that did not happen


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU exit")
def test_no_gpu_exits_without_a_result_line():
    r = _bench("--steps", "1", "--warmup", "0")
    assert r.returncode == 1
    assert "needs a GPU" in r.stderr
    assert r.stdout == ""
