"""Host-side contract of the bench script and the Python binding (no GPU).

bench.py measures one GPU: asked for several it must refuse with a message
and print no result line.  The binding has no CPU fallback: with the HIP
library absent it must raise instead of computing anything.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""  # no JSON result line


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import transformer_lm_step_flat_amd.gpt2 as g
    monkeypatch.setattr(g, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(g, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        g.lib()
