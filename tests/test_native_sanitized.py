"""Host code built with AddressSanitizer and UndefinedBehaviorSanitizer on
the CPU (g++/gcc, no device code): the checkpoint file module of the library
(tests/native/checkpoint_driver.cpp) and the oracle
(tests/native/oracle_driver.c).  A sanitizer report makes the driver exit
non-zero with the report on stderr."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_checkpoint_module_under_sanitizers(tmp_path):
    exe = str(tmp_path / "ck")
    _run(["g++", "-std=c++17", "-Wall", *SAN, "-o", exe,
          os.path.join(ROOT, "tests", "native", "checkpoint_driver.cpp"),
          os.path.join(ROOT, "transformer_lm_step_flat_amd", "csrc", "checkpoint.cpp")])
    r = _run([exe, str(tmp_path)], timeout=300)
    assert "all checks passed" in r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle")
    _run(["gcc", "-std=c11", "-D_GNU_SOURCE", "-Wall", "-Wno-unknown-pragmas", *SAN, "-o", exe,
          os.path.join(ROOT, "tests", "native", "oracle_driver.c"), os.path.join(ROOT, "oracle", "gpt2_ref.c"),
          "-lm"])
    r = _run([exe], timeout=300)
    assert r.stdout.count("loss") == 3
