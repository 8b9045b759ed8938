"""Host-side checks of bench.py that need no GPU: the one-GPU guard and the rocminfo parser."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

ROCMINFO = """\
*******
Agent 1
*******
  Name:                    Some CPU
  Device Type:             CPU
  Compute Unit:            64
  Max Clock Freq. (MHz):   3000
*******
Agent 2
*******
  Name:                    gfx950
  Marketing Name:          AMD Instinct MI355X
  Device Type:             GPU
  Max Clock Freq. (MHz):   2400
  Compute Unit:            256
  ISA Info:
    ISA 1
      Name:                    amdgcn-amd-amdhsa--gfx950:sramecc+:xnack-
"""


def test_device_info_parses_the_gpu_agent(monkeypatch):
    class Done:
        stdout = ROCMINFO
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: Done())
    d = bench.device_info()
    assert d == {"name": "AMD Instinct MI355X", "arch": "gfx950", "compute_units": 256,
                 "max_sclk_mhz": 2400, "peak_bf16_tflops_from_clock": 2516.6}


def test_device_info_without_rocminfo(monkeypatch):
    def missing(*a, **k):
        raise FileNotFoundError("rocminfo")
    monkeypatch.setattr(subprocess, "run", missing)
    assert bench.device_info() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
