"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
parsing of rocminfo's agent listing."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


ROCMINFO = """
*******
Agent 1
*******
  Name:                    AMD EPYC 9575F 64-Core Processor
  Compute Unit:            128
  Max Clock Freq. (MHz):   5008
*******
Agent 2
*******
  Name:                    gfx950
  Marketing Name:          AMD Instinct MI355X
  Compute Unit:            256
  Max Clock Freq. (MHz):   2400
"""


def test_device_info_reads_the_gpu_agent(monkeypatch):
    class Done:
        stdout = ROCMINFO

    monkeypatch.setattr(subprocess, "run", lambda *a, **k: Done())
    info = bench.device_info()
    assert info == {"arch": "gfx950", "compute_units": 256, "max_clock_mhz": 2400,
                    "nominal_bf16_tflops": 2516.6}


def test_device_info_without_rocminfo(monkeypatch):
    def missing(*a, **k):
        raise FileNotFoundError("rocminfo")

    monkeypatch.setattr(subprocess, "run", missing)
    assert bench.device_info() is None
