"""Shared pytest configuration.

Markers
  gpu -- needs an MI355X (gfx950) and the built HIP library; skipped by
         ``-m "not gpu"`` runs.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: test runs HIP kernels on a gfx950 GPU through the C-ABI")
