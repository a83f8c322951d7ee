"""Shared pytest configuration.

Markers:
  gpu -- needs an MI355X (gfx950) and the built HIP library; the CPU suite runs
         with ``-m "not gpu"``.
"""
from __future__ import annotations

import os
import sys

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU and the built HIP library")
