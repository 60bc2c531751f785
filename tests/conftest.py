"""Shared pytest setup.

* registers the ``gpu`` marker (tests that need an MI355X);
* keeps large freed blocks on the glibc heap so the float64 oracle reuses
  pages instead of faulting fresh ones for every temporary (first-touch page
  faults are slow in some containers).  This changes no arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _keep_heap() -> None:
    try:
        libc = ctypes.CDLL("libc.so.6")
        libc.mallopt(-4, 0)            # M_MMAP_MAX: serve large blocks from the heap
        libc.mallopt(-1, 1 << 30)      # M_TRIM_THRESHOLD: do not hand freed memory back
    except OSError:
        pass


_keep_heap()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False
