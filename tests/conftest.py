"""Shared test setup: repo root on sys.path and the `gpu` marker.

Tests marked `gpu` need a real MI355X (gfx950) and the built HIP library; the
CPU suite (`-m "not gpu"`) covers the oracle against its pins, the synthetic
input generator, host-side logic of the boundary, and that the C-ABI library
loads and exports every symbol its header declares.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of CPU oracle time)")
