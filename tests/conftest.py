"""Shared pytest setup: the `gpu` marker and import paths.

Tests marked `gpu` need an MI355X (gfx950) and the built HIP library; everything
else runs on a CPU-only host.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle._load()
    return oracle


def _ensure_built():
    """Tests load what is built; they build only when nothing is."""
    import memory_bound_row_sm_amd as sm
    import oracle
    if not os.path.exists(oracle.LIB_PATH):
        from oracle import build as ob
        ob.build()
    if not os.path.exists(sm.lib_path):
        from memory_bound_row_sm_amd import build as sb
        sb.build()


_ensure_built()
