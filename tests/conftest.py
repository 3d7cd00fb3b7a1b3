import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libpisa")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of host-side generation)")


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _has_gpu():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


# A planted oracle mistake for tests/test_oracle_mutations.py (set only in its subprocesses).
if os.environ.get("PISA_ORACLE_MUTANT"):
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import oracle_mutants

    oracle_mutants.apply(os.environ["PISA_ORACLE_MUTANT"])
