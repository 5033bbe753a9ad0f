import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    return oracle.load()


@pytest.fixture(scope="session")
def full_size():
    """Seeded inputs and oracle results of the full-size GEMM workloads
    (4096^3 and 4000x4032x4104), each computed once per test session and
    shared by every test that compares a kernel with them in full."""
    import functools
    from types import SimpleNamespace

    import datagen
    import oracle

    @functools.lru_cache(maxsize=None)
    def inputs(cfg_id, integer=False, bf16=False):
        return datagen.gemm_inputs(datagen.WORKLOADS[cfg_id], integer=integer, bf16=bf16)

    @functools.lru_cache(maxsize=None)
    def reference(cfg_id, integer=False, bf16=False):
        A, B = inputs(cfg_id, integer, bf16)
        return (oracle.gemm_bf16 if bf16 else oracle.gemm)(A, B)

    return SimpleNamespace(inputs=inputs, reference=reference)
