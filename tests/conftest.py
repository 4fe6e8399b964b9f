import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle.lib()
    return oracle


@pytest.fixture(scope="session")
def syn():
    import synth

    synth.lib()
    return synth


@pytest.fixture
def tune():
    """Force launch choices (moe_tuning fields) on every MoELayer the test
    creates after the call: tune(ffn_path=2, skinny_mt=4, ...)."""
    from mixture_experts_layer_gemv_amd import layer as layer_mod

    saved = layer_mod.default_tuning
    cur = {}

    def set_(**fields):
        cur.update(fields)
        layer_mod.default_tuning = dict(cur)

    yield set_
    layer_mod.default_tuning = saved
