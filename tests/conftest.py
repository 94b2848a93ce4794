import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def oracle_mod():
    from oracle import oracle
    oracle.build()
    return oracle


@pytest.fixture(scope="session")
def synth_mod():
    from synth import synth
    synth.build()
    return synth


@pytest.fixture(scope="session")
def verify_experts(synth_mod):
    """The 256 MXFP4 experts of the full-size workloads (d=7168, ffn=2048), host
    arrays, generated once per session."""
    cfg = synth_mod.get_config("verify")
    print("\n[full] generating 256 MXFP4 experts (d=7168, ffn=2048)", flush=True)
    return synth_mod.expert_weights(cfg)
