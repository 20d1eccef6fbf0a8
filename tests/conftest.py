import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# The native helpers (oracle/liboracle.so, libtpsynth.so, libtpmlp.so) are
# compiled by __graft_entry__.build() only; the tests load them and raise if
# one is missing or was built from another version of its source, so that no
# test starts a compiler from a process that may already drive the GPU.

@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle._L()
    return oracle


@pytest.fixture(scope="session")
def inputs_mod():
    from tensor_transformer_mlp_amd import inputs
    inputs._synth()
    return inputs

