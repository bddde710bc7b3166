import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture
def ncc_opts():
    """Sets library options (ncc_set_option) for one test and restores the
    previous values afterwards: ncc_opts(route="generic", sat_build=...)."""
    import normalized_cross_correlation_amd as ncc
    saved = {}

    def set_(**settings):
        for k, v in settings.items():
            if k not in saved:
                saved[k] = ncc.get_option(k)
            ncc.set_option(k, v)

    yield set_
    for k, v in saved.items():
        ncc.set_option(k, v)


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build(force=False)
    return oracle
