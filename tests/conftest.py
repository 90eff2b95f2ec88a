import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


_IMPLS = [x for x in os.environ.get("SG_ORACLE_IMPLS", "c,numpy").split(",") if x]


@pytest.fixture(params=_IMPLS)
def oracle_impl(request):
    """Both oracle implementations: the plain C loops (the default `oracle`)
    and the numpy cross-check (SG_ORACLE_IMPLS=c or =numpy selects one)."""
    import oracle
    return oracle.IMPLEMENTATIONS[request.param]
