import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # The full-size parity tests run the fp64 oracle on every (batch, head)
    # in a process pool.  Its workers are forked here, before any test
    # touches the GPU, so that none of them inherits GPU state.
    markexpr = (config.getoption("markexpr", "") or "").replace(" ", "")
    if "notgpu" not in markexpr:
        from oracle import heads
        heads.start()


def pytest_unconfigure(config):
    from oracle import heads
    heads.stop()


@pytest.fixture(scope="session")
def lib():
    """The C-ABI library through the Python binding (GPU tests only)."""
    import kernelized_linear_attention_elu_amd as la
    la.load_library()
    return la


def pytest_runtest_logreport(report):
    """Print a failing test's report at once, so that it survives even if a
    later test takes the process down."""
    if report.failed:
        print(f"\n---- {report.nodeid} ({report.when}) failed ----\n{report.longreprtext}\n", flush=True)


@pytest.fixture
def span(lib):
    """Set the library's span length (tokens per workgroup; None: its own
    choice) for one test; restored afterwards."""
    def _set(tokens):
        lib.set_span_tokens(tokens or 0)
    _set(None)
    yield _set
    _set(None)
