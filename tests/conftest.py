import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU oracle runs")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build()
    return oracle


def pytest_terminal_summary(terminalreporter):
    """Near-tie tokens of every GPU selection check (tokens whose GPU and
    oracle selections differ only by reordering logits within the certified
    rounding bound), so the count stays in the log of a quiet run."""
    try:
        import gpu_util
    except ImportError:
        return
    if not gpu_util.NEAR_TIES:
        return
    rows = gpu_util.NEAR_TIES
    terminalreporter.section("near-tie tokens per selection check")
    tot_t = sum(r[1] for r in rows)
    tot_n = sum(r[2] for r in rows)
    for test, n, near in rows:
        if near:
            terminalreporter.write_line(f"{test}: {near} of {n}")
    terminalreporter.write_line(f"all checks: {tot_n} near-tie tokens of {tot_t} "
                                f"({len(rows)} checks, {sum(1 for r in rows if r[2])} with any)")
