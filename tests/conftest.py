import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (seconds to minutes)")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle._load()


def pytest_terminal_summary(terminalreporter):
    """Near ties of the oracle among the sampled cells the GPU tests compared
    (the cells excused from token equality)."""
    mod = sys.modules.get("gpu_helpers")
    tally = getattr(mod, "NEAR_TIE_TALLY", None) if mod else None
    if not tally:
        return
    terminalreporter.section("oracle near ties among compared sampled cells")
    sampled = sum(t[1] for t in tally)
    near = sum(t[2] for t in tally)
    mism = sum(t[3] for t in tally)
    for name, n, k, m in tally:
        if k:
            terminalreporter.write_line(f"{name}: {k} near ties in {n} sampled cells, {m} drew another kept id")
    terminalreporter.write_line(f"total: {near} near ties in {sampled} sampled cells over {len(tally)} checks, "
                                f"{mism} drew another kept id within the band")
