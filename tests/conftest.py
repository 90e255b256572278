import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle

    oracle.build(force=False)
    return oracle


def pytest_terminal_summary(terminalreporter):
    """Whole-output error figures of the parity tests that ran (see
    gpu_helpers.record_parity), one line each, so that a quiet run keeps them."""
    helpers = sys.modules.get("gpu_helpers")
    recs = getattr(helpers, "PARITY_RECORDS", None) if helpers else None
    if not recs:
        return
    terminalreporter.section("whole-output parity against the fp64 oracle")
    for what, name, sd, ey, ef, tol in recs:
        efs = "-" if ef is None else f"{ef:.3e}"
        ok = "ok" if ey <= tol and (ef is None or ef <= tol) else "FAIL"
        terminalreporter.write_line(f"{what:10s} {name:10s} states={sd:5s} err_y={ey:.3e} err_final={efs} "
                                    f"tol={tol:g} {ok}")
