import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Prints the parity figures the attention tests recorded (errors against the fp64 oracle)."""
    helpers = sys.modules.get("tests.helpers")
    recs = getattr(helpers, "PARITY_RECORDS", None) if helpers else None
    if not recs:
        return
    terminalreporter.write_sep("-", "attention parity against the fp64 oracle")
    for what, st in recs:
        terminalreporter.write_line(
            f"{what}: rows={st.get('rows')} max_abs={st['max_abs']:.3g} mean_abs={st['mean_abs']:.3g} "
            f"rel_fro={st.get('rel_fro', 0.0):.3g} lse_max_abs={st.get('lse_max_abs', float('nan')):.3g}")
