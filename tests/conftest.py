import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_sessionfinish(session, exitstatus):
    """With MLORA_PARITY_LOG set, write the observed parity figures of every
    fold comparison (label, relative L2, max abs, max abs / limit) there."""
    path = os.environ.get("MLORA_PARITY_LOG")
    if not path:
        return
    from tests.common import PARITY_LOG
    rows = [{"label": l, "rel_l2": r, "max_abs": m, "max_abs_over_limit": e}
            for (l, r, m, e) in PARITY_LOG]
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump(rows, f, indent=1)


@pytest.fixture
def overrides(monkeypatch):
    """Sets / removes MLORA_* launch-shape overrides for one test: the library
    reads them once per process, so each change is followed by a re-read, and
    the test's end restores the environment and re-reads it again."""
    import moe_expert_lora_amd as ml

    class _Overrides:
        def set(self, name, value):
            monkeypatch.setenv(name, str(value))
            ml.mlora_reload_launch_overrides()

        def delete(self, name):
            monkeypatch.delenv(name, raising=False)
            ml.mlora_reload_launch_overrides()

    yield _Overrides()
    monkeypatch.undo()
    ml.mlora_reload_launch_overrides()
