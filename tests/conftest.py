import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


import pytest  # noqa: E402


@pytest.fixture
def tune():
    """Set the library's tuning variables for one test (mmb_set_tuning: the
    library reads the environment only when it loads) and restore them
    afterwards: ``tune.set("MMB_SPLITS_DWEIGHT", "4")``, ``tune.clear(name)``."""
    from linear_layer_backward_amd import mmb
    saved = {}

    class Tune:
        def set(self, name, value):
            if name not in saved:
                saved[name] = mmb._tuning_now.get(name)
            mmb.mmb_set_tuning(name, value)

        def clear(self, name):
            self.set(name, None)

    yield Tune()
    for k, v in saved.items():
        mmb.mmb_set_tuning(k, v)
