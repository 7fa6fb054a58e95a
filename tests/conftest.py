import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


class Knobs:
    """Tuning overrides of the library (fa_set_knob), restored after the test."""
    NAMES = {"FA_KERNEL": 1, "FA_TILE_QB": 2, "FA_WG_GROUP": 3, "FA_WG_LIGHT": 4, "FA_DEBUG": 5}

    def __init__(self):
        self.touched = set()

    def set(self, name, value):
        import exact_attention_02_amd as fa
        knob = self.NAMES[name]
        fa.set_knob(knob, int(value))
        self.touched.add(knob)

    def restore(self):
        import exact_attention_02_amd as fa
        for knob in self.touched:
            fa.set_knob(knob, -1)


@pytest.fixture
def knobs():
    k = Knobs()
    yield k
    k.restore()
