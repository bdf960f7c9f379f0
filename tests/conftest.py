"""Shared pytest set-up: the ``gpu`` marker and the CPU-side libraries.

GPU tests are marked ``@pytest.mark.gpu`` and run only on a machine with an
MI355X; everything else runs on the CPU. The CPU libraries (input generator,
oracle) are compiled here only when no built copy exists.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    import oracle
    import synth
    for mod in (synth, oracle):
        if not os.path.exists(mod.LIB_PATH):
            mod.build()
