"""Test configuration: the ``gpu`` marker and import paths.

``-m "not gpu"`` runs the oracle pins, host logic and library-load checks on
any machine; ``-m gpu`` runs the parity tests on an MI355X through the C ABI.
"""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libpa.so")
