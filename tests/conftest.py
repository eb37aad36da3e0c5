import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _ensure_built():
    """Load what is built; build only if a library is missing."""
    need = [os.path.join(ROOT, "oracle", "liboracle.so"),
            os.path.join(ROOT, "synth", "libsynth_host.so")]
    if not all(os.path.exists(p) for p in need):
        import __graft_entry__
        __graft_entry__.build_oracle()
        __graft_entry__.build_synth()


_ensure_built()
