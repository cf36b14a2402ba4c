import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # Host-side libraries are built on demand when absent (CPU-only builds).
    for mod, lib in (("oracle", "liboracle.so"), ("ds4gen", "libds4gen.so")):
        if not os.path.exists(os.path.join(ROOT, mod, lib)):
            import importlib
            importlib.import_module(mod + ".build").build(**({"device": False} if mod == "ds4gen" else {}))
