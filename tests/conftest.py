import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def ensure_built():
    """Build libglu.so and libglu_ref.so only if they are not there yet (the
    tests never rebuild)."""
    from mlp_gated_activation_amd import build
    if not os.path.exists(build.LIB) or not os.path.exists(build.REF_LIB):
        build.build()
