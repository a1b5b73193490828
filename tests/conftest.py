import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# The host sanitizer run (tests/test_host_sanitizer.py) points the binding at
# the host-check build of the C ABI through this variable.
if os.environ.get("KVSEL_TEST_LIB"):
    from token_selection_tsp_amd import kvsel as _kvsel
    _kvsel.LIB_PATH = os.environ["KVSEL_TEST_LIB"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
