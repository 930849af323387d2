import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.append(ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _point_binding_at_test_library():
    """NQ_TEST_LIB=<path> runs the suite against another build of the library
    (a tuning variant); by default the in-tree libnq.so is used."""
    path = os.environ.get("NQ_TEST_LIB")
    if path:
        import block_quantized_weight_nq_amd as nq
        nq.LIB_PATH = path
        nq._LIB = None


_point_binding_at_test_library()
