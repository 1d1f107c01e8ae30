import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size case (minutes of host work)")


def pytest_sessionstart(session):
    """Checker builds (the host-sanitizer run of test_sanitizers.py) point the
    tests at other builds of the library and the oracle through these two
    variables; unset, the in-tree builds are used."""
    lib = os.environ.get("POSTMIX_TEST_LIB")
    if lib:
        from rope_head_mixing_amd import postmix
        postmix.LIB_PATH = lib
        postmix._lib = None
    olib = os.environ.get("ORACLE_TEST_LIB")
    if olib:
        import oracle
        oracle.use_library(olib)
