import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: statistical test that takes more than a few seconds")


# Alternative builds for the sanitizer test, which runs the CPU tests in a
# child process against AddressSanitizer / UndefinedBehaviorSanitizer builds
# of the library's host code and of the oracle.
if os.environ.get("SV_TEST_LIB"):
    import lossless_draft_verification_amd._lib as _svlib

    _svlib.LIB_PATH = os.environ["SV_TEST_LIB"]
if os.environ.get("SV_TEST_ORACLE_LIB"):
    import oracle as _oracle

    _oracle._LIB_PATH = os.environ["SV_TEST_ORACLE_LIB"]
