import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# The library reads its testing switches (TITANS_MEM_FORCE_GENERIC, ..._GENERIC_MODE,
# ..._LINEAR, ..._FUSED_SINGLE, ..._TEST_PAIR_TIMEOUT) only while this is set; the tests
# set those per case with monkeypatch.
os.environ["TITANS_MEM_DEBUG"] = "1"


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")
