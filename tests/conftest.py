import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_runtest_logreport(report):
    # one line per finished test with its duration, so a long GPU run shows
    # its progress and the cost of every test
    if report.when == "call" and "gpu" in report.keywords:
        import sys
        sys.stdout.write(f"\n[{report.duration:7.1f} s] {report.nodeid} {report.outcome}\n")
        sys.stdout.flush()
