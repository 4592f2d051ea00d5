import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct MI355X (gfx950) GPU and the built HIP library")


def pytest_report_header(config):
    return "draft_verification_sv_amd test-suite"


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Counts of the long parity runs (positions compared and disagreements
    excused by a low oracle margin), shown whatever the verbosity."""
    try:
        from harness import PARITY_LOG
    except ImportError:
        return
    if PARITY_LOG:
        terminalreporter.section("parity against the oracle")
        for line in PARITY_LOG:
            terminalreporter.write_line(line)
