"""Shared pytest setup: the `gpu` marker, the repository root on sys.path, and a session
summary of every oracle comparison (one line per test: the bf16 rule's floor-active and
unfloored-failure counts, the largest error in ulps, copy and sentinel checks)."""
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))
TESTS = Path(__file__).resolve().parent
if str(TESTS) not in sys.path:
    sys.path.insert(0, str(TESTS))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    parity = sys.modules.get("parity")
    if parity is None or not parity.REPORTS:
        return
    merged = {}
    for test, rep in parity.REPORTS:
        merged.setdefault(test, parity.Report()).merge(rep)
    terminalreporter.section("oracle comparisons")
    total = parity.Report()
    for test, rep in merged.items():
        terminalreporter.write_line(f"{test}: {rep.line()}")
        total.merge(rep)
    terminalreporter.write_line(f"ALL ({len(merged)} comparisons): {total.line()}")
