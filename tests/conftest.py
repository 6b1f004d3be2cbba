import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_terminal_summary(terminalreporter):
    h = sys.modules.get("tests.echo_harness")
    if h is not None and h.STATS["set_checked"]:
        s = h.STATS
        terminalreporter.write_line(
            f"score parity: largest relative error {s['max_rel']:.3g} (more than 4 heads); top-k set "
            f"clause checked "
            f"{s['set_checked']} times, {s['set_diffs']} tokens differed (all within the "
            f"tolerance of the k-th score)")
