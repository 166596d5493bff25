import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Threshold parity bookkeeping: keep/skip choices compared with the fp64
    walks, those inside the rounding band that went the other way, and walks
    replayed on the GPU's choices."""
    try:
        import checks
    except ImportError:
        return
    st = checks.THRESH_STATS
    if st["decisions"]:
        terminalreporter.write_line(
            f"threshold parity: {st['decisions']} keep/skip choices checked, {st['flips']} flips within "
            f"{checks.THRESH_EPS:g} of the fp64 threshold (largest |margin| {st['max_flip_margin']:.3g}), "
            f"{st['replays']} of {st['walks']} walks replayed on the GPU's choices")
