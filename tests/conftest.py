import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Largest parity error per quantity over the session's GPU comparisons,
    with the raw max-abs (grad_loc) and max |g - r| / max(1, |r|)."""
    try:
        from tests.gpu_util import ERRORS
    except Exception:  # the GPU helpers need torch; nothing to report without them
        return
    if not ERRORS:
        return
    worst = {}
    for test, name, err, raw, rel in ERRORS:
        if name not in worst or err > worst[name][1]:
            worst[name] = (test, err, raw, rel)
    tr = terminalreporter
    tr.section("parity errors against the fp64 oracle (largest per quantity)")
    for name in sorted(worst):
        test, err, raw, rel = worst[name]
        raw_s = "" if raw is None else f"  raw {raw:.3e}"
        tr.write_line(f"{name:28s} {err:.3e}{raw_s}  rel {rel:.3e}  ({len([e for e in ERRORS if e[1] == name])} "
                      f"comparisons; worst in {test})")
