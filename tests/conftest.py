import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")
    config.addinivalue_line("markers", "slow: large CPU case")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Reports every selection that differed from the fp64 oracle's (near
    ties), so that the count is visible under -q as well."""
    mod = sys.modules.get("tests.parity_util")
    if mod is None:
        return
    flips = getattr(mod, "FLIPS", [])
    checked = getattr(mod, "CHECKED", [0])[0]
    terminalreporter.write_line(f"selection parity: {checked} selections compared with the fp64 oracle, "
                                f"{len(flips)} near-tie flips (relative gap <= {mod.NEAR_TIE:g})")
    for f in flips:
        terminalreporter.write_line(f"  flip {f['what']}: {f['members']} members, gap {f['relative_gap']:.2e}, "
                                    f"gpu-only {f['only_gpu']}, oracle-only {f['only_oracle']}")
