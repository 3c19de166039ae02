import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (minutes)")


import pytest


@pytest.fixture
def force_path():
    """Forces the forward path and row splits for one test through the
    library's test hook (ssd_set_path_override) and restores the shape's own
    choice afterwards.  rows: "" = chosen by the shape, "0" = the four stages,
    "4" / "2" / "1" = the one-pass state stage with that many row sets per
    workgroup, "fused" = the fused pass; adj_rows likewise for the backward's
    adjoint scan ("" = by shape)."""
    from selective_state_space_amd import ssd

    def apply(rows="", adj_rows=""):
        rows = str(rows)
        if rows == "":
            fwd, sr = -1, 0
        elif rows == "0":
            fwd, sr = ssd.PATH_FOUR_STAGE, 0
        elif rows == "fused":
            fwd, sr = ssd.PATH_FUSED, 0
        else:
            fwd, sr = ssd.PATH_STATE_FWD, int(rows)
        ssd.set_path_override(fwd, sr, int(adj_rows) if str(adj_rows) else 0)

    yield apply
    ssd.set_path_override(-1, 0, 0)
