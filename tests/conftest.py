import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name):
    """Parse ``key = v1 v2 ...`` lines of tests/golden/<name>.txt into floats."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            vals = [float(x) for x in v.split()]
            out[k] = vals[0] if len(vals) == 1 else vals
    return out


@pytest.fixture
def golden():
    return load_golden


def _track_workspaces():
    """Remember every Workspace the tests create (weakly), so that the status
    word of each can be checked after a GPU test."""
    import weakref

    import draft_token_verification_spec_amd as sv

    live = weakref.WeakSet([sv._default_ws])
    init = sv.Workspace.__init__

    def tracked(self, *a, **kw):
        init(self, *a, **kw)
        live.add(self)

    sv.Workspace.__init__ = tracked
    return live


_LIVE_WORKSPACES = None


@pytest.fixture(autouse=True)
def _gpu_case_bookkeeping(request):
    """For GPU tests: name the running test in the flip log, and afterwards
    assert that no bounded wait expired in any workspace the test used
    (sv_workspace_status reads and clears each status word)."""
    global _LIVE_WORKSPACES
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import gpu_harness
    import torch

    import draft_token_verification_spec_amd as sv

    if _LIVE_WORKSPACES is None:
        _LIVE_WORKSPACES = _track_workspaces()
    gpu_harness.CURRENT = request.node.nodeid.split("::", 1)[-1]
    yield
    if not torch.cuda.is_available():
        return
    bad = []
    for ws in list(_LIVE_WORKSPACES):
        for key in list(ws._buf):
            st = sv.sv_workspace_status(ws, torch.device(*key))
            if int(st.item()) != 0:
                bad.append((key, int(st.item())))
    assert not bad, f"workspace status words set (a bounded wait expired): {bad}"


def pytest_terminal_summary(terminalreporter):
    """Within-margin flips of every parity comparison, at the end of the run."""
    try:
        import gpu_harness
    except Exception:
        return
    if not gpu_harness.FLIP_LOG:
        return
    tr = terminalreporter
    tr.section("parity: within-margin flips per comparison")
    total_req = total_flips = 0
    total_tight = 0
    for case, n, flips, ed, et, tight in gpu_harness.FLIP_LOG:
        tr.write_line(f"{case}: {n} requests compared, {tight} with a margin <= 1e-5, {flips} flips, "
                      f"max rel err pd(d) {ed:.2e} pt(d) {et:.2e}")
        total_req += n
        total_flips += flips
        total_tight += tight
    tr.write_line(f"total: {total_req} requests compared, {total_tight} with a margin <= 1e-5, "
                  f"{total_flips} within-margin flips")
