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


VERIFY_KERNELS = {"streaming": 1, "resident": 2}  # sv_kernel values of include/specverify.h


@pytest.fixture(params=sorted(VERIFY_KERNELS))
def verify_kernel(request):
    """Run a test once per verification kernel (process-wide selector),
    restoring the previous selection afterwards."""
    import draft_token_verification_spec_amd as sv

    prev = sv.sv_set_verify_kernel(VERIFY_KERNELS[request.param])
    print(f"[kernel {request.param}]", flush=True)
    yield request.param
    sv.sv_set_verify_kernel(prev)
