"""The library's benchmark timing: HIP events recorded around the kernels
of each sv_spec_verify call on its stream (both kernels, and the resident
kernel as phase 0 with an empty phase 1)."""
import numpy as np
import pytest
import torch

import draft_token_verification_spec_amd as sv
from gpu_harness import gpu_verify, to_device
from synth import gen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP device")]


def test_timing_ring_records_each_call(verify_kernel):
    b = gen.make_batch("tiny_fp32_b4_k4_v1024", trial=0)
    d = to_device(b)
    print(f"case timing kernel={verify_kernel}", flush=True)
    sv.sv_timing_enable(3)
    try:
        outs = [gpu_verify(b, d=d) for _ in range(5)]
        ms = sv.sv_timing_read(8)
    finally:
        sv.sv_timing_enable(0)
    assert ms.shape == (3, 2)  # the ring keeps the last three calls
    assert np.all(ms[:, 0] > 0) and np.all(np.isfinite(ms))
    if verify_kernel == "resident":
        assert np.all(ms[:, 1] < 0.05)
    else:
        assert np.all(ms[:, 1] > 0)
    assert sv.sv_timing_read(8).shape == (0, 2)  # read empties the ring
    for o in outs[1:]:  # timing changes nothing in the outputs
        for k in o:
            np.testing.assert_array_equal(o[k], outs[0][k])
