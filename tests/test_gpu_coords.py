"""Bit-exact sampling corners: the GPU's coordinate stage vs the oracle.

The fused kernel and dcn_debug_coords share one device function for the
sampling point (page 1, "deform_conv.py": exact integer grid + one fp32 add
of the offset, floor, per-corner validity), so this checks the code that runs
on the timed path.  (y0, x0) and the 4-bit validity mask must be equal at
every (b, tap, ho, wo) of every workload.
"""
import numpy as np
import pytest

import oracle
from modulated_deformable_convolution_dcn_amd import synth
from dcn_testlib import oracle_shape, device_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_corners_bit_exact(name):
    import torch
    from modulated_deformable_convolution_dcn_amd import Desc, Plan
    spec = synth.WORKLOADS[name]
    d = synth.make_inputs(spec)
    print("case", name, flush=True)
    y_ref, v_ref = oracle.coords(oracle_shape(spec), d["offset"])
    dev = device_inputs(spec, d)
    plan = Plan(Desc(spec.B, spec.C, spec.H, spec.W, spec.O, spec.kh, spec.kw, spec.ph, spec.pw,
                     spec.dtype))
    y_gpu, v_gpu = plan.debug_coords(dev["offset"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(v_gpu.cpu().numpy(), v_ref)
    # compare corners where they matter: any point with a corner inside
    y_gpu = y_gpu.cpu().numpy()
    inside = v_ref != 0
    np.testing.assert_array_equal(y_gpu[inside], y_ref[inside])
    # and everywhere for moderate offsets (saturation aside, still equal)
    np.testing.assert_array_equal(y_gpu, y_ref)


def test_corners_at_exact_integers_and_halves():
    """Offsets that land exactly on integers, half-integers and -1 / H-1 / H."""
    import torch
    from modulated_deformable_convolution_dcn_amd import Desc, Plan
    H, W = 6, 5
    s = oracle.Shape(1, 4, H, W, 4, 3, 3, 1, 1)
    vals = np.array([-2.0, -1.5, -1.0, -0.5, -1e-7, 0.0, 0.5, 1.0, 2.5, H - 1.0, H - 0.5,
                     float(H), 1e30, -1e30], np.float32)
    rng = np.random.default_rng(0)
    off = rng.choice(vals, size=(1, 2 * 9, s.Ho, s.Wo)).astype(np.float32)
    y_ref, v_ref = oracle.coords(s, off)
    plan = Plan(Desc(1, 4, H, W, 4, 3, 3, 1, 1))
    y_gpu, v_gpu = plan.debug_coords(torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(v_gpu.cpu().numpy(), v_ref)
    np.testing.assert_array_equal(y_gpu.cpu().numpy(), y_ref)
