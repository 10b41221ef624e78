"""dcn_forward_noalloc (the forward without a caller workspace) against dcn_forward.

Both run the same kernels with the same tap split, so their outputs must be
bit-identical.  Two calls in a row share the library's static scratch; the
second is a smaller problem, so stale contents of the first call's larger
packed weight and partial sums must not leak into it.  Calls go through the
C ABI (ctypes), not the Python convenience layer.
"""
import ctypes

import numpy as np
import pytest

from modulated_deformable_convolution_dcn_amd import Desc, Plan, _lib, synth
from dcn_testlib import device_inputs

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _noalloc(plan, dev, out):
    import torch
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = _lib.load().dcn_forward_noalloc(
        plan._h, p(dev["x"]), p(dev["offset"]), p(dev["mask"]), p(dev["weight"]), p(dev["bias"]),
        p(out), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    _lib.check(st, "dcn_forward_noalloc")


def _pair(spec, layout):
    """(dcn_forward output, dcn_forward_noalloc output) of one workload, as numpy."""
    import torch
    d = synth.make_inputs(spec)
    dev = device_inputs(spec, d)
    plan = Plan(Desc(spec.B, spec.C, spec.H, spec.W, spec.O, spec.kh, spec.kw, spec.ph, spec.pw,
                     spec.dtype, layout))
    ref = plan.forward(dev["x"], dev["offset"], dev["mask"], dev["weight"], dev["bias"])
    out = torch.full(plan.out_shape(), float("nan"), device="cuda")
    _noalloc(plan, dev, out)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), out.cpu().numpy()


# first call large (split tap sum: partial sums in the scratch), second smaller
SEQUENCES = [
    ("birefnet512_fp32", W["birefnet512_fp32"], W["birefnet512_fp32"].scaled(H=40, W=36)),
    ("detection_bf16", W["detection_bf16"].scaled(B=2), W["detection_bf16"].scaled(B=1, H=20, W=20)),
    ("edge_stress_fp32", W["edge_stress_fp32"].scaled(B=1, H=64, W=48),
     W["edge_stress_fp32"].scaled(B=1, C=64, O=32, H=17, W=19, kh=3, kw=3, ph=1, pw=1)),
]


@pytest.mark.parametrize("layout", ["nchw", "nhwc"])
@pytest.mark.parametrize("name,first,second", SEQUENCES, ids=[s[0] for s in SEQUENCES])
def test_noalloc_matches_forward(name, first, second, layout):
    for i, spec in enumerate((first, second)):
        print("case", name, layout, "call", i, spec, flush=True)
        ref, got = _pair(spec, layout)
        assert np.isfinite(got).all()
        assert np.array_equal(ref.view(np.uint32), got.view(np.uint32)), (name, i)


def test_noalloc_refuses_a_weight_larger_than_the_scratch():
    # 512 x 512 x 7 x 7 fp32 packed weight = 49 MiB > 32 MiB
    import torch
    plan = Plan(Desc(1, 512, 8, 8, 512, 7, 7, 3, 3))
    x = torch.zeros((1, 8, 8, 512), device="cuda")
    off = torch.zeros((1, 98, 8, 8), device="cuda")
    w = torch.zeros((512, 512, 7, 7), device="cuda")
    out = torch.zeros(plan.out_shape(), device="cuda")
    st = _lib.load().dcn_forward_noalloc(plan._h, ctypes.c_void_p(x.data_ptr()),
                                         ctypes.c_void_p(off.data_ptr()), None,
                                         ctypes.c_void_p(w.data_ptr()), None,
                                         ctypes.c_void_p(out.data_ptr()), None)
    assert st == 4, _lib.load().dcn_last_error()
