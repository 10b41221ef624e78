"""DCN_VALIDATE on the GPU path: a non-finite offset or mask is refused before
any launch; finite inputs run as usual."""
import math

import numpy as np
import pytest

from modulated_deformable_convolution_dcn_amd import synth
from dcn_testlib import device_inputs

pytestmark = pytest.mark.gpu


def test_validate_refuses_non_finite_offsets(monkeypatch):
    import torch
    from modulated_deformable_convolution_dcn_amd import Desc, Plan
    monkeypatch.setenv("DCN_VALIDATE", "1")
    spec = synth.WORKLOADS["tiny_fp32"]
    d = synth.make_inputs(spec)
    dev = device_inputs(spec, d)
    plan = Plan(Desc(spec.B, spec.C, spec.H, spec.W, spec.O, spec.kh, spec.kw, spec.ph, spec.pw))
    out = plan.forward(dev["x"], dev["offset"], dev["mask"], dev["weight"], dev["bias"])
    torch.cuda.synchronize()
    assert np.isfinite(out.cpu().numpy()).all()
    bad = dev["offset"].clone()
    bad[0, 3, 2, 2] = math.nan
    sentinel = torch.full(plan.out_shape(), 7.0, device="cuda")
    with pytest.raises(ValueError, match="offset"):
        plan.forward(dev["x"], bad, dev["mask"], dev["weight"], dev["bias"], out=sentinel)
    m = dev["mask"].clone()
    m[0, 0, 0, 0] = math.inf
    with pytest.raises(ValueError, match="mask"):
        plan.forward(dev["x"], dev["offset"], m, dev["weight"], dev["bias"], out=sentinel)
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())  # nothing was launched
