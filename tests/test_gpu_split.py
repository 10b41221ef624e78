"""GPU parity of the split tap sum (fp32 plans of 17..64 output channels whose
grid would leave most of the GPU idle): each workgroup runs two tap groups
of four waves over the two halves of its taps, added on chip, and when even
that leaves most of the GPU idle the taps are also divided into runs that
workgroups compute side by side into partial outputs, then a reduce adds the
runs and the bias.

Every case runs both ways -- with the full workspace (split) and with only
the packed weight (no split: tap groups only) -- and both are held to the
parity bar against the oracle; the split result is also checked to be
deterministic.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from dcn_testlib import compare, device_inputs, oracle_shape, pixel_major
from modulated_deformable_convolution_dcn_amd import synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
E = W["edge_stress_fp32"]
B5 = W["birefnet512_fp32"]

CASES = {
    # 36 workgroups: four runs of 13, 13, 13 and 10 taps
    "k49_48x48": B5.scaled(H=48, W=48),
    # two channel chunks (one ragged), 40 outputs; runs of 7, 7, 7, 4 taps
    "k25_c96_o40": E.scaled(B=1, C=96, O=40, H=21, W=17),
    # K = 4: two runs of two taps, one per tap group
    "k4_c32_o64": E.scaled(B=1, C=32, O=64, H=15, W=14, kh=1, kw=4, ph=0, pw=0),
    # two images, K = 9 over three runs; odd Ho*Wo
    "k9_b2_c32_o64": E.scaled(B=2, C=32, O=64, H=9, W=11, kh=3, kw=3, ph=1, pw=1),
}


def _run(spec, dev, layout, split, use_mask=True, use_bias=True, repeat=1):
    import torch
    from modulated_deformable_convolution_dcn_amd import Desc, Plan
    plan = Plan(Desc(spec.B, spec.C, spec.H, spec.W, spec.O, spec.kh, spec.kw, spec.ph, spec.pw,
                     spec.dtype, layout))
    assert plan.workspace_bytes > plan.packed_weight_bytes, "case does not split its taps"
    assert plan.tap_groups == 2
    packed = plan.pack_weight(dev["weight"], split=split)
    outs = []
    for _ in range(repeat):
        o = plan.forward_packed(dev["x"], dev["offset"], dev["mask"] if use_mask else None, packed,
                                dev["bias"] if use_bias else None)
        outs.append(o)
    torch.cuda.synchronize()
    return [pixel_major(o.cpu().numpy(), layout) for o in outs]


@pytest.mark.parametrize("layout", ["nchw", "nhwc"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_split_and_unsplit_match_the_oracle(name, layout):
    spec = CASES[name]
    d = synth.make_inputs(spec)
    ref, norm = oracle.forward(oracle_shape(spec), d["x"], d["offset"], d["mask"], d["weight"],
                               d["bias"])
    dev = device_inputs(spec, d)
    print("case", name, layout, spec, flush=True)
    s1, s2 = _run(spec, dev, layout, split=True, repeat=2)
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))  # fixed summation order
    (u,) = _run(spec, dev, layout, split=False)
    ws = compare(s1, ref, norm, d["bias"], "f32", "%s/%s split" % (name, layout))
    wu = compare(u, ref, norm, d["bias"], "f32", "%s/%s unsplit" % (name, layout))
    print("worst err/N split %.3g unsplit %.3g" % (ws, wu))


@pytest.mark.parametrize("use_mask,use_bias", [(False, False), (True, False), (False, True)])
def test_split_without_mask_or_bias(use_mask, use_bias):
    spec = CASES["k25_c96_o40"]
    d = synth.make_inputs(spec)
    ref, norm = oracle.forward(oracle_shape(spec), d["x"], d["offset"],
                               d["mask"] if use_mask else None, d["weight"],
                               d["bias"] if use_bias else None)
    dev = device_inputs(spec, d)
    (got,) = _run(spec, dev, "nchw", split=True, use_mask=use_mask, use_bias=use_bias)
    compare(got, ref, norm, d["bias"] if use_bias else None, "f32", "split options")


def test_scratch_is_rewritten_on_every_call():
    """One packed workspace, two calls on different inputs: the second result
    is the second problem's (the partial outputs are fully overwritten)."""
    import torch
    from modulated_deformable_convolution_dcn_amd import Desc, Plan
    spec = CASES["k49_48x48"]
    plan = Plan(Desc(spec.B, spec.C, spec.H, spec.W, spec.O, spec.kh, spec.kw, spec.ph, spec.pw))
    d1 = synth.make_inputs(spec)
    d2 = synth.make_inputs(spec.scaled(seed=77))
    dev1, dev2 = device_inputs(spec, d1), device_inputs(spec, d2)
    packed = plan.pack_weight(dev1["weight"])
    plan.forward_packed(dev1["x"], dev1["offset"], dev1["mask"], packed, dev1["bias"])
    out = plan.forward_packed(dev2["x"], dev2["offset"], dev2["mask"], packed, dev1["bias"])
    torch.cuda.synchronize()
    ref, norm = oracle.forward(oracle_shape(spec), d2["x"], d2["offset"], d2["mask"], d1["weight"],
                               d1["bias"])
    compare(pixel_major(out.cpu().numpy(), "nchw"), ref, norm, d1["bias"], "f32", "second call")


# tap groups without runs: 8-wave workgroups, the two groups' sums added on chip
GROUP_CASES = {
    # 256 tiles: the birefnet512 grid, 25 + 24 taps
    "k49_128x128": B5,
    # K = 2: one tap per group; ragged last tile
    "k2_c32_o64": E.scaled(B=1, C=32, O=64, H=15, W=14, kh=1, kw=2, ph=0, pw=0),
    # K = 3 (groups of 2 and 1), two channel chunks, one ragged
    "k3_c96_o24": E.scaled(B=1, C=96, O=24, H=31, W=29, kh=1, kw=3, ph=0, pw=1),
}


@pytest.mark.parametrize("layout", ["nchw", "nhwc"])
@pytest.mark.parametrize("name", sorted(GROUP_CASES))
def test_tap_groups_match_the_oracle(name, layout):
    import torch
    from modulated_deformable_convolution_dcn_amd import Desc, Plan
    spec = GROUP_CASES[name]
    plan = Plan(Desc(spec.B, spec.C, spec.H, spec.W, spec.O, spec.kh, spec.kw, spec.ph, spec.pw,
                     spec.dtype, layout))
    assert (plan.tap_runs, plan.tap_groups) == (1, 2), "case does not run tap groups alone"
    d = synth.make_inputs(spec)
    ref, norm = oracle.forward(oracle_shape(spec), d["x"], d["offset"], d["mask"], d["weight"],
                               d["bias"])
    dev = device_inputs(spec, d)
    print("case", name, layout, spec, flush=True)
    packed = plan.pack_weight(dev["weight"])
    o1 = plan.forward_packed(dev["x"], dev["offset"], dev["mask"], packed, dev["bias"])
    o2 = plan.forward_packed(dev["x"], dev["offset"], dev["mask"], packed, dev["bias"])
    torch.cuda.synchronize()
    g1 = pixel_major(o1.cpu().numpy(), layout)
    g2 = pixel_major(o2.cpu().numpy(), layout)
    assert np.array_equal(g1.view(np.uint32), g2.view(np.uint32))  # fixed summation order
    w = compare(g1, ref, norm, d["bias"], "f32", "%s/%s tap groups" % (name, layout))
    print("worst err/N %.3g" % w)
