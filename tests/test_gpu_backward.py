"""GPU parity of the fp32 backward (dcn_backward) against the oracle's backward.

Per gradient element: |gpu - ref| <= 1e-4 * N + ulp32(|ref|), N = the sum of
the absolute values of the terms that element adds up (the oracle's
normaliser; the inner contraction over outputs expanded too).  N == 0 means
no term reaches the element: the GPU value must then be exactly 0.  The
input / offset / mask gradients are accumulated with fp32 atomics (their
order is not fixed), which the same bound covers.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from dcn_testlib import bound_used, device_inputs, oracle_shape, record_margin
from modulated_deformable_convolution_dcn_amd import synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
E = W["edge_stress_fp32"]

CASES = {
    "c64_o64_k7": W["birefnet512_fp32"].scaled(H=24, W=21),
    "c128_o128_k5": E.scaled(B=1, H=19, W=17),
    "c72_o100_k3_b2": E.scaled(B=2, C=72, O=100, H=11, W=13, kh=3, kw=3, ph=1, pw=1),
    "c36_o16_k1": E.scaled(B=1, C=36, O=16, H=9, W=10, kh=1, kw=1, ph=0, pw=0),
    "c4_o4_tiny": W["tiny_fp32"],
    "c64_o256_k3": W["p1_k3"].scaled(H=14, W=12),
    "c32_o200_k2x3": E.scaled(B=1, C=32, O=200, H=12, W=9, kh=2, kw=3, ph=0, pw=1),
}


def _grad_out(spec, seed=123):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((spec.B, spec.O, spec.Ho, spec.Wo)).astype(np.float32)


def _check(name, got, ref, norm):
    got = got.astype(np.float64)
    err = np.abs(got - ref)
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    zero = norm == 0
    assert not (zero & (got != 0)).any(), "%s: %d elements with no terms are not 0" % (
        name, int((zero & (got != 0)).sum()))
    bad = (~zero) & (err > 1e-4 * norm + ulp)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d / %d outside tolerance; first %s gpu %.9g ref %.9g N %.3g" % (
            name, int(bad.sum()), bad.size, tuple(i), got[tuple(i)], ref[tuple(i)], norm[tuple(i)]))
    nz = ~zero
    worst = float((err[nz] / norm[nz]).max()) if nz.any() else 0.0
    record_margin("backward " + name, got.size, worst, 1e-4,
                  bound_used(err, 1e-4 * norm + ulp, nz))
    return worst


def _run(spec, d, gout, layout, use_mask=True, want=("x", "offset", "mask", "weight", "bias")):
    import torch
    from modulated_deformable_convolution_dcn_amd import Desc, Plan
    dev = device_inputs(spec, d)
    plan = Plan(Desc(spec.B, spec.C, spec.H, spec.W, spec.O, spec.kh, spec.kw, spec.ph, spec.pw,
                     spec.dtype, layout))
    g = torch.from_numpy(gout).cuda()
    if layout == "nhwc":
        g = g.permute(0, 2, 3, 1).contiguous()
    grads = plan.backward(dev["x"], dev["offset"], dev["mask"] if use_mask else None,
                          dev["weight"], g, want=want)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in grads.items()}


@pytest.mark.parametrize("layout", ["nchw", "nhwc"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_parity(name, layout):
    spec = CASES[name]
    d = synth.make_inputs(spec)
    gout = _grad_out(spec)
    ref, norm = oracle.backward(oracle_shape(spec), d["x"], d["offset"], d["mask"], d["weight"],
                                gout)
    print("case", name, layout, spec, flush=True)
    got = _run(spec, d, gout, layout)
    for k in ("x", "offset", "mask", "weight", "bias"):
        worst = _check("%s/%s grad_%s" % (name, layout, k), got[k], ref[k], norm[k])
        print("  grad_%s worst err/N %.3g" % (k, worst))


def test_backward_without_mask_and_partial_outputs():
    spec = CASES["c64_o64_k7"].scaled(H=15, W=14)
    d = synth.make_inputs(spec)
    gout = _grad_out(spec, 5)
    ref, norm = oracle.backward(oracle_shape(spec), d["x"], d["offset"], None, d["weight"], gout)
    got = _run(spec, d, gout, "nchw", use_mask=False)
    for k in ("x", "offset", "mask", "weight", "bias"):
        _check("nomask grad_%s" % k, got[k], ref[k], norm[k])
    only = _run(spec, d, gout, "nchw", use_mask=False, want=("weight",))
    assert set(only) == {"weight"}
    _check("weight only", only["weight"], ref["weight"], norm["weight"])


def test_backward_all_corners_outside():
    """Every sampling point outside the map: only the weight... nothing but the
    bias gradient is non-zero (the samples and their derivatives vanish)."""
    spec = CASES["c72_o100_k3_b2"]
    d = synth.make_inputs(spec)
    d["offset"] = np.full_like(d["offset"], float(spec.H + spec.kh + 2))
    gout = _grad_out(spec, 9)
    got = _run(spec, d, gout, "nchw")
    for k in ("x", "offset", "mask", "weight"):
        assert not got[k].any(), k
    assert np.allclose(got["bias"], gout.astype(np.float64).sum(axis=(0, 2, 3)), rtol=1e-5,
                       atol=1e-4)


@pytest.mark.parametrize("name", ["birefnet512_fp32", "birefnet1024_fp32"])
def test_backward_full_size(name):
    """The 128 x 128 and 256 x 256 (benchmarked) 64-channel 7x7 workloads at
    full size, NCHW, every element of all five gradients."""
    spec = W[name]
    d = synth.make_inputs(spec)
    gout = _grad_out(spec, 17)
    print("case %s backward full: oracle" % name, flush=True)
    ref, norm = oracle.backward(oracle_shape(spec), d["x"], d["offset"], d["mask"], d["weight"],
                                gout)
    print("case %s backward full: gpu" % name, flush=True)
    got = _run(spec, d, gout, "nchw")
    for k in ("x", "offset", "mask", "weight", "bias"):
        worst = _check("%s full grad_%s" % (name, k), got[k], ref[k], norm[k])
        print("  grad_%s worst err/N %.3g" % (k, worst))


@pytest.mark.parametrize("want", [("offset", "mask"), ("offset",), ("mask", "bias"), ("x",)])
def test_backward_partial_outputs_without_grad_x(want):
    """Offset / mask gradients without the input gradient: the data kernel
    runs its sums but no input-gradient scatter (there is no grad_x buffer)."""
    spec = CASES["c64_o64_k7"].scaled(H=13, W=15)
    d = synth.make_inputs(spec)
    gout = _grad_out(spec, 31)
    ref, norm = oracle.backward(oracle_shape(spec), d["x"], d["offset"], d["mask"], d["weight"],
                                gout)
    print("case partial", want, flush=True)
    got = _run(spec, d, gout, "nchw", want=want)
    assert set(got) == set(want)
    for k in want:
        _check("partial %s grad_%s" % ("+".join(want), k), got[k], ref[k], norm[k])


# bf16 operands: widened exactly to fp32 before the fp32 backward, so the
# oracle (which reads the same bf16-rounded values) bounds them with the fp32
# tolerance
D = W["detection_bf16"]
BF16_CASES = {
    "bf16_c64_o64_k3": D.scaled(B=1, C=64, O=64, H=14, W=13),
    "bf16_c32_o200_k2x3": D.scaled(B=2, C=32, O=200, H=9, W=11, kh=2, kw=3, ph=0, pw=1),
    "bf16_c256_o256_k3": D.scaled(B=1, H=12, W=10),
}


@pytest.mark.parametrize("layout", ["nchw", "nhwc"])
@pytest.mark.parametrize("name", sorted(BF16_CASES))
def test_backward_bf16_parity(name, layout):
    spec = BF16_CASES[name]
    d = synth.make_inputs(spec)
    gout = _grad_out(spec, 61)
    ref, norm = oracle.backward(oracle_shape(spec), d["x"], d["offset"], d["mask"], d["weight"],
                                gout)
    print("case", name, layout, spec, flush=True)
    got = _run(spec, d, gout, layout)
    for k in ("x", "offset", "mask", "weight", "bias"):
        worst = _check("%s/%s grad_%s" % (name, layout, k), got[k], ref[k], norm[k])
        print("  grad_%s worst err/N %.3g" % (k, worst))


def test_backward_bf16_detection_full_size():
    """The detection workload (B=8, 256 -> 256 channels, 64 x 64, 3x3, bf16) at
    full size, NCHW, all five gradients."""
    spec = W["detection_bf16"]
    d = synth.make_inputs(spec)
    gout = _grad_out(spec, 63)
    print("case detection_bf16 backward full: oracle", flush=True)
    ref, norm = oracle.backward(oracle_shape(spec), d["x"], d["offset"], d["mask"], d["weight"],
                                gout)
    print("case detection_bf16 backward full: gpu", flush=True)
    got = _run(spec, d, gout, "nchw")
    for k in ("x", "offset", "mask", "weight", "bias"):
        worst = _check("detection_bf16 full grad_%s" % k, got[k], ref[k], norm[k])
        print("  grad_%s worst err/N %.3g" % (k, worst))


# A seeded sweep of small random shapes through the whole backward: every
# data-gradient variant (padded outputs 16 / 64 / 128 / 256), both weight-
# gradient kernels, fp32 and bf16 plans, odd channel counts, rectangular
# kernels, one-pixel and kernel-wider-than-map maps, optional mask, both
# gradient layouts, every offset spread.
def _sweep(n=24, seed=7):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        dtype = "bf16" if rng.random() < 0.25 else "f32"
        C = int(rng.choice([8, 16, 40, 64, 72, 128] if dtype == "bf16" else
                           [4, 8, 12, 32, 36, 64, 72, 128, 132]))
        O = int(rng.choice([1, 3, 16, 17, 40, 64, 65, 100, 128, 129, 200, 256]))
        kh, kw = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        ph, pw = int(rng.integers(0, kh)), int(rng.integers(0, kw))
        H = int(rng.integers(max(1, kh - 2 * ph), 21))
        W = int(rng.integers(max(1, kw - 2 * pw), 21))
        spec = synth.Spec("bsweep%d" % len(out), int(rng.integers(1, 3)), C, O, H, W, kh, kw,
                          ph, pw, dtype, 2000 + len(out),
                          str(rng.choice(["normal1.5", "normal4", "uniform2", "edge_mix", "zero"])),
                          str(rng.choice(["sigmoid_normal", "uniform", "none"])),
                          float(1.0 / np.sqrt(kh * kw * C)), "none")
        if spec.Ho < 1 or spec.Wo < 1 or spec.pixels * O * spec.K * C > 20e6:
            continue
        out.append((spec, "nhwc" if rng.random() < 0.5 else "nchw"))
    return out


SWEEP = _sweep()


@pytest.mark.parametrize("i", range(len(SWEEP)))
def test_backward_sweep(i):
    spec, layout = SWEEP[i]
    d = synth.make_inputs(spec)
    gout = _grad_out(spec, 100 + i)
    print("case", i, layout, spec, flush=True)
    ref, norm = oracle.backward(oracle_shape(spec), d["x"], d["offset"], d["mask"], d["weight"],
                                gout)
    got = _run(spec, d, gout, layout)
    for k in ("x", "offset", "mask", "weight", "bias"):
        _check("%s/%s grad_%s" % (spec.name, layout, k), got[k], ref[k], norm[k])
