"""Bit-exact sampling corners: the kernels' corner stage against the oracle.

Two checks of page 1's corner step ("deform_conv.py", deform_conv2d_gather:
the point as the exact integer grid plus one fp32 add of the offset,
torch.floor, and the per-corner `valid` comparison):

* test_corner_table_*: the fused forward kernel that a plan launches (the
  same kernel and launch as dcn_forward_packed; its output is checked equal
  to the plain call's) exports the corner table it gathers from.  Every
  corner's validity and input-pixel index must equal the oracle's, bit for
  bit, for every (b, tap, pixel) of every workload, and for points exactly on
  integers, half-integers, -1, H-1, H and +-1e30 on each kernel variant.
  The corner weights (bilinear weight x mask) are compared against an
  independent float32 numpy derivation within the rounding of their few fp32
  products (bf16 rounding for the two wide bf16 kernels).
* test_coords_*: dcn_debug_coords, the stage alone from the same device
  functions, for the floor of every point (also those with no corner inside).
"""
import numpy as np
import pytest

import oracle
from modulated_deformable_convolution_dcn_amd import synth
from dcn_testlib import oracle_shape, device_inputs

pytestmark = pytest.mark.gpu


def _expected_index(y0x0, valid4, H, W):
    """[B,K,Ho,Wo,4] input-pixel index of each corner (-1 outside) from the
    oracle's floor and validity."""
    B = y0x0.shape[0]
    y0 = y0x0[..., 0].astype(np.int64)
    x0 = y0x0[..., 1].astype(np.int64)
    bimg = np.arange(B, dtype=np.int64).reshape(B, 1, 1, 1)
    idx = np.empty(y0x0.shape[:4] + (4,), np.int64)
    for c in range(4):
        a, bb = c >> 1, c & 1
        v = ((valid4 >> c) & 1).astype(bool)
        idx[..., c] = np.where(v, (bimg * H + y0 + a) * W + x0 + bb, -1)
    return idx


def _expected_weight(s, offset, mask, valid4):
    """Corner weight = bilinear weight x mask from the fp32 fractions
    (one fp32 add for the point, fp32 floor and subtraction), in fp64."""
    B, K, Ho, Wo = s.B, s.K, s.Ho, s.Wo
    off = offset.reshape(B, K, 2, Ho, Wo).astype(np.float32)
    i = (np.arange(K) // s.kw).reshape(1, K, 1, 1)
    j = (np.arange(K) % s.kw).reshape(1, K, 1, 1)
    gy = (np.arange(Ho).reshape(1, 1, Ho, 1) - s.ph + i).astype(np.float32)
    gx = (np.arange(Wo).reshape(1, 1, 1, Wo) - s.pw + j).astype(np.float32)
    py = (gy + off[:, :, 0]).astype(np.float32)
    px = (gx + off[:, :, 1]).astype(np.float32)
    ly = (py - np.floor(py)).astype(np.float64)
    lx = (px - np.floor(px)).astype(np.float64)
    m = np.ones((B, K, Ho, Wo)) if mask is None else mask.astype(np.float64)
    w = np.stack([(1 - ly) * (1 - lx), (1 - ly) * lx, ly * (1 - lx), ly * lx], axis=-1)
    w = w * m[..., None]
    for c in range(4):
        w[..., c] = np.where((valid4 >> c) & 1, w[..., c], 0.0)
    return w


def _corner_table(spec, d, layout="nchw"):
    import torch
    from modulated_deformable_convolution_dcn_amd import Desc, Plan
    dev = device_inputs(spec, d)
    plan = Plan(Desc(spec.B, spec.C, spec.H, spec.W, spec.O, spec.kh, spec.kw, spec.ph, spec.pw,
                     spec.dtype, layout))
    ws = plan.pack_weight(dev["weight"])
    out, idx, wgt = plan.debug_corner_table(dev["x"], dev["offset"], dev["mask"], ws, dev["bias"])
    plain = plan.forward_packed(dev["x"], dev["offset"], dev["mask"], ws, dev["bias"])
    torch.cuda.synchronize()
    # the hook runs the same kernel: same output, bit for bit
    assert torch.equal(out, plain)
    return idx.cpu().numpy(), wgt.cpu().numpy()


def _check_table(s, offset, mask, idx, wgt, dtype, what):
    y_ref, v_ref = oracle.coords(s, offset)
    want = _expected_index(y_ref, v_ref, s.H, s.W)
    bad = idx != want
    if bad.any():
        e = np.argwhere(bad)[0]
        raise AssertionError("%s: %d corner entries differ; first %s gpu %d oracle %d" % (
            what, int(bad.sum()), tuple(e), idx[tuple(e)], want[tuple(e)]))
    ref_w = _expected_weight(s, offset, mask, v_ref)
    outside = want < 0
    assert not (wgt[outside] != 0).any(), "%s: weight of an outside corner is not 0" % what
    rtol = 1e-6 if dtype == "f32" else 2.0 ** -8 + 1e-6
    err = np.abs(wgt.astype(np.float64) - ref_w)
    assert (err <= rtol * np.abs(ref_w) + 1e-30).all(), "%s: corner weight off by %.3g rel" % (
        what, float((err / np.maximum(np.abs(ref_w), 1e-30)).max()))


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_corner_table_bit_exact(name):
    spec = synth.WORKLOADS[name]
    d = synth.make_inputs(spec)
    print("case", name, flush=True)
    idx, wgt = _corner_table(spec, d)
    _check_table(oracle_shape(spec), d["offset"], d["mask"], idx, wgt, spec.dtype, name)


# one plan shape per kernel variant: (dtype, C, O, kernel size) -> general,
# k split, 32 x 32 per wave, wide bf16 (5 x 5: no window), wide bf16 with the
# LDS input window (3 x 3)
VARIANTS = {
    "general_f32": ("f32", 4, 4, 3),
    "general_bf16": ("bf16", 32, 64, 3),
    "ksplit_f32": ("f32", 64, 128, 3),
    "quad_f32": ("f32", 64, 64, 3),
    "wide_bf16": ("bf16", 64, 256, 5),
    "window_bf16": ("bf16", 64, 256, 3),
}
SPECIAL = np.array([-2.0, -1.5, -1.0, -0.5, -1e-7, 0.0, 0.5, 1.0, 2.5, 5.0, 5.5, 6.0, 1e30, -1e30],
                   np.float32)  # H = 6: -1, H - 1 = 5, H = 6 and half-integers around them


@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_corner_table_at_exact_integers_and_halves(variant):
    dtype, C, O, k = VARIANTS[variant]
    spec = synth.Spec(name="special", B=2, C=C, O=O, H=6, W=5, kh=k, kw=k, ph=k // 2, pw=k // 2,
                      dtype=dtype, seed=5, offset_dist="normal1.5", mask_dist="uniform",
                      weight_std=0.3, bias_dist="normal1")
    d = synth.make_inputs(spec)
    rng = np.random.default_rng(0)
    off = rng.choice(SPECIAL, size=d["offset"].shape).astype(np.float32)
    if dtype == "bf16":
        # every special value except 1e30 / -1e7 is exact in bf16; use the rounded ones
        d["offset"], d["bits"]["offset"] = synth.round_bf16(off)
    else:
        d["offset"] = off
    print("case", variant, flush=True)
    idx, wgt = _corner_table(spec, d)
    _check_table(oracle_shape(spec), d["offset"], d["mask"], idx, wgt, dtype, variant)


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_coords_bit_exact(name):
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
    np.testing.assert_array_equal(y_gpu.cpu().numpy(), y_ref)


def test_coords_at_exact_integers_and_halves():
    """Offsets that land exactly on integers, half-integers and -1 / H-1 / H."""
    import torch
    from modulated_deformable_convolution_dcn_amd import Desc, Plan
    H, W = 6, 5
    s = oracle.Shape(1, 4, H, W, 4, 3, 3, 1, 1)
    rng = np.random.default_rng(0)
    off = rng.choice(SPECIAL, size=(1, 2 * 9, s.Ho, s.Wo)).astype(np.float32)
    y_ref, v_ref = oracle.coords(s, off)
    plan = Plan(Desc(1, 4, H, W, 4, 3, 3, 1, 1))
    y_gpu, v_gpu = plan.debug_coords(torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(v_gpu.cpu().numpy(), v_ref)
    np.testing.assert_array_equal(y_gpu.cpu().numpy(), y_ref)
