"""Helpers shared by the GPU parity tests: run the HIP path, compare to the oracle.

Tolerances (per output element, N = sum over taps and channels of
|weight| * |modulated sample|, computed by the oracle; N excludes the bias):
  fp32 operands:                  |gpu - ref| <= 1e-4 * N + ulp32(|ref|)
  bf16 operands, fp32 accumulate: |gpu - ref| <= 2e-2 * N + ulp32(|ref|)
  N == 0 (every corner outside or mask 0): gpu == bias exactly.
The ulp term covers the final fp32 rounding of acc + bias when |bias| >> N.
"""
from __future__ import annotations

import numpy as np

import oracle
from modulated_deformable_convolution_dcn_amd import synth

TOL = {"f32": 1e-4, "bf16": 2e-2}

# Per comparison of this session: what, elements compared, the worst
# err / N, the tolerance factor on N, and the largest share of the whole
# per-element bound (tol * N + ulp32(|ref|)) that any element used.  Written
# out at session end when DCN_PARITY_MARGINS names a file (tests/conftest.py).
MARGINS = []


def record_margin(what: str, n: int, worst: float, tol: float, used: float) -> None:
    MARGINS.append({"what": what, "elements": int(n), "worst_err_over_N": float(worst),
                    "tol": float(tol), "bound_used": float(used)})


def bound_used(err: np.ndarray, bound: np.ndarray, mask: np.ndarray) -> float:
    """max over masked elements of err / bound (0 when none)."""
    return float((err[mask] / bound[mask]).max()) if mask.any() else 0.0


def oracle_shape(spec: synth.Spec) -> oracle.Shape:
    return oracle.Shape(spec.B, spec.C, spec.H, spec.W, spec.O, spec.kh, spec.kw, spec.ph, spec.pw)


def to_device(arr, dtype: str, bits=None):
    """float32 numpy -> device tensor of the workload dtype (bf16 from its bit patterns)."""
    import torch
    if arr is None:
        return None
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()
    assert bits is not None
    t = torch.from_numpy(bits.astype(np.int16).copy()).cuda()
    return t.view(torch.bfloat16)


def device_inputs(spec: synth.Spec, d: dict) -> dict:
    bits = d.get("bits", {})
    return {k: to_device(d[k], spec.dtype, bits.get(k)) for k in ("x", "offset", "mask", "weight", "bias")}


def run_gpu(spec: synth.Spec, d: dict, layout: str = "nchw", use_mask=True, use_bias=True):
    """Whole forward on the GPU; returns the output as numpy, pixel-major [P, O]."""
    import torch
    from modulated_deformable_convolution_dcn_amd import Desc, Plan
    dev = device_inputs(spec, d)
    plan = Plan(Desc(spec.B, spec.C, spec.H, spec.W, spec.O, spec.kh, spec.kw, spec.ph, spec.pw,
                     spec.dtype, layout))
    out = plan.forward(dev["x"], dev["offset"], dev["mask"] if use_mask else None, dev["weight"],
                       dev["bias"] if use_bias else None)
    torch.cuda.synchronize()
    return pixel_major(out.cpu().numpy(), layout)


def pixel_major(out: np.ndarray, layout: str) -> np.ndarray:
    if layout == "nchw":
        B, O, Ho, Wo = out.shape
        return out.transpose(0, 2, 3, 1).reshape(-1, O)
    B, Ho, Wo, O = out.shape
    return out.reshape(-1, O)


def compare(gpu: np.ndarray, ref: np.ndarray, norm: np.ndarray, bias, dtype: str, what: str):
    """Assert the parity bar element by element; returns the worst err / N."""
    gpu = gpu.astype(np.float64)
    err = np.abs(gpu - ref)
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    tol = TOL[dtype] * norm + ulp
    zero = norm == 0
    if zero.any():
        b = np.zeros(ref.shape[1]) if bias is None else np.asarray(bias, dtype=np.float32).astype(np.float64)
        bb = np.broadcast_to(b, ref.shape)
        bad0 = zero & (gpu != bb)
        assert not bad0.any(), "%s: %d outputs with N == 0 differ from the bias" % (what, int(bad0.sum()))
    bad = (~zero) & (err > tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        msg = ["%s: %d / %d outputs outside tolerance" % (what, int(bad.sum()), bad.size)]
        for p, o in idx:
            msg.append("  pixel %d o %d: gpu %.9g ref %.9g N %.3g err/N %.3g" % (
                p, o, gpu[p, o], ref[p, o], norm[p, o], err[p, o] / max(norm[p, o], 1e-300)))
        raise AssertionError("\n".join(msg))
    nz = ~zero
    worst = float((err[nz] / norm[nz]).max()) if nz.any() else 0.0
    record_margin(what, gpu.size, worst, TOL[dtype], bound_used(err, tol, nz))
    return worst
