"""MI355X-native modulated deformable conv2d forward (DCNv2, gfx950).

The operator (page 1, "deform_conv.py": module docstring; page 5, deformops
README, "Deformable convolution"): for each output pixel and kernel tap,
sample the NHWC input bilinearly at the offset point (corners outside the
image count as zero), multiply by the tap's mask, contract over
(tap, channel) with the weight and add the bias.  Stride 1, dilation 1, one
offset group.

Everything is computed by the HIP kernels of ``libdcn_mi355x.so`` behind the C
ABI of ``include/dcn.h``; this module only marshals torch tensors (device
memory and the current stream) into those calls.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

from . import _lib
from ._lib import DcnError  # noqa: F401

__all__ = ["Plan", "MsdaPlan", "DsamplePlan", "deform_conv2d", "deform_conv2d_nhwc",
           "forward_multi", "msda", "dsample", "nchw_to_nhwc", "DcnError"]

_DTYPES = {"f32": _lib.DCN_F32, "bf16": _lib.DCN_BF16}
_LAYOUTS = {"nchw": _lib.DCN_OUT_NCHW, "nhwc": _lib.DCN_OUT_NHWC}


def _torch():
    import torch
    return torch


def _stream_handle(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def validation_enabled() -> bool:
    """DCN_VALIDATE=1 turns on the opt-in input check (page 5's
    DEFORMOPS_VALIDATE works the same way): before each call, offsets,
    masks, sampling locations and aggregation weights must be finite.  The
    check synchronises with the device, so it is off by default and never on
    a timed path; non-finite offsets are otherwise outside the contract."""
    return os.environ.get("DCN_VALIDATE", "") not in ("", "0")


def _validate(**tensors):
    if not validation_enabled():
        return
    torch = _torch()
    for name, t in tensors.items():
        if t is not None and not bool(torch.isfinite(t).all()):
            raise ValueError("DCN_VALIDATE: %s holds non-finite values" % name)


@dataclass(frozen=True)
class Desc:
    batch: int
    in_ch: int
    height: int
    width: int
    out_ch: int
    kernel_h: int
    kernel_w: int
    pad_h: int
    pad_w: int
    dtype: str = "f32"          # storage type of x, offset, mask, weight, bias
    out_layout: str = "nchw"    # "nchw" -> [B,O,Ho,Wo], "nhwc" -> [B,Ho,Wo,O]; fp32


class Plan:
    """One validated problem size (``dcn_create``); reusable, immutable."""

    def __init__(self, desc: Desc):
        lib = _lib.load()
        if desc.dtype not in _DTYPES:
            raise ValueError("dtype must be one of %s" % list(_DTYPES))
        if desc.out_layout not in _LAYOUTS:
            raise ValueError("out_layout must be one of %s" % list(_LAYOUTS))
        self.desc = desc
        c = _lib.DcnDesc(desc.batch, desc.in_ch, desc.height, desc.width, desc.out_ch,
                         desc.kernel_h, desc.kernel_w, desc.pad_h, desc.pad_w,
                         _DTYPES[desc.dtype], _lib.DCN_F32, _LAYOUTS[desc.out_layout])
        h = ctypes.c_void_p()
        _lib.check(lib.dcn_create(ctypes.byref(c), ctypes.byref(h)), "dcn_create")
        self._h = h
        ho, wo = ctypes.c_int32(), ctypes.c_int32()
        _lib.check(lib.dcn_output_size(h, ctypes.byref(ho), ctypes.byref(wo)), "dcn_output_size")
        self.Ho, self.Wo = ho.value, wo.value
        ws = ctypes.c_size_t()
        _lib.check(lib.dcn_workspace_bytes(h, ctypes.byref(ws)), "dcn_workspace_bytes")
        self.workspace_bytes = ws.value
        _lib.check(lib.dcn_packed_weight_bytes(h, ctypes.byref(ws)), "dcn_packed_weight_bytes")
        self.packed_weight_bytes = ws.value
        runs, kper, groups = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _lib.check(lib.dcn_tap_schedule(h, ctypes.byref(runs), ctypes.byref(kper),
                                        ctypes.byref(groups)), "dcn_tap_schedule")
        # tap runs (with a full workspace), taps per run, tap groups per workgroup
        self.tap_runs, self.taps_per_run, self.tap_groups = runs.value, kper.value, groups.value

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                _lib.load().dcn_destroy(h)
            except Exception:
                pass
            self._h = None

    # -- shapes -------------------------------------------------------------
    @property
    def K(self) -> int:
        return self.desc.kernel_h * self.desc.kernel_w

    def _torch_dtype(self):
        torch = _torch()
        return torch.float32 if self.desc.dtype == "f32" else torch.bfloat16

    def out_shape(self):
        d = self.desc
        if d.out_layout == "nchw":
            return (d.batch, d.out_ch, self.Ho, self.Wo)
        return (d.batch, self.Ho, self.Wo, d.out_ch)

    def _check(self, name, t, shape, dtype=None, optional=False):
        if t is None:
            if optional:
                return
            raise ValueError("%s is required" % name)
        if not t.is_cuda:
            raise ValueError("%s must be a device tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if tuple(t.shape) != tuple(shape):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
        want = dtype if dtype is not None else self._torch_dtype()
        if t.dtype != want:
            raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, want))

    def _check_inputs(self, x, offset, mask, bias):
        d = self.desc
        self._check("x", x, (d.batch, d.height, d.width, d.in_ch))
        self._check("offset", offset, (d.batch, 2 * self.K, self.Ho, self.Wo))
        self._check("mask", mask, (d.batch, self.K, self.Ho, self.Wo), optional=True)
        self._check("bias", bias, (d.out_ch,), optional=True)
        _validate(offset=offset, mask=mask)

    # -- calls --------------------------------------------------------------
    def new_workspace(self, split=True):
        """A workspace of ``dcn_workspace_bytes`` bytes, or with ``split=False``
        only ``dcn_packed_weight_bytes`` (forward calls then never split taps)."""
        torch = _torch()
        n = self.workspace_bytes if split else self.packed_weight_bytes
        return torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")

    def new_output(self):
        torch = _torch()
        return torch.empty(self.out_shape(), dtype=torch.float32, device="cuda")

    def pack_weight(self, weight, workspace=None, stream=None, split=True):
        """``dcn_pack_weight``: weight [O,C,kh,kw] -> packed workspace (returned;
        ``split`` as for ``new_workspace``)."""
        d = self.desc
        self._check("weight", weight, (d.out_ch, d.in_ch, d.kernel_h, d.kernel_w))
        ws = workspace if workspace is not None else self.new_workspace(split)
        _lib.check(_lib.load().dcn_pack_weight(self._h, _ptr(weight), _ptr(ws), ws.numel(),
                                               ctypes.c_void_p(_stream_handle(stream))),
                   "dcn_pack_weight")
        return ws

    def forward_packed(self, x, offset, mask, packed, bias=None, out=None, stream=None):
        """``dcn_forward_packed``: the fused forward from a packed weight."""
        self._check_inputs(x, offset, mask, bias)
        out = out if out is not None else self.new_output()
        self._check("out", out, self.out_shape(), dtype=_torch().float32)
        _lib.check(_lib.load().dcn_forward_packed(
            self._h, _ptr(x), _ptr(offset), _ptr(mask), _ptr(packed), packed.numel(),
            _ptr(bias), _ptr(out), ctypes.c_void_p(_stream_handle(stream))),
            "dcn_forward_packed")
        return out

    def forward(self, x, offset, mask, weight, bias=None, out=None, workspace=None,
                stream=None):
        """``dcn_forward``: pack the weight and run the fused forward."""
        d = self.desc
        self._check_inputs(x, offset, mask, bias)
        self._check("weight", weight, (d.out_ch, d.in_ch, d.kernel_h, d.kernel_w))
        out = out if out is not None else self.new_output()
        self._check("out", out, self.out_shape(), dtype=_torch().float32)
        ws = workspace if workspace is not None else self.new_workspace()
        _lib.check(_lib.load().dcn_forward(
            self._h, _ptr(x), _ptr(offset), _ptr(mask), _ptr(weight), _ptr(bias), _ptr(out),
            _ptr(ws), ws.numel(), ctypes.c_void_p(_stream_handle(stream))), "dcn_forward")
        return out

    def forward_rows(self, row0, x, offset, mask, packed, bias=None, out=None, stream=None):
        """``dcn_forward_rows``: output rows [row0, row0 + rows) where rows is
        offset.shape[2]; offset/mask/out cover those rows only, x is whole."""
        d = self.desc
        rows = offset.shape[2] if offset is not None and offset.dim() == 4 else -1
        self._check("x", x, (d.batch, d.height, d.width, d.in_ch))
        self._check("offset", offset, (d.batch, 2 * self.K, rows, self.Wo))
        self._check("mask", mask, (d.batch, self.K, rows, self.Wo), optional=True)
        self._check("bias", bias, (d.out_ch,), optional=True)
        _validate(offset=offset, mask=mask)
        shape = ((d.batch, d.out_ch, rows, self.Wo) if d.out_layout == "nchw"
                 else (d.batch, rows, self.Wo, d.out_ch))
        if out is None:
            out = _torch().empty(shape, dtype=_torch().float32, device="cuda")
        self._check("out", out, shape, dtype=_torch().float32)
        _lib.check(_lib.load().dcn_forward_rows(
            self._h, int(row0), int(rows), _ptr(x), _ptr(offset), _ptr(mask), _ptr(packed),
            packed.numel(), _ptr(bias), _ptr(out), ctypes.c_void_p(_stream_handle(stream))),
            "dcn_forward_rows")
        return out

    def backward_workspace_bytes(self) -> int:
        n = ctypes.c_size_t()
        _lib.check(_lib.load().dcn_backward_workspace_bytes(self._h, ctypes.byref(n)),
                   "dcn_backward_workspace_bytes")
        return n.value

    def backward(self, x, offset, mask, weight, grad_out, want=("x", "offset", "mask", "weight",
                                                                 "bias"),
                 grads=None, workspace=None, stream=None):
        """``dcn_backward``: returns {name: gradient} for the names in ``want``
        (x [B,H,W,C], offset, mask [B,K,Ho,Wo], weight, bias [O]; fp32)."""
        torch = _torch()
        d = self.desc
        self._check_inputs(x, offset, mask, None)
        self._check("weight", weight, (d.out_ch, d.in_ch, d.kernel_h, d.kernel_w))
        self._check("grad_out", grad_out, self.out_shape(), dtype=torch.float32)
        shapes = {"x": (d.batch, d.height, d.width, d.in_ch),
                  "offset": (d.batch, 2 * self.K, self.Ho, self.Wo),
                  "mask": (d.batch, self.K, self.Ho, self.Wo),
                  "weight": (d.out_ch, d.in_ch, d.kernel_h, d.kernel_w), "bias": (d.out_ch,)}
        grads = dict(grads or {})
        for k in want:
            if k not in shapes:
                raise ValueError("unknown gradient %r" % k)
            if k not in grads:
                grads[k] = torch.empty(shapes[k], dtype=torch.float32, device="cuda")
            self._check("grad_" + k, grads[k], shapes[k], dtype=torch.float32)
        ws = workspace
        if ws is None:
            ws = torch.empty(max(self.backward_workspace_bytes(), 16), dtype=torch.uint8,
                             device="cuda")
        g = lambda k: _ptr(grads.get(k)) if k in want else None  # noqa: E731
        _lib.check(_lib.load().dcn_backward(
            self._h, _ptr(x), _ptr(offset), _ptr(mask), _ptr(weight), _ptr(grad_out),
            g("x"), g("offset"), g("mask"), g("weight"), g("bias"), _ptr(ws), ws.numel(),
            ctypes.c_void_p(_stream_handle(stream))), "dcn_backward")
        return {k: grads[k] for k in want}

    def debug_corner_table(self, x, offset, mask, packed, bias=None, out=None, stream=None):
        """``dcn_debug_corner_table``: the forward from a packed weight (as
        ``forward_packed``) plus the corner table its kernel built:
        (out, corner_index [B,K,Ho,Wo,4] int32, corner_weight [B,K,Ho,Wo,4] fp32)."""
        torch = _torch()
        d = self.desc
        self._check_inputs(x, offset, mask, bias)
        out = out if out is not None else self.new_output()
        self._check("out", out, self.out_shape(), dtype=torch.float32)
        shape = (d.batch, self.K, self.Ho, self.Wo, 4)
        idx = torch.full(shape, -2, dtype=torch.int32, device="cuda")
        wgt = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
        _lib.check(_lib.load().dcn_debug_corner_table(
            self._h, _ptr(x), _ptr(offset), _ptr(mask), _ptr(packed), packed.numel(), _ptr(bias),
            _ptr(out), _ptr(idx), _ptr(wgt), ctypes.c_void_p(_stream_handle(stream))),
            "dcn_debug_corner_table")
        return out, idx, wgt

    def debug_coords(self, offset, stream=None):
        """``dcn_debug_coords``: (y0x0 [B,K,Ho,Wo,2] int32, valid4 [B,K,Ho,Wo] uint8)."""
        torch = _torch()
        d = self.desc
        self._check("offset", offset, (d.batch, 2 * self.K, self.Ho, self.Wo))
        y0x0 = torch.empty((d.batch, self.K, self.Ho, self.Wo, 2), dtype=torch.int32,
                           device="cuda")
        valid4 = torch.empty((d.batch, self.K, self.Ho, self.Wo), dtype=torch.uint8,
                             device="cuda")
        _lib.check(_lib.load().dcn_debug_coords(self._h, _ptr(offset), _ptr(y0x0), _ptr(valid4),
                                                ctypes.c_void_p(_stream_handle(stream))),
                   "dcn_debug_coords")
        return y0x0, valid4


_PLANS = {}


def plan_for(desc: Desc) -> Plan:
    p = _PLANS.get(desc)
    if p is None:
        p = Plan(desc)
        _PLANS[desc] = p
    return p


def deform_conv2d_nhwc(x, offset, weight, bias=None, padding=0, mask=None, out_layout="nchw"):
    """Modulated deformable conv2d on an NHWC input (stride 1, dilation 1).

    x [B,H,W,C]; offset [B,2*kh*kw,Ho,Wo] (dy, dx per tap); mask [B,kh*kw,Ho,Wo]
    or None; weight [O,C,kh,kw]; bias [O] or None; all float32 or all bfloat16
    device tensors.  Returns fp32 [B,O,Ho,Wo] (``out_layout="nchw"``) or
    [B,Ho,Wo,O] (``"nhwc"``).
    """
    torch = _torch()
    ph, pw = (padding, padding) if isinstance(padding, int) else tuple(padding)
    B, H, W, C = x.shape
    O, _, kh, kw = weight.shape
    dtype = {torch.float32: "f32", torch.bfloat16: "bf16"}.get(x.dtype)
    if dtype is None:
        raise ValueError("x must be float32 or bfloat16, got %s" % x.dtype)
    plan = plan_for(Desc(B, C, H, W, O, kh, kw, ph, pw, dtype, out_layout))
    return plan.forward(x, offset, mask, weight, bias)


def nchw_to_nhwc(x, out=None, stream=None):
    """``dcn_nchw_to_nhwc``: [B,C,H,W] -> [B,H,W,C] on the GPU (float32 or bfloat16)."""
    torch = _torch()
    dtype = {torch.float32: _lib.DCN_F32, torch.bfloat16: _lib.DCN_BF16}.get(x.dtype)
    if dtype is None:
        raise ValueError("x must be float32 or bfloat16, got %s" % x.dtype)
    if x.dim() != 4 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous 4-d device tensor")
    B, C, H, W = x.shape
    if out is None:
        out = torch.empty((B, H, W, C), dtype=x.dtype, device=x.device)
    if tuple(out.shape) != (B, H, W, C) or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B,H,W,C] tensor of x's dtype")
    _lib.check(_lib.load().dcn_nchw_to_nhwc(_ptr(x), _ptr(out), B, C, H, W, dtype,
                                            ctypes.c_void_p(_stream_handle(stream))),
               "dcn_nchw_to_nhwc")
    return out


def deform_conv2d(input, offset, weight, bias=None, padding=0, mask=None, out_layout="nchw"):
    """torchvision-order drop-in (page 5's torchvision integration): NCHW
    ``input`` [B,C,H,W], offset [B,2*kh*kw,Ho,Wo], weight [O,C,kh,kw], bias
    [O] or None, mask [B,kh*kw,Ho,Wo] or None; stride 1, dilation 1.  The input
    is moved to NHWC by the library's transpose kernel, then the fused forward
    runs.  Returns fp32 [B,O,Ho,Wo] (or [B,Ho,Wo,O] with ``out_layout="nhwc"``)."""
    return deform_conv2d_nhwc(nchw_to_nhwc(input), offset, weight, bias, padding, mask,
                              out_layout)


def forward_multi(plans, x, offsets, masks, packeds, biases=None, outs=None, stream=None):
    """``dcn_forward_multi``: branch i = plans[i] on the shared NHWC ``x`` with
    offsets[i], masks[i] (or None), packed weight packeds[i] (from
    plans[i].pack_weight), biases[i] (or None); returns the list of outputs.
    Branches that run the same kernel variant share one launch."""
    n = len(plans)
    masks = masks if masks is not None else [None] * n
    biases = biases if biases is not None else [None] * n
    outs = outs if outs is not None else [p.new_output() for p in plans]
    if not (len(offsets) == len(masks) == len(packeds) == len(biases) == len(outs) == n):
        raise ValueError("one offset, mask, packed weight, bias and output per plan")
    for p, off, m, b, o in zip(plans, offsets, masks, biases, outs):
        p._check_inputs(x, off, m, b)
        p._check("out", o, p.out_shape(), dtype=_torch().float32)
    arr = lambda items: (ctypes.c_void_p * n)(*[None if t is None else t.data_ptr()  # noqa: E731
                                                for t in items])
    handles = (ctypes.c_void_p * n)(*[p._h.value for p in plans])
    sizes = (ctypes.c_size_t * n)(*[w.numel() for w in packeds])
    _lib.check(_lib.load().dcn_forward_multi(
        n, handles, _ptr(x), arr(offsets), arr(masks), arr(packeds), sizes, arr(biases),
        arr(outs), ctypes.c_void_p(_stream_handle(stream))), "dcn_forward_multi")
    return outs


class MsdaPlan:
    """``dcn_msda_create``: multi-scale deformable attention sampling of one size."""

    def __init__(self, batch, num_queries, num_heads, head_dim, shapes, num_points,
                 softmax=False, dtype="f32"):
        lib = _lib.load()
        if dtype not in _DTYPES:
            raise ValueError("dtype must be one of %s" % list(_DTYPES))
        self.dtype = dtype
        shapes = [(int(h), int(w)) for h, w in shapes]
        self.shapes = shapes
        self.B, self.Q, self.G, self.D = batch, num_queries, num_heads, head_dim
        self.L, self.K = len(shapes), num_points
        self.softmax = bool(softmax)
        d = _lib.MsdaDesc(batch, num_queries, num_heads, head_dim, len(shapes), num_points,
                          _DTYPES[dtype], int(bool(softmax)))
        hw = (ctypes.c_int32 * (2 * len(shapes)))(*[v for s in shapes for v in s])
        h = ctypes.c_void_p()
        _lib.check(lib.dcn_msda_create(ctypes.byref(d), hw, ctypes.byref(h)), "dcn_msda_create")
        self._h = h
        n = ctypes.c_int32()
        _lib.check(lib.dcn_msda_value_positions(h, ctypes.byref(n)), "dcn_msda_value_positions")
        self.S = n.value

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                _lib.load().dcn_msda_destroy(h)
            except Exception:
                pass
            self._h = None

    def forward(self, value, locations, weights, out=None, stream=None):
        """value [B,S,G,D], locations [B,Q,G,L,K,2], weights [B,Q,G,L*K] (device
        tensors of the plan's dtype) -> out [B,Q,G*D] fp32."""
        torch = _torch()
        want = torch.float32 if self.dtype == "f32" else torch.bfloat16
        shapes = {"value": (self.B, self.S, self.G, self.D),
                  "locations": (self.B, self.Q, self.G, self.L, self.K, 2),
                  "weights": (self.B, self.Q, self.G, self.L * self.K)}
        for name, t in (("value", value), ("locations", locations), ("weights", weights)):
            if not t.is_cuda or not t.is_contiguous() or t.dtype != want:
                raise ValueError("%s must be a contiguous %s device tensor" % (name, want))
            if tuple(t.shape) != shapes[name]:
                raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape),
                                                                    shapes[name]))
        _validate(locations=locations, weights=weights)
        if out is None:
            out = torch.empty((self.B, self.Q, self.G * self.D), dtype=torch.float32,
                              device="cuda")
        if tuple(out.shape) != (self.B, self.Q, self.G * self.D) or not out.is_contiguous():
            raise ValueError("out must be a contiguous [B, Q, G*D] float32 tensor")
        _lib.check(_lib.load().dcn_msda_forward(self._h, _ptr(value), _ptr(locations),
                                                _ptr(weights), _ptr(out),
                                                ctypes.c_void_p(_stream_handle(stream))),
                   "dcn_msda_forward")
        return out


_MSDA_PLANS = {}


def msda(value, shapes, locations, weights, softmax=False):
    """Multi-scale deformable attention sampling (page 5's functional form):
    value [B,S,G,D], shapes [(H, W), ...], locations [B,Q,G,L,K,2] normalised
    (x, y), weights [B,Q,G,L*K] (logits when ``softmax``) -> [B,Q,G*D]."""
    torch = _torch()
    B, S, G, D = value.shape
    _, Q, _, L, K, _ = locations.shape
    dtype = {torch.float32: "f32", torch.bfloat16: "bf16"}.get(value.dtype)
    if dtype is None:
        raise ValueError("value must be float32 or bfloat16, got %s" % value.dtype)
    key = (B, Q, G, D, tuple((int(h), int(w)) for h, w in shapes), K, bool(softmax), dtype)
    p = _MSDA_PLANS.get(key)
    if p is None:
        p = MsdaPlan(B, Q, G, D, shapes, K, softmax, dtype)
        _MSDA_PLANS[key] = p
    return p.forward(value, locations, weights)


class DsamplePlan:
    """``dcn_dsample_create``: single-scale deformable sampling (page 5's DCNv3
    form) of one size: x [B,H,W,G*D] NHWC, offset [B,G*2K,Ho,Wo] (channel
    (g*K + k)*2 = dy, +1 = dx), weights [B,G*K,Ho,Wo] (logits when
    ``softmax``); out fp32 [B,Ho,Wo,G*D] ("nhwc") or [B,G*D,Ho,Wo] ("nchw")."""

    def __init__(self, batch, groups, group_ch, height, width, kernel_h, kernel_w, pad_h, pad_w,
                 dtype="f32", softmax=True, out_layout="nhwc"):
        lib = _lib.load()
        if dtype not in _DTYPES or out_layout not in _LAYOUTS:
            raise ValueError("dtype in %s, out_layout in %s" % (list(_DTYPES), list(_LAYOUTS)))
        self.B, self.G, self.D = batch, groups, group_ch
        self.H, self.W, self.kh, self.kw = height, width, kernel_h, kernel_w
        self.dtype, self.softmax, self.out_layout = dtype, bool(softmax), out_layout
        d = _lib.DsDesc(batch, groups, group_ch, height, width, kernel_h, kernel_w, pad_h, pad_w,
                        _DTYPES[dtype], int(bool(softmax)), _LAYOUTS[out_layout])
        h = ctypes.c_void_p()
        _lib.check(lib.dcn_dsample_create(ctypes.byref(d), ctypes.byref(h)), "dcn_dsample_create")
        self._h = h
        ho, wo = ctypes.c_int32(), ctypes.c_int32()
        _lib.check(lib.dcn_dsample_output_size(h, ctypes.byref(ho), ctypes.byref(wo)),
                   "dcn_dsample_output_size")
        self.Ho, self.Wo = ho.value, wo.value

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                _lib.load().dcn_dsample_destroy(h)
            except Exception:
                pass
            self._h = None

    @property
    def K(self) -> int:
        return self.kh * self.kw

    def out_shape(self):
        C = self.G * self.D
        return ((self.B, self.Ho, self.Wo, C) if self.out_layout == "nhwc"
                else (self.B, C, self.Ho, self.Wo))

    def forward(self, x, offset, weights, out=None, stream=None):
        torch = _torch()
        want = torch.float32 if self.dtype == "f32" else torch.bfloat16
        shapes = {"x": (self.B, self.H, self.W, self.G * self.D),
                  "offset": (self.B, self.G * 2 * self.K, self.Ho, self.Wo),
                  "weights": (self.B, self.G * self.K, self.Ho, self.Wo)}
        for name, t in (("x", x), ("offset", offset), ("weights", weights)):
            if not t.is_cuda or not t.is_contiguous() or t.dtype != want:
                raise ValueError("%s must be a contiguous %s device tensor" % (name, want))
            if tuple(t.shape) != shapes[name]:
                raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape),
                                                                    shapes[name]))
        _validate(offset=offset, weights=weights)
        if out is None:
            out = torch.empty(self.out_shape(), dtype=torch.float32, device="cuda")
        if (tuple(out.shape) != self.out_shape() or out.dtype != torch.float32 or
                not out.is_contiguous()):
            raise ValueError("out must be a contiguous float32 tensor of shape %s"
                             % (self.out_shape(),))
        _lib.check(_lib.load().dcn_dsample_forward(self._h, _ptr(x), _ptr(offset),
                                                   _ptr(weights), _ptr(out),
                                                   ctypes.c_void_p(_stream_handle(stream))),
                   "dcn_dsample_forward")
        return out


_DS_PLANS = {}


def dsample(x, offset, weights, groups, kernel_size, padding=0, softmax=True, out_layout="nhwc"):
    """Single-scale deformable sampling (page 5, DCNv3 form) on NHWC ``x``
    [B,H,W,G*D]; ``kernel_size`` and ``padding`` an int or a pair."""
    torch = _torch()
    kh, kw = (kernel_size, kernel_size) if isinstance(kernel_size, int) else tuple(kernel_size)
    ph, pw = (padding, padding) if isinstance(padding, int) else tuple(padding)
    B, H, W, C = x.shape
    if C % groups:
        raise ValueError("channels %d are not a multiple of groups %d" % (C, groups))
    dtype = {torch.float32: "f32", torch.bfloat16: "bf16"}.get(x.dtype)
    if dtype is None:
        raise ValueError("x must be float32 or bfloat16, got %s" % x.dtype)
    key = (B, groups, C // groups, H, W, kh, kw, ph, pw, dtype, bool(softmax), out_layout)
    p = _DS_PLANS.get(key)
    if p is None:
        p = DsamplePlan(*key)
        _DS_PLANS[key] = p
    return p.forward(x, offset, weights)
