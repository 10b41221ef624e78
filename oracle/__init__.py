"""CPU oracle for the modulated deformable conv2d forward -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never loads it and it
loads nothing of the GPU library: the two share no code.

The arithmetic lives in ``dcn_oracle.cpp`` (a plain C++ loop nest written from
page 1, "deform_conv.py": module docstring and ``deform_conv2d_gather``).  This
module only compiles it with g++ and marshals numpy arrays through ctypes.

Every function here is pinned by ``tests/test_oracle_pins.py`` against facts
that do not come from the oracle itself (direct convolution, integer shifts,
out-of-image sampling, a hand-derived 2x2 example, tap order, partition of
unity, linearity, and an independent numpy formulation).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dcn_oracle.cpp")
_LIB = os.path.join(_HERE, "libdcn_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/libdcn_oracle.so`` (g++, no SIMD flags)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-shared",
           "-fPIC", "-pthread", "-o", tmp, _SRC]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


class _Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "batch", "in_ch", "height", "width", "out_ch", "kernel_h", "kernel_w", "pad_h", "pad_w")]


class _DsShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "batch", "groups", "group_ch", "height", "width", "kernel_h", "kernel_w", "pad_h",
        "pad_w")]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        vp = ctypes.c_void_p
        lib.dcn_oracle_forward.argtypes = [ctypes.POINTER(_Shape), vp, vp, vp, vp, vp, vp,
                                           ctypes.c_int64, vp, vp, ctypes.c_int]
        lib.dcn_oracle_forward.restype = ctypes.c_int
        lib.dcn_oracle_coords.argtypes = [ctypes.POINTER(_Shape), vp, vp, vp, ctypes.c_int]
        lib.dcn_oracle_coords.restype = ctypes.c_int
        lib.dcn_oracle_backward.argtypes = [ctypes.POINTER(_Shape)] + [vp] * 15 + [ctypes.c_int]
        lib.dcn_oracle_backward.restype = ctypes.c_int
        i64 = ctypes.c_int64
        lib.dcn_oracle_msda.argtypes = [i64] * 7 + [vp] * 4 + [ctypes.c_int, vp, vp, ctypes.c_int]
        lib.dcn_oracle_msda.restype = ctypes.c_int
        lib.dcn_oracle_dsample.argtypes = [ctypes.POINTER(_DsShape), vp, vp, vp, ctypes.c_int, vp,
                                           vp, ctypes.c_int]
        lib.dcn_oracle_dsample.restype = ctypes.c_int
        _lib = lib
    return _lib


@dataclass(frozen=True)
class Shape:
    """Problem size: x [B,H,W,C] NHWC, weight [O,C,kh,kw], padding (ph, pw)."""
    B: int
    C: int
    H: int
    W: int
    O: int
    kh: int
    kw: int
    ph: int
    pw: int

    @property
    def K(self) -> int:
        return self.kh * self.kw

    @property
    def Ho(self) -> int:
        return self.H + 2 * self.ph - self.kh + 1

    @property
    def Wo(self) -> int:
        return self.W + 2 * self.pw - self.kw + 1

    def _c(self) -> _Shape:
        return _Shape(self.B, self.C, self.H, self.W, self.O, self.kh, self.kw, self.ph, self.pw)


def _f32(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    """Threads for a call that asks for 0: this process's CPU share (the
    affinity mask, or OMP_NUM_THREADS when set), at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, 16))


def _threads(n: int) -> int:
    return int(n) if n and n > 0 else default_threads()


def forward(shape: Shape, x, offset, mask, weight, bias, pixels=None, nthreads: int = 0,
            with_norm: bool = True):
    """Oracle forward.

    Returns ``(out, norm)`` as float64 arrays of shape [npix, O] (pixel-major;
    ``pixels`` are linear ids ``(b*Ho + ho)*Wo + wo``; None = all pixels in
    order).  ``norm`` = sum over (tap, channel) of |weight|*|sample|, the
    normaliser of the parity tolerance; None when ``with_norm`` is False.
    """
    s = shape
    x, offset, mask, weight, bias = (_f32(a) for a in (x, offset, mask, weight, bias))
    assert x.shape == (s.B, s.H, s.W, s.C), x.shape
    assert offset.shape == (s.B, 2 * s.K, s.Ho, s.Wo), offset.shape
    assert mask is None or mask.shape == (s.B, s.K, s.Ho, s.Wo), mask.shape
    assert weight.shape == (s.O, s.C, s.kh, s.kw), weight.shape
    assert bias is None or bias.shape == (s.O,), bias.shape
    if pixels is None:
        npix = s.B * s.Ho * s.Wo
        pix = None
    else:
        pix = np.ascontiguousarray(pixels, dtype=np.int64)
        npix = int(pix.size)
    out = np.empty((npix, s.O), dtype=np.float64)
    norm = np.empty((npix, s.O), dtype=np.float64) if with_norm else None
    cs = s._c()
    rc = _load().dcn_oracle_forward(ctypes.byref(cs), _ptr(x), _ptr(offset), _ptr(mask),
                                    _ptr(weight), _ptr(bias), _ptr(pix), npix, _ptr(out),
                                    _ptr(norm), _threads(nthreads))
    if rc != 0:
        raise ValueError("dcn_oracle_forward failed with code %d" % rc)
    return out, norm


def forward_nchw(shape: Shape, x, offset, mask, weight, bias, nthreads: int = 0):
    """Whole output as [B, O, Ho, Wo] float64, plus the normaliser in the same layout."""
    s = shape
    out, norm = forward(s, x, offset, mask, weight, bias, None, nthreads)
    to = lambda a: a.reshape(s.B, s.Ho, s.Wo, s.O).transpose(0, 3, 1, 2).copy()
    return to(out), to(norm)


def coords(shape: Shape, offset, nthreads: int = 0):
    """Sampling corners: ``(y0x0 [B,K,Ho,Wo,2] int32, valid4 [B,K,Ho,Wo] uint8)``."""
    s = shape
    offset = _f32(offset)
    assert offset.shape == (s.B, 2 * s.K, s.Ho, s.Wo), offset.shape
    y0x0 = np.empty((s.B, s.K, s.Ho, s.Wo, 2), dtype=np.int32)
    valid4 = np.empty((s.B, s.K, s.Ho, s.Wo), dtype=np.uint8)
    cs = s._c()
    rc = _load().dcn_oracle_coords(ctypes.byref(cs), _ptr(offset), _ptr(y0x0), _ptr(valid4),
                                   _threads(nthreads))
    if rc != 0:
        raise ValueError("dcn_oracle_coords failed with code %d" % rc)
    return y0x0, valid4


def backward(shape: Shape, x, offset, mask, weight, grad_out, nthreads: int = 0):
    """Oracle backward: the exact derivative of ``forward`` (see dcn_oracle.h).

    ``grad_out`` is dL/dout in the forward's NCHW layout [B, O, Ho, Wo].
    Returns ``(grads, norms)``: dicts with keys ``x`` [B,H,W,C], ``offset``
    [B,2K,Ho,Wo], ``mask`` [B,K,Ho,Wo], ``weight`` [O,C,kh,kw], ``bias`` [O],
    float64; ``norms`` holds each element's absolute-term sum (the parity
    normaliser).
    """
    s = shape
    x, offset, mask, weight, grad_out = (_f32(a) for a in (x, offset, mask, weight, grad_out))
    assert x.shape == (s.B, s.H, s.W, s.C), x.shape
    assert offset.shape == (s.B, 2 * s.K, s.Ho, s.Wo), offset.shape
    assert mask is None or mask.shape == (s.B, s.K, s.Ho, s.Wo), mask.shape
    assert weight.shape == (s.O, s.C, s.kh, s.kw), weight.shape
    assert grad_out.shape == (s.B, s.O, s.Ho, s.Wo), grad_out.shape
    shapes = {"x": (s.B, s.H, s.W, s.C), "offset": (s.B, 2 * s.K, s.Ho, s.Wo),
              "mask": (s.B, s.K, s.Ho, s.Wo), "weight": (s.O, s.C, s.kh, s.kw), "bias": (s.O,)}
    g = {k: np.empty(v, dtype=np.float64) for k, v in shapes.items()}
    n = {k: np.empty(v, dtype=np.float64) for k, v in shapes.items()}
    order = ("x", "offset", "mask", "weight", "bias")
    cs = s._c()
    rc = _load().dcn_oracle_backward(ctypes.byref(cs), _ptr(x), _ptr(offset), _ptr(mask),
                                     _ptr(weight), _ptr(grad_out),
                                     *[_ptr(g[k]) for k in order], *[_ptr(n[k]) for k in order],
                                     _threads(nthreads))
    if rc != 0:
        raise ValueError("dcn_oracle_backward failed with code %d" % rc)
    return g, n


def msda(value, shapes, locations, weights, softmax: bool, nthreads: int = 0):
    """Oracle multi-scale deformable attention sampling (see dcn_oracle.h).

    value (B, S, G, D), shapes [(H, W), ...], locations (B, Q, G, L, K, 2)
    with component 0 = x (column), 1 = y (row), weights (B, Q, G, L*K).
    Returns ``(out, norm)``, float64 (B, Q, G, D).
    """
    value, locations, weights = (_f32(a) for a in (value, locations, weights))
    B, S, G, D = value.shape
    _, Q, _, L, K, _ = locations.shape
    assert locations.shape == (B, Q, G, L, K, 2), locations.shape
    assert weights.shape == (B, Q, G, L * K), weights.shape
    sh = np.ascontiguousarray(np.asarray(shapes, dtype=np.int64).reshape(L, 2))
    out = np.empty((B, Q, G, D), dtype=np.float64)
    norm = np.empty((B, Q, G, D), dtype=np.float64)
    rc = _load().dcn_oracle_msda(B, S, G, D, Q, L, K, _ptr(sh), _ptr(value), _ptr(locations),
                                 _ptr(weights), int(bool(softmax)), _ptr(out), _ptr(norm),
                                 _threads(nthreads))
    if rc != 0:
        raise ValueError("dcn_oracle_msda failed with code %d" % rc)
    return out, norm


@dataclass(frozen=True)
class DsShape:
    """Single-scale deformable sampling size: x [B,H,W,G*D] NHWC, a kh x kw
    kernel grid, padding (ph, pw)."""
    B: int
    G: int
    D: int
    H: int
    W: int
    kh: int
    kw: int
    ph: int
    pw: int

    @property
    def C(self) -> int:
        return self.G * self.D

    @property
    def K(self) -> int:
        return self.kh * self.kw

    @property
    def Ho(self) -> int:
        return self.H + 2 * self.ph - self.kh + 1

    @property
    def Wo(self) -> int:
        return self.W + 2 * self.pw - self.kw + 1


def dsample(shape: DsShape, x, offset, weights, softmax: bool, nthreads: int = 0):
    """Oracle single-scale deformable sampling (see dcn_oracle.h).

    x [B,H,W,G*D], offset [B,G*2K,Ho,Wo] (channel (g*K+k)*2 = dy, +1 = dx),
    weights [B,G*K,Ho,Wo] (logits when ``softmax``).  Returns ``(out, norm)``,
    float64 [B, Ho, Wo, G*D] (NHWC).
    """
    s = shape
    x, offset, weights = (_f32(a) for a in (x, offset, weights))
    assert x.shape == (s.B, s.H, s.W, s.C), x.shape
    assert offset.shape == (s.B, s.G * 2 * s.K, s.Ho, s.Wo), offset.shape
    assert weights.shape == (s.B, s.G * s.K, s.Ho, s.Wo), weights.shape
    out = np.empty((s.B, s.Ho, s.Wo, s.C), dtype=np.float64)
    norm = np.empty((s.B, s.Ho, s.Wo, s.C), dtype=np.float64)
    cs = _DsShape(s.B, s.G, s.D, s.H, s.W, s.kh, s.kw, s.ph, s.pw)
    rc = _load().dcn_oracle_dsample(ctypes.byref(cs), _ptr(x), _ptr(offset), _ptr(weights),
                                    int(bool(softmax)), _ptr(out), _ptr(norm),
                                    _threads(nthreads))
    if rc != 0:
        raise ValueError("dcn_oracle_dsample failed with code %d" % rc)
    return out, norm
