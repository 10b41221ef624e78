"""Seeded synthetic inputs for the deformable-convolution workloads.

This module only draws random numbers (numpy PCG64 via ``default_rng``, in
float64, then rounded to float32 and, for the bf16 workload, to bfloat16 with
round-to-nearest-even).  It holds none of the operator's arithmetic, so both
the GPU path and the CPU oracle can be fed from it.

Workloads (shapes and value distributions):

* ``tiny_fp32``          B=1, C=O=4, 8x8, 3x3 pad 1.
* ``birefnet512_fp32``   B=1, C=O=64, 128x128, 7x7 pad 3 -- the deformable 3x3..7x7
  ASPP branches of BiRefNet's decoder at 512 input (page 2, "patch_deform.py":
  [1,1,64,49,256,256] gathers at 1024 input, i.e. 64 channels, 49 taps, a
  256^2 map; 128^2 at 512).
* ``birefnet1024_fp32``  the same at 1024 input: 256x256 (the headline shape).
* ``detection_bf16``     B=8, C=O=256, 64x64, 3x3 pad 1, all operands bf16.
* ``edge_stress_fp32``   B=2, C=O=128, 200x176, 5x5 pad 2, offsets a per-location
  mix of exact integers, far out-of-image values and N(0,1).
* ``p1_k1/p1_k3/p1_k7``  page 1's own self-test shapes ("deform_conv.py",
  ``__main__``): x[1,64,33,40], O=256, (ks, pad) in {(1,0),(3,1),(7,3)},
  offsets N(0,4^2), mask U(0,2), weight N(0,1)*0.05, no bias.

Distribution notation ``N(0, s)`` in the workload list is read as a standard
deviation ``s`` (``N(0, 1.5^2)`` -> std 1.5).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Spec:
    name: str
    B: int
    C: int
    O: int
    H: int
    W: int
    kh: int
    kw: int
    ph: int
    pw: int
    dtype: str            # "f32" or "bf16": storage type of every operand
    seed: int
    offset_dist: str      # "uniform2", "normal1.5", "normal2", "normal4", "edge_mix", "zero"
    mask_dist: str        # "uniform", "sigmoid_normal", "uniform2", "ones", "none"
    weight_std: float
    bias_dist: str        # "normal0.1", "normal1", "zero", "none"

    @property
    def K(self) -> int:
        return self.kh * self.kw

    @property
    def Ho(self) -> int:
        return self.H + 2 * self.ph - self.kh + 1

    @property
    def Wo(self) -> int:
        return self.W + 2 * self.pw - self.kw + 1

    @property
    def pixels(self) -> int:
        return self.B * self.Ho * self.Wo

    @property
    def gemm_flops(self) -> int:
        """2 * P * O * K * C: the dense contraction's flop count."""
        return 2 * self.pixels * self.O * self.K * self.C

    def scaled(self, **kw) -> "Spec":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_fp32": Spec("tiny_fp32", 1, 4, 4, 8, 8, 3, 3, 1, 1, "f32", 1,
                      "uniform2", "uniform", 0.1, "normal0.1"),
    "birefnet512_fp32": Spec("birefnet512_fp32", 1, 64, 64, 128, 128, 7, 7, 3, 3, "f32", 2,
                             "normal1.5", "sigmoid_normal", 1.0 / np.sqrt(49 * 64), "normal0.1"),
    "birefnet1024_fp32": Spec("birefnet1024_fp32", 1, 64, 64, 256, 256, 7, 7, 3, 3, "f32", 3,
                              "normal1.5", "sigmoid_normal", 1.0 / np.sqrt(49 * 64), "normal0.1"),
    "detection_bf16": Spec("detection_bf16", 8, 256, 256, 64, 64, 3, 3, 1, 1, "bf16", 4,
                           "normal2", "sigmoid_normal", 1.0 / np.sqrt(9 * 256), "zero"),
    "edge_stress_fp32": Spec("edge_stress_fp32", 2, 128, 128, 200, 176, 5, 5, 2, 2, "f32", 5,
                             "edge_mix", "uniform", 1.0 / np.sqrt(25 * 128), "normal1"),
    "p1_k1": Spec("p1_k1", 1, 64, 256, 33, 40, 1, 1, 0, 0, "f32", 0,
                  "normal4", "uniform2", 0.05, "none"),
    "p1_k3": Spec("p1_k3", 1, 64, 256, 33, 40, 3, 3, 1, 1, "f32", 0,
                  "normal4", "uniform2", 0.05, "none"),
    "p1_k7": Spec("p1_k7", 1, 64, 256, 33, 40, 7, 7, 3, 3, "f32", 0,
                  "normal4", "uniform2", 0.05, "none"),
}


def round_bf16(a: np.ndarray):
    """Round float32 -> bfloat16 (nearest-even).  Returns (values as float32, uint16 bits)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    return back, bits


def _offsets(rng, spec: Spec, shape):
    d = spec.offset_dist
    if d == "zero":
        return np.zeros(shape)
    if d == "uniform2":
        return rng.uniform(-2.0, 2.0, size=shape)
    if d.startswith("normal"):
        return rng.standard_normal(shape) * float(d[len("normal"):])
    if d == "edge_mix":
        # Per (b, tap, ho, wo) location one class, shared by dy and dx:
        # exact integers in [-3, 3], U(-H/2, H/2) (mostly far outside), N(0, 1).
        B, K2, Ho, Wo = shape
        K = K2 // 2
        cls = rng.integers(0, 3, size=(B, K, 1, Ho, Wo))
        ints = rng.integers(-3, 4, size=(B, K, 2, Ho, Wo)).astype(np.float64)
        wide = rng.uniform(-spec.H / 2.0, spec.H / 2.0, size=(B, K, 2, Ho, Wo))
        norm = rng.standard_normal((B, K, 2, Ho, Wo))
        out = np.where(cls == 0, ints, np.where(cls == 1, wide, norm))
        return out.reshape(shape)
    raise ValueError(d)


def _mask(rng, spec: Spec, shape):
    d = spec.mask_dist
    if d == "none":
        return None
    if d == "ones":
        return np.ones(shape)
    if d == "uniform":
        return rng.uniform(0.0, 1.0, size=shape)
    if d == "uniform2":
        return rng.uniform(0.0, 2.0, size=shape)
    if d == "sigmoid_normal":
        return 1.0 / (1.0 + np.exp(-rng.standard_normal(shape)))
    raise ValueError(d)


def _bias(rng, spec: Spec):
    d = spec.bias_dist
    if d == "none":
        return None
    if d == "zero":
        return np.zeros(spec.O)
    if d.startswith("normal"):
        return rng.standard_normal(spec.O) * float(d[len("normal"):])
    raise ValueError(d)


def make_inputs(spec: Spec):
    """Draw one workload's operands.

    Returns a dict with float32 numpy arrays ``x`` [B,H,W,C] (NHWC), ``offset``
    [B,2K,Ho,Wo], ``mask`` [B,K,Ho,Wo] or None, ``weight`` [O,C,kh,kw], ``bias``
    [O] or None.  For ``dtype == "bf16"`` every array already holds bf16-
    representable values and ``bits`` maps each name to its uint16 patterns.
    """
    rng = np.random.default_rng(spec.seed)
    K = spec.K
    x = rng.standard_normal((spec.B, spec.H, spec.W, spec.C))
    offset = _offsets(rng, spec, (spec.B, 2 * K, spec.Ho, spec.Wo))
    mask = _mask(rng, spec, (spec.B, K, spec.Ho, spec.Wo))
    weight = rng.standard_normal((spec.O, spec.C, spec.kh, spec.kw)) * spec.weight_std
    bias = _bias(rng, spec)
    arrs = {"x": x, "offset": offset, "mask": mask, "weight": weight, "bias": bias}
    out = {k: (None if v is None else np.ascontiguousarray(v, dtype=np.float32))
           for k, v in arrs.items()}
    if spec.dtype == "bf16":
        bits = {}
        for k, v in list(out.items()):
            if v is None:
                continue
            out[k], bits[k] = round_bf16(v)
        out["bits"] = bits
    return out


@dataclass(frozen=True)
class MsdaSpec:
    """A multi-scale deformable attention sampling workload (page 5)."""
    name: str
    B: int
    Q: int
    G: int
    D: int
    shapes: tuple
    K: int
    softmax: bool
    seed: int
    loc_lo: float = -0.05   # locations ~ U(loc_lo, loc_hi): a few points fall outside
    loc_hi: float = 1.05
    dtype: str = "f32"      # "f32" or "bf16": value, locations and weights

    @property
    def L(self) -> int:
        return len(self.shapes)

    @property
    def S(self) -> int:
        return sum(h * w for h, w in self.shapes)

    def scaled(self, **kw) -> "MsdaSpec":
        return replace(self, **kw)


# Deformable-DETR-like encoder: every position of a 4-level pyramid
# (64^2, 32^2, 16^2, 8^2 -- page 5's example shapes) queries 4 points per
# level in each of 8 heads of 32 channels; softmax over the 16 logits.
MSDA_WORKLOADS = {
    "msda_encoder_fp32": MsdaSpec("msda_encoder_fp32", 4, 5440, 8, 32,
                                  ((64, 64), (32, 32), (16, 16), (8, 8)), 4, True, 21),
    "msda_decoder_fp32": MsdaSpec("msda_decoder_fp32", 8, 300, 8, 32,
                                  ((64, 64), (32, 32), (16, 16), (8, 8)), 4, True, 22),
    # page 5 recommends bfloat16 for training: the encoder workload in bf16
    "msda_encoder_bf16": MsdaSpec("msda_encoder_bf16", 4, 5440, 8, 32,
                                  ((64, 64), (32, 32), (16, 16), (8, 8)), 4, True, 23,
                                  dtype="bf16"),
}


def make_msda_inputs(spec: MsdaSpec) -> dict:
    """value ~ N(0,1) [B,S,G,D]; locations ~ U(loc_lo, loc_hi) [B,Q,G,L,K,2];
    weights (logits) ~ N(0,1) [B,Q,G,L*K]; drawn in that order, float32 (bf16-
    rounded with ``bits`` when spec.dtype is "bf16")."""
    rng = np.random.default_rng(spec.seed)
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)  # noqa: E731
    value = f32(rng.standard_normal((spec.B, spec.S, spec.G, spec.D)))
    loc = f32(rng.uniform(spec.loc_lo, spec.loc_hi,
                          size=(spec.B, spec.Q, spec.G, spec.L, spec.K, 2)))
    w = f32(rng.standard_normal((spec.B, spec.Q, spec.G, spec.L * spec.K)))
    out = {"value": value, "locations": loc, "weights": w}
    if spec.dtype == "bf16":
        bits = {}
        for k in list(out):
            out[k], bits[k] = round_bf16(out[k])
        out["bits"] = bits
    return out


@dataclass(frozen=True)
class DsSpec:
    """A single-scale deformable sampling workload (page 5, DCNv3 form):
    x [B,H,W,G*D] NHWC, offset [B,G*2K,Ho,Wo], aggregation weights [B,G*K,Ho,Wo]."""
    name: str
    B: int
    G: int
    D: int
    H: int
    W: int
    kh: int
    kw: int
    ph: int
    pw: int
    dtype: str          # "f32" or "bf16"
    softmax: bool       # weights are logits normalised over the K taps in the kernel
    seed: int
    offset_std: float = 1.5

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

    @property
    def pixels(self) -> int:
        return self.B * self.Ho * self.Wo

    def scaled(self, **kw) -> "DsSpec":
        return replace(self, **kw)


# page 5's example layer: DeformSample2d(dim=64, kernel_size=3, groups=4) on a
# 32 x 32 map; the same layer on the 256 x 256 decoder map of the BiRefNet
# workloads (page 2) for throughput, in fp32 and bf16
DS_WORKLOADS = {
    "dcnv3_page5_fp32": DsSpec("dcnv3_page5_fp32", 1, 4, 16, 32, 32, 3, 3, 1, 1, "f32", True, 31),
    "dcnv3_map256_fp32": DsSpec("dcnv3_map256_fp32", 1, 4, 16, 256, 256, 3, 3, 1, 1, "f32", True,
                                32),
    "dcnv3_map256_bf16": DsSpec("dcnv3_map256_bf16", 1, 4, 16, 256, 256, 3, 3, 1, 1, "bf16", True,
                                33),
}


def make_ds_inputs(spec: DsSpec) -> dict:
    """x ~ N(0,1) [B,H,W,G*D]; offsets ~ N(0, offset_std^2) [B,G*2K,Ho,Wo];
    weights (logits when spec.softmax, else U(0,1)) [B,G*K,Ho,Wo]; drawn in that
    order in fp64, rounded to fp32 (and to bf16 with ``bits`` for bf16)."""
    rng = np.random.default_rng(spec.seed)
    K = spec.K
    x = rng.standard_normal((spec.B, spec.H, spec.W, spec.C))
    off = rng.standard_normal((spec.B, spec.G * 2 * K, spec.Ho, spec.Wo)) * spec.offset_std
    shape = (spec.B, spec.G * K, spec.Ho, spec.Wo)
    w = rng.standard_normal(shape) if spec.softmax else rng.uniform(0.0, 1.0, size=shape)
    out = {k: np.ascontiguousarray(v, dtype=np.float32)
           for k, v in (("x", x), ("offset", off), ("weights", w))}
    if spec.dtype == "bf16":
        bits = {}
        for k in list(out):
            out[k], bits[k] = round_bf16(out[k])
        out["bits"] = bits
    return out
