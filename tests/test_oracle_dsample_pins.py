"""Pins of the oracle's single-scale deformable sampling (DCNv3 form).

Page 5 ("Single-scale deformable sampling") defines the operator as the
deformable convolution's sampling and aggregation without its spatial
weight.  Each pin comes from outside dcn_oracle_dsample's code:

* per channel group it equals the (separately pinned) deformable-convolution
  oracle on that group's channels with an identity weight (O = D,
  weight[o, c, i, j] = 1 if o == c) and the aggregation weights as the mask;
* scipy's bilinear sampler (map_coordinates, order 1, zero outside) on the
  same fp32 points, weighted and summed in numpy -- the values and, on |x|
  with |a|, the normaliser, both two-sided;
* a numpy softmax for the softmax-normalised weights, and partition of unity
  (a constant image is returned unchanged);
* exact cases: a 1x1 kernel with zero offsets and weight 1 is the identity;
  integer offsets are a brute-force gather.
"""
from __future__ import annotations

import numpy as np
import pytest
from scipy import ndimage

import oracle

SHAPES = [
    oracle.DsShape(1, 4, 16, 9, 8, 3, 3, 1, 1),    # page 5's DeformSample2d: 64 ch, 4 groups, 3x3
    oracle.DsShape(2, 3, 4, 7, 10, 3, 2, 1, 0),
    oracle.DsShape(1, 1, 8, 6, 6, 5, 5, 2, 2),
    oracle.DsShape(1, 2, 12, 5, 7, 1, 1, 0, 0),
]


def _inputs(s, seed, scale=1.7, softmax=False):
    rng = np.random.default_rng(seed)
    f32 = lambda a: np.asarray(a, dtype=np.float32)  # noqa: E731
    x = f32(rng.standard_normal((s.B, s.H, s.W, s.C)))
    off = f32(rng.standard_normal((s.B, s.G * 2 * s.K, s.Ho, s.Wo)) * scale)
    a = f32(rng.standard_normal((s.B, s.G * s.K, s.Ho, s.Wo)) if softmax else
            rng.uniform(-0.5, 1.5, size=(s.B, s.G * s.K, s.Ho, s.Wo)))
    return x, off, a


def _points(s, off):
    """fp32 points [B, G, K, Ho, Wo]: exact integer grid + one fp32 add."""
    o = off.reshape(s.B, s.G, s.K, 2, s.Ho, s.Wo)
    i = (np.arange(s.K) // s.kw).reshape(1, 1, s.K, 1, 1)
    j = (np.arange(s.K) % s.kw).reshape(1, 1, s.K, 1, 1)
    gy = (np.arange(s.Ho).reshape(1, 1, 1, s.Ho, 1) - s.ph + i).astype(np.float32)
    gx = (np.arange(s.Wo).reshape(1, 1, 1, 1, s.Wo) - s.pw + j).astype(np.float32)
    return (gy + o[:, :, :, 0]).astype(np.float32), (gx + o[:, :, :, 1]).astype(np.float32)


def _scipy(s, x, off, a):
    """sum_k a * bilinear sample, per channel, with scipy's sampler: [B,Ho,Wo,C]."""
    py, px = _points(s, off)
    aa = a.reshape(s.B, s.G, s.K, s.Ho, s.Wo).astype(np.float64)
    out = np.zeros((s.B, s.Ho, s.Wo, s.C))
    for b in range(s.B):
        for g in range(s.G):
            for c in range(s.D):
                img = x[b, :, :, g * s.D + c].astype(np.float64)
                smp = ndimage.map_coordinates(
                    img, [py[b, g].astype(np.float64).ravel(), px[b, g].astype(np.float64).ravel()],
                    order=1, mode="grid-constant", cval=0.0).reshape(s.K, s.Ho, s.Wo)
                out[b, :, :, g * s.D + c] = (aa[b, g] * smp).sum(axis=0)
    return out


def _softmax(s, logits):
    z = logits.reshape(s.B, s.G, s.K, s.Ho, s.Wo).astype(np.float64)
    e = np.exp(z - z.max(axis=2, keepdims=True))
    return (e / e.sum(axis=2, keepdims=True)).reshape(logits.shape)


@pytest.mark.parametrize("si", range(len(SHAPES)))
def test_each_group_is_the_convolution_with_an_identity_weight(si):
    s = SHAPES[si]
    x, off, a = _inputs(s, 10 + si)
    got, norm = oracle.dsample(s, x, off, a, softmax=False, nthreads=2)
    eye = np.zeros((s.D, s.D, s.kh, s.kw), np.float32)
    for c in range(s.D):
        eye[c, c] = 1.0
    cs = oracle.Shape(s.B, s.D, s.H, s.W, s.D, s.kh, s.kw, s.ph, s.pw)
    for g in range(s.G):
        xg = np.ascontiguousarray(x[..., g * s.D:(g + 1) * s.D])
        og = np.ascontiguousarray(off[:, g * 2 * s.K:(g + 1) * 2 * s.K])
        ag = np.ascontiguousarray(a[:, g * s.K:(g + 1) * s.K])
        ref, rn = oracle.forward(cs, xg, og, ag, eye, None, nthreads=2)
        want = ref.reshape(s.B, s.Ho, s.Wo, s.D)
        part = got[..., g * s.D:(g + 1) * s.D]
        assert np.allclose(part, want, rtol=0, atol=1e-13 * (1 + np.abs(want).max())), g
        # the convolution's normaliser takes |sample| as one term; this one
        # expands the corners (sum w |x|), so it bounds it from above
        assert (norm[..., g * s.D:(g + 1) * s.D] >= rn.reshape(want.shape) * (1 - 1e-13)).all()


@pytest.mark.parametrize("softmax", [False, True])
@pytest.mark.parametrize("si", range(len(SHAPES)))
def test_matches_scipy_bilinear_sampler(si, softmax):
    """scipy takes the fraction of the fp32 point in fp64, the oracle in fp32
    (it rounds for negative points): 2.5e-7 of the absolute-term sum."""
    s = SHAPES[si]
    x, off, a = _inputs(s, 30 + si, softmax=softmax)
    got, norm = oracle.dsample(s, x, off, a, softmax=softmax, nthreads=2)
    aw = _softmax(s, a) if softmax else a.astype(np.float64)
    want = _scipy(s, x, off, aw)
    assert (np.abs(got - want) <= 2.5e-7 * norm + 1e-300).all()
    # normaliser, two-sided: scipy on |x| with |a|
    want_n = _scipy(s, np.abs(x), off, np.abs(aw))
    assert (np.abs(norm - want_n) <= 2.5e-7 * want_n + 1e-300).all()
    # without |a| it would not match (a dropped factor fails)
    if not softmax:
        plain = _scipy(s, np.abs(x), off, np.abs(aw) * 0 + 1)
        assert (np.abs(norm - plain) > 2.5e-7 * plain).any()


def test_softmax_weights_keep_a_constant_image():
    """Softmax weights sum to 1 over the taps; with every point at least one
    pixel inside, a constant image comes back unchanged."""
    s = oracle.DsShape(1, 2, 4, 12, 12, 3, 3, 1, 1)
    x = np.full((1, 12, 12, 8), 0.75, np.float32)
    rng = np.random.default_rng(4)
    # base grid in [-1, 12] for 3x3 pad 1; keep points in [1, 10]
    py, px = _points(s, np.zeros((1, 2 * 2 * 9, 12, 12), np.float32))
    off = np.zeros((1, 2, 9, 2, 12, 12), np.float32)
    off[:, :, :, 0] = np.clip(rng.uniform(-2, 2, size=py.shape), 1 - py, 10 - py)
    off[:, :, :, 1] = np.clip(rng.uniform(-2, 2, size=px.shape), 1 - px, 10 - px)
    off = off.reshape(1, 36, 12, 12).astype(np.float32)
    logits = rng.standard_normal((1, 18, 12, 12)).astype(np.float32)
    got, _ = oracle.dsample(s, x, off, logits, softmax=True, nthreads=2)
    assert np.allclose(got, 0.75, rtol=0, atol=1e-14)


def test_one_by_one_zero_offsets_unit_weight_is_identity():
    s = oracle.DsShape(2, 3, 4, 5, 6, 1, 1, 0, 0)
    x, _, _ = _inputs(s, 7)
    off = np.zeros((s.B, s.G * 2, 5, 6), np.float32)
    a = np.ones((s.B, s.G, 5, 6), np.float32)
    got, norm = oracle.dsample(s, x, off, a, softmax=False, nthreads=1)
    assert np.array_equal(got, x.astype(np.float64))
    assert np.array_equal(norm, np.abs(x).astype(np.float64))


def test_integer_offsets_are_an_exact_gather():
    s = oracle.DsShape(1, 2, 3, 6, 7, 3, 3, 1, 1)
    x, _, a = _inputs(s, 8)
    rng = np.random.default_rng(9)
    off = rng.integers(-3, 4, size=(1, s.G * 2 * s.K, s.Ho, s.Wo)).astype(np.float32)
    got, _ = oracle.dsample(s, x, off, a, softmax=False, nthreads=1)
    want = np.zeros_like(got)
    o = off.reshape(1, s.G, s.K, 2, s.Ho, s.Wo)
    aa = a.reshape(1, s.G, s.K, s.Ho, s.Wo).astype(np.float64)
    for g in range(s.G):
        for k in range(s.K):
            i, j = divmod(k, s.kw)
            for ho in range(s.Ho):
                for wo in range(s.Wo):
                    y = ho - s.ph + i + int(o[0, g, k, 0, ho, wo])
                    xx = wo - s.pw + j + int(o[0, g, k, 1, ho, wo])
                    if 0 <= y < s.H and 0 <= xx < s.W:
                        want[0, ho, wo, g * s.D:(g + 1) * s.D] += (
                            aa[0, g, k, ho, wo] * x[0, y, xx, g * s.D:(g + 1) * s.D])
    assert np.allclose(got, want, rtol=0, atol=1e-13)
