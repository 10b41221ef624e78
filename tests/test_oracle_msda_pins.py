"""Pins of the oracle's multi-scale deformable attention sampling.

Each check comes from outside the oracle's code: a brute-force gather where
every sampling point is an exact pixel centre, scipy's bilinear sampler
(map_coordinates, order 1, zero outside) on the same fp32 pixel
coordinates, a numpy softmax, partition of unity and linearity.
"""
from __future__ import annotations

import numpy as np
import pytest
from scipy import ndimage

import oracle

CASES = [
    dict(B=1, G=2, D=8, Q=5, shapes=[(8, 8), (4, 4)], K=3),
    dict(B=2, G=3, D=4, Q=7, shapes=[(6, 10), (3, 5), (2, 3)], K=2),
    dict(B=1, G=1, D=16, Q=9, shapes=[(16, 8)], K=4),
]


def _inputs(c, seed, lo=-0.1, hi=1.1):
    rng = np.random.default_rng(seed)
    S = sum(h * w for h, w in c["shapes"])
    L = len(c["shapes"])
    f32 = lambda a: np.asarray(a, dtype=np.float32)  # noqa: E731
    v = f32(rng.standard_normal((c["B"], S, c["G"], c["D"])))
    loc = f32(rng.uniform(lo, hi, size=(c["B"], c["Q"], c["G"], L, c["K"], 2)))
    w = f32(rng.standard_normal((c["B"], c["Q"], c["G"], L * c["K"])))
    return v, loc, w


def _pixel(loc, size):
    # the fp32 pixel coordinate: one rounded product, one rounded difference
    return (np.float32(loc) * np.float32(size)).astype(np.float32) - np.float32(0.5)


def _scipy_msda(c, v, loc, w):
    B, S, G, D = v.shape
    L, K = len(c["shapes"]), c["K"]
    out = np.zeros((B, c["Q"], G, D))
    start = 0
    for l, (H, W) in enumerate(c["shapes"]):
        lv = v[:, start:start + H * W].reshape(B, H, W, G, D).astype(np.float64)
        for b in range(B):
            for g in range(G):
                px = _pixel(loc[b, :, g, l, :, 0], W).astype(np.float64).ravel()
                py = _pixel(loc[b, :, g, l, :, 1], H).astype(np.float64).ravel()
                a = w[b, :, g, l * K:(l + 1) * K].astype(np.float64).ravel()
                for d in range(D):
                    s = ndimage.map_coordinates(lv[b, :, :, g, d], [py, px], order=1,
                                                mode="grid-constant", cval=0.0)
                    out[b, :, g, d] += (a * s).reshape(c["Q"], K).sum(axis=1)
        start += H * W
    return out


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_matches_scipy_bilinear_sampler(ci):
    """scipy takes the fraction of the (fp32) pixel coordinate in fp64; the
    oracle in fp32, which rounds for negative coordinates (their fraction
    has a larger exponent than the coordinate): at most 2^-24 relative per
    weight factor, hence 2.5e-7 of the absolute-term sum.  With every pixel
    coordinate >= 0 the two agree to fp64 rounding."""
    c = CASES[ci]
    v, loc, w = _inputs(c, 100 + ci)
    got, norm = oracle.msda(v, c["shapes"], loc, w, softmax=False, nthreads=2)
    want = _scipy_msda(c, v, loc, w)
    assert (np.abs(got - want) <= 2.5e-7 * norm + 1e-12).all()
    assert (np.abs(got) <= norm * (1 + 1e-12) + 1e-300).all()
    v, loc, w = _inputs(c, 150 + ci, lo=0.5, hi=1.05)   # pixel coordinates >= 0.5
    got, norm = oracle.msda(v, c["shapes"], loc, w, softmax=False, nthreads=2)
    want = _scipy_msda(c, v, loc, w)
    assert np.allclose(got, want, rtol=0, atol=1e-12 * (1 + norm.max()))


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_softmax_is_the_softmax_of_the_logits(ci):
    c = CASES[ci]
    v, loc, w = _inputs(c, 200 + ci)
    w64 = w.astype(np.float64)
    e = np.exp(w64 - w64.max(axis=-1, keepdims=True))
    a = (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)
    got, _ = oracle.msda(v, c["shapes"], loc, w, softmax=True)
    ref, norm = oracle.msda(v, c["shapes"], loc, a, softmax=False)
    # a was rounded to fp32 for the second call: compare to that rounding
    assert np.allclose(got, ref, rtol=0, atol=1e-6 * (1 + norm.max()))


def test_exact_pixel_centres_are_a_plain_gather():
    c = dict(B=1, G=2, D=5, Q=6, shapes=[(8, 4), (2, 16)], K=3)
    rng = np.random.default_rng(3)
    v, _, w = _inputs(c, 4)
    L = len(c["shapes"])
    loc = np.zeros((1, c["Q"], c["G"], L, c["K"], 2), dtype=np.float32)
    pick = np.zeros((1, c["Q"], c["G"], L, c["K"], 2), dtype=np.int64)
    for l, (H, W) in enumerate(c["shapes"]):
        # sizes are powers of two, so (i + 0.5) / size and the pixel
        # coordinate are exact: every point is a pixel centre
        ix = rng.integers(0, W, size=(1, c["Q"], c["G"], c["K"]))
        iy = rng.integers(0, H, size=(1, c["Q"], c["G"], c["K"]))
        loc[:, :, :, l, :, 0] = ((ix + 0.5) / W).astype(np.float32)
        loc[:, :, :, l, :, 1] = ((iy + 0.5) / H).astype(np.float32)
        pick[:, :, :, l, :, 0] = ix
        pick[:, :, :, l, :, 1] = iy
    got, _ = oracle.msda(v, c["shapes"], loc, w, softmax=False)
    want = np.zeros_like(got)
    starts = np.cumsum([0] + [h * w_ for h, w_ in c["shapes"]])
    for q in range(c["Q"]):
        for g in range(c["G"]):
            for l, (H, W) in enumerate(c["shapes"]):
                for k in range(c["K"]):
                    pix = starts[l] + pick[0, q, g, l, k, 1] * W + pick[0, q, g, l, k, 0]
                    want[0, q, g] += float(w[0, q, g, l * c["K"] + k]) * v[0, pix, g].astype(np.float64)
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_partition_of_unity_linearity_and_far_points():
    c = CASES[0]
    v, loc, w = _inputs(c, 9, lo=0.3, hi=0.7)   # every point well inside every level
    const = np.broadcast_to(np.arange(c["G"] * c["D"], dtype=np.float32).reshape(1, 1, c["G"], c["D"]),
                            v.shape).copy()
    out, _ = oracle.msda(const, c["shapes"], loc, w, softmax=True)
    assert np.allclose(out, np.broadcast_to(const[:, :1], out.shape), rtol=0, atol=1e-9)
    a, _ = oracle.msda(v, c["shapes"], loc, w, softmax=False)
    b2, _ = oracle.msda(2 * v, c["shapes"], loc, w, softmax=False)
    h, _ = oracle.msda(v, c["shapes"], loc, w * np.float32(0.5), softmax=False)
    assert np.array_equal(b2, 2 * a) and np.array_equal(h, 0.5 * a)
    far = np.full_like(loc, 3.0)
    z, n = oracle.msda(v, c["shapes"], far, w, softmax=True)
    assert not z.any() and not n.any()


@pytest.mark.parametrize("softmax", [False, True])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_normaliser_two_sided(ci, softmax):
    """N = sum over points and corners of |a| * w * |v|: with w >= 0 that is
    scipy's bilinear sample of |v| weighted by |a|; two-sided, so an N
    missing its |a| factor (or with |a| inflated) fails as a low one does."""
    c = CASES[ci]
    v, loc, w = _inputs(c, 300 + ci)
    _, norm = oracle.msda(v, c["shapes"], loc, w, softmax=softmax, nthreads=2)
    if softmax:
        L, K = len(c["shapes"]), c["K"]
        e = np.exp(w.astype(np.float64) - w.astype(np.float64).max(axis=-1, keepdims=True))
        a = (e / e.sum(axis=-1, keepdims=True))
    else:
        a = w.astype(np.float64)
    want = _scipy_msda(c, np.abs(v.astype(np.float64)), loc, np.abs(a))
    assert (np.abs(norm - want) <= 2.5e-7 * want + 1e-300).all()
    # sensitivity: without |a| the sum is far off
    plain = _scipy_msda(c, np.abs(v.astype(np.float64)), loc, np.ones_like(a))
    assert (np.abs(norm - plain) > 2.5e-7 * plain).any()
