"""Pins of the oracle's backward against facts that do not come from its code.

The forward oracle is itself pinned (test_oracle_pins.py); the backward is
the derivative of that forward, so it is pinned by identities that hold for
any correct derivative:

* adjoint identities -- the forward is linear in x, in the weight and in the
  mask (bias off), so <g, F(dx)> = <grad_x, dx>, <g, F(dW)> = <grad_W, dW>,
  <g, F(dm)> = <grad_mask, dm> for any directions (exact up to fp64 rounding);
* the bias gradient is the sum of g over pixels (closed form);
* exact central differences for the offsets: inside one floor cell the
  sample is bilinear in (row, column), and a bilinear function's central
  difference along any direction equals its directional derivative exactly.
  Offsets are dyadic with fractions in [1/4, 3/4] and the step is 2^-10, so
  every sampling point stays in its cell and the fp32 coordinates are exact;
* zero offsets with mask 1: grad_x is the textbook adjoint of a
  cross-correlation (a brute-force numpy loop).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle

SHAPES = [
    oracle.Shape(1, 4, 6, 5, 3, 3, 3, 1, 1),
    oracle.Shape(2, 8, 7, 9, 5, 3, 2, 1, 0),
    oracle.Shape(1, 3, 5, 6, 2, 1, 1, 0, 0),
    oracle.Shape(1, 4, 9, 8, 3, 5, 5, 2, 2),
]


def _inputs(s: oracle.Shape, seed: int, dyadic: bool = False):
    rng = np.random.default_rng(seed)
    f32 = lambda a: np.asarray(a, dtype=np.float32)  # noqa: E731
    x = f32(rng.standard_normal((s.B, s.H, s.W, s.C)))
    if dyadic:
        # integer part in [-3, 3], fraction a multiple of 2^-8 in [1/4, 3/4]
        ip = rng.integers(-3, 4, size=(s.B, 2 * s.K, s.Ho, s.Wo))
        fr = rng.integers(64, 193, size=ip.shape) / 256.0
        off = f32(ip + fr)
    else:
        off = f32(rng.standard_normal((s.B, 2 * s.K, s.Ho, s.Wo)) * 1.7)
    m = f32(rng.random((s.B, s.K, s.Ho, s.Wo)) * 1.5)
    w = f32(rng.standard_normal((s.O, s.C, s.kh, s.kw)) * 0.3)
    g = f32(rng.standard_normal((s.B, s.O, s.Ho, s.Wo)))
    return x, off, m, w, g


def _fwd(s, x, off, m, w):
    out, _ = oracle.forward_nchw(s, x, off, m, w, None, nthreads=2)
    return out


def _close(a: float, b: float, scale: float, rel: float = 1e-11):
    assert abs(a - b) <= rel * scale + 1e-300, (a, b, scale)


@pytest.mark.parametrize("si", range(len(SHAPES)))
def test_adjoint_identities(si):
    s = SHAPES[si]
    x, off, m, w, g = _inputs(s, 10 + si)
    grads, norms = oracle.backward(s, x, off, m, w, g, nthreads=3)
    rng = np.random.default_rng(99 + si)
    f32 = lambda a: np.asarray(a, dtype=np.float32)  # noqa: E731
    g64 = g.astype(np.float64)
    # x
    dx = f32(rng.standard_normal(x.shape))
    lhs = float((g64 * _fwd(s, dx, off, m, w)).sum())
    rhs = float((grads["x"] * dx).sum())
    _close(lhs, rhs, float((norms["x"] * np.abs(dx)).sum()))
    # weight
    dw = f32(rng.standard_normal(w.shape))
    lhs = float((g64 * _fwd(s, x, off, m, dw)).sum())
    rhs = float((grads["weight"] * dw).sum())
    _close(lhs, rhs, float((norms["weight"] * np.abs(dw)).sum()))
    # mask
    dm = f32(rng.standard_normal(m.shape))
    lhs = float((g64 * _fwd(s, x, off, dm, w)).sum())
    rhs = float((grads["mask"] * dm).sum())
    _close(lhs, rhs, float((norms["mask"] * np.abs(dm)).sum()))
    # bias: closed form
    assert np.allclose(grads["bias"], g64.sum(axis=(0, 2, 3)), rtol=0, atol=1e-12)
    # normalisers bound the gradients
    for k in grads:
        assert (np.abs(grads[k]) <= norms[k] * (1 + 1e-12) + 1e-300).all(), k


@pytest.mark.parametrize("si", range(len(SHAPES)))
def test_offset_gradient_is_the_exact_central_difference(si):
    s = SHAPES[si]
    x, off, m, w, g = _inputs(s, 20 + si, dyadic=True)
    grads, _ = oracle.backward(s, x, off, m, w, g, nthreads=2)
    rng = np.random.default_rng(7 + si)
    eps = 2.0 ** -10
    delta = (rng.integers(0, 2, size=off.shape) * 2 - 1) * eps
    fp = _fwd(s, x, (off + delta).astype(np.float32), m, w)
    fm = _fwd(s, x, (off - delta).astype(np.float32), m, w)
    lhs = float((g.astype(np.float64) * (fp - fm)).sum()) / 2.0
    rhs = float((grads["offset"] * delta).sum())
    _close(lhs, rhs, float((np.abs(g) * (np.abs(fp) + np.abs(fm))).sum()), rel=1e-12)
    # one coordinate at a time, on a few elements: dy and dx are not swapped
    for idx in [(0, 0, 0, 0), (0, 1, s.Ho - 1, s.Wo - 1), (0, 2 * s.K - 1, s.Ho // 2, 0)]:
        e = np.zeros(off.shape)
        e[idx] = eps
        d = _fwd(s, x, (off + e).astype(np.float32), m, w) - _fwd(s, x, (off - e).astype(np.float32), m, w)
        num = float((g.astype(np.float64) * d).sum()) / (2 * eps)
        assert abs(num - grads["offset"][idx]) <= 1e-9 * (1 + abs(num)), (idx, num,
                                                                           grads["offset"][idx])


def test_zero_offsets_give_the_correlation_adjoint():
    s = oracle.Shape(1, 3, 6, 7, 4, 3, 3, 1, 1)
    x, off, m, w, g = _inputs(s, 5)
    off[:] = 0
    m[:] = 1
    grads, _ = oracle.backward(s, x, off, m, w, g, nthreads=1)
    # brute force: x[y, x'] feeds out[ho, wo] through tap (i, j) when
    # y = ho - ph + i and x' = wo - pw + j
    want = np.zeros((s.B, s.H, s.W, s.C))
    for ho in range(s.Ho):
        for wo in range(s.Wo):
            for i in range(s.kh):
                for j in range(s.kw):
                    y, xx = ho - s.ph + i, wo - s.pw + j
                    if 0 <= y < s.H and 0 <= xx < s.W:
                        want[0, y, xx] += np.einsum("o,oc->c", g[0, :, ho, wo].astype(np.float64),
                                                    w[:, :, i, j].astype(np.float64))
    assert np.allclose(grads["x"], want, rtol=1e-12, atol=1e-12)


def test_null_mask_is_mask_one_and_thread_count_is_deterministic():
    s = SHAPES[1]
    x, off, m, w, g = _inputs(s, 3)
    ones = np.ones_like(m)
    a, _ = oracle.backward(s, x, off, None, w, g, nthreads=2)
    b, _ = oracle.backward(s, x, off, ones, w, g, nthreads=2)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    c, _ = oracle.backward(s, x, off, ones, w, g, nthreads=2)
    for k in a:
        assert np.array_equal(b[k], c[k]), k


# ---------------------------------------------------------------- normalisers
# Each gradient element is a sum of products; its normaliser N is the sum of
# the absolute values of those products.  Because every bilinear weight is
# >= 0, the absolute-term sums are themselves bilinear samples of |x| (with
# per-corner zero fill), which scipy's sampler computes independently of the
# oracle's code.  The pins below are two-sided: a dropped factor (an inflated
# N) fails them as surely as a missing term.  scipy takes the fraction of the
# fp32 point in fp64, the oracle in fp32 (it rounds for negative points), so
# the two agree to 2.5e-7 relative (two fp32 fraction roundings per weight).

def _fp32_points(s, off):
    """fp32 sampling points [B, K, Ho, Wo]: exact integer grid + one fp32 add."""
    o = off.reshape(s.B, s.K, 2, s.Ho, s.Wo)
    i = (np.arange(s.K) // s.kw).reshape(1, s.K, 1, 1)
    j = (np.arange(s.K) % s.kw).reshape(1, s.K, 1, 1)
    gy = (np.arange(s.Ho).reshape(1, 1, s.Ho, 1) - s.ph + i).astype(np.float32)
    gx = (np.arange(s.Wo).reshape(1, 1, 1, s.Wo) - s.pw + j).astype(np.float32)
    return (gy + o[:, :, 0]).astype(np.float32), (gx + o[:, :, 1]).astype(np.float32)


def _sample_abs(x, b, c, yy, xx):
    """Bilinear sample of |x[b, :, :, c]| at (yy, xx), zero outside (per corner)."""
    from scipy import ndimage
    img = np.abs(x[b, :, :, c].astype(np.float64))
    return ndimage.map_coordinates(img, [yy.astype(np.float64).ravel(),
                                         xx.astype(np.float64).ravel()],
                                   order=1, mode="grid-constant", cval=0.0).reshape(yy.shape)


def _normalisers(s, x, off, m, w, g):
    """The five absolute-term sums, from scipy samples of |x| (and, for grad_x,
    an explicit scatter of the fp32 bilinear weights)."""
    py, px = _fp32_points(s, off)
    y0, x0 = np.floor(py), np.floor(px)
    am = np.ones((s.B, s.K, s.Ho, s.Wo)) if m is None else np.abs(m.astype(np.float64))
    ag = np.abs(g.astype(np.float64)).reshape(s.B, s.O, s.Ho, s.Wo)
    aw = np.abs(w.astype(np.float64)).reshape(s.O, s.C, s.K)
    # gsa[b, k, ho, wo, c] = sum_o |g| |W[o, c, k]|
    gsa = np.einsum("bohw,ock->bkhwc", ag, aw)
    samp = np.zeros((s.B, s.K, s.Ho, s.Wo, s.C))      # sample of |x| at the point
    rows = np.zeros_like(samp)                         # rows y0, y0+1 at column px
    cols = np.zeros_like(samp)                         # columns x0, x0+1 at row py
    for b in range(s.B):
        for c in range(s.C):
            samp[b, ..., c] = _sample_abs(x, b, c, py[b], px[b])
            rows[b, ..., c] = (_sample_abs(x, b, c, y0[b], px[b]) +
                               _sample_abs(x, b, c, y0[b] + 1, px[b]))
            cols[b, ..., c] = (_sample_abs(x, b, c, py[b], x0[b]) +
                               _sample_abs(x, b, c, py[b], x0[b] + 1))
    n = {}
    n["mask"] = (gsa * samp).sum(axis=-1)
    noff = np.zeros((s.B, s.K, 2, s.Ho, s.Wo))
    noff[:, :, 0] = am * (gsa * rows).sum(axis=-1)
    noff[:, :, 1] = am * (gsa * cols).sum(axis=-1)
    n["offset"] = noff.reshape(s.B, 2 * s.K, s.Ho, s.Wo)
    nw = np.einsum("bohw,bkhw,bkhwc->ock", ag, am, samp)
    n["weight"] = nw.reshape(s.O, s.C, s.kh, s.kw)
    n["bias"] = ag.sum(axis=(0, 2, 3))
    # grad_x: scatter gsa * |m| * w_q to each inside corner
    ly = (py - y0.astype(np.float32)).astype(np.float64)
    lx = (px - x0.astype(np.float32)).astype(np.float64)
    nx = np.zeros((s.B, s.H, s.W, s.C))
    for a in (0, 1):
        for bb in (0, 1):
            wq = (ly if a else 1 - ly) * (lx if bb else 1 - lx)
            yy, xx = y0 + a, x0 + bb
            ok = (yy >= 0) & (yy <= s.H - 1) & (xx >= 0) & (xx <= s.W - 1)
            bi, ki, hi, wi = np.nonzero(ok)
            vals = (gsa * (am * wq)[..., None])[bi, ki, hi, wi]
            np.add.at(nx, (bi, yy[bi, ki, hi, wi].astype(np.int64),
                           xx[bi, ki, hi, wi].astype(np.int64)), vals)
    n["x"] = nx
    return n


@pytest.mark.parametrize("use_mask", [True, False])
@pytest.mark.parametrize("si", range(len(SHAPES)))
def test_normalisers_two_sided(si, use_mask):
    s = SHAPES[si]
    x, off, m, w, g = _inputs(s, 40 + si)
    m = m if use_mask else None
    _, norms = oracle.backward(s, x, off, m, w, g, nthreads=2)
    want = _normalisers(s, x, off, m, w, g)
    for k in ("x", "offset", "mask", "weight", "bias"):
        err = np.abs(norms[k] - want[k])
        assert (err <= 2.5e-7 * want[k] + 1e-300).all(), (k, float((err / want[k]).max()))
    # sensitivity: the same sums without |mask| (a plausible slip in the
    # input, offset and weight normalisers) lie far outside that bound
    if use_mask:
        loose = _normalisers(s, x, off, None, w, g)
        for k in ("x", "offset", "weight"):
            assert (np.abs(norms[k] - loose[k]) > 2.5e-7 * loose[k]).any(), k
