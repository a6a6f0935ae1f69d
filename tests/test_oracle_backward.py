"""Pins of the oracle's site backward (CPU only).

The backward ("Attention Residuals 阅读补充", gradients along the tangent;
"Attention Residuals" notes, section 7, logit gradient) is pinned to the
oracle's forward, a separate code path already pinned by test_oracle_pins:
central finite differences of L = sum_t dx_t . x_t in fp64 must equal every
analytic gradient, plus special cases with closed forms.
"""
import numpy as np
import pytest

import oracle


def _rand(rng, *shape, scale=1.0):
    # values exactly representable in fp32 (the backward widens fp32 inputs)
    return (rng.standard_normal(shape) * scale).astype(np.float32).astype(np.float64)


def _loss(src, w, g, gamma, eps, dx, prenorm):
    """L = sum_t dx_t . x_t through the oracle's forward functions."""
    n, T, d = src.shape
    tot = 0.0
    for t in range(T):
        h = oracle.depth_softmax([src[i, t] for i in range(n)], w, g, eps)["h"]
        x = oracle.rmsnorm(h, gamma, eps) if prenorm else h
        tot += float(np.dot(dx[t], x))
    return tot


def _fd(f, arr, delta=1e-6):
    """Central differences of f() w.r.t. every element of arr (in place)."""
    out = np.empty_like(arr)
    flat, g = arr.reshape(-1), out.reshape(-1)
    for j in range(flat.size):
        keep = flat[j]
        flat[j] = keep + delta
        up = f()
        flat[j] = keep - delta
        dn = f()
        flat[j] = keep
        g[j] = (up - dn) / (2 * delta)
    return out


def _close(a, b, tol):
    scale = max(1.0, float(np.max(np.abs(b))))
    assert float(np.max(np.abs(a - b))) <= tol * scale, (float(np.max(np.abs(a - b))), scale)


@pytest.mark.parametrize("n,T,d,prenorm,eps", [(3, 2, 8, True, 1e-6), (1, 2, 6, True, 1e-6), (4, 1, 5, False, 1e-3),
                                               (2, 3, 4, True, 0.0)])
def test_backward_matches_finite_differences(n, T, d, prenorm, eps):
    rng = np.random.default_rng(100 + n * 10 + d)
    src = _rand(rng, n, T, d, scale=2.0)
    w = _rand(rng, d)
    g = 0.8 + 0.4 * rng.random(d).astype(np.float32).astype(np.float64)
    gamma = 0.5 + rng.random(d).astype(np.float32).astype(np.float64)
    dx = _rand(rng, T, d)
    b = oracle.site_backward(src, w, g, gamma if prenorm else None, eps, dx, prenorm=prenorm)
    f = lambda: _loss(src, w, g, gamma, eps, dx, prenorm)  # noqa: E731
    _close(b["du"], _fd(f, src), 1e-6)
    _close(b["dw"], _fd(f, w), 1e-6)
    _close(b["dg"], _fd(f, g), 1e-6)
    if prenorm:
        _close(b["dgamma"], _fd(f, gamma), 1e-6)


def test_single_source_has_no_score_gradient():
    # one source: alpha = 1 regardless of z, so w and g get no gradient and
    # the source receives the PreNorm backward of h = u unchanged
    rng = np.random.default_rng(7)
    src = _rand(rng, 1, 3, 16)
    w, dx = _rand(rng, 16), _rand(rng, 3, 16)
    b = oracle.site_backward(src, w, None, None, 1e-6, dx)
    assert np.all(b["dw"] == 0.0) and np.all(b["dg"] == 0.0)
    f = lambda: _loss(src, w, None, None, 1e-6, dx, True)  # noqa: E731
    _close(b["du"], _fd(f, src), 1e-6)


def test_identical_sources_share_the_gradient():
    # identical sources: alpha = 1/n, u_i - h = 0, so dz = 0 and every source
    # receives 1/n of the gradient of h
    rng = np.random.default_rng(8)
    row = _rand(rng, 1, 2, 12)
    src = np.repeat(row, 5, axis=0)
    w, dx = _rand(rng, 12), _rand(rng, 2, 12)
    b = oracle.site_backward(src, w, None, None, 1e-6, dx, prenorm=False)
    for i in range(5):
        np.testing.assert_allclose(b["du"][i], dx / 5.0, rtol=0, atol=1e-15)
    assert np.max(np.abs(b["dw"])) < 1e-15 and np.max(np.abs(b["dg"])) < 1e-15


def test_zero_upstream_gradient_gives_zero():
    rng = np.random.default_rng(9)
    src = _rand(rng, 3, 2, 7)
    b = oracle.site_backward(src, _rand(rng, 7), None, None, 1e-6, np.zeros((2, 7)))
    for k in ("du", "dw", "dg", "dgamma"):
        assert np.all(b[k] == 0.0), k


def test_logit_gradient_formula_of_the_notes():
    # with g = 1 and no PreNorm, dL/dw = sum_i dz_i y_i where the notes give
    # dz_i = alpha_i dh^T (u_i - h); check it by hand on one token
    rng = np.random.default_rng(10)
    n, d = 4, 9
    src = _rand(rng, n, 1, d)
    w, dx = _rand(rng, d), _rand(rng, 1, d)
    b = oracle.site_backward(src, w, None, None, 1e-6, dx, prenorm=False)
    f = oracle.depth_softmax([src[i, 0] for i in range(n)], w, None, 1e-6)
    dz = f["alpha"] * np.array([np.dot(dx[0], src[i, 0] - f["h"]) for i in range(n)])
    ys = np.array([src[i, 0] / oracle.rms(src[i, 0], 1e-6) for i in range(n)])
    np.testing.assert_allclose(b["dw"], dz @ ys, rtol=1e-12, atol=1e-14)
