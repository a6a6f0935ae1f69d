"""Pins of the oracle's backward through the whole Block AttnRes structure
(CPU only).

The loss is L = sum_l dx_l . x_l + dhf . hfinal with the sublayer outputs v_l
as inputs.  Its gradients are pinned to central finite differences of a
forward written here from the oracle's one-site functions (depth_softmax,
rmsnorm) in fp64 -- a path that shares no loop with oracle_block_backward --
and to closed forms of degenerate structures.
"""
import numpy as np
import pytest

import oracle


def _rand(rng, *shape, scale=1.0):
    # values exactly representable in fp32 (the oracle widens fp32 inputs)
    return (rng.standard_normal(shape) * scale).astype(np.float32).astype(np.float64)


def _gain(rng, *shape):
    return (0.8 + 0.4 * rng.random(shape)).astype(np.float32).astype(np.float64)


def _forward_loss(emb, given, v, w, g, gamma, blocks, eps, dx, dhf, final_site):
    """sum_l dx_l . x_l + dhf . hfinal, one token at a time ("Attention
    Residuals" notes, section 8: sources b_0..b_{n-1} plus the block's partial
    sum after its first sublayer; the final site reads b_0..b_N)."""
    T, d = emb.shape
    L = int(sum(blocks))
    tot = 0.0
    for t in range(T):
        reps = [emb[t]] + [given[i, t] for i in range(0 if given is None else given.shape[0])]
        l = 0
        for S in blocks:
            part = np.zeros(d)
            for j in range(S):
                srcs = reps + ([part] if j > 0 else [])
                h = oracle.depth_softmax(srcs, w[l], g[l], eps)["h"]
                tot += float(np.dot(dx[l, t], oracle.rmsnorm(h, gamma[l], eps)))
                part = part + v[l, t]
                l += 1
            reps.append(part)
        if final_site:
            hf = oracle.depth_softmax(reps, w[L], g[L], eps)["h"]
            tot += float(np.dot(dhf[t], hf))
    return tot


def _fd(f, arr, delta=1e-6):
    out = np.empty_like(arr)
    flat, o = arr.reshape(-1), out.reshape(-1)
    for j in range(flat.size):
        keep = flat[j]
        flat[j] = keep + delta
        up = f()
        flat[j] = keep - delta
        dn = f()
        flat[j] = keep
        o[j] = (up - dn) / (2 * delta)
    return out


def _close(a, b, tol):
    scale = max(1.0, float(np.max(np.abs(b))))
    assert float(np.max(np.abs(a - b))) <= tol * scale, (float(np.max(np.abs(a - b))), scale)


def _case(seed, T, d, blocks, n_given, final_site):
    rng = np.random.default_rng(seed)
    L = int(sum(blocks))
    c = dict(emb=_rand(rng, T, d), given=_rand(rng, n_given, T, d, scale=3.0) if n_given else None,
             v=_rand(rng, L, T, d, scale=2.0), w=_rand(rng, L + 1, d, scale=0.5), g=_gain(rng, L + 1, d),
             gamma=_gain(rng, L, d), dx=_rand(rng, L, T, d), dhf=_rand(rng, T, d) if final_site else None)
    return c


@pytest.mark.parametrize("T,d,blocks,n_given,final_site,eps", [
    (2, 5, (2, 3), 1, True, 1e-6),
    (1, 4, (3,), 0, True, 1e-3),
    (2, 6, (1, 2, 2), 0, False, 1e-6),
    (1, 3, (4, 1), 2, True, 0.0),
])
def test_block_backward_matches_finite_differences(T, d, blocks, n_given, final_site, eps):
    c = _case(300 + T + d + len(blocks), T, d, blocks, n_given, final_site)
    b = oracle.block_backward(c["emb"], c["v"], c["w"], c["g"], c["gamma"], blocks, eps, c["dx"], c["dhf"],
                              given=c["given"], final_site=final_site)

    def f():
        return _forward_loss(c["emb"], c["given"], c["v"], c["w"], c["g"], c["gamma"], blocks, eps, c["dx"],
                             c["dhf"], final_site)

    _close(b["dv"], _fd(f, c["v"]), 1e-6)
    _close(b["demb"], _fd(f, c["emb"]), 1e-6)
    if n_given:
        _close(b["dgiven"], _fd(f, c["given"]), 1e-6)
    _close(b["dw"], _fd(f, c["w"]), 1e-6)
    _close(b["dg"], _fd(f, c["g"]), 1e-6)
    _close(b["dgamma"], _fd(f, c["gamma"]), 1e-6)


def test_zero_upstream_gives_zero():
    c = _case(5, 2, 4, (2, 2), 1, True)
    b = oracle.block_backward(c["emb"], c["v"], c["w"], c["g"], c["gamma"], (2, 2), 1e-6,
                              np.zeros_like(c["dx"]), np.zeros_like(c["dhf"]), given=c["given"])
    for k in ("dv", "demb", "dgiven", "dw", "dg", "dgamma"):
        assert np.all(b[k] == 0.0), k


def test_one_sublayer_closed_form():
    # one block of one sublayer, no final site: the only site reads b_0 alone
    # (alpha = 1, h = b_0), so dL/db_0 is the PreNorm backward of dx and v_0
    # reaches nothing
    rng = np.random.default_rng(6)
    T, d, eps = 3, 7, 1e-6
    emb, v, dx = _rand(rng, T, d), _rand(rng, 1, T, d), _rand(rng, 1, T, d)
    w, g, gamma = _rand(rng, 1, d), _gain(rng, 1, d), _gain(rng, 1, d)
    b = oracle.block_backward(emb, v, w, g, gamma, (1,), eps, dx, None, final_site=False)
    assert np.all(b["dv"] == 0.0)
    assert np.all(b["dw"] == 0.0) and np.all(b["dg"] == 0.0)
    r = np.sqrt(np.mean(emb * emb, axis=1, keepdims=True) + eps)
    y = emb / r
    G = gamma[0] * dx[0]
    want = (G - y * np.sum(y * G, axis=1, keepdims=True) / d) / r
    np.testing.assert_allclose(b["demb"], want, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b["dgamma"][0], np.sum(dx[0] * y, axis=0), rtol=1e-12, atol=1e-13)


def test_last_output_of_the_last_block_without_final_site_gets_nothing():
    # v of the last sublayer enters only the last block sum, which no site
    # reads without the final aggregation; every earlier output of that
    # block reaches later sites through the partial sum
    c = _case(8, 2, 5, (2, 3), 0, False)
    b = oracle.block_backward(c["emb"], c["v"], c["w"], c["g"], c["gamma"], (2, 3), 1e-6, c["dx"], None,
                              final_site=False)
    assert np.all(b["dv"][-1] == 0.0)
    assert np.all(np.any(b["dv"][:-1] != 0.0, axis=-1))
