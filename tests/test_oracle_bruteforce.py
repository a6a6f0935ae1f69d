"""Brute force against the oracle: an independent pure-Python Block AttnRes
forward (lists, math.fsum, the softmax in exp-ratio form
alpha_i = 1 / sum_k e^(z_k - z_i)) on tiny shapes (3 tokens of 8 channels),
over every partition of up to six sublayers into blocks (ragged tails
included), with and without given block sums.  It follows the definitions directly: "Attention
Residuals" (structured notes on arXiv 2603.15031), section 7 (the depth
softmax over RMS-normalised keys) and section 8 (Block sources: the
embedding, the completed block sums, and after a block's first sublayer the
running partial sum; the final aggregation over all block sums);
"Attention Residuals 阅读补充", RMSNorm.  Shares nothing with the oracle's C
code; agreement to 1e-13 (both sides are fp64; they differ only in
rounding order, about 1e-15 here) pins the oracle's source sets, partial sums,
phase-1 statistics and block sums index by index."""
import itertools
import math

import numpy as np
import pytest

import oracle


def rms(u, eps):
    return math.sqrt(math.fsum(x * x for x in u) / len(u) + eps)


def score(u, w, g, eps):
    r = rms(u, eps)
    return math.fsum(w[k] * g[k] * u[k] / r for k in range(len(u)))


def site(sources, w, g, eps):
    """Softmax over the sources' scores: weights by exp ratios, h, max, log-sum-exp."""
    z = [score(u, w, g, eps) for u in sources]
    alpha = [1.0 / math.fsum(math.exp(zk - zi) for zk in z) for zi in z]
    d = len(sources[0])
    h = [math.fsum(alpha[i] * sources[i][k] for i in range(len(sources))) for k in range(d)]
    m = max(z)
    lse = z[0] + math.log(math.fsum(math.exp(zk - z[0]) for zk in z))
    return h, m, lse


def brute_block_forward(emb, v, w, g, gamma, blocks, eps, given):
    """One token: emb [d]; v [L][d]; w, g [L+1][d]; gamma [L][d]; given [n][d]."""
    d = len(emb)
    out = {k: [] for k in ("x", "h", "o1", "m1", "lse1", "lse")}
    done = [emb] + list(given)       # b_0, the given block sums, then this pass's blocks
    l = 0
    for S in blocks:
        for j in range(S):
            sources = list(done)
            o1, m1, lse1 = site(sources, w[l], g[l], eps)
            if j >= 1:
                sources = sources + [[math.fsum(v[l - j + i][k] for i in range(j)) for k in range(d)]]
            h, _, lse = site(sources, w[l], g[l], eps)
            rh = rms(h, eps)
            out["x"].append([gamma[l][k] * h[k] / rh for k in range(d)])
            out["h"].append(h)
            out["o1"].append(o1)
            out["m1"].append(m1)
            out["lse1"].append(lse1)
            out["lse"].append(lse)
            l += 1
        done.append([math.fsum(v[l - S + i][k] for i in range(S)) for k in range(d)])
    hf, _, _ = site(done, w[l], g[l], eps)
    out["hfinal"] = hf
    out["reps"] = done
    return out


def compositions(L):
    """Every ordered partition of L sublayers into blocks."""
    for cuts in itertools.product((0, 1), repeat=L - 1):
        parts, n = [], 1
        for c in cuts:
            if c:
                parts.append(n)
                n = 1
            else:
                n += 1
        parts.append(n)
        yield tuple(parts)


CASES = [(blocks, ng) for L in range(1, 7) for blocks in compositions(L) for ng in (0, 1)]


@pytest.mark.parametrize("blocks,n_given", CASES)
def test_oracle_block_forward_equals_brute_force(blocks, n_given):
    rng = np.random.default_rng(hash((blocks, n_given)) % (1 << 32))
    T, d, eps = 3, 8, 1e-6
    L = sum(blocks)
    f32 = lambda a: np.asarray(a, dtype=np.float32)  # noqa: E731  (inputs as delivered: fp32)
    emb = f32(rng.normal(size=(T, d)))
    v = f32(rng.normal(size=(L, T, d)) * rng.uniform(0.5, 4, size=(L, 1, 1)))
    given = f32(rng.normal(size=(n_given, T, d)) * 2) if n_given else None
    w = f32(rng.normal(size=(L + 1, d)) * 0.7)
    g = f32(rng.uniform(0.8, 1.2, size=(L + 1, d)))
    gamma = f32(rng.uniform(0.8, 1.2, size=(L, d)))
    o = oracle.block_forward(emb, v, w, g, gamma, blocks, eps, given=given)
    tol = 1e-13
    for t in range(T):
        ref = brute_block_forward(emb[t].tolist(), v[:, t].tolist(), w.tolist(), g.tolist(), gamma.tolist(),
                                  blocks, eps, [] if given is None else given[:, t].tolist())
        for key in ("x", "h", "o1"):
            got = o[key][:, t]
            want = np.asarray(ref[key])
            assert np.max(np.abs(got - want)) <= tol * max(1.0, np.max(np.abs(want))), (key, t)
        for key in ("m1", "lse1", "lse"):
            assert np.max(np.abs(o[key][:, t] - np.asarray(ref[key]))) <= tol * 10, (key, t)
        assert np.max(np.abs(o["hfinal"][t] - np.asarray(ref["hfinal"]))) <= tol * 10
        assert np.max(np.abs(o["reps"][:, t] - np.asarray(ref["reps"]))) <= tol * 10
