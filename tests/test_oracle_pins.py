"""Pins of the fp64 oracle to facts the pages and the mathematics fix.

Each test names the passage it relies on by page title and section.  The
checks are chosen so that a plausible slip in the oracle -- a dropped eps, a
LayerNorm in place of RMSNorm, a wrong sign, normalised values in place of raw
sources, the wrong pseudo-query at a site, the empty partial sum counted as a
source, a wrong block boundary -- fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle

RNG = np.random.default_rng(20260316)


# ---------------------------------------------------------------- RMSNorm
# "Attention Residuals 阅读补充", section "从均方根到欧氏范数": at eps = 0 the
# normalised vector lies on the sphere of radius sqrt(d); mean square is 1.
@pytest.mark.parametrize("d", [1, 2, 7, 256, 7168])
def test_rmsnorm_sphere_radius_sqrt_d(oracle_lib, d):
    x = RNG.normal(size=d) * RNG.uniform(0.01, 100)
    y = oracle.rmsnorm(x, None, eps=0.0)
    assert np.isclose(np.dot(y, y), d, rtol=1e-13)
    assert np.isclose(np.mean(y * y), 1.0, rtol=1e-13)
    # direction preserved
    assert np.allclose(y / np.linalg.norm(y), x / np.linalg.norm(x), rtol=1e-12, atol=1e-15)


# Same page, section "ε 与 γ 改变了什么": with eps > 0 the squared length is
# d ||x||^2 / (||x||^2 + d eps), strictly below d.
@pytest.mark.parametrize("eps", [1e-6, 1e-2, 0.5])
def test_rmsnorm_eps_closed_form(oracle_lib, eps):
    d = 64
    x = RNG.normal(size=d) * 0.05
    y = oracle.rmsnorm(x, None, eps=eps)
    n2 = float(np.dot(x, x))
    assert np.isclose(np.dot(y, y), d * n2 / (n2 + d * eps), rtol=1e-13)
    assert np.dot(y, y) < d


# Same page, section "二阶原点矩与方差": m2 = sigma^2 + mu^2, so RMSNorm is not
# shift invariant and coincides with LayerNorm (no bias, same eps) iff mu = 0.
def test_rmsnorm_is_not_layernorm(oracle_lib):
    d = 32
    x = RNG.normal(size=d)
    eps = 1e-6
    r = oracle.rms(x, eps)
    assert np.isclose(r * r, np.var(x) + np.mean(x) ** 2 + eps, rtol=1e-13)
    shifted = oracle.rmsnorm(x + 0.7, None, eps)
    assert not np.allclose(shifted, oracle.rmsnorm(x, None, eps), atol=1e-3)
    xc = x - x.mean()
    ln = torch.nn.functional.layer_norm(torch.from_numpy(xc), (d,), eps=eps).numpy()
    assert np.allclose(oracle.rmsnorm(xc, None, eps), ln, rtol=1e-12, atol=1e-12)
    # and it differs from LayerNorm when the mean is not zero
    ln2 = torch.nn.functional.layer_norm(torch.from_numpy(x + 0.7), (d,), eps=eps).numpy()
    assert not np.allclose(shifted, ln2, atol=1e-3)


def test_rmsnorm_gain_is_per_channel(oracle_lib):
    d = 16
    x = RNG.normal(size=d)
    g = RNG.uniform(0.5, 2.0, size=d)
    base = oracle.rmsnorm(x, None, 1e-6)
    assert np.allclose(oracle.rmsnorm(x, g, 1e-6), g * base, rtol=1e-14)


# ---------------------------------------------------------- scoring / softmax
# "Attention Residuals 阅读补充", section "尺度变化与平移" and "回到 AttnRes":
# at eps = 0, RMSNorm(a x) = RMSNorm(x) for a > 0 and = -RMSNorm(x) for a < 0,
# so the score of a source does not see its scale, only its sign.
@pytest.mark.parametrize("a", [1e-3, 0.5, 3.0, 1e4])
def test_score_scale_invariance(oracle_lib, a):
    d = 48
    v = RNG.normal(size=d)
    w = RNG.normal(size=d) * 0.02
    g = RNG.uniform(0.8, 1.2, size=d)
    z = oracle.depth_softmax([v, a * v, -a * v], w, g, eps=0.0)["z"]
    assert np.isclose(z[1], z[0], rtol=1e-12)
    assert np.isclose(z[2], -z[0], rtol=1e-12)


def test_key_gain_folds_into_query(oracle_lib):
    # z = w^T (g (.) v / r) = (w (.) g)^T (v / r): the key gain acts per
    # channel, exactly like a gain on the query.  A gain of 2 doubles scores.
    d = 40
    srcs = [RNG.normal(size=d) for _ in range(4)]
    w = RNG.normal(size=d) * 0.02
    g = RNG.uniform(0.8, 1.2, size=d)
    z1 = oracle.depth_softmax(srcs, w, g, 1e-6)["z"]
    z2 = oracle.depth_softmax(srcs, w * g, None, 1e-6)["z"]
    assert np.allclose(z1, z2, rtol=1e-12)
    z3 = oracle.depth_softmax(srcs, w, np.full(d, 2.0), 1e-6)["z"]
    z4 = oracle.depth_softmax(srcs, w, None, 1e-6)["z"]
    assert np.allclose(z3, 2 * z4, rtol=1e-13)


# "Attention Residuals" notes, section 7: the weights are a softmax over depth
# of the scores (no 1/sqrt(d), no temperature); they are positive, sum to 1.
def test_softmax_weights(oracle_lib):
    d = 1024
    srcs = [RNG.normal(size=d) * s for s in (0.5, 1, 4, 8, 2)]
    w = RNG.normal(size=d) * 0.02
    r = oracle.depth_softmax(srcs, w, None, 1e-6)
    assert np.all(r["alpha"] > 0)
    assert np.isclose(r["alpha"].sum(), 1.0, rtol=1e-14)
    assert np.allclose(r["alpha"], scipy.special.softmax(r["z"]), rtol=1e-13)
    assert np.isclose(r["lse"], scipy.special.logsumexp(r["z"]), rtol=1e-14)
    assert np.isclose(r["m"], r["z"].max())
    # the scores are plain dot products with the RMS-normalised keys
    keys = [s / math.sqrt(np.mean(s * s) + 1e-6) for s in srcs]
    assert np.allclose(r["z"], [float(np.dot(w, k)) for k in keys], rtol=1e-12)


# Same section: values are the unnormalised sources, so identical sources give
# that source back, a single source gives itself with weight 1, and the
# output is a convex combination (||h|| <= max ||v_i||, channelwise hull).
def test_identical_and_single_sources(oracle_lib):
    d = 64
    v = RNG.normal(size=d) * 7.0
    w = RNG.normal(size=d) * 0.5
    r = oracle.depth_softmax([v, v, v], w, None, 1e-6)
    assert np.allclose(r["h"], v, rtol=1e-14)
    assert np.allclose(r["alpha"], 1 / 3, rtol=1e-14)
    r1 = oracle.depth_softmax([v], w, None, 1e-6)
    assert np.array_equal(r1["h"], v)
    assert r1["alpha"][0] == 1.0
    assert np.isclose(r1["lse"], r1["z"][0], rtol=0, atol=0)


def test_convexity_bound(oracle_lib):
    d = 128
    for _ in range(20):
        n = int(RNG.integers(1, 10))
        srcs = [RNG.normal(size=d) * RNG.uniform(0.1, 10) for _ in range(n)]
        w = RNG.normal(size=d) * RNG.uniform(0.01, 1.0)
        h = oracle.depth_softmax(srcs, w, None, 1e-6)["h"]
        assert np.linalg.norm(h) <= max(np.linalg.norm(s) for s in srcs) * (1 + 1e-12)
        S = np.stack(srcs)
        assert np.all(h <= S.max(0) + 1e-12) and np.all(h >= S.min(0) - 1e-12)


# Same section: zero pseudo-queries give equal weights, i.e. the plain mean.
def test_zero_query_is_mean(oracle_lib):
    d = 32
    srcs = [RNG.normal(size=d) for _ in range(5)]
    r = oracle.depth_softmax(srcs, np.zeros(d), None, 1e-6)
    assert np.allclose(r["h"], np.mean(srcs, axis=0), rtol=1e-13)
    assert np.isclose(r["lse"], math.log(5), rtol=1e-15)


# Worked example derived here from the definitions (not printed on the pages):
# d = 2, eps = 0, unit gains, v0 = (1, 0), v1 = (0, 2), w = (a, b).
# RMSNorm(v0) = sqrt(2) (1, 0), RMSNorm(v1) = sqrt(2) (0, 1), so
# z = (sqrt2 a, sqrt2 b) and h = (s, 2 (1 - s)) with s = 1 / (1 + e^{sqrt2 (b - a)}).
@pytest.mark.parametrize("a,b", [(0.0, 0.0), (1.0, -1.0), (-2.0, 0.5), (0.3, 0.31), (5.0, -5.0)])
def test_worked_example_d2(oracle_lib, a, b):
    r = oracle.depth_softmax([np.array([1.0, 0.0]), np.array([0.0, 2.0])], [a, b], None, 0.0)
    s = 1.0 / (1.0 + math.exp(math.sqrt(2.0) * (b - a)))
    assert np.allclose(r["z"], [math.sqrt(2) * a, math.sqrt(2) * b], rtol=1e-14)
    assert np.allclose(r["h"], [s, 2 * (1 - s)], rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------ two-phase merge
# "Attention Residuals 阅读补充", two-phase section, and the notes' section 10:
# merging the statistics of any two disjoint, complete partitions equals the
# one-shot softmax over their union.
def test_two_partition_merge_equals_one_shot(oracle_lib):
    d = 24
    for n in range(2, 7):
        srcs = [RNG.normal(size=d) * RNG.uniform(0.3, 9) for _ in range(n)]
        w = RNG.normal(size=d) * 0.3
        g = RNG.uniform(0.8, 1.2, size=d)
        ref = oracle.depth_softmax(srcs, w, g, 1e-6)["h"]
        for k in range(1, n):
            for A in itertools.combinations(range(n), k):
                B = [i for i in range(n) if i not in A]
                mA, lA, oA = oracle.partition_stats([srcs[i] for i in A], w, g, 1e-6)
                mB, lB, oB = oracle.partition_stats([srcs[i] for i in B], w, g, 1e-6)
                h = oracle.merge_two(mA, lA, oA, mB, lB, oB)
                assert np.allclose(h, ref, rtol=1e-13, atol=1e-13)
                # order of the two partitions does not matter
                assert np.allclose(oracle.merge_two(mB, lB, oB, mA, lA, oA), ref, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------- Block AttnRes
def _int_inputs(L, n_tok, d, n_given=0, lo=-4, hi=5):
    emb = RNG.integers(lo, hi, size=(n_tok, d)).astype(np.float32)
    v = RNG.integers(lo, hi, size=(L, n_tok, d)).astype(np.float32)
    given = RNG.integers(lo, hi, size=(n_given, n_tok, d)).astype(np.float32) if n_given else None
    return emb, v, given


def _expected_sources(emb_t, v_t, given_t, blocks):
    """Enumerate each site's source list from block membership (integers)."""
    reps = [emb_t] + ([] if given_t is None else list(given_t))
    sites = []
    l = 0
    for S in blocks:
        block_sum = None
        for j in range(S):
            srcs = list(reps) + ([block_sum] if j > 0 else [])
            sites.append(srcs)
            block_sum = v_t[l].astype(np.int64) if block_sum is None else block_sum + v_t[l]
            l += 1
        reps.append(block_sum)
    return sites, reps


# "Attention Residuals" notes, section 8: the first sublayer of block n sees
# b_0..b_{n-1}; later ones add the partial sum b_n^{i-1}; b_n^0 = 0 is not a
# source; the final output reads b_0..b_N.  With zero queries every site's
# output is the mean of exactly those sources and lse = ln(#sources).
@pytest.mark.parametrize("blocks,n_given", [((4, 4), 0), ((3, 1, 2), 0), ((1,), 0), ((5,), 3),
                                            ((2, 3, 1), 2), ((1, 1, 1, 1), 0)])
def test_block_source_sets_zero_query(oracle_lib, blocks, n_given):
    L, n_tok, d = sum(blocks), 3, 8
    emb, v, given = _int_inputs(L, n_tok, d, n_given)
    w = np.zeros((L + 1, d), np.float32)
    out = oracle.block_forward(emb, v, w, None, None, blocks, eps=1e-6, given=given)
    for t in range(n_tok):
        sites, reps = _expected_sources(emb[t], v[:, t], None if given is None else given[:, t], blocks)
        for l, srcs in enumerate(sites):
            mean = np.sum(np.stack(srcs).astype(np.float64), axis=0) / len(srcs)
            assert np.allclose(out["h"][l, t], mean, rtol=1e-14, atol=1e-14), (l, t)
            assert np.isclose(out["lse"][l, t], math.log(len(srcs)), rtol=1e-14)
        # exact block sums
        for i, r in enumerate(reps):
            assert np.array_equal(out["reps"][i, t], np.asarray(r, np.float64)), (i, t)
        fin = np.sum(np.stack(reps).astype(np.float64), axis=0) / len(reps)
        assert np.allclose(out["hfinal"][t], fin, rtol=1e-14, atol=1e-14)


def test_block_phase1_quantities_zero_query(oracle_lib):
    blocks, n_given = (3, 4), 2
    L, n_tok, d = sum(blocks), 2, 8
    emb, v, given = _int_inputs(L, n_tok, d, n_given)
    out = oracle.block_forward(emb, v, np.zeros((L + 1, d), np.float32), None, None, blocks,
                               eps=1e-6, given=given)
    for t in range(n_tok):
        sites, reps = _expected_sources(emb[t], v[:, t], given[:, t], blocks)
        l = 0
        for b, S in enumerate(blocks):
            done = reps[:1 + n_given + b]
            for j in range(S):
                mean = np.sum(np.stack(done).astype(np.float64), axis=0) / len(done)
                assert np.allclose(out["o1"][l, t], mean, rtol=1e-14, atol=1e-14)
                assert np.isclose(out["lse1"][l, t], math.log(len(done)), rtol=1e-14)
                assert out["m1"][l, t] == 0.0
                l += 1


# "Attention Residuals" notes, section 8 (extremes of the block count): with
# one sublayer per block, Block AttnRes is exactly Full AttnRes.  The two are
# separate code paths in the oracle.
def test_block_with_N_equal_L_is_full(oracle_lib):
    L, n_tok, d = 7, 4, 40
    emb = RNG.normal(size=(n_tok, d)).astype(np.float32)
    v = (RNG.normal(size=(L, n_tok, d)) * RNG.uniform(0.5, 8, size=(L, 1, 1))).astype(np.float32)
    w = (RNG.normal(size=(L + 1, d)) * 0.3).astype(np.float32)
    g = RNG.uniform(0.8, 1.2, size=(L + 1, d)).astype(np.float32)
    gam = RNG.uniform(0.8, 1.2, size=(L, d)).astype(np.float32)
    b = oracle.block_forward(emb, v, w, g, gam, (1,) * L, eps=1e-6)
    f = oracle.full_forward(emb, v, w, g, gam, eps=1e-6)
    for k in ("x", "h", "lse", "hfinal"):
        assert np.allclose(b[k], f[k], rtol=1e-13, atol=1e-13), k


# Hard selection: with one-hot pseudo-queries of large magnitude and +-1
# sources (RMS exactly 1 at eps = 0), site l must return the one source that
# is +1 on the channel its own query selects.  A wrong sign, the query of a
# neighbouring site, or normalised values in place of raw ones all fail.
def test_full_hard_selection_uses_each_sites_query(oracle_lib):
    L, d, n_tok = 6, 8, 2
    rng = np.random.default_rng(7)
    emb = np.empty((n_tok, d), np.float32)
    v = np.empty((L, n_tok, d), np.float32)
    for t in range(n_tok):
        srcs = -np.ones((L + 1, d), np.float32)
        for k in range(d):
            srcs[rng.integers(0, L + 1), k] = 1.0
        emb[t], v[:, t] = srcs[0], srcs[1:]
    chan = rng.integers(0, d, size=L + 1)
    w = np.zeros((L + 1, d), np.float32)
    w[np.arange(L + 1), chan] = 30.0
    out = oracle.full_forward(emb, v, w, None, None, eps=0.0)
    for t in range(n_tok):
        hist = np.concatenate([emb[t][None], v[:, t]], 0)
        for l in range(L):
            cand = hist[:l + 1]
            pos = np.where(cand[:, chan[l]] > 0)[0]
            if len(pos) == 1:
                assert np.allclose(out["h"][l, t], cand[pos[0]], atol=1e-12)
            else:  # all candidates tie at -1 or several at +1: mean of the tied ones
                top = pos if len(pos) else np.arange(l + 1)
                assert np.allclose(out["h"][l, t], cand[top].mean(0), atol=1e-12)


# PreNorm of the consumer (read as RMSNorm with that sublayer's gain): scaling
# every input by a > 0 at eps = 0 scales each h by a and leaves x unchanged;
# with unit gain ||x|| = sqrt(d); a constant gain c scales x by c.
def test_prenorm_output_invariances(oracle_lib):
    blocks = (3, 2)
    L, n_tok, d = sum(blocks), 3, 32
    emb = RNG.normal(size=(n_tok, d)).astype(np.float32)
    v = RNG.normal(size=(L, n_tok, d)).astype(np.float32)
    w = (RNG.normal(size=(L + 1, d)) * 0.3).astype(np.float32)
    a = 4.0  # a power of two keeps the scaled fp32 inputs exact
    o1 = oracle.block_forward(emb, v, w, None, None, blocks, eps=0.0)
    o2 = oracle.block_forward(a * emb, a * v, w, None, None, blocks, eps=0.0)
    assert np.allclose(o2["h"], a * o1["h"], rtol=1e-12)
    assert np.allclose(o2["x"], o1["x"], rtol=1e-12)
    assert np.allclose(np.sum(o1["x"] ** 2, -1), d, rtol=1e-12)
    gam = np.full((L, d), 3.0, np.float32)
    o3 = oracle.block_forward(emb, v, w, None, gam, blocks, eps=0.0)
    assert np.allclose(o3["x"], 3.0 * o1["x"], rtol=1e-13)


# "Attention Residuals" notes, section 7: the aggregation acts along depth
# only; tokens do not interact.  Permuting tokens permutes every output, and a
# token computed alone equals the same token computed in a batch.
def test_tokens_are_independent(oracle_lib):
    blocks = (2, 3)
    L, n_tok, d = sum(blocks), 5, 16
    emb = RNG.normal(size=(n_tok, d)).astype(np.float32)
    v = RNG.normal(size=(L, n_tok, d)).astype(np.float32)
    w = (RNG.normal(size=(L + 1, d)) * 0.3).astype(np.float32)
    perm = RNG.permutation(n_tok)
    a = oracle.block_forward(emb, v, w, None, None, blocks, eps=1e-6)
    b = oracle.block_forward(emb[perm], v[:, perm], w, None, None, blocks, eps=1e-6)
    for k in ("x", "h", "o1", "lse"):
        assert np.array_equal(b[k], a[k][:, perm]), k
    one = oracle.block_forward(emb[2:3], v[:, 2:3], w, None, None, blocks, eps=1e-6)
    assert np.array_equal(one["x"][:, 0], a["x"][:, 2])


def test_empty_token_set(oracle_lib):
    out = oracle.block_forward(np.zeros((0, 8), np.float32), np.zeros((2, 0, 8), np.float32),
                               np.zeros((3, 8), np.float32), None, None, (2,), eps=1e-6)
    assert out["x"].shape == (2, 0, 8)
