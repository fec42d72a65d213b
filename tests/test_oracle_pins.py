"""Pins of the CPU oracle against what the pages and the mathematics fix (CPU only).

Each test ties one part of the oracle to something other than itself: a library routine for a
special case (numpy's Philox, scipy's softmax, an optimiser for Theorem 12), brute force on tiny
inputs, the lossless theorem integrated exactly over the uniforms with the oracle treated as a
black box, the pages' worked example (Theorem 19) and closed forms.
"""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.optimize
import scipy.special
import scipy.stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------------------------------
# Philox4x64-10 against numpy's independent implementation
# ------------------------------------------------------------------------------------------
def _numpy_philox_block(ctr, key):
    """numpy's Philox4x64 increments its counter before each block: start one below."""
    c = [int(x) for x in ctr]
    prev = list(c)
    for i in range(4):  # subtract one with borrow
        if prev[i] > 0:
            prev[i] -= 1
            break
        prev[i] = (1 << 64) - 1
    bg = np.random.Philox(key=0)
    st = bg.state
    st["state"]["counter"] = np.array(prev, dtype=np.uint64)
    st["state"]["key"] = np.array([int(k) for k in key], dtype=np.uint64)
    st["buffer_pos"] = 4
    bg.state = st
    return bg.random_raw(4)


@pytest.mark.parametrize("ctr,key", [
    ([1, 0, 0, 0], [1, 2]),
    ([0, 0, 0, 0], [0, 0]),
    ([5, 7, 11, 13], [0xDEADBEEF, 42]),
    ([0, 1, 0, 0], [0xC0FFEE03, 0]),
    ([(1 << 64) - 1, (1 << 64) - 1, 3, 9], [(1 << 64) - 1, 1 << 63]),
    ([123456789, 15, 5, 0], [0xC0FFEE01, 0]),
])
def test_philox_matches_numpy(ctr, key):
    assert (oracle.philox4x64_10(ctr, key) == _numpy_philox_block(ctr, key)).all()


def test_uniforms_open_interval_and_uniform():
    U = oracle.uniforms(0xC0FFEE01, 0, 20000, 4)
    assert U.min() > 0.0 and U.max() < 1.0
    for lane in range(3):
        counts, _ = np.histogram(U[:, :, lane].ravel(), bins=64, range=(0.0, 1.0))
        assert scipy.stats.chisquare(counts).pvalue > 1e-4


# ------------------------------------------------------------------------------------------
# Processing: temperature, top-k, softmax, nucleus
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("T", [0.25, 0.8, 1.0, 2.5])
def test_softmax_matches_scipy(T):
    rng = np.random.default_rng(1)
    z = rng.normal(0, 3, 4096)
    p, bad, _, n = oracle.process_row(z, T, 0, 1.0)
    assert not bad and n == 4096
    # the temperature is an fp32 request parameter
    np.testing.assert_allclose(p, scipy.special.softmax(z / float(np.float32(T))), rtol=1e-12, atol=1e-300)


def _brute_order(z):
    return sorted(range(len(z)), key=lambda i: (-z[i], i))


@pytest.mark.parametrize("seed", range(6))
def test_topk_and_nucleus_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    V = 9
    z = rng.integers(-3, 3, V).astype(np.float64)  # integer logits force ties
    for T in (0.7, 1.0):
        for top_k in (0, 1, 3, 5, 9, 12):
            for top_p in (0.1, 0.5, 0.77, 0.95, 1.0):
                p, bad, _, _ = oracle.process_row(z, T, top_k, top_p)
                order = _brute_order(z)
                kept = order[: top_k] if 0 < top_k < V else order
                Tf = float(np.float32(T))
                e = {i: np.exp((z[i] - z[order[0]]) / Tf) for i in kept}
                S = sum(e.values())
                if top_p < 1.0:
                    cum, nuc = 0.0, []
                    for i in kept:
                        nuc.append(i)
                        cum += e[i]
                        if cum >= float(np.float32(top_p)) * S:
                            break
                else:
                    nuc = kept
                Sn = sum(e[i] for i in nuc)
                ref = np.zeros(V)
                for i in nuc:
                    ref[i] = e[i] / Sn
                np.testing.assert_allclose(p, ref, rtol=1e-13, atol=1e-15)


def test_bad_rows():
    p, bad, _, _ = oracle.process_row([0.0, np.nan, 1.0], 1.0, 0, 1.0)
    assert bad
    p, bad, _, _ = oracle.process_row([0.0, np.inf, 1.0], 1.0, 0, 1.0)
    assert bad
    p, bad, _, _ = oracle.process_row([-np.inf, -np.inf], 1.0, 0, 1.0)
    assert bad
    p, bad, _, n = oracle.process_row([-np.inf, 3.0, -np.inf], 1.0, 0, 0.5)
    assert not bad and n == 1 and p[1] == 1.0


# ------------------------------------------------------------------------------------------
# Saguaro sampling: Theorem 19 worked example, and Theorem 15 monotonicity
# ------------------------------------------------------------------------------------------
def test_theorem19_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "theorem19.json")))
    pt = np.array(g["p_target"])
    pd = np.array(g["p_draft"])
    C = g["C_num"] / g["C_den"]
    # logits = ln p at T = 1 reproduce p exactly up to rounding
    q, *_ = oracle.process_row(np.log(pt), 1.0, 0, 1.0)
    p, *_ = oracle.process_row(np.log(pd), 1.0, 0, 1.0)
    pp, Z, ids, deg = oracle.downweight_probs(np.log(pd), p, g["F"], C)
    assert not deg
    assert sorted(ids.tolist()) == [0, 1]
    np.testing.assert_allclose(pp, g["p_draft_after"], atol=1e-14)
    np.testing.assert_allclose(Z, 1.0 / 3.0, atol=1e-14)
    assert abs(np.minimum(p, q).sum() - g["alpha_before"]) < 1e-14
    assert abs(np.minimum(pp, q).sum() - g["alpha_after"]) < 1e-14
    assert np.flatnonzero(np.maximum(q - p, 0) > 1e-12).tolist() == g["residual_support_before"]
    assert np.flatnonzero(np.maximum(q - pp, 0) > 1e-12).tolist() == g["residual_support_after"]


@pytest.mark.parametrize("seed", range(5))
def test_theorem15_monotone_in_C(seed):
    rng = np.random.default_rng(200 + seed)
    V, F = 64, 4
    zq = rng.normal(0, 2, V)
    zp = zq + rng.normal(0, 1, V)
    q, *_ = oracle.process_row(zq, 1.0, 0, 1.0)
    p, *_ = oracle.process_row(zp, 1.0, 0, 1.0)
    mass_on_S, frac_on_S = [], []
    for C in np.linspace(1.0, 0.0, 21):
        pp, Z, ids, deg = oracle.downweight_probs(zp, p, F, C)
        assert not deg
        r = np.maximum(q - pp, 0)
        mass_on_S.append(r[ids].sum())
        frac_on_S.append(r[ids].sum() / r.sum())
    # residual mass (and its share) on the downweighted set never decrease as C -> 0
    assert np.all(np.diff(mass_on_S) >= -1e-15)
    assert np.all(np.diff(frac_on_S) >= -1e-15)
    assert mass_on_S[-1] > mass_on_S[0]


def test_downweight_set_is_top_F_with_mass():
    z = np.array([1.0, 3.0, 3.0, -np.inf, 2.0, 0.5])
    p, *_ = oracle.process_row(z, 1.0, 0, 1.0)
    pp, Z, ids, _ = oracle.downweight_probs(z, p, 3, 0.5)
    assert ids.tolist() == [1, 2, 4]        # ties by id, -inf carries no mass
    # nucleus leaves fewer than F tokens with mass: the set stops there
    p2, *_ = oracle.process_row(z, 1.0, 0, 0.3)
    _, _, ids2, _ = oracle.downweight_probs(z, p2, 3, 0.5)
    assert ids2.tolist()[0] == 1 and ids2.tolist()[2] == -1


# ------------------------------------------------------------------------------------------
# Lossless theorem by exact integration over the uniforms (oracle as a black box)
# ------------------------------------------------------------------------------------------
def _tile(a, n):
    return np.ascontiguousarray(np.repeat(a[None], n, axis=0))


def _bisect(decide, n, iters=64):
    """Per probe, sup{x in (0,1): decide(x) is True}, decide monotone (True for small x)."""
    lo = np.zeros(n)
    hi = np.ones(n)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        d = decide(mid)
        lo = np.where(d, mid, lo)
        hi = np.where(d, hi, mid)
    # never True -> 0, never False -> 1, else the bracket's midpoint (width 2^-64)
    return np.where(lo == 0.0, 0.0, np.where(hi == 1.0, 1.0, 0.5 * (lo + hi)))


def exact_law(zd, zt, T=1.0, top_k=0, top_p=1.0, F=0, C=1.0, uniform=False, tau=None, assisted=False):
    """Law of the oracle's output over s ~ p' and the uniforms, integrated exactly.

    ``uniform``: the draft distribution is the uniform one on [0, V) (the backup speculator);
    zd then only gives the shape.  Returns (law, p', q): law maps (k, emitted tokens) -> probability.
    """
    K, V = zd.shape
    # inputs are given to the oracle as fp32; the distributions below come from the same values
    q = [oracle.process_row(zt[j].astype(np.float32).astype(np.float64), T, top_k, top_p)[0] for j in range(K + 1)]
    pp = []
    for j in range(K):
        if uniform:
            pp.append(np.full(V, 1.0 / V))
            continue
        zz = zd[j].astype(np.float32).astype(np.float64)
        pj = oracle.process_row(zz, T, top_k, top_p)[0]
        pp.append(oracle.downweight_probs(zz, pj, F, C)[0])
    seqs = [s for s in itertools.product(range(V), repeat=K) if np.prod([pp[j][s[j]] for j in range(K)]) > 0]
    N = len(seqs)
    tok = np.array(seqs, dtype=np.int32)
    prm = oracle.params_array(T, top_k, top_p, B=N)
    D = _tile(zd.astype(np.float32), N)
    Tt = _tile(zt.astype(np.float32), N)
    ps = np.array([np.prod([pp[j][s[j]] for j in range(K)]) for s in seqs])

    def run(U, tokens=tok):
        n = U.shape[0]
        return oracle.verify(None if uniform else D[:n], Tt[:n], oracle.FP32, K, prm[:n], F=F, C=C, tokens=tokens,
                             U=U, uniform_draft=uniform, tau=tau, assisted=assisted)

    # acceptance thresholds a[n, j] with the earlier positions accepting
    a = np.zeros((N, K))
    for j in range(K):
        def dec(x, j=j):
            U = np.full((N, K + 1, 3), 0.5)
            U[:, :j, 0] = np.maximum(a[:, :j] * 0.5, 1e-300)
            U[:, j, 0] = np.maximum(x, 1e-300)
            return run(U).k > j
        a[:, j] = _bisect(dec, N)
    # law of t* as a function of v at each stopping position m: cut points by bisection
    law = {}
    for m in range(K + 1):
        reach = np.prod(a[:, :m], axis=1) * ((1.0 - a[:, m]) if m < K else 1.0)
        idx = np.flatnonzero(reach * ps > 0)
        if len(idx) == 0:
            continue
        n_i = len(idx)
        cuts = np.zeros((n_i, V + 1))
        cuts[:, V] = 1.0
        for y in range(V - 1):
            def dec(x, y=y):
                U = np.full((n_i, K + 1, 3), 0.5)
                U[:, :m, 0] = np.maximum(a[idx, :m] * 0.5, 1e-300)
                if m < K:
                    U[:, m, 0] = 0.5 * (1.0 + a[idx, m])
                U[:, m, 1] = np.maximum(x, 1e-300)
                r = oracle.verify(None if uniform else D[:n_i], Tt[:n_i], oracle.FP32, K, prm[:n_i], F=F, C=C,
                                  tokens=tok[idx], U=U, uniform_draft=uniform, tau=tau, assisted=assisted)
                assert (r.k == m).all()
                return r.t <= y
            cuts[:, y + 1] = _bisect(dec, n_i)
        width = np.diff(cuts, axis=1)
        for row, n in enumerate(idx):
            for y in range(V):
                w = ps[n] * reach[n] * width[row, y]
                if w > 0:
                    key = (m,) + tuple(int(x) for x in tok[n, :m]) + (y,)
                    law[key] = law.get(key, 0.0) + w
    return law, pp, q


def _check_lossless(law, pp, q, K, V):
    total = sum(law.values())
    assert abs(total - 1.0) < 1e-12
    # each depth's emitted token, given the output reaches that depth, has law q_j
    for d in range(K + 1):
        reach = 0.0
        dist = np.zeros(V)
        for key, w in law.items():
            m = key[0]
            if m >= d:
                dist[key[1 + d]] += w
                reach += w
        if reach > 1e-9:
            assert np.abs(dist / reach - q[d]).sum() < 1e-11, (d, dist / reach, q[d])
    # the joint law in closed form: prod_{i<m} min(p', q)(y_i) * (q_m - p'_m)+(y_m), or q_K at m = K
    for key, w in law.items():
        m, ys = key[0], key[1:]
        ref = np.prod([min(pp[i][ys[i]], q[i][ys[i]]) for i in range(m)])
        ref *= max(q[m][ys[m]] - pp[m][ys[m]], 0.0) if m < K else q[K][ys[K]]
        assert abs(w - ref) < 1e-12
    # acceptance-length law: P(k >= j) = prod_{i<j} alpha_i, alpha_i = sum min(p'_i, q_i)
    alpha = [np.minimum(pp[i], q[i]).sum() for i in range(K)]
    for j in range(K + 1):
        pk = sum(w for key, w in law.items() if key[0] >= j)
        assert abs(pk - np.prod(alpha[:j])) < 1e-12


@pytest.mark.parametrize("V,K,T,top_k,top_p,F,C,seed", [
    (4, 1, 1.0, 0, 1.0, 0, 1.0, 0),
    (8, 2, 1.0, 0, 1.0, 0, 1.0, 1),
    (4, 3, 0.8, 0, 1.0, 0, 1.0, 2),
    (5, 2, 1.0, 3, 1.0, 0, 1.0, 3),
    (6, 2, 1.0, 0, 0.8, 0, 1.0, 4),
    (5, 2, 0.9, 0, 1.0, 2, 0.3, 5),
    (6, 2, 1.0, 4, 0.9, 1, 0.5, 6),
])
def test_lossless_exact_enumeration(V, K, T, top_k, top_p, F, C, seed):
    rng = np.random.default_rng(300 + seed)
    zt = rng.normal(0, 1.5, (K + 1, V))
    zd = zt[:K] + rng.normal(0, 0.8, (K, V))
    law, pp, q = exact_law(zd, zt, T, top_k, top_p, F, C)
    _check_lossless(law, pp, q, K, V)


def test_mass_identity_random_rows():
    rng = np.random.default_rng(7)
    for _ in range(20):
        V = int(rng.integers(2, 3000))
        zq = rng.normal(0, 2, V)
        zp = zq + rng.normal(0, 1, V)
        T = float(rng.uniform(0.3, 1.5))
        tk = int(rng.integers(0, V + 2))
        tp = float(rng.uniform(0.2, 1.0))
        q, *_ = oracle.process_row(zq, T, tk, tp)
        p, *_ = oracle.process_row(zp, T, tk, tp)
        pp, *_ = oracle.downweight_probs(zp, p, int(rng.integers(0, 6)), float(rng.uniform(0, 1)))
        for d in (p, pp):
            assert abs(np.minimum(d, q).sum() + np.maximum(q - d, 0).sum() - 1.0) < 1e-13


def test_chi_square_monte_carlo():
    """10^6 Philox-driven rounds with sampled draft tokens against the exact law of (k, t*)."""
    rng = np.random.default_rng(11)
    V, K, N = 6, 2, 1_000_000
    zt = rng.normal(0, 1.2, (K + 1, V)).astype(np.float32)
    zd = (zt[:K] + rng.normal(0, 0.8, (K, V))).astype(np.float32)
    law, pp, q = exact_law(zd.astype(np.float64), zt.astype(np.float64), 1.0, 0, 1.0, 1, 0.5)
    _check_lossless(law, pp, q, K, V)
    prm = oracle.params_array(1.0, 0, 1.0, B=N)
    r = oracle.verify(_tile(zd, N), _tile(zt, N), oracle.FP32, K, prm, F=1, C=0.5, tokens=None,
                      seed=0x5EED, round_=3)
    exp = np.zeros((K + 1, V))
    for key, w in law.items():
        exp[key[0], key[-1]] += w
    obs = np.zeros((K + 1, V))
    np.add.at(obs, (r.k, r.t), 1)
    mask = exp.ravel() > 0
    assert obs.ravel()[~mask].sum() == 0
    stat = scipy.stats.chisquare(obs.ravel()[mask], exp.ravel()[mask] * N)
    assert stat.pvalue > 1e-4, stat


# ------------------------------------------------------------------------------------------
# Greedy verification
# ------------------------------------------------------------------------------------------
def test_greedy_longest_argmax_prefix():
    rng = np.random.default_rng(5)
    V, K, B = 50, 4, 64
    zt = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    zd = (zt[:, :K] + rng.normal(0, 0.5, (B, K, V))).astype(np.float32)
    amax = zt.argmax(axis=2)
    tok = np.zeros((B, K), np.int32)
    want_k = rng.integers(0, K + 1, B)
    for b in range(B):
        for j in range(K):
            tok[b, j] = amax[b, j] if j < want_k[b] else (amax[b, j] + 1 + rng.integers(0, V - 1)) % V
    prm = oracle.params_array(0.0, 0, 1.0, B=B)
    r = oracle.verify(zd, zt, oracle.FP32, K, prm, tokens=tok, seed=1)
    assert (r.k == want_k).all()
    assert (r.t == amax[np.arange(B), want_k]).all()
    # the stochastic rule at a tiny temperature with well separated logits reduces to the same
    zt2 = zt.copy()
    zd2 = zd.copy()
    for b in range(B):
        for j in range(K + 1):
            zt2[b, j, amax[b, j]] += 60.0
    prm2 = oracle.params_array(0.05, 0, 1.0, B=B)
    r2 = oracle.verify(zd2, zt2, oracle.FP32, K, prm2, tokens=tok, seed=1)
    assert (r2.k == want_k).all() and (r2.t == r.t).all()


def test_greedy_samples_draft_argmax():
    rng = np.random.default_rng(6)
    V, K, B = 40, 3, 16
    zt = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    zd = zt[:, :K].copy()
    prm = oracle.params_array(0.0, 0, 1.0, B=B)
    r = oracle.verify(zd, zt, oracle.FP32, K, prm, tokens=None, seed=1)
    assert (r.tokens == zd.argmax(axis=2)).all()
    assert (r.k == K).all()


# ------------------------------------------------------------------------------------------
# Status bits and near-tie flags
# ------------------------------------------------------------------------------------------
def test_status_and_flags():
    V, K = 4, 2
    zt = np.log(np.array([[0.25, 0.25, 0.25, 0.25], [0.4, 0.3, 0.2, 0.1], [0.1, 0.2, 0.3, 0.4]], np.float64))
    zd = np.log(np.array([[0.5, 0.2, 0.2, 0.1], [0.1, 0.2, 0.3, 0.4]], np.float64))
    prm = oracle.params_array(1.0, 0, 1.0, B=1)
    U = np.full((1, K + 1, 3), 0.5)
    # u * p(s0) = 0.5 * 0.5 = 0.25 = q(s0): a near tie of the acceptance test
    r = oracle.verify(zd[None].astype(np.float32), zt[None].astype(np.float32), oracle.FP32, K, prm,
                      tokens=[[0, 1]], U=U)
    assert r.flags[0] & oracle.FL_NEAR_ACCEPT
    # invalid token
    r = oracle.verify(zd[None].astype(np.float32), zt[None].astype(np.float32), oracle.FP32, K, prm,
                      tokens=[[0, 9]], U=U)
    assert r.status[0] & oracle.ST_BAD_TOKEN and r.k[0] == 0 and r.t[0] == -1
    # NaN logit
    zbad = zt.copy()
    zbad[1, 2] = np.nan
    r = oracle.verify(zd[None].astype(np.float32), zbad[None].astype(np.float32), oracle.FP32, K, prm,
                      tokens=[[0, 1]], U=U)
    assert r.status[0] & oracle.ST_BAD_LOGIT and r.t[0] == -1
    # token outside the draft's support (top-k 1 keeps token 0 only): accepted iff q(s) > 0
    prm1 = oracle.params_array(1.0, 1, 1.0, B=1)
    r = oracle.verify(zd[None].astype(np.float32), zt[None].astype(np.float32), oracle.FP32, K, prm1,
                      tokens=[[3, 1]], U=U)
    assert r.status[0] & oracle.ST_OUTSIDE_DRAFT_SUPPORT
    assert r.k[0] == 0   # q_0 under top-k 1 keeps token 0 only, so q(3) = 0
    # identical draft and target rows: never a rejection, bonus token from q_K
    r = oracle.verify(zt[None, :K].astype(np.float32), zt[None].astype(np.float32), oracle.FP32, K, prm,
                      tokens=[[0, 1]], U=np.full((1, K + 1, 3), 0.999))
    assert r.k[0] == K and r.W[0] == 0.0


# ------------------------------------------------------------------------------------------
# Theorem 12 fan-out
# ------------------------------------------------------------------------------------------
def test_fanout_golden_and_closed_form():
    g = json.load(open(os.path.join(GOLDEN, "fanout.json")))
    for c in g["cases"]:
        real, ints = oracle.fanout(c["K"], c["budget"], c["a"], c["r"])
        assert ints.tolist() == c["F_int"]
        assert abs(real.sum() - c["budget"]) < 1e-12
        assert ints.sum() == c["budget"]


@pytest.mark.parametrize("K,budget,a,r", [(5, 32, 0.7, 1.0), (4, 23, 0.6, 0.5), (7, 100, 0.85, 2.0), (3, 8, 0.3, 1.0)])
def test_fanout_is_the_optimum(K, budget, a, r):
    """F maximises sum_k P_k (1 - F_k^-r) under sum F_k = B, P_k = a^k (1-a) (k<K), a^K."""
    real, ints = oracle.fanout(K, budget, a, r)
    P = np.array([a ** k * (1 - a) for k in range(K)] + [a ** K])
    assert abs(P.sum() - 1.0) < 1e-12
    obj = lambda F: -np.sum(P * (1.0 - np.power(F, -r)))
    res = scipy.optimize.minimize(obj, np.full(K + 1, budget / (K + 1)), method="SLSQP",
                                  bounds=[(1e-6, budget)] * (K + 1),
                                  constraints=[{"type": "eq", "fun": lambda F: F.sum() - budget}],
                                  options={"ftol": 1e-14, "maxiter": 1000})
    assert res.success
    np.testing.assert_allclose(real, res.x, rtol=2e-4)
    assert obj(real) <= obj(res.x) + 1e-12
    assert ints.sum() == budget and np.all(np.abs(ints - real) < 1.0)


# ------------------------------------------------------------------------------------------
# Cache build / lookup / branch reuse
# ------------------------------------------------------------------------------------------
def test_cache_build_brute_force():
    rng = np.random.default_rng(9)
    B, K, V = 5, 3, 12
    draft = rng.integers(-2, 3, (B, K + 1, V)).astype(np.float32)  # many ties
    draft[0, 1, 4] = np.nan
    tok = rng.integers(0, V, (B, K)).astype(np.int32)
    fan = np.array([3, 2, 4, 5], np.int32)
    cache = oracle.cache_build(draft, oracle.FP32, K, tok, fan)
    for b in range(B):
        off = 0
        for k in range(K + 1):
            z = draft[b, k]
            order = sorted([i for i in range(V) if not np.isnan(z[i])], key=lambda i: (-z[i], i))
            order += [i for i in range(V) if np.isnan(z[i])]
            if k < K:
                order = [i for i in order if i != tok[b, k]]
            assert cache[b, off:off + fan[k]].tolist() == order[: fan[k]]
            off += fan[k]


def test_cache_lookup_definition():
    fan = np.array([2, 1, 3], np.int32)  # K = 2, budget 6
    cache = np.array([[10, 11, 20, 30, 31, 32], [5, 6, 7, 8, 9, 4]], np.int32)
    slot, hit, batch = oracle.cache_lookup(0, cache, fan, 2, 2, k=[2, 1], t=[31, 7])
    assert slot.tolist() == [4, 2] and hit.tolist() == [1, 1] and batch.tolist() == [2, 1]
    slot, hit, batch = oracle.cache_lookup(0, cache, fan, 2, 2, k=[0, 1], t=[20, 7])
    assert slot.tolist() == [-1, 2] and batch.tolist() == [1, 0]


def test_branch_reuse_definition():
    kappa, gamma = 3, 3
    br = np.array([[[1, 2, 3], [1, 5, 6], [1, 2, 9]],
                   [[4, 4, 4], [7, 7, 7], [4, 8, 8]]], np.int32)
    shape = np.array([kappa, gamma], np.int32)
    # request 0: chain 0 accepted 2 then correction 9 -> branch 2; request 1: k=1, t*=8 -> branch 2
    k = np.array([[2, 0, 0], [1, 0, 0]], np.int32)
    t = np.array([[9, 0, 0], [8, 0, 0]], np.int32)
    slot, hit, batch = oracle.cache_lookup(1, br, shape, 0, 2, k, t)
    assert slot.tolist() == [2, 2] and batch.tolist() == [2, 1]
    k[0, 0], t[0, 0] = 1, 7   # (1, 7) is no path
    k[1, 0] = gamma           # every token accepted: FULL
    slot, hit, batch = oracle.cache_lookup(1, br, shape, 0, 2, k, t)
    assert slot.tolist() == [-1, -2] and hit.tolist() == [0, 0]


def test_corollary16_whole_batch_hit():
    """Requests hit independently, so the all-hit frequency is the product of the hit rates."""
    rng = np.random.default_rng(12)
    B, K, V, R = 3, 2, 24, 3000
    zt = rng.normal(0, 1.5, (B, K + 1, V)).astype(np.float32)
    zd = np.concatenate([zt[:, :K] + rng.normal(0, 0.6, (B, K, V)), zt[:, K:] + rng.normal(0, 0.6, (B, 1, V))],
                        axis=1).astype(np.float32)
    fan = np.array([3, 2, 2], np.int32)
    prm = oracle.params_array(1.0, 0, 1.0, B=B)
    hits = np.zeros((R, B), bool)
    for rd in range(R):
        r = oracle.verify(zd[:, :K], zt, oracle.FP32, K, prm, F=2, C=0.3, tokens=None, seed=77, round_=rd)
        cache = oracle.cache_build(zd, oracle.FP32, K, r.tokens, fan)
        _, hit, batch = oracle.cache_lookup(0, cache, fan, K, B, r.k, r.t)
        hits[rd] = hit.astype(bool)
        assert batch[1] == int(hit.all())
    ph = hits.mean(axis=0)
    allhit = hits.all(axis=1).mean()
    se = np.sqrt(np.prod(ph) * (1 - np.prod(ph)) / R)
    assert abs(allhit - np.prod(ph)) < 5 * se + 1e-3


# ------------------------------------------------------------------------------------------
# Random-token backup speculation (SSD reading notes, section 7.1; hyper.ai summary, fallback)
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("V,K,T,top_k,top_p,seed", [
    (4, 1, 1.0, 0, 1.0, 0),
    (6, 2, 1.0, 0, 1.0, 1),
    (5, 2, 0.7, 3, 1.0, 2),
    (6, 2, 1.0, 0, 0.7, 3),
])
def test_uniform_draft_lossless_exact_enumeration(V, K, T, top_k, top_p, seed):
    # verifying uniform random tokens against the target leaves every emitted token with law q_j:
    # the lossless law of the speculative-sampling page with p = 1/V at every position
    rng = np.random.default_rng(900 + seed)
    zt = rng.normal(0, 1.5, (K + 1, V))
    zd = np.zeros((K, V))
    law, pp, q = exact_law(zd, zt, T, top_k, top_p, uniform=True)
    _check_lossless(law, pp, q, K, V)


def test_uniform_token_is_exact_floor_and_inverse_cdf():
    from fractions import Fraction
    U = oracle.uniforms(seed=77, round_=3, B=64, K=7)[:, :, 2].ravel()
    for V in (1, 2, 3, 7, 1000, 128256, 151936, (1 << 31) - 1):
        t = oracle.uniform_tokens(U, V)
        for u, ti in zip(U, t):
            fu = Fraction(float(u))          # the exact dyadic value of the uniform
            assert ti == (fu * V).numerator // (fu * V).denominator
            if V <= 1000:                    # inverse CDF of the uniform law by its definition
                assert ti == min(i for i in range(V) if Fraction(i + 1, V) > fu)


def test_uniform_tokens_are_uniform():
    V, n = 7, 70000
    U = oracle.uniforms(seed=5, round_=0, B=n // 7, K=6)[:, :, 2].ravel()[:n]
    counts = np.bincount(oracle.uniform_tokens(U, V), minlength=V)
    chi2 = ((counts - n / V) ** 2 / (n / V)).sum()
    assert chi2 < 22.46   # chi^2(6) at p = 0.001


def test_uniform_draft_acceptance_and_residual_definitions():
    # p'(s) = 1/V: accept iff u / V < q(s); the residual is (q - 1/V)+; sampled tokens are the
    # uniform draws of lane 2
    rng = np.random.default_rng(31)
    B, K, V = 40, 3, 50
    zt = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    prm = oracle.params_array(1.0, 0, 1.0, B=B)
    r = oracle.verify(None, zt, oracle.FP32, K, prm, tokens=None, seed=11, uniform_draft=True)
    U = oracle.uniforms(11, 0, B, K)
    assert (r.tokens == oracle.uniform_tokens(U[:, :K, 2], V)).all()
    for b in range(B):
        q = [oracle.process_row(zt[b, j].astype(np.float64))[0] for j in range(K + 1)]
        k = K
        for j in range(K):
            if not (U[b, j, 0] * (1.0 / V) < q[j][r.tokens[b, j]]):
                k = j
                break
        assert r.k[b] == k
        assert (r.status[b] & oracle.ST_OUTSIDE_DRAFT_SUPPORT) == 0
        if k < K:
            w = np.maximum(q[k] - 1.0 / V, 0.0)
            assert abs(r.W[b] - w.sum()) < 1e-12
            cum = np.cumsum(w)
            assert r.t[b] == int(np.argmax(cum > U[b, k, 1] * w.sum())) or r.flags[b] != 0


def test_backup_plan_switch():
    hit = np.array([1, 0, 1, 1, 0, 1], np.uint8)
    use, sw = oracle.backup_plan(6, hit, all_hit=0, b_star=4)
    assert sw == 1 and use.tolist() == [0, 1, 0, 0, 1, 0]
    use, sw = oracle.backup_plan(6, hit, all_hit=0, b_star=7)     # below b*: the primary drafter
    assert sw == 0 and use.tolist() == [0] * 6
    use, sw = oracle.backup_plan(6, np.ones(6, np.uint8), all_hit=1, b_star=1)   # every request hit
    assert sw == 0 and use.tolist() == [0] * 6


# ------------------------------------------------------------------------------------------
# Mirror-SD signposts: top-kappa of the early-exit distribution with log-probabilities
# ------------------------------------------------------------------------------------------
def _bf16(x):
    x = np.asarray(x, np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_signposts_brute_force_and_log_softmax():
    rng = np.random.default_rng(41)
    for trial in range(60):
        V = int(rng.integers(1, 40))
        B = 3
        z = np.round(rng.normal(0, 2, (B, V)) * 2) / 2          # many ties
        z[rng.random((B, V)) < 0.1] = -np.inf
        z[rng.random((B, V)) < 0.1] = -0.0
        z[:, 0] = np.where(np.isinf(z[:, 0]), 1.0, z[:, 0])       # at least one finite logit
        z = z.astype(np.float32)
        kappa = int(rng.integers(1, V + 3))
        for dtype, arr in ((oracle.FP32, z), (oracle.BF16, _bf16(z))):
            ids, lp, st = oracle.signposts(arr, dtype, kappa)
            zz = z if dtype == oracle.FP32 else (arr.astype(np.uint32) << 16).view(np.float32)
            assert (st == 0).all()
            for b in range(B):
                want = sorted(range(V), key=lambda i: (-float(zz[b, i]), i))[:kappa]
                assert ids[b, :len(want)].tolist() == want
                assert (ids[b, len(want):] == -1).all() and np.isneginf(lp[b, len(want):]).all()
                ref = scipy.special.log_softmax(zz[b].astype(np.float64))
                np.testing.assert_allclose(lp[b, :len(want)], ref[want], rtol=1e-12, atol=1e-12)


def test_signposts_special_rows():
    V = 1000
    ids, lp, st = oracle.signposts(np.full((1, V), 3.25, np.float32), oracle.FP32, 8)
    assert ids[0].tolist() == list(range(8))                   # a flat row: ties to the lower id
    np.testing.assert_allclose(lp[0], -np.log(V), rtol=1e-14)
    one = np.full((1, V), -np.inf, np.float32)
    one[0, 417] = -7.0
    ids, lp, st = oracle.signposts(one, oracle.FP32, 3)
    assert ids[0, 0] == 417 and lp[0, 0] == 0.0 and np.isneginf(lp[0, 1:]).all()
    full = np.random.default_rng(3).normal(0, 3, (2, 50)).astype(np.float32)
    ids, lp, st = oracle.signposts(full, oracle.FP32, 50)      # kappa = V: a distribution
    np.testing.assert_allclose(np.exp(lp).sum(axis=1), 1.0, rtol=1e-13)
    assert (np.diff(lp, axis=1) <= 0).all()
    shifted = (full + np.float32(16.0)).astype(np.float32)
    ids2, lp2, _ = oracle.signposts(shifted, oracle.FP32, 50)
    assert (ids2 == ids).all()
    np.testing.assert_allclose(lp2, lp, atol=1e-5)            # the shift rounds in fp32
    bad = np.zeros((3, 20), np.float32)
    bad[0, 5] = np.nan
    bad[1, 7] = np.inf
    bad[2, :] = -np.inf
    ids, lp, st = oracle.signposts(bad, oracle.FP32, 4)
    assert (st == oracle.ST_BAD_LOGIT).all() and (ids == -1).all() and np.isnan(lp).all()


# ------------------------------------------------------------------------------------------
# Mirror-SD reuse against a draft tree with internal branching
# ------------------------------------------------------------------------------------------
def _mirror_example_tree(ex, case, names):
    """Roots first, the verified branch under root 0, filler branches under the others, then
    the fork's extra children; returns (tokens, parents)."""
    gamma = len(ex["verified_path"])
    tok, par = [], []
    for r in ex["roots"]:
        tok.append(names[r]); par.append(-1)
    depth_node = {1: 0}
    prev = 0
    for d, name in enumerate(ex["verified_path"][1:], start=2):
        tok.append(names[name]); par.append(prev)
        prev = len(tok) - 1
        depth_node[d] = prev
    for r in range(1, len(ex["roots"])):
        prev = r
        for d in range(2, gamma + 1):
            tok.append(names[f"filler{r}_{d}"]); par.append(prev)
            prev = len(tok) - 1
    fork = depth_node[ex["fork_parent_depth"]]
    for name in case["fork_children"]:
        tok.append(names[name]); par.append(fork)
    return np.array(tok, np.int32), np.array(par, np.int32)


def test_tree_reuse_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "mirror_reuse_example.json")))
    labels = list(ex["roots"]) + list(ex["verified_path"]) + ["zhong1", "shang4"]
    labels += [f"filler{r}_{d}" for r in range(8) for d in range(2, 9)]
    names = {}
    for lab in labels:
        names.setdefault(lab, len(names))
    path = np.array([[names[x] for x in ex["verified_path"]]], np.int32)
    for case in ex["cases"]:
        tok, par = _mirror_example_tree(ex, case, names)
        node, hit, batch = oracle.tree_lookup(tok[None], par[None], path, [case["k"]], [names[case["t"]]])
        n = int(node[0])
        if case["expect"] == "full":
            assert n == -2 and hit[0] == 0, case["name"]
        elif case["expect"] == "miss":
            assert n == -1 and hit[0] == 0 and batch.tolist() == [0, 0], case["name"]
        else:
            assert n >= 0 and hit[0] == 1 and batch.tolist() == [1, 1], case["name"]
            assert tok[n] == names[case["t"]]
            d, cur = 0, n
            while cur != -1:
                d, cur = d + 1, par[cur]
            assert d == case["depth"], case["name"]


def _paths_top_down(tok, par):
    """Brute force: every root-to-node path, walking down from the roots over child lists."""
    N = len(tok)
    valid = [tok[n] >= 0 and -1 <= par[n] < n for n in range(N)]
    kids = {n: [] for n in range(-1, N)}
    for n in range(N):
        if valid[n]:
            kids[int(par[n])].append(n)
    best = {}
    stack = [(c, (int(tok[c]),)) for c in kids[-1]]
    while stack:
        n, p = stack.pop()
        best[p] = min(best.get(p, N), n)
        stack.extend((c, p + (int(tok[c]),)) for c in kids[n])
    return best


def test_tree_reuse_brute_force():
    rng = np.random.default_rng(17)
    gamma = 5
    for trial in range(200):
        N = int(rng.integers(1, 60))
        tok = rng.integers(0, 4, N).astype(np.int32)             # small alphabet: many equal paths
        par = np.array([int(rng.integers(-1, n)) if n else -1 for n in range(N)], np.int32)
        if trial % 3 == 0:                                       # padding and broken parents
            tok[rng.random(N) < 0.1] = -1
            par[rng.random(N) < 0.05] = N + 3
        best = _paths_top_down(tok, par)
        B = 8
        path = rng.integers(0, 4, (B, gamma)).astype(np.int32)
        k = rng.integers(0, gamma + 1, B).astype(np.int32)
        t = rng.integers(0, 4, B).astype(np.int32)
        if best:                                                 # steer some requests onto tree paths
            keys = list(best)
            for b in range(0, B, 2):
                p = keys[int(rng.integers(len(keys)))]
                if len(p) - 1 < gamma:
                    k[b] = len(p) - 1
                    path[b, :k[b]] = p[:-1]
                    t[b] = p[-1]
        node, hit, batch = oracle.tree_lookup(np.tile(tok, (B, 1)), np.tile(par, (B, 1)), path, k, t)
        for b in range(B):
            if k[b] == gamma:
                want = -2
            else:
                want = best.get(tuple(int(x) for x in path[b, :k[b]]) + (int(t[b]),), -1)
            assert node[b] == want, (trial, b)
        assert batch[0] == hit.sum() and batch[1] == int(hit.all())


def test_tree_reuse_on_a_comb_is_branch_reuse():
    # a tree without internal branching is the branch-complete comb: node // gamma is the branch
    rng = np.random.default_rng(23)
    B, kappa, gamma = 30, 8, 7
    br = rng.integers(0, 3, (B, kappa, gamma)).astype(np.int32)
    k = np.zeros((B, kappa), np.int32)
    t = np.zeros((B, kappa), np.int32)
    k[:, 0] = rng.integers(0, gamma + 1, B)
    t[:, 0] = rng.integers(0, 3, B)
    slot, hit, batch = oracle.cache_lookup(1, br, [kappa, gamma], 0, B, k, t)
    tok = br.reshape(B, kappa * gamma)
    par = np.tile(np.array([-1 if d == 0 else j * gamma + d - 1 for j in range(kappa) for d in range(gamma)],
                           np.int32), (B, 1))
    node, hit2, batch2 = oracle.tree_lookup(tok, par, br[:, 0], k[:, 0], t[:, 0])
    assert (np.where(node >= 0, node // gamma, node) == slot).all()
    assert (hit2 == hit).all() and (batch2 == batch).all()



# ------------------------------------------------------------------------------------------
# PyramidSD fuzzy acceptance (Jensen-Shannon divergence in bits against a threshold)
# ------------------------------------------------------------------------------------------
import scipy.spatial.distance


def test_jsd_matches_scipy():
    rng = np.random.default_rng(8)
    for trial in range(200):
        V = int(rng.integers(1, 30))
        p = rng.random(V) * (rng.random(V) < 0.7)
        q = rng.random(V) * (rng.random(V) < 0.7)
        if p.sum() == 0:
            p[0] = 1.0
        if q.sum() == 0:
            q[-1] = 1.0
        p /= p.sum()
        q /= q.sum()
        ref = scipy.spatial.distance.jensenshannon(p, q, base=2) ** 2   # scipy gives the distance
        d = oracle.jsd_bits(p, q)
        assert abs(d - ref) <= 1e-12 and abs(oracle.jsd_bits(q, p) - d) <= 1e-15
        assert -1e-15 <= d <= 1.0 + 1e-15
    assert oracle.jsd_bits([1.0, 0.0], [0.0, 1.0]) == 1.0            # disjoint supports
    assert oracle.jsd_bits([0.3, 0.7], [0.3, 0.7]) == 0.0            # identical


def _fuzzy_inputs(rng, B, K, V):
    zt = rng.normal(0, 1.5, (B, K + 1, V)).astype(np.float32)
    zd = (zt[:, :K] + rng.normal(0, 1.0, (B, K, V))).astype(np.float32)
    return zd, zt


def test_fuzzy_divergences_and_extremes():
    rng = np.random.default_rng(12)
    B, K, V = 30, 3, 40
    zd, zt = _fuzzy_inputs(rng, B, K, V)
    T = rng.choice([0.0, 0.7, 1.0], B).astype(np.float32)
    tk = rng.choice([0, 5], B).astype(np.int32)
    tp = rng.choice([0.8, 1.0], B).astype(np.float32)
    prm = oracle.params_array(T, tk, tp)
    tok = rng.integers(0, V, (B, K))
    base = oracle.verify(zd, zt, oracle.FP32, K, prm, F=2, C=0.5, tokens=tok, seed=3)
    # divergences: the Jensen-Shannon divergence of the processed rows (scipy)
    r = oracle.verify(zd, zt, oracle.FP32, K, prm, F=2, C=0.5, tokens=tok, seed=3, tau=np.full(B, -1.0))
    for b in range(B):
        for j in range(K):
            zz = zd[b, j].astype(np.float64)
            pj = oracle.process_row(zz, float(T[b]), int(tk[b]), float(tp[b]))[0]
            pj = oracle.downweight_probs(zz, pj, 2, 0.5)[0] if T[b] > 0 else pj
            qj = oracle.process_row(zt[b, j].astype(np.float64), float(T[b]), int(tk[b]), float(tp[b]))[0]
            ref = scipy.spatial.distance.jensenshannon(pj, qj, base=2) ** 2
            assert abs(r.div[b, j] - ref) <= 1e-12, (b, j)
    # a threshold below every divergence is the lossless rule
    assert (r.k == base.k).all() and (r.t == base.t).all() and (r.status == base.status).all()
    # the divergence never exceeds 1 bit: tau = 1 passes every drafted token
    full = oracle.verify(zd, zt, oracle.FP32, K, prm, F=2, C=0.5, tokens=tok, seed=3, tau=np.ones(B))
    assert (full.k == K).all()
    # more tolerance never shortens the accepted run (same uniforms)
    mid = oracle.verify(zd, zt, oracle.FP32, K, prm, F=2, C=0.5, tokens=tok, seed=3, tau=np.median(r.div, axis=1))
    assert (mid.k >= base.k).all() and (mid.k <= full.k).all()


def _fuzzy_law_closed_form(pp, q, tau_pass, assisted):
    """Law of (k, emitted tokens) from the rule: a position whose divergence passes keeps its
    drafted token; elsewhere s is kept with probability min(1, q/p), and a rejection emits
    the residual (q - p)+ (or, assisted, beta q with beta the rejection probability)."""
    K = len(pp)
    law = {}

    def walk(j, prefix, prob):
        if prob == 0.0:
            return
        if j == K:
            for y in range(len(q[K])):
                key = (K,) + prefix + (y,)
                law[key] = law.get(key, 0.0) + prob * q[K][y]
            return
        p_j, q_j = pp[j], q[j]
        if tau_pass[j]:
            for x in range(len(p_j)):
                walk(j + 1, prefix + (x,), prob * p_j[x])
            return
        for x in range(len(p_j)):
            walk(j + 1, prefix + (x,), prob * min(p_j[x], q_j[x]))
        beta = float(np.maximum(p_j - q_j, 0.0).sum())
        corr = q_j * beta if assisted else np.maximum(q_j - p_j, 0.0)
        for y in range(len(q_j)):
            key = (j,) + prefix + (y,)
            law[key] = law.get(key, 0.0) + prob * corr[y]

    walk(0, (), 1.0)
    return law


@pytest.mark.parametrize("assisted", [False, True])
def test_fuzzy_law_exact_enumeration(assisted):
    rng = np.random.default_rng(21 + assisted)
    K, V = 2, 3
    zd = rng.normal(0, 1.2, (K, V))
    zt = rng.normal(0, 1.2, (K + 1, V))
    pp = [oracle.process_row(zd[j].astype(np.float32).astype(np.float64), 1.0, 0, 1.0)[0] for j in range(K)]
    q = [oracle.process_row(zt[j].astype(np.float32).astype(np.float64), 1.0, 0, 1.0)[0] for j in range(K + 1)]
    div = [scipy.spatial.distance.jensenshannon(pp[j], q[j], base=2) ** 2 for j in range(K)]
    tau = 0.5 * (div[0] + div[1])            # one position passes, the other is tested
    law, _, _ = exact_law(zd, zt, tau=tau, assisted=assisted)
    want = _fuzzy_law_closed_form(pp, q, [d <= tau for d in div], assisted)
    keys = set(law) | set(want)
    assert max(abs(law.get(x, 0.0) - want.get(x, 0.0)) for x in keys) < 1e-9
    assert abs(sum(law.values()) - 1.0) < 1e-9


# ------------------------------------------------------------------------------------------
# The uniforms' counter layout, the near-tie predicates and the readings for degenerate
# inputs, each against values worked out by hand from their definitions
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("seed,round_,B,K", [
    (0xC0FFEE03, 0, 5, 4),
    (0x5EED0001, 17, 3, 6),
    ((1 << 64) - 3, (1 << 40) + 5, 2, 2),
])
def test_uniforms_counter_layout_against_numpy_philox(seed, round_, B, K):
    """U[b, j, w] is word w of Philox4x64-10 with counter (round, b, j, 0) and key (seed, 0),
    mapped to ((w >> 12) + 1/2) 2^-52; numpy's generator supplies the words."""
    U = oracle.uniforms(seed, round_, B, K)
    for b in range(B):
        for j in range(K + 1):
            words = _numpy_philox_block([round_, b, j, 0], [seed, 0])
            for lane in range(3):
                expect = (float(int(words[lane]) >> 12) + 0.5) * 2.0 ** -52
                assert U[b, j, lane] == expect, (b, j, lane)


def test_near_nucleus_flag_band():
    """The nucleus flag is raised exactly when the cut's running mass lies within 1e-9 of the
    total of top_p * S, on either side of the token that reaches it."""
    # four equal masses: two tokens reach top_p * S = 2 exactly
    _, _, near, n = oracle.process_row(np.zeros(4), 1.0, 0, 0.5)
    assert near and n == 2
    # the next float32 above 0.5: the target lies 2^-22 past the second breakpoint
    tp = float(np.nextafter(np.float32(0.5), np.float32(1.0)))
    _, _, near, n = oracle.process_row(np.zeros(4), 1.0, 0, tp)
    assert not near and n == 3
    # above the target: the first token heavier by d, masses (1, e^-d, e^-d, e^-d); the two
    # leading tokens overshoot top_p * S by d/2 (in units of the leading mass)
    for d, flagged in ((2e-10, True), (2e-8, False)):
        z = np.array([np.log1p(d), 0.0, 0.0, 0.0])
        _, _, near, n = oracle.process_row(z, 1.0, 0, 0.5)
        assert n == 2 and near == flagged, (d, near, n)
    # below the target: masses (1, 1/2 + d, 1/2); one token falls short of top_p * S by d/2
    for d, flagged in ((2e-10, True), (2e-8, False)):
        z = np.array([np.log(2.0), np.log1p(2 * d), 0.0])
        _, _, near, n = oracle.process_row(z, 1.0, 0, 0.5)
        assert n == 2 and near == flagged, (d, near, n)


def _bonus_draw(v):
    """K = 1, V = 4, draft row = target row = four equal logits, drafted token 0 (accepted for
    any u < 1): the bonus token is the inverse CDF of q_1 = (1/4, 1/4, 1/4, 1/4) at v."""
    z = np.zeros((1, 2, 4), np.float32)
    U = np.full((1, 2, 3), 0.5)
    U[0, 1, 1] = v
    return oracle.verify(z[:, :1], z, oracle.FP32, 1, oracle.params_array(1.0, 0, 1.0, B=1), tokens=[[0]], U=U)


def test_near_cdf_flag_band():
    # v W lands exactly on the breakpoint after token 1: the draw is token 2, flagged
    r = _bonus_draw(0.5)
    assert r.k[0] == 1 and r.t[0] == 2 and r.flags[0] & oracle.FL_NEAR_CDF
    r = _bonus_draw(0.5 + 2e-10)
    assert r.t[0] == 2 and r.flags[0] & oracle.FL_NEAR_CDF
    # outside the 1e-9 band on either side: no flag, the draws on both sides of the breakpoint
    r = _bonus_draw(0.5 + 5e-9)
    assert r.t[0] == 2 and not r.flags[0] & oracle.FL_NEAR_CDF
    r = _bonus_draw(0.5 - 5e-9)
    assert r.t[0] == 1 and not r.flags[0] & oracle.FL_NEAR_CDF


def test_empty_residual_draws_from_the_target():
    """Reading R7: a rejection whose residual (q - p')+ is empty draws t* from q_k itself.  Draft
    and target rows agree (top-k 2 keeps q = p = (0.6, 0.4, 0, 0)); the drafted token 2 lies
    outside both supports, so u p(2) < q(2) fails (reading R8) and W = 0."""
    z = np.log(np.array([0.6, 0.4, 0.05, 0.05], np.float64)).astype(np.float32)
    rows = np.stack([z, z])[None]
    prm = oracle.params_array(1.0, 2, 1.0, B=1)
    for v, t in ((0.3, 0), (0.7, 1)):
        U = np.full((1, 2, 3), 0.5)
        U[0, 0, 1] = v
        r = oracle.verify(rows[:, :1], rows, oracle.FP32, 1, prm, tokens=[[2]], U=U)
        assert r.k[0] == 0 and r.t[0] == t and r.W[0] == 0.0
        assert r.status[0] == oracle.ST_EMPTY_RESIDUAL | oracle.ST_OUTSIDE_DRAFT_SUPPORT


def test_bad_parameters_reject_the_request():
    """Reading R20: a negative, infinite or NaN temperature, or top_p <= 0, yields k = 0,
    t* = -1 and the bad-parameter status alone; the other requests of the batch are unaffected."""
    rng = np.random.default_rng(5)
    B, K, V = 7, 2, 16
    zt = rng.normal(0, 1, (B, K + 1, V)).astype(np.float32)
    zd = zt[:, :K] + rng.normal(0, 0.3, (B, K, V)).astype(np.float32)
    T = np.array([-1.0, np.nan, np.inf, 1.0, 1.0, 1.0, 0.0], np.float32)
    tp = np.array([1.0, 1.0, 1.0, 0.0, -0.5, 0.9, 1.0], np.float32)
    prm = oracle.params_array(T, 0, tp)
    r = oracle.verify(zd, zt, oracle.FP32, K, prm, tokens=np.zeros((B, K), np.int32), seed=3)
    for b in range(5):
        assert r.status[b] == oracle.ST_BAD_PARAM and r.k[b] == 0 and r.t[b] == -1
    for b in (5, 6):
        assert not r.status[b] & oracle.ST_BAD_PARAM and r.t[b] >= 0
        one = oracle.verify(zd[b:b + 1], zt[b:b + 1], oracle.FP32, K, prm[b:b + 1],
                            tokens=np.zeros((1, K), np.int32), U=oracle.uniforms(3, 0, B, K)[b:b + 1])
        assert (one.k[0], one.t[0], one.status[0]) == (r.k[b], r.t[b], r.status[b])


def test_degenerate_downweight_leaves_the_row():
    """Reading R21: with C = 0 and the downweighted set holding every token with mass, the
    normaliser 1 - (1 - C) P_S is 0; the row is verified undownweighted, with its status bit.
    Draft p = (0.6, 0.4, 0, 0), target q = (0.3, 0.7, 0, 0) under top-k 2; drafted token 0."""
    zd = np.log(np.array([0.6, 0.4, 0.05, 0.05]))
    zt = np.log(np.array([0.3, 0.7, 0.05, 0.05]))
    p, _, _, _ = oracle.process_row(zd, 1.0, 2, 1.0)
    pp, Z, ids, deg = oracle.downweight_probs(zd, p, 4, 0.0)
    assert deg and Z == 1.0 and list(ids[:2]) == [0, 1] and (pp == p).all()
    # a proper set (F = 1): p' = (0, 1, 0, 0)
    pp1, Z1, ids1, deg1 = oracle.downweight_probs(zd, p, 1, 0.0)
    assert not deg1 and ids1[0] == 0 and abs(Z1 - 0.4) < 1e-15 and pp1[0] == 0.0 and abs(pp1[1] - 1.0) < 1e-15
    draft = np.stack([zd, zd])[None].astype(np.float32)
    target = np.stack([zt, zt])[None].astype(np.float32)
    prm = oracle.params_array(1.0, 2, 1.0, B=1)
    for u, acc in ((0.45, True), (0.55, False)):  # accept iff u p(0) < q(0): u < 0.3 / 0.6
        U = np.full((1, 2, 3), 0.5)
        U[0, 0, 0] = u
        r = oracle.verify(draft[:, :1], target, oracle.FP32, 1, prm, F=4, C=0.0, tokens=[[0]], U=U)
        assert r.status[0] & oracle.ST_DEGENERATE_DOWNWEIGHT
        if acc:
            assert r.k[0] == 1
        else:  # residual (q - p)+ = (0, 0.3): W = 0.3 and t* = 1 whatever v is
            assert r.k[0] == 0 and r.t[0] == 1 and abs(r.W[0] - 0.3) < 1e-6  # float32 logits
    # with F = 1 the drafted token has p'(0) = 0 and q(0) > 0: accepted for every u (reading R8)
    U = np.full((1, 2, 3), 0.99)
    r = oracle.verify(draft[:, :1], target, oracle.FP32, 1, prm, F=1, C=0.0, tokens=[[0]], U=U)
    assert r.k[0] == 1 and r.status[0] == oracle.ST_OUTSIDE_DRAFT_SUPPORT
