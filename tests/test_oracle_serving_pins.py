"""Pins of the decode-serving helpers of the oracle (running V mean, fitted
thresholds) against facts fixed outside them: the plain mean over the whole
cache, data that lie exactly on the fitted family, and an independent least
squares solve (numpy.linalg.lstsq on the Vandermonde matrix)."""
import math

import numpy as np
import pytest

from oracle import serving


def test_running_mean_append_equals_mean_of_the_cache():
    rng = np.random.default_rng(0)
    V = rng.standard_normal((1000, 16))
    mu = None
    n = 0
    for m in [1, 7, 0, 200, 31, 761]:
        mu = serving.running_mean_append(mu, n, V[n:n + m]) if n + m > 0 else mu
        n += m
        np.testing.assert_allclose(mu, V[:n].mean(axis=0), rtol=1e-12, atol=1e-14)


def test_running_mean_closed_form():
    # mean of rows [2, 4] is [3]; append [6] and [9]: mean of 2, 4, 6, 9 is 21/4
    mu = serving.running_mean_append(None, 0, [[2.0], [4.0]])
    assert mu[0] == 3.0
    mu = serving.running_mean_append(mu, 2, [[6.0], [9.0]])
    assert mu[0] == pytest.approx(21 / 4, abs=1e-15)
    with pytest.raises(ValueError):
        serving.running_mean_append(None, 0, np.zeros((0, 3)))


def test_fit_recovers_a_power_law_exactly():
    """Post-softmax thresholds that fall as c * (p + 1)^-b are a line in
    ln(p + 1) after the log: the degree-1 fit recovers -b and ln c exactly and
    extrapolates them to any row."""
    R = 600
    p = np.arange(R)
    th = np.stack([0.7 * (p + 1.0) ** -0.9, 2.0 * (p + 1.0) ** -1.2])
    obs = np.zeros_like(th, dtype=bool)
    obs[:, [40, 90, 200, 350]] = True
    coef = serving.fit_theta(th, obs, 1, True)
    np.testing.assert_allclose(coef[:, 0], [-0.9, -1.2], rtol=1e-12)
    np.testing.assert_allclose(coef[:, 1], [math.log(0.7), math.log(2.0)], rtol=1e-12)
    out = serving.eval_theta(coef, 32, 40000, True)
    assert np.isneginf(out[:, :32]).all()
    q = np.arange(32, 40000)
    np.testing.assert_allclose(out[0, 32:], 0.7 * (q + 1.0) ** -0.9, rtol=1e-10)


def test_fit_recovers_a_quadratic_in_log_rows():
    """Pre-softmax thresholds (scores) exactly quadratic in ln(p + 1)."""
    x = np.log(np.arange(300) + 1.0)
    th = (0.5 + 0.3 * x - 0.01 * x * x)[None, :]
    obs = np.zeros_like(th, dtype=bool)
    obs[0, ::17] = True
    coef = serving.fit_theta(th, obs, 2, False)
    np.testing.assert_allclose(coef[0], [-0.01, 0.3, 0.5], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(serving.eval_theta(coef, 0, 300, False)[0], th[0], rtol=1e-12)


def test_fit_is_the_least_squares_solution():
    """Noisy rows: the coefficients equal numpy.linalg.lstsq on the Vandermonde
    matrix of ln(p + 1) (a second, independent least-squares routine)."""
    rng = np.random.default_rng(3)
    R = 2048
    th = np.exp(-1.0 * np.log(np.arange(R) + 1.0) + 0.05 * rng.standard_normal(R))[None, :]
    obs = np.zeros_like(th, dtype=bool)
    obs[0, rng.choice(R, 50, replace=False)] = True
    obs[0, :5] = False
    coef = serving.fit_theta(th, obs, 2, True)
    x = np.log(np.flatnonzero(obs[0]) + 1.0)
    A = np.stack([x * x, x, np.ones_like(x)], axis=1)
    want, *_ = np.linalg.lstsq(A, np.log(th[0, obs[0]]), rcond=None)
    np.testing.assert_allclose(coef[0], want, rtol=1e-9, atol=1e-12)


def test_fit_from_a_minimum_row_ignores_the_short_rows():
    """Rows below min_row are left out: thresholds on a power law from row 255
    on but corrupted below it give back the exact power law, while a fit over
    every row does not."""
    R = 3000
    p = np.arange(R)
    th = (0.5 * (p + 1.0) ** -1.1)[None, :]
    th[0, :255] = 0.001 * (p[:255] + 1.0) ** 0.7          # rising near p + 1 = k
    obs = np.zeros_like(th, dtype=bool)
    obs[0, ::37] = True
    coef = serving.fit_theta(th, obs, 1, True, min_row=255)
    np.testing.assert_allclose(coef[0], [-1.1, math.log(0.5)], rtol=1e-12)
    assert abs(serving.fit_theta(th, obs, 1, True)[0, 0] + 1.1) > 0.1


def test_fit_needs_enough_rows_and_skips_unusable_ones():
    th = np.full((3, 50), 0.1)
    obs = np.zeros_like(th, dtype=bool)
    obs[0, [10, 20]] = True          # two rows: a line fits, a quadratic does not
    obs[1, [10, 20, 30]] = True
    th[1, 30] = -1.0                 # not usable in the log domain
    obs[2, [5, 6, 7]] = True
    assert np.isfinite(serving.fit_theta(th, obs, 1, True)[0]).all()
    assert np.isnan(serving.fit_theta(th, obs, 2, True)[0]).all()
    assert np.isnan(serving.fit_theta(th, obs, 2, True)[1]).all()
    assert np.isfinite(serving.fit_theta(th, obs, 2, False)[1]).all()
    assert np.isfinite(serving.fit_theta(th, obs, 2, True)[2]).all()


# ----------------------------------------------------- GQA selection variants
def _gqa_case(seed, B=2, Hq=8, Hkv=2, n=40, d=6):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, d))
    K = rng.standard_normal((B, Hkv, n, d)) * 1.5
    V = rng.standard_normal((B, Hkv, n, d))
    theta = np.full((Hq, n), 0.03)
    vm = V.mean(axis=2)
    return q, K, V, [n, n - 13], theta, vm


def test_gqa_default_is_plain_decode():
    import oracle
    q, K, V, lens, th, vm = _gqa_case(1)
    a = serving.decode_gqa(q, K, V, lens, th, vm, 0.5, vmc=True)
    b = oracle.decode(q, K, V, lens, th, vm, 0.5, vmc=True)
    np.testing.assert_allclose(a.out, b.out, rtol=1e-13, atol=1e-15)
    assert (a.kept_count == b.kept_count).all() and (a.vrows_read == b.vrows_read).all()


def test_gqa_loaded_sets_by_subset_enumeration():
    """The loaded set for min_votes = m is the union, over every m-subset of the
    group's heads, of the keys all heads of the subset keep (itertools);
    m = 1 is the union, m = g the intersection (Python sets)."""
    import itertools
    import oracle
    q, K, V, lens, th, vm = _gqa_case(2)
    g = 4
    base = oracle.decode(q, K, V, lens, th, vm, 0.5, vmc=False)
    for m in range(1, g + 2):
        r = serving.decode_gqa(q, K, V, lens, th, vm, 0.5, vmc=False, min_votes=m, augment=True)
        for b in range(2):
            for kv in range(2):
                sets = [set(np.flatnonzero(base.keep[b][h]).tolist()) for h in range(kv * g, (kv + 1) * g)]
                want = set()
                for sub in itertools.combinations(range(g), m):
                    want |= set.intersection(*[sets[i] for i in sub])
                assert r.vrows_read[b, kv] == len(want)
                for h in range(kv * g, (kv + 1) * g):
                    assert set(np.flatnonzero(r.keep[b][h]).tolist()) == want
                if m == 1:
                    assert want == set.union(*sets)
                if m == g:
                    assert want == set.intersection(*sets)


def test_gqa_discard_keeps_own_keys_inside_the_loaded_set():
    import oracle
    q, K, V, lens, th, vm = _gqa_case(3)
    base = oracle.decode(q, K, V, lens, th, vm, 0.5, vmc=True)
    r = serving.decode_gqa(q, K, V, lens, th, vm, 0.5, vmc=True, min_votes=2)
    for b in range(2):
        for h in range(8):
            assert not (r.keep[b][h] & ~base.keep[b][h]).any()
            s = base.s[b][h]
            w = np.where(r.keep[b][h], s, 0.0)
            mu = vm[b, h // 4]
            np.testing.assert_allclose(r.out[b, h], w @ V[b, h // 4, :lens[b]] + (1 - w.sum()) * mu,
                                       rtol=1e-12, atol=1e-14)
