"""Pins of the pre-softmax oracle (scores thresholded before softmax, with the
three estimates of the discarded softmax mass) against facts fixed outside it.

Each test checks ``oracle.presoftmax`` against hand-derived closed forms
(``tests/golden/topth_presoftmax_closed_form.json``), library routines the
oracle does not call (torch SDPA, SciPy softmax / logsumexp, NumPy
argpartition), brute force on tiny inputs, or identities of "Top-Theta
Attention: Sparsifying Transformers by Compensated Thresholding" (Eq. 4-7).
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import presoftmax as pre

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "topth_presoftmax_closed_form.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _val(x):
    """'-inf', 'lnX' (natural log of X), 'lnX/2', or a rational 'p/q'."""
    if x == "-inf":
        return -math.inf
    if isinstance(x, str) and x.startswith("ln"):
        body = x[2:]
        if body.endswith("/2"):
            return math.log(float(body[:-2])) / 2
        return math.log(float(body))
    return float(Fraction(x)) if isinstance(x, str) else float(x)


def _rand(rng, B, Hq, Hkv, L, d):
    q = rng.standard_normal((B, Hq, L, d))
    k = rng.standard_normal((B, Hkv, L, d)) * np.exp(0.5 * rng.standard_normal((B, Hkv, L, 1)))
    v = rng.standard_normal((B, Hkv, L, d))
    return q, k, v


# ---------------------------------------------------------------- closed forms
def test_golden_rows():
    g = _golden()["row_cases"]
    K = np.array([[math.log(c), g["k_second_column"]] for c in g["k_rows_log_of"]])
    a = oracle.scores(g["q"], K, g["scale"])
    for c in g["cases"]:
        r = pre.pre_row(a, g["v"], _val(c["theta"]), g["mu"], sdc=c["sdc"], vmc=c["vmc"],
                        gamma=g["gamma"], e_tilde=c["e_tilde"])
        assert r.keep.tolist() == c["keep"], c
        assert r.kept_count == c["kept"]
        assert r.beta == pytest.approx(_val(c["beta"]), abs=1e-12), c
        np.testing.assert_allclose(r.out, [_val(x) for x in c["out"]], rtol=1e-12, atol=1e-12)


def test_golden_calibration():
    g = _golden()["calibration_case"]
    cal = pre.PreCalibrator(g["ks"], 1, 4)
    for rows in g["sequences_k_rows_log_of"]:
        K = np.array([[[math.log(c), g["k_second_column"]] for c in rows]])
        Q = np.array([[g["q"]]])
        cal.observe(Q, K, g["scale"], q_pos0=3)
    th = cal.finalize()
    et = cal.finalize_etilde()
    for ki in range(len(g["ks"])):
        want = _val(g["theta_alpha0"][ki])
        if math.isinf(want):
            assert th[ki, 0, 3] == -np.inf
        else:
            assert th[ki, 0, 3] == pytest.approx(want, abs=1e-12)
        assert et[ki, 0, 3] == pytest.approx(_val(g["etilde"][ki]), abs=1e-12)
    assert cal.finalize(alpha=1.0)[1, 0, 3] == pytest.approx(_val(g["theta_alpha1_k2"]), abs=1e-12)
    # k = 2: rows 0, 1 keep all (theta -inf, E~ 0); row 2 copies the observed row 3
    assert np.isneginf(th[1, 0, :2]).all() and (et[1, 0, :2] == 0).all()
    assert th[1, 0, 2] == th[1, 0, 3] and et[1, 0, 2] == et[1, 0, 3]


# ------------------------------------------------------- dense and library pins
@pytest.mark.parametrize("sdc", ["exact", "expth", "none"])
def test_theta_minus_inf_is_dense_attention(sdc):
    """theta = -inf keeps every element; exact, exp-threshold (n - k~ = 0) and
    uncompensated SDC then all reduce to dense causal attention (torch SDPA)."""
    rng = np.random.default_rng(1)
    B, Hq, Hkv, L, d = 1, 4, 2, 9, 8
    q, k, v = _rand(rng, B, Hq, Hkv, L, d)
    theta = np.full((Hq, L), -np.inf)
    r = pre.prefill_pre(q, k, v, theta, 1 / math.sqrt(d), sdc=sdc, vmc=True)
    g = Hq // Hkv
    kk = torch.tensor(np.repeat(k, g, axis=1))
    vv = torch.tensor(np.repeat(v, g, axis=1))
    ref = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q), kk, vv, is_causal=True).numpy()
    np.testing.assert_allclose(r.out, ref, rtol=1e-12, atol=1e-12)
    assert (r.beta == 0).all()


def test_exact_sdc_weights_are_post_softmax_values():
    """Eq. 4: softmax(a~) * R / (R + E) equals softmax(a) on the kept set."""
    rng = np.random.default_rng(2)
    for _ in range(20):
        a = rng.standard_normal(40) * 2
        theta = float(np.quantile(a, 0.7))
        keep, w, beta = pre.pre_weights(a, theta, sdc="exact")
        s = scipy.special.softmax(a)
        np.testing.assert_allclose(w[keep], s[keep], rtol=1e-13)
        assert (w[~keep] == 0).all()
        assert beta == pytest.approx(s[~keep].sum(), abs=1e-13)


def test_none_is_softmax_over_kept_scores():
    rng = np.random.default_rng(3)
    a = rng.standard_normal(30)
    theta = float(np.quantile(a, 0.5))
    keep, w, beta = pre.pre_weights(a, theta, sdc="none")
    np.testing.assert_allclose(w[keep], scipy.special.softmax(a[keep]), rtol=1e-13)
    assert beta == 0.0


def test_expth_closed_form_and_shift_invariance():
    """E~ = gamma (n - k~) exp(theta - max): weights = exp(a - max) / (R + E~).
    Shifting every score and theta by one constant leaves the result unchanged
    (the estimate is taken in the same frame as R)."""
    rng = np.random.default_rng(4)
    a = rng.standard_normal(25)
    theta = float(np.sort(a)[-6])
    gamma = 0.05
    keep, w, beta = pre.pre_weights(a, theta, sdc="expth", gamma=gamma)
    m = a.max()
    R = np.exp(a[keep] - m).sum()
    Et = gamma * (a.size - keep.sum()) * np.exp(theta - m)
    np.testing.assert_allclose(w[keep], np.exp(a[keep] - m) / (R + Et), rtol=1e-13)
    assert beta == pytest.approx(Et / (R + Et), rel=1e-12)
    k2, w2, b2 = pre.pre_weights(a + 37.5, theta + 37.5, sdc="expth", gamma=gamma)
    assert (k2 == keep).all()
    np.testing.assert_allclose(w2, w, rtol=1e-12, atol=1e-15)
    assert b2 == pytest.approx(beta, rel=1e-12)


def test_theta_at_kth_score_is_brute_force_topk():
    """theta equal to the row's exact k-th largest score keeps exactly the top k."""
    rng = np.random.default_rng(5)
    for n, k in [(10, 3), (33, 7), (64, 1), (5, 5)]:
        a = rng.standard_normal(n)
        theta = oracle.kth_largest(a, k)
        keep, _, _ = pre.pre_weights(a, theta, sdc="exact")
        top = set(np.argpartition(-a, k - 1)[:k].tolist())
        assert set(np.flatnonzero(keep).tolist()) == top


def test_pre_and_post_thresholds_select_the_same_set():
    """softmax is monotone: keeping a >= a_(k) is keeping s >= s_(k), and the
    exact-SDC outputs of the two oracle paths agree."""
    rng = np.random.default_rng(6)
    d = 6
    for n, k in [(12, 4), (30, 10)]:
        q = rng.standard_normal(d)
        K = rng.standard_normal((n, d))
        V = rng.standard_normal((n, d))
        mu = V.mean(0)
        a = oracle.scores(q, K, 0.4)
        s = scipy.special.softmax(a)
        r_pre = pre.pre_row(a, V, oracle.kth_largest(a, k), mu, sdc="exact", vmc=True)
        r_post = oracle.topth_row(a, V, oracle.kth_largest(s, k), mu, vmc=True)
        assert (r_pre.keep == r_post.keep).all()
        np.testing.assert_allclose(r_pre.out, r_post.out, rtol=1e-12, atol=1e-14)
        assert r_pre.beta == pytest.approx(r_post.beta, abs=1e-13)


@pytest.mark.parametrize("sdc", ["exact", "expth", "offline"])
def test_identical_v_rows_give_that_row(sdc):
    """VMC: the kept weights and beta sum to one, so identical V rows give that
    row for any threshold (mu is then the same row)."""
    rng = np.random.default_rng(7)
    n, d = 20, 5
    a = rng.standard_normal(n)
    row = rng.standard_normal(d)
    V = np.tile(row, (n, 1))
    for theta in [-np.inf, float(np.median(a)), float(a.max())]:
        r = pre.pre_row(a, V, theta, row, sdc=sdc, vmc=True, e_tilde=0.3)
        np.testing.assert_allclose(r.out, row, rtol=1e-12)
        assert r.weights.sum() + r.beta == pytest.approx(1.0, abs=1e-13)


def test_monotone_in_theta():
    rng = np.random.default_rng(8)
    a = rng.standard_normal(50)
    ths = np.sort(rng.standard_normal(12))
    prev = None
    for t in ths:
        keep, _, _ = pre.pre_weights(a, float(t), sdc="none")
        if prev is not None:
            assert not (keep & ~prev).any()
        prev = keep


def test_decode_equals_prefill_row_and_union():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, L, d = 2, 4, 2, 11, 8
    q, k, v = _rand(rng, B, Hq, Hkv, L, d)
    theta = rng.standard_normal((Hq, L)) * 0.3 + 0.4
    et = np.abs(rng.standard_normal((Hq, L)))
    lens = [L, 6]
    scale = 1 / math.sqrt(d)
    vm = np.stack([[v[b, h, :lens[b]].mean(0) for h in range(Hkv)] for b in range(B)])
    dec = pre.decode_pre(np.stack([q[b, :, lens[b] - 1] for b in range(B)]), k, v, lens,
                         theta, vm, scale, sdc="offline", vmc=True, e_tilde=et)
    pf = pre.prefill_pre(q, k, v, theta, scale, sdc="offline", vmc=True, e_tilde=et)
    g = Hq // Hkv
    for b in range(B):
        p = lens[b] - 1
        np.testing.assert_allclose(dec.out[b], pf.out[b, :, p], rtol=1e-12, atol=1e-12)
        assert (dec.kept_count[b] == pf.kept_count[b, :, p]).all()
        for kv in range(Hkv):
            u = set()
            for h in range(kv * g, (kv + 1) * g):
                u |= set(np.flatnonzero(dec.keep[b][h]).tolist())
            assert dec.vrows_read[b, kv] == len(u)


# ------------------------------------------------------------- calibration pins
def test_calibration_samples_brute_force():
    """k-th largest score by argpartition; discarded mass by enumerating the
    subsets of size k of a tiny row and taking the largest-sum one."""
    rng = np.random.default_rng(10)
    Hq, Hkv, L, d = 2, 1, 7, 4
    Q = rng.standard_normal((Hq, L, d))
    K = rng.standard_normal((Hkv, L, d))
    obs = pre.calibration_samples_pre(Q, K, [1, 3], 0.5, 0)
    for (ki, h, p), (t, E) in obs.items():
        k = [1, 3][ki]
        a = oracle.scores(Q[h, p], K[0, :p + 1], 0.5)
        assert t == a[np.argpartition(-a, k - 1)[k - 1]]
        e = np.exp(a - a.max())
        best = max(itertools.combinations(range(p + 1), k), key=lambda c: e[list(c)].sum())
        assert E == pytest.approx(e.sum() - e[list(best)].sum(), rel=1e-12, abs=1e-15)
    assert set(obs) == {(ki, h, p) for ki, k in enumerate([1, 3]) for h in range(Hq)
                        for p in range(L) if p + 1 > k}


def test_calibration_pre_equals_post_through_lse():
    """On one sequence, the post-softmax sample is exp(pre sample - LSE) of the
    row (SciPy logsumexp), so the two calibrations agree up to that map."""
    rng = np.random.default_rng(11)
    Hq, L, d = 2, 16, 8
    Q = rng.standard_normal((Hq, L, d))
    K = rng.standard_normal((1, L, d))
    pre_obs = pre.calibration_samples_pre(Q, K, [4], 0.35, 0)
    post_obs = oracle.calibration_samples(Q, K, [4], 0.35, 0)
    assert set(pre_obs) == set(post_obs)
    for key, (t, _) in pre_obs.items():
        _, h, p = key
        lse = scipy.special.logsumexp(oracle.scores(Q[h, p], K[0, :p + 1], 0.35))
        assert post_obs[key] == pytest.approx(math.exp(t - lse), rel=1e-12)


def test_self_calibrated_offline_equals_exact():
    """Calibrating theta and E~ on one sequence and applying them to it keeps
    the top-k of every calibrated row, and E~ then equals the exact E."""
    rng = np.random.default_rng(12)
    B, Hq, Hkv, L, d, k = 1, 2, 1, 24, 8, 5
    q, kk, v = _rand(rng, B, Hq, Hkv, L, d)
    scale = 1 / math.sqrt(d)
    cal = pre.PreCalibrator([k], Hq, L)
    cal.observe(q[0], kk[0], scale, 0)
    th = cal.finalize()[0]
    et = cal.finalize_etilde()[0]
    off = pre.prefill_pre(q, kk, v, th, scale, sdc="offline", vmc=True, e_tilde=et)
    ex = pre.prefill_pre(q, kk, v, th, scale, sdc="exact", vmc=True)
    np.testing.assert_allclose(off.out, ex.out, rtol=1e-10, atol=1e-12)
    assert (off.kept_count[0, :, k:] == k).all()


def test_calibration_identical_copies_and_associativity():
    rng = np.random.default_rng(13)
    Hq, L, d = 1, 12, 4
    seqs = [(rng.standard_normal((Hq, L, d)), rng.standard_normal((1, L, d))) for _ in range(3)]
    one = pre.PreCalibrator([3], Hq, L)
    one.observe(*seqs[0], 0.5, 0)
    rep = pre.PreCalibrator([3], Hq, L)
    for _ in range(4):
        rep.observe(*seqs[0], 0.5, 0)
    np.testing.assert_allclose(rep.finalize(), one.finalize(), rtol=1e-14)
    np.testing.assert_allclose(rep.finalize_etilde(), one.finalize_etilde(), rtol=1e-14)
    # mean over A + B equals the count-weighted mean of the two parts
    a = pre.PreCalibrator([3], Hq, L)
    b = pre.PreCalibrator([3], Hq, L)
    ab = pre.PreCalibrator([3], Hq, L)
    a.observe(*seqs[0], 0.5, 0)
    b.observe(*seqs[1], 0.5, 0); b.observe(*seqs[2], 0.5, 0)
    for s in seqs:
        ab.observe(*s, 0.5, 0)
    w = (a.finalize_etilde() * 1 + b.finalize_etilde() * 2) / 3
    np.testing.assert_allclose(ab.finalize_etilde(), w, rtol=1e-12)
