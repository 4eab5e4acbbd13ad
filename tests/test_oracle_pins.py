"""Pins of the CPU oracle against facts fixed outside of it.

Each test checks the oracle against a hand-derived closed form, a library
routine the oracle does not call, brute force on tiny inputs, or an identity
of "Top-Theta Attention: Sparsifying Transformers by Compensated Thresholding".
"""
import itertools
import json
import os
import statistics

import numpy as np
import pytest
import scipy.special
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "topth_closed_form.json")


def _num(x):
    return -np.inf if x == "-inf" else float(x)


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _rand_qkv(rng, B, Hq, Hkv, L, d, lam_sigma=0.5):
    q = rng.standard_normal((B, Hq, L, d))
    k = rng.standard_normal((B, Hkv, L, d)) * np.exp(lam_sigma * rng.standard_normal((B, Hkv, L, 1)))
    v = rng.standard_normal((B, Hkv, L, d))
    return q, k, v


# ---------------------------------------------------------------- closed forms
def test_golden_rows():
    g = _golden()["row_cases"]
    K = np.array([[np.log(c), g["k_second_column"]] for c in g["k_rows_log_of"]])
    a = oracle.scores(g["q"], K, g["scale"])
    for c in g["cases"]:
        r = oracle.topth_row(a, g["v"], _num(c["theta"]), g["mu"], vmc=c["vmc"], renorm=c["renorm"])
        assert r.keep.tolist() == c["keep"]
        assert r.kept_count == c["kept"]
        assert r.beta == pytest.approx(c["beta"], abs=1e-12)
        np.testing.assert_allclose(r.out, c["out"], rtol=1e-12, atol=1e-12)


def test_golden_prefill():
    g = _golden()["prefill_case"]
    L = len(g["k_rows_log_of"])
    Q = np.tile(np.array(g["q_row"]), (1, 1, L, 1))
    K = np.array([[[[np.log(c), g["k_second_column"]] for c in g["k_rows_log_of"]]]])
    V = np.array([[g["v"]]])
    theta = np.array([[_num(t) for t in g["theta"]]])
    r = oracle.prefill(Q, K, V, theta, g["scale"], vmc=True)
    assert r.kept_count[0, 0].tolist() == g["kept"]
    np.testing.assert_allclose(r.beta[0, 0], g["beta"], atol=1e-12)
    np.testing.assert_allclose(r.out[0, 0], g["out"], rtol=1e-12, atol=1e-12)


def _golden_calib_inputs(g):
    seqs = []
    for cs in g["sequences_k_rows_log_of"]:
        L = len(cs)
        Q = np.tile(np.array(g["q_row"]), (1, L, 1))
        K = np.array([[[np.log(c), 0.0] for c in cs]])
        seqs.append((Q, K))
    return seqs


def test_golden_calibration():
    g = _golden()["calibration_case"]
    seqs = _golden_calib_inputs(g)
    cal = oracle.Calibrator([2, 1], Hq=1, n_rows=g["n_rows"])
    for Q, K in seqs:
        cal.observe(Q, K, g["scale"], q_pos0=0)
    th0 = cal.finalize(alpha=0.0)
    th1 = cal.finalize(alpha=1.0)
    np.testing.assert_allclose(th0[0, 0], [_num(x) for x in g["k2_alpha0"]], rtol=1e-12)
    np.testing.assert_allclose(th1[0, 0], [_num(x) for x in g["k2_alpha1"]], rtol=1e-12)
    np.testing.assert_allclose(th0[1, 0], [_num(x) for x in g["k1_alpha0"]], rtol=1e-12)
    # decode-style: the query is the last position only
    Q, K = seqs[0]
    cal = oracle.Calibrator([2], Hq=1, n_rows=g["n_rows"])
    cal.observe(Q[:, -1:], K, g["scale"], q_pos0=K.shape[1] - 1)
    np.testing.assert_allclose(cal.finalize()[0, 0], [_num(x) for x in g["decode_style_seqA_k2"]],
                               rtol=1e-12)


# ------------------------------------------------- library / textbook routines
def test_scores_bruteforce():
    rng = np.random.default_rng(1)
    q = rng.standard_normal(8); K = rng.standard_normal((5, 8))
    a = oracle.scores(q, K, 0.37)
    for j in range(5):
        acc = 0.0
        for t in range(8):
            acc += q[t] * K[j, t]
        assert a[j] == pytest.approx(0.37 * acc, rel=1e-13)


def test_post_softmax_matches_scipy():
    rng = np.random.default_rng(2)
    a = 4.0 * rng.standard_normal(300)
    s, lse = oracle.post_softmax(a)
    np.testing.assert_allclose(s, scipy.special.softmax(a), rtol=1e-13)
    assert lse == pytest.approx(scipy.special.logsumexp(a), rel=1e-14)


def test_kth_largest_counting_definition():
    rng = np.random.default_rng(3)
    for _ in range(200):
        n = int(rng.integers(1, 12))
        x = rng.integers(0, 5, size=n).astype(float)    # many ties
        for k in range(1, n + 1):
            t = oracle.kth_largest(x, k)
            # t is the k-th largest iff fewer than k elements exceed it and at least k reach it
            assert (x > t).sum() < k <= (x >= t).sum()
            assert t == np.partition(x, n - k)[n - k]


def test_prefix_mean_cumsum():
    rng = np.random.default_rng(4)
    V = rng.standard_normal((17, 3))
    np.testing.assert_allclose(oracle.prefix_mean(V),
                               np.cumsum(V, axis=0) / np.arange(1, 18)[:, None], rtol=1e-13)


def test_dense_prefill_equals_sdpa():
    """T1: theta = -inf everywhere reproduces causal softmax attention (torch SDPA, fp64)."""
    rng = np.random.default_rng(5)
    B, Hq, Hkv, L, d = 2, 4, 2, 23, 16
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, L, d)
    theta = np.full((Hq, L), -np.inf)
    r = oracle.prefill(q, k, v, theta, 1 / np.sqrt(d), vmc=True)
    g = Hq // Hkv
    kt = torch.from_numpy(k).repeat_interleave(g, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(g, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), kt, vt,
                                                           is_causal=True).numpy()
    np.testing.assert_allclose(r.out, ref, rtol=1e-11, atol=1e-12)
    assert (r.kept_count == np.arange(1, L + 1)[None, None, :]).all()
    np.testing.assert_allclose(r.beta, 0.0, atol=1e-13)


def test_dense_decode_equals_sdpa():
    rng = np.random.default_rng(6)
    B, Hq, Hkv, L, d = 3, 8, 2, 40, 16
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, L, d)
    lens = np.array([40, 17, 1])
    theta = np.full((Hq, 1), -np.inf)
    vm = np.stack([[v[b, h, :lens[b]].mean(0) for h in range(Hkv)] for b in range(B)])
    r = oracle.decode(q[:, :, 0], k, v, lens, theta, vm, 0.25, vmc=True)
    for b in range(B):
        n = lens[b]
        kt = torch.from_numpy(k[b:b + 1, :, :n]).repeat_interleave(4, dim=1)
        vt = torch.from_numpy(v[b:b + 1, :, :n]).repeat_interleave(4, dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b:b + 1, :, :1]), kt, vt, scale=0.25).numpy()[0, :, 0]
        np.testing.assert_allclose(r.out[b], ref, rtol=1e-11, atol=1e-12)
        assert (r.kept_count[b] == n).all()
        assert (r.vrows_read[b] == n).all()


# --------------------------------------------------------- method identities
def test_exact_kth_threshold_is_topk():
    """T2: theta = the exact k-th largest s of the row keeps exactly the top-k set."""
    rng = np.random.default_rng(7)
    for trial in range(50):
        n = int(rng.integers(2, 64))
        a = 3 * rng.standard_normal(n)
        k = int(rng.integers(1, n + 1))
        s = scipy.special.softmax(a)
        srt = np.sort(s)[::-1]
        if k < n and srt[k - 1] - srt[k] < 1e-9 * srt[k - 1]:
            continue                      # near-tie: the top-k set is not unique
        theta = np.partition(s, n - k)[n - k] * (1 - 1e-12)   # below the k-th value by far less than any gap
        r = oracle.topth_row(a, np.eye(n), theta, np.zeros(n), vmc=False)
        top = set(np.argpartition(-a, k - 1)[:k].tolist())
        assert set(np.flatnonzero(r.keep).tolist()) == top
        assert r.kept_count == k


def test_sdc_equation_4():
    """Exact SDC: softmax over the kept pre-softmax scores times R/(R+E) equals s
    on the kept set, with R and E the exp-sums of kept / discarded elements
    after subtracting the row max (Eq. 4)."""
    rng = np.random.default_rng(8)
    for _ in range(30):
        n = int(rng.integers(3, 200))
        a = 2.5 * rng.standard_normal(n)
        theta = float(np.exp(rng.uniform(-8, -1)))
        V = rng.standard_normal((n, 5))
        r = oracle.topth_row(a, V, theta, np.zeros(5), vmc=False)
        if r.kept_count == 0:
            continue
        m = a.max()
        R = np.exp(a[r.keep] - m).sum()
        E = np.exp(a[~r.keep] - m).sum()
        sm_kept = torch.softmax(torch.from_numpy(a[r.keep]), 0).numpy()
        w, beta = oracle.row_weights(r.s, r.keep, renorm=False)
        np.testing.assert_allclose(w[r.keep], sm_kept * R / (R + E), rtol=1e-12)
        assert beta == pytest.approx(E / (R + E), rel=1e-9, abs=1e-15)
        np.testing.assert_allclose(r.out, (sm_kept * R / (R + E)) @ V[r.keep], rtol=1e-10, atol=1e-12)


def test_renorm_is_softmax_over_kept_set():
    rng = np.random.default_rng(9)
    n = 50
    a = 2 * rng.standard_normal(n); V = rng.standard_normal((n, 4))
    r = oracle.topth_row(a, V, 0.02, np.ones(4), vmc=True, renorm=True)
    assert r.kept_count > 0
    ref = torch.softmax(torch.from_numpy(a[r.keep]), 0).numpy() @ V[r.keep]
    np.testing.assert_allclose(r.out, ref, rtol=1e-12)
    assert r.beta == 0.0


def test_mass_identity():
    """sum of kept weights + beta = 1 (Eq. 6)."""
    rng = np.random.default_rng(10)
    for _ in range(40):
        n = int(rng.integers(1, 300))
        a = 3 * rng.standard_normal(n)
        r = oracle.topth_row(a, np.zeros((n, 1)), float(np.exp(rng.uniform(-9, 0))), [0.0], vmc=True)
        w, beta = oracle.row_weights(r.s, r.keep, renorm=False)
        assert w.sum() + beta == pytest.approx(1.0, abs=1e-13)


def test_identical_v_rows():
    """T3: identical V rows make the VMC output equal to the dense output for any theta."""
    rng = np.random.default_rng(11)
    B, Hq, Hkv, L, d = 1, 2, 1, 30, 8
    q, k, _ = _rand_qkv(rng, B, Hq, Hkv, L, d)
    row = rng.standard_normal(d)
    v = np.broadcast_to(row, (B, Hkv, L, d)).copy()
    for theta_val in (-np.inf, 1e-3, 0.05, 0.3, 2.0):
        theta = np.full((Hq, L), theta_val)
        r = oracle.prefill(q, k, v, theta, 0.3, vmc=True)
        np.testing.assert_allclose(r.out, np.broadcast_to(row, r.out.shape), rtol=1e-12, atol=1e-12)
        r2 = oracle.prefill(q, k, v, theta, 0.3, vmc=False)
        np.testing.assert_allclose(r2.out, (1 - r2.beta)[..., None] * row, rtol=1e-12, atol=1e-12)


def test_vmc_unbiased_under_independent_v():
    """T5 (Lemma E.1): with V drawn independently of the scores, E[VMC output]
    equals E[dense output] = m, while the uncompensated output is biased by -beta*m."""
    rng = np.random.default_rng(12)
    n, d, m, draws = 64, 4, 1.5, 4000
    a = 2.0 * rng.standard_normal(n)
    s = scipy.special.softmax(a)
    theta = np.sort(s)[::-1][9]          # keep 10 elements
    tot_vmc = np.zeros(d); tot_no = np.zeros(d); tot_dense = np.zeros(d)
    for _ in range(draws):
        V = m + rng.standard_normal((n, d))
        mu = V.mean(0)
        r = oracle.topth_row(a, V, theta, mu, vmc=True)
        r0 = oracle.topth_row(a, V, theta, mu, vmc=False)
        tot_vmc += r.out; tot_no += r0.out; tot_dense += s @ V
    beta = r.beta
    assert 0.05 < beta < 0.95
    se = 4.0 / np.sqrt(draws)            # generous: every output has unit-order variance
    np.testing.assert_allclose(tot_vmc / draws, m, atol=se)
    np.testing.assert_allclose(tot_dense / draws, m, atol=se)
    np.testing.assert_allclose(tot_no / draws, (1 - beta) * m, atol=se)
    assert np.all(np.abs(tot_no / draws - m) > 0.5 * beta * m)


def test_monotone_in_theta():
    rng = np.random.default_rng(13)
    a = 3 * rng.standard_normal(500)
    prev = None
    for t in np.exp(np.linspace(-12, 0, 40)):
        r = oracle.topth_row(a, np.zeros((500, 1)), t, [0.0], vmc=False)
        if prev is not None:
            assert not (r.keep & ~prev).any()
        prev = r.keep


def test_ties_keep_at_least_k():
    """T6: duplicated keys and theta = the k-th value keep every tie (k~ >= k)."""
    rng = np.random.default_rng(14)
    d, n = 8, 40
    K = rng.standard_normal((n, d))
    K[10] = K[3]; K[11] = K[3]; K[20] = K[5]
    q = rng.standard_normal(d)
    a = oracle.scores(q, K, 0.5)
    s, _ = oracle.post_softmax(a)
    for k in range(1, n + 1):
        r = oracle.topth_row(a, np.zeros((n, 1)), oracle.kth_largest(s, k), [0.0], vmc=False)
        assert r.kept_count >= k
        assert r.kept_count == (s >= np.sort(s)[::-1][k - 1]).sum()


def test_decode_permutation_invariance():
    rng = np.random.default_rng(15)
    B, Hq, Hkv, L, d = 1, 4, 2, 33, 8
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, L, d)
    theta = np.full((Hq, L), 0.01)
    vm = v.mean(2)
    r = oracle.decode(q[:, :, 0], k, v, [L], theta, vm, 0.35, vmc=True)
    perm = rng.permutation(L)
    rp = oracle.decode(q[:, :, 0], k[:, :, perm], v[:, :, perm], [L], theta, vm, 0.35, vmc=True)
    np.testing.assert_allclose(rp.out, r.out, rtol=1e-12, atol=1e-13)
    assert (rp.kept_count == r.kept_count).all() and (rp.vrows_read == r.vrows_read).all()


def test_decode_equals_prefill_row():
    rng = np.random.default_rng(16)
    B, Hq, Hkv, L, d = 1, 4, 2, 21, 8
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, L, d)
    theta = np.exp(rng.uniform(-5, -1, size=(Hq, L)))
    pre = oracle.prefill(q, k, v, theta, 0.35, vmc=True)
    for p in (0, 5, 20):
        vm = v[:, :, :p + 1].mean(2)
        dec = oracle.decode(q[:, :, p], k, v, [p + 1], theta, vm, 0.35, vmc=True)
        np.testing.assert_allclose(dec.out, pre.out[:, :, p], rtol=1e-12, atol=1e-13)
        assert (dec.kept_count == pre.kept_count[:, :, p]).all()


def test_gqa_equals_replicated_mha():
    rng = np.random.default_rng(17)
    B, Hq, Hkv, L, d = 2, 6, 2, 15, 8
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, L, d)
    theta = np.exp(rng.uniform(-4, -1, size=(Hq, L)))
    r = oracle.prefill(q, k, v, theta, 0.35, vmc=True)
    rm = oracle.prefill(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), theta, 0.35, vmc=True)
    np.testing.assert_allclose(r.out, rm.out, rtol=1e-13)
    assert (r.kept_count == rm.kept_count).all()


def test_vrows_is_union_bruteforce():
    rng = np.random.default_rng(18)
    B, Hq, Hkv, L, d = 2, 8, 2, 50, 8
    q, k, v = _rand_qkv(rng, B, Hq, Hkv, L, d)
    theta = np.full((Hq, L), 0.03)
    r = oracle.decode(q[:, :, 0], k, v, [50, 31], theta, v.mean(2), 0.35, vmc=True)
    for b in range(B):
        for kv in range(Hkv):
            used = set()
            for h in range(kv * 4, kv * 4 + 4):
                used |= {j for j in range(len(r.keep[b][h])) if r.keep[b][h][j]}
            assert r.vrows_read[b, kv] == len(used)


# -------------------------------------------------------------- calibration
def test_self_calibration_keeps_k():
    """Calibrating on one sequence and applying theta to the same sequence keeps
    exactly k elements in every calibrated row (distinct scores)."""
    rng = np.random.default_rng(19)
    Hq, Hkv, L, d, k = 2, 1, 40, 16, 5
    q, kk, v = _rand_qkv(rng, 1, Hq, Hkv, L, d)
    cal = oracle.Calibrator([k], Hq, L)
    cal.observe(q[0], kk[0], 0.25)
    theta = cal.finalize()[0]
    assert np.isneginf(theta[:, :k]).all() and np.isfinite(theta[:, k:]).all()
    r = oracle.prefill(q, kk, v, theta, 0.25, vmc=True)
    assert (r.kept_count[0, :, k:] == k).all()
    assert (r.kept_count[0, :, :k] == np.arange(1, k + 1)).all()


def test_calibration_associative_and_copies():
    rng = np.random.default_rng(20)
    Hq, Hkv, L, d = 2, 2, 24, 8
    seqs = [_rand_qkv(rng, 1, Hq, Hkv, L, d)[:2] for _ in range(5)]
    ks = [3, 7]
    allc = oracle.Calibrator(ks, Hq, L)
    ca = oracle.Calibrator(ks, Hq, L); cb = oracle.Calibrator(ks, Hq, L)
    for i, (q, k) in enumerate(seqs):
        allc.observe(q[0], k[0], 0.3)
        (ca if i < 2 else cb).observe(q[0], k[0], 0.3)
    th, tha, thb = allc.finalize(), ca.finalize(), cb.finalize()
    fin = np.isfinite(th)
    np.testing.assert_allclose(th[fin], ((2 * tha + 3 * thb) / 5)[fin], rtol=1e-12)
    one = oracle.Calibrator(ks, Hq, L); many = oracle.Calibrator(ks, Hq, L)
    one.observe(seqs[0][0][0], seqs[0][1][0], 0.3)
    for _ in range(4):
        many.observe(seqs[0][0][0], seqs[0][1][0], 0.3)
    np.testing.assert_allclose(many.finalize(alpha=0.7), one.finalize(alpha=0.7), rtol=1e-12)


def test_calibration_alpha_uses_population_std():
    rng = np.random.default_rng(21)
    Hq, L, d = 1, 12, 8
    cal = oracle.Calibrator([4], Hq, L)
    obs = []
    for _ in range(6):
        q, k, _ = _rand_qkv(rng, 1, Hq, 1, L, d)
        cal.observe(q[0], k[0], 0.3)
        s = scipy.special.softmax(0.3 * (k[0, 0, :L] @ q[0, 0, L - 1]))
        obs.append(sorted(s)[-4])
    th = cal.finalize(alpha=0.5)
    assert th[0, 0, L - 1] == pytest.approx(statistics.fmean(obs) + 0.5 * statistics.pstdev(obs), rel=1e-12)


def test_nearest_fill_rule():
    """Rows no sequence reached copy the nearest observed row, the smaller one on a tie."""
    rng = np.random.default_rng(22)
    d, L = 8, 30
    cal = oracle.Calibrator([2], 1, L)
    for n in (10, 20):           # decode-style observations at rows 9 and 19
        q, k, _ = _rand_qkv(rng, 1, 1, 1, n, d)
        cal.observe(q[0][:, -1:], k[0], 0.3, q_pos0=n - 1)
    th = cal.finalize()[0, 0]
    assert np.isneginf(th[:2]).all()
    assert (th[2:15] == th[9]).all()        # row 14 is 5 from both 9 and 19: the smaller wins
    assert (th[15:] == th[19]).all()
    assert th[9] != th[19]


def test_calibration_samples_bruteforce_small():
    """Every sample equals the k-th largest of a brute-force enumeration of the row."""
    rng = np.random.default_rng(23)
    Hq, L, d = 1, 7, 4
    q, k, _ = _rand_qkv(rng, 1, Hq, 1, L, d)
    obs = oracle.calibration_samples(q[0], k[0], [1, 3], 0.5, 0)
    for (ki, h, p), t in obs.items():
        kk = [1, 3][ki]
        e = [np.exp(0.5 * sum(q[0, h, p, c] * k[0, 0, j, c] for c in range(d))) for j in range(p + 1)]
        z = sum(e)
        vals = [x / z for x in e]
        # brute force: the value whose rank (count of strictly larger values) is below k
        best = [v for v in vals if sum(1 for w in vals if w > v) < kk and sum(1 for w in vals if w >= v) >= kk]
        assert t == pytest.approx(best[0], rel=1e-12)
    assert {p for (ki, h, p) in obs if ki == 1} == set(range(3, L))
    assert {p for (ki, h, p) in obs if ki == 0} == set(range(1, L))


def test_kept_zero_row():
    """G13: a theta above every s keeps nothing: out = mu with VMC, 0 without."""
    a = np.array([0.0, 0.1, -0.2])
    V = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    mu = np.array([-1.0, 7.0])
    r = oracle.topth_row(a, V, 0.9, mu, vmc=True)
    assert r.kept_count == 0 and r.beta == pytest.approx(1.0)
    np.testing.assert_allclose(r.out, mu)
    np.testing.assert_allclose(oracle.topth_row(a, V, 0.9, mu, vmc=False).out, 0.0)
    np.testing.assert_allclose(oracle.topth_row(a, V, 0.9, mu, vmc=True, renorm=True).out, 0.0)


def test_theta_row_clamps_to_last_row():
    t = np.arange(12, dtype=float).reshape(2, 6)
    assert oracle.theta_row(t, 1, 3) == 9.0
    assert oracle.theta_row(t, 1, 100) == 11.0
    assert oracle.theta_row(t, 0, 5) == 5.0


def test_bruteforce_tiny_prefill():
    """Whole prefill on a tiny case against an itertools brute force of the definitions."""
    rng = np.random.default_rng(24)
    L, d = 5, 3
    q, k, v = _rand_qkv(rng, 1, 1, 1, L, d)
    theta = np.array([[-np.inf, 0.3, 0.2, 0.25, 0.1]])
    r = oracle.prefill(q, k, v, theta, 0.8, vmc=True)
    for p in range(L):
        e = [np.exp(0.8 * sum(q[0, 0, p, c] * k[0, 0, j, c] for c in range(d))) for j in range(p + 1)]
        s = [x / sum(e) for x in e]
        keep = [x >= theta[0, p] for x in s]
        mu = [sum(v[0, 0, j, c] for j in range(p + 1)) / (p + 1) for c in range(d)]
        beta = 1 - sum(x for x, kp in zip(s, keep) if kp)
        out = [sum(s[j] * v[0, 0, j, c] for j in range(p + 1) if keep[j]) + beta * mu[c] for c in range(d)]
        np.testing.assert_allclose(r.out[0, 0, p], out, rtol=1e-12, atol=1e-14)
        assert r.kept_count[0, 0, p] == sum(keep)
    assert list(itertools.islice(r.kept_count[0, 0], 1)) == [1]
