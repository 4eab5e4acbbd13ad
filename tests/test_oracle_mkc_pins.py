"""Pins of the multi-k cumulative calibration oracle (oracle/mkc.py) against
things other than itself: closed forms that Appendix D and Eq. 8 fix for
special inputs, a brute force that evaluates Eq. 8 over explicit interval
lists, NumPy/SciPy routines the oracle does not call, and invariants.

Source: "Top-Theta Attention: Sparsifying Transformers by Compensated
Thresholding", Appendix D (Algorithm 2, Eq. 8, Fig. 14)."""
import heapq
import itertools

import numpy as np
import pytest
from scipy.special import softmax

from oracle import mkc


def brute_intervals(values):
    """Algorithm 2, step 1, written out: for the values sorted ascending, the
    tuples <effective k, lo, hi> of the intervals (lo, hi] between neighbours,
    effective k = number of values >= any theta inside (counted directly)."""
    v = sorted(float(x) for x in values)
    out = []
    for lo, hi in zip(v[:-1], v[1:]):
        if lo < hi:
            mid = (lo + hi) / 2.0
            out.append((sum(1 for x in v if x >= mid), lo, hi))
    return out


def brute_theta(samples, k):
    """Eq. 8 at every sample value and every midpoint between neighbouring
    distinct values (kbar is constant between them), then the largest probe
    whose mean effective k over the covering intervals is at least k."""
    sets = [brute_intervals(s) for s in samples]
    vals = sorted(set(float(x) for s in samples for x in s))
    probes = vals + [(a + b) / 2.0 for a, b in zip(vals[:-1], vals[1:])]
    best = -np.inf
    for t in probes:
        ks = [ke for iv in sets for (ke, lo, hi) in iv if lo < t <= hi]
        if ks and sum(ks) / len(ks) >= k and t > best:
            best = t
    return best


@pytest.mark.parametrize("seed", range(6))
def test_single_sample_gives_the_kth_largest(seed):
    rng = np.random.default_rng(seed)
    m = int(rng.integers(2, 40))
    v = rng.standard_normal(m)
    got = mkc.theta_of_ks([v], list(range(1, m + 2)))
    for k in range(1, m):
        assert got[k - 1] == heapq.nlargest(k, v.tolist())[-1]
    assert got[m - 1] == -np.inf and got[m] == -np.inf       # k >= m: keep everything


def test_identical_copies_equal_one_sample():
    rng = np.random.default_rng(7)
    v = rng.random(25)
    ks = list(range(1, 25))
    np.testing.assert_array_equal(mkc.theta_of_ks([v] * 9, ks), mkc.theta_of_ks([v], ks))


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_over_interval_lists(seed):
    # small integers: many ties within and across samples
    rng = np.random.default_rng(100 + seed)
    S = int(rng.integers(1, 5))
    m = int(rng.integers(2, 8))
    samples = [rng.integers(0, 6, size=m).astype(float) for _ in range(S)]
    for k in range(1, m + 1):
        assert mkc.theta_of_k(samples, k) == brute_theta(samples, k), (samples, k)


def test_hand_computed_two_samples():
    # A = {0.05, 0.1, 0.3, 0.5}, B = {0.01, 0.02, 0.2, 0.9}.  Going down from the
    # top, Eq. 8 averages only the samples whose range covers theta:
    #   theta = 0.9: only B covers, 1 kept -> kbar 1            => theta(1) = 0.9
    #   0.5: A 1, B 1 -> 1;  0.3: A 2, B 1 -> 1.5;  0.2: A 2, B 2 -> 2  => theta(2) = 0.2
    #   0.1: A 3, B 2 -> 2.5;  0.05: A's range (0.05, 0.5] no longer covers,
    #   B 2 -> 2;  0.02: B 3 -> 3                                 => theta(3) = 0.02
    #   0.01: nobody covers                                       => theta(4) = -inf
    # Counting uncovered samples as keeping 0 or all 4 elements would give
    # theta(1) = 0.5 and theta(3) = 0.05 instead.
    A = [0.05, 0.1, 0.3, 0.5]
    B = [0.9, 0.2, 0.01, 0.02]
    np.testing.assert_array_equal(mkc.theta_of_ks([A, B], [1, 2, 3, 4]), [0.9, 0.2, 0.02, -np.inf])


@pytest.mark.parametrize("seed", range(5))
def test_pooled_quantile_where_every_sample_covers(seed):
    # every sample holds +100 and -100, so every theta strictly between is
    # covered by all S samples and kbar(theta) = #{pooled values >= theta} / S:
    # theta(k) is the (k S)-th largest pooled value for 2 <= k <= m - 1
    rng = np.random.default_rng(200 + seed)
    S, mid = 6, 30
    samples = [np.concatenate([[100.0, -100.0], rng.standard_normal(mid)]) for _ in range(S)]
    m = mid + 2
    pooled = np.concatenate(samples)
    ks = list(range(2, m))
    got = mkc.theta_of_ks(samples, ks)
    for k, t in zip(ks, got):
        assert t == -np.partition(-pooled, k * S - 1)[k * S - 1], k
    assert mkc.theta_of_k(samples, 1) == 100.0


@pytest.mark.parametrize("seed", range(5))
def test_monotone_in_k_and_attained_at_sample_values(seed):
    rng = np.random.default_rng(300 + seed)
    samples = [rng.lognormal(size=int(rng.integers(5, 30))) for _ in range(4)]
    m = min(len(s) for s in samples)
    got = mkc.theta_of_ks(samples, list(range(1, m)))
    assert np.all(np.diff(got) <= 0)
    allv = set(np.concatenate(samples).tolist())
    assert all((t in allv) or t == -np.inf for t in got)


def test_merged_kbar_is_eq8_on_explicit_intervals():
    rng = np.random.default_rng(9)
    samples = [rng.integers(0, 9, size=6).astype(float) for _ in range(3)]
    sets = [brute_intervals(s) for s in samples]
    probes = np.linspace(-1.0, 10.0, 221)
    kb = mkc.merged_kbar([mkc.sample_intervals(s) for s in samples], probes)
    for t, got in zip(probes, kb):
        ks = [ke for iv in sets for (ke, lo, hi) in iv if lo < t <= hi]
        if ks:
            assert got == pytest.approx(sum(ks) / len(ks), abs=1e-12)
        else:
            assert np.isnan(got)


def test_mkc_calibrate_rows_of_one_sequence():
    # one calibration sequence: theta_p(k) is the k-th largest softmax value of
    # row p (SciPy softmax), for prefill rows; and the k-th largest score in
    # the pre-softmax form
    rng = np.random.default_rng(11)
    d, L = 16, 12
    q = rng.standard_normal((1, 2, L, d))
    K = rng.standard_normal((1, 1, L, d))
    ks = [1, 2, 3, 5]
    sc = 0.25
    th = mkc.mkc_calibrate(q, K, sc, 0, ks)
    thp = mkc.mkc_calibrate(q, K, sc, 0, ks, pre=True)
    for h, p in itertools.product(range(2), range(L)):
        a = sc * (K[0, 0, :p + 1] @ q[0, h, p])
        s = softmax(a)
        for t, k in enumerate(ks):
            if k < p + 1:
                assert th[t, h, p] == pytest.approx(np.sort(s)[::-1][k - 1], rel=1e-12)
                assert thp[t, h, p] == pytest.approx(np.sort(a)[::-1][k - 1], rel=1e-12)
            else:
                assert th[t, h, p] == -np.inf and thp[t, h, p] == -np.inf


def test_mkc_calibrate_decode_row_and_gqa():
    # a decoding row (q_pos0 = Lk - 1) of two sequences; query heads 2 and 3
    # read KV head 1
    rng = np.random.default_rng(12)
    d, Lk = 8, 20
    q = rng.standard_normal((2, 4, 1, d))
    K = rng.standard_normal((2, 2, Lk, d))
    th = mkc.mkc_calibrate(q, K, 0.5, Lk - 1, [1, 4, 10])
    for h in range(4):
        samples = [softmax(0.5 * (K[c, h // 2] @ q[c, h, 0])) for c in range(2)]
        for t, k in enumerate([1, 4, 10]):
            assert th[t, h, 0] == pytest.approx(brute_theta(samples, k), rel=1e-12)
