"""Float64 reference of multi-k cumulative calibration (test infrastructure only).

Source: "Top-Theta Attention: Sparsifying Transformers by Compensated
Thresholding" (arXiv 2502.08363), Appendix D ("Multi-k Cumulative
Calibration"), Algorithm 2, Eq. 8 and Fig. 14.  Instead of one threshold per
target k, MKC builds for every (head, row) a function theta(k) that can be
queried for any k after one pass over the calibration set.

Steps, in the order of Appendix D:
  1. Each calibration sample's row r (m = r + 1 causal elements, or the n keys
     of a decoding step) is sorted ascending, v_0 <= ... <= v_{m-1}, and read as
     the intervals between consecutive values, each tagged with its effective
     k: the number of elements a threshold inside the interval keeps.
  2. MergeIntervals (Eq. 8): kbar(theta) is the mean effective k over the
     intervals, one per sample at most, that contain theta.
  3. theta(k) is the inverse of kbar at natural k.

Readings of steps the pages leave open (each also listed in the design notes):
  * Compare convention.  The appendix counts elements strictly greater than
    the threshold and writes the intervals [v_i, v_{i+1}); the thresholds of
    this library keep s >= theta.  Here the intervals are (v_i, v_{i+1}] with
    effective k = m - 1 - i = #{v >= theta}: the same counts for every theta
    except the sample values themselves, where ">=" is the count the kernels
    apply.  A sample's range is (v_0, v_{m-1}].
  * Samples outside their range.  As Eq. 8 defines the set of intervals that
    contain theta, a sample whose range does not contain theta is left out of
    the mean (it is neither counted as keeping 0 nor m elements).  kbar is
    then not monotone: near the top a sample whose maximum is passed joins the
    mean with effective k 1.
  * The inverse.  kbar is a step function that may skip integers and is not
    monotone, so inverting it at whole numbers k is read as
        theta(k) = max { theta : kbar(theta) >= k },
    the largest threshold that keeps at least k elements on average over the
    samples that cover it.  It is attained at a sample value, is non-increasing
    in k, and for a single sample equals the k-th largest value (the Algorithm 1
    sample).  Where kbar reaches k nowhere (k >= m in particular), theta(k) is
    -inf: keep every element, as for rows with at most k keys in Algorithm 1.
  * Values: post-softmax s = softmax(a) by default (the form of the main path),
    or the scores a themselves (pre-softmax); both appear in Fig. 15.
"""
from __future__ import annotations

import numpy as np

from .topth import post_softmax, scores


def sample_intervals(values):
    """Step 1 for one sample row: its values sorted ascending, v_0 <= ... <=
    v_{m-1}.  They stand for the intervals (v_i, v_{i+1}], i = 0 .. m-2, whose
    effective k is m - 1 - i; the sample's range is (v_0, v_{m-1}]."""
    return np.sort(np.asarray(values, dtype=np.float64))


def merged_kbar(sorted_samples, thetas):
    """Eq. 8 at each theta of `thetas`: the mean effective k over the samples
    whose range (v_0, v_{m-1}] contains theta.  In a sample that covers theta,
    the interval (v_i, v_{i+1}] holding it is found by binary search
    (i = #{v < theta} - 1) and contributes m - 1 - i.  NaN where no sample
    covers theta."""
    thetas = np.asarray(thetas, dtype=np.float64)
    total = np.zeros(thetas.shape)
    covering = np.zeros(thetas.shape)
    for v in sorted_samples:
        m = v.size
        inside = (v[0] < thetas) & (thetas <= v[-1])
        i = np.searchsorted(v, thetas, side="left") - 1
        total += np.where(inside, m - 1 - i, 0)
        covering += inside
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(covering > 0, total / np.maximum(covering, 1), np.nan)


def theta_of_ks(samples, ks):
    """Step 3: theta(k) = max { theta : kbar(theta) >= k } for every k of ks;
    -inf where kbar never reaches k.

    kbar is constant on each piece (x', x] between consecutive distinct sample
    values, so the largest qualifying theta is a sample value: every distinct
    value is a candidate and the largest one that qualifies is taken."""
    sorted_samples = [sample_intervals(s) for s in samples]
    cands = np.unique(np.concatenate(sorted_samples))
    kb = merged_kbar(sorted_samples, cands)
    out = np.full(len(ks), -np.inf)
    for t, k in enumerate(ks):
        ok = np.flatnonzero(kb >= k)          # NaN (no covering sample) never qualifies
        if ok.size:
            out[t] = cands[ok[-1]]
    return out


def theta_of_k(samples, k: int) -> float:
    """theta(k) of one target k (see theta_of_ks)."""
    return float(theta_of_ks(samples, [k])[0])


def row_values(q, K, scale: float, pre: bool):
    """The values Algorithm 2 sorts for one row: post-softmax s (default) or the
    scores a (pre-softmax)."""
    a = scores(q, K, scale)
    if pre:
        return a
    s, _ = post_softmax(a)
    return s


def mkc_calibrate(qs, ks_, scale: float, q_pos0: int, targets, pre: bool = False):
    """Algorithm 2 over a calibration set, for one attention layer.

    qs [S][Hq][Lq][d], ks_ [S][Hkv][Lk][d] (float64), query row i at position
    p = q_pos0 + i seeing keys 0..p (prefill rows, or one decoding row with
    q_pos0 = Lk - 1).  Returns theta [len(targets)][Hq][Lq]: theta_p(k) of the
    merged function of the S samples of row p of head h."""
    qs = np.asarray(qs, dtype=np.float64)
    ks_ = np.asarray(ks_, dtype=np.float64)
    S, Hq, Lq, _ = qs.shape
    Hkv = ks_.shape[1]
    g = Hq // Hkv
    out = np.full((len(targets), Hq, Lq), -np.inf)
    for h in range(Hq):
        for i in range(Lq):
            p = q_pos0 + i
            samples = [row_values(qs[c, h, i], ks_[c, h // g, :p + 1], scale, pre) for c in range(S)]
            out[:, h, i] = theta_of_ks(samples, targets)
    return out
