"""Float64 reference of the decode-serving helpers around Top-theta (test
infrastructure only).

Source: "Top-Theta Attention: Sparsifying Transformers by Compensated
Thresholding" (arXiv 2502.08363), cited as [TT], and the Pith verdict page on
the same paper, which paraphrases the paper's lost technical details.

* Running mean of V ([TT] §3.2.2, after Eq. 7: in generative decoding the
  paper keeps mu up to date as a running mean): appending rows n_old..n_new-1 to a
  cache whose first n_old rows have mean mu_old gives the mean of the first
  n_new rows, mu_new = (n_old * mu_old + sum of the new rows) / n_new.  This is
  Eq. 5 over the longer cache, rewritten; a cache with n_old = 0 starts fresh.
* Fitted thresholds (Pith verdict page, technical details: for rows beyond
  the calibrated ones the paper takes the closest calibrated row's threshold
  or a function of the row length fitted to the calibrated thresholds, which
  replaces a per-row table by a handful of coefficients; the function itself
  is lost with the paper's Fig. 3 and technical details).  Reading: a
  least-squares polynomial of low degree in x = ln(p + 1) through the
  calibrated rows of each (k, head) -- on ln(theta) for post-softmax thresholds
  (probabilities, which fall roughly as a power of the row length) and on theta
  itself for pre-softmax thresholds (scores).  Evaluated at every row with
  p + 1 > k; rows with p + 1 <= k keep everything (-inf).  **Parity unpinned**
  by the pages: the function form is a reading; the pins check the fit itself
  (exact recovery of data that lie on such a polynomial, library least squares).
"""
from __future__ import annotations

import numpy as np

from .topth import _as64


def running_mean_append(mu_old, n_old: int, V_new) -> np.ndarray:
    """mu of the first n_old + m rows from mu of the first n_old rows and the m
    appended rows V_new [m, d]."""
    V_new = _as64(V_new)
    n_new = int(n_old) + V_new.shape[0]
    if n_new <= 0:
        raise ValueError("empty cache")
    total = V_new.sum(axis=0)
    if n_old > 0:
        total = total + int(n_old) * _as64(mu_old)
    return total / n_new


def fit_theta(theta_table, observed, degree: int, log_domain: bool, min_row: int = 0):
    """Coefficients (highest power first) of the least-squares polynomial of
    ``degree`` in ln(p + 1) through the rows p >= min_row where ``observed``
    is true, on ln(theta) if ``log_domain`` else on theta; one row of
    coefficients per head.  theta_table and observed are [Hq, R].  A head with
    fewer than degree + 1 usable rows gets NaN coefficients; in the log domain
    rows with theta <= 0 are not usable.  (Near p + 1 = k the k-th largest
    value of a row sits close to the row's minimum, so thresholds first rise
    with the row length and then fall; leaving out the rows below a few k
    keeps that rise out of a fit that is extrapolated to longer rows.)"""
    th = _as64(theta_table)
    obs = np.asarray(observed, dtype=bool)
    Hq, R = th.shape
    coef = np.full((Hq, degree + 1), np.nan)
    x_all = np.log(np.arange(R) + 1.0)
    for h in range(Hq):
        use = obs[h] & np.isfinite(th[h]) & (np.arange(R) >= min_row)
        if log_domain:
            use &= th[h] > 0
        if use.sum() < degree + 1:
            continue
        y = np.log(th[h][use]) if log_domain else th[h][use]
        coef[h] = np.polyfit(x_all[use], y, degree)
    return coef


def eval_theta(coef, k: int, n_out: int, log_domain: bool) -> np.ndarray:
    """theta [Hq, n_out] from the fitted coefficients: the polynomial at
    ln(p + 1) (exponentiated in the log domain) for p + 1 > k, -inf below."""
    coef = _as64(coef)
    Hq = coef.shape[0]
    x = np.log(np.arange(n_out) + 1.0)
    out = np.full((Hq, n_out), -np.inf)
    for h in range(Hq):
        v = np.polyval(coef[h], x)
        if log_domain:
            v = np.exp(v)
        rows = np.arange(n_out) + 1 > k
        out[h, rows] = v[rows]
    return out


def decode_gqa(q, K_cache, V_cache, seq_lens, theta, v_mean, scale: float, *, vmc: bool,
               min_votes: int = 1, augment: bool = False, renorm: bool = False):
    """One decoding step with the GQA selection variants of [TT] §4.6: a key is
    loaded for a (b, KV head) group when at least ``min_votes`` of its g heads
    keep it (s >= theta), so rows wanted by fewer heads are dropped; each head
    then uses its own kept keys among those (``augment`` False) or all of them
    (``augment`` True: every head takes the group's whole selection), weighted
    by its own post-softmax values (exact SDC) and VMC as in Eq. 5-7.
    min_votes = 1 without augment is the plain per-head selection."""
    from .topth import DecodeResult, post_softmax, row_output, scores, theta_row
    q = _as64(q); K_cache = _as64(K_cache); V_cache = _as64(V_cache)
    B, Hq, d = q.shape
    Hkv = K_cache.shape[1]
    g = Hq // Hkv
    out = np.zeros((B, Hq, d)); kept = np.zeros((B, Hq), dtype=np.int64)
    beta = np.zeros((B, Hq)); vrows = np.zeros((B, Hkv), dtype=np.int64)
    s_rows = [[None] * Hq for _ in range(B)]
    k_rows = [[None] * Hq for _ in range(B)]
    for b in range(B):
        n = int(seq_lens[b])
        for kv in range(Hkv):
            heads = range(kv * g, (kv + 1) * g)
            s = {h: post_softmax(scores(q[b, h], K_cache[b, kv, :n], scale))[0] for h in heads}
            own = {h: s[h] >= theta_row(theta, h, n - 1) for h in heads}
            votes = np.sum([own[h] for h in heads], axis=0)
            loaded = votes >= min_votes
            vrows[b, kv] = int(loaded.sum())
            for h in heads:
                keep = loaded if augment else (loaded & own[h])
                mu = _as64(v_mean[b, kv]) if vmc else np.zeros(d)
                o, bt = row_output(s[h], keep, V_cache[b, kv, :n], mu, vmc=vmc, renorm=renorm)
                out[b, h] = o; kept[b, h] = int(keep.sum()); beta[b, h] = bt
                s_rows[b][h] = s[h]; k_rows[b][h] = keep
    return DecodeResult(out, kept, beta, vrows, s_rows, k_rows)
