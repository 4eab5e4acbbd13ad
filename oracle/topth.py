"""Float64 reference of Top-theta attention (test infrastructure only).

Source: "Top-Theta Attention: Sparsifying Transformers by Compensated
Thresholding" (arXiv 2502.08363), cited below as [TT] with its section,
equation or algorithm number.  Readings of steps the paper leaves open:

* Scores carry the 1/sqrt(d) factor and the causal mask that [TT] §2.2 says it
  leaves out of Eq. 1 to keep it short; query row p sees keys 0..p.
* Post-softmax thresholding ([TT] §3.1, last paragraph): the calibrated sample of
  a row is taken on s = softmax(a), not on a.
* The per-row quantile of [TT] Alg. 1 is read as the k-th largest valid
  element of the row (its printed quantile index is garbled); rows with at most
  k keys are not calibrated and keep every element (theta = -inf).
* A row is kept element-wise when s >= theta (">=": theta equal to the exact
  k-th value then keeps exactly k distinct values).
* Row id of a query = its 0-based position p; a decode step with n cached keys
  is row p = n - 1.  Rows past the end of a table use its last row; calibrated
  tables fill rows no calibration sequence reached from the nearest calibrated
  row (smaller row on a tie): the closest-calibrated-row rule that the Pith
  verdict page on arXiv 2502.08363 (skeptic critique) reports from the paper's
  lost technical details.
* SDC ([TT] §3.2.1, Eq. 4) in its "exact" form: the kept weights keep the full
  denominator R + E, i.e. they are the post-softmax values s themselves.  The
  alternative ``renorm`` divides by R only (softmax over the kept set).
* VMC ([TT] §3.2.2, Eq. 5-7): beta = 1 - sum of kept s; out += beta * mu.  In
  prefill mu_p is the causal prefix mean of V rows 0..p (Eq. 5 read causally);
  in decode mu is the caller's running mean of the cached V rows.  Under
  ``renorm`` the kept weights already sum to one, so beta = 0; a row with no
  kept element then outputs zero.
* GQA: query head h reads KV head floor(h / g), g = Hq / Hkv ([TT] §2.2, §4.6);
  every head keeps its own selection.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Eq. 1-2: scores and the post-softmax row
# ---------------------------------------------------------------------------
def scores(q, K, scale: float) -> np.ndarray:
    """a_j = scale * <q, K_j> for the keys given ([TT] §2.2, Eq. 1 with 1/sqrt(d))."""
    q = _as64(q)
    K = _as64(K)
    return (K @ q) * float(scale)


def post_softmax(a):
    """Return (s, lse): s = softmax(a) ([TT] Eq. 2) and lse = log(sum exp a)."""
    a = _as64(a)
    m = a.max()
    e = np.exp(a - m)
    z = e.sum()
    return e / z, m + math.log(z)


def kth_largest(x, k: int) -> float:
    """k-th largest element (1-based k) of x, by a full descending sort."""
    x = _as64(x)
    if not 1 <= k <= x.size:
        raise ValueError("k out of range")
    return float(np.sort(x)[::-1][k - 1])


def theta_row(theta_table, h: int, p: int) -> float:
    """theta for query head h at row p; rows past the table use its last row."""
    t = np.asarray(theta_table)
    return float(t[h, min(p, t.shape[1] - 1)])


# ---------------------------------------------------------------------------
# §3.2.1 (SDC) and §3.2.2 (VMC) on one row, for a given keep mask
# ---------------------------------------------------------------------------
@dataclass
class RowResult:
    out: np.ndarray       # [d] compensated output p_hat
    keep: np.ndarray      # [n] bool mask of kept keys
    kept_count: int       # k~
    beta: float           # mass added by VMC (Eq. 6)
    s: np.ndarray         # [n] post-softmax values (for ambiguity bands)


def row_weights(s, keep, renorm: bool):
    """Weights of the kept keys and beta.

    Exact SDC (Eq. 4 with E~ = E): w = s on the kept set, beta = 1 - sum w.
    ``renorm``: w = s / sum_kept s (beta = 0); an empty kept set gives no weights.
    """
    s = _as64(s)
    keep = np.asarray(keep, dtype=bool)
    kept_mass = float(s[keep].sum())
    w = np.where(keep, s, 0.0)
    if renorm:
        if keep.any():
            w = w / kept_mass
        return w, 0.0
    return w, 1.0 - kept_mass


def row_output(s, keep, V, mu, *, vmc: bool, renorm: bool):
    """p_hat = sum_kept w_j V_j (+ beta * mu with VMC): Eq. 7."""
    w, beta = row_weights(s, keep, renorm)
    V = _as64(V)
    out = w @ V
    if vmc and not renorm:
        out = out + beta * _as64(mu)
    return out, beta


def topth_row(a, V, theta: float, mu, *, vmc: bool, renorm: bool = False) -> RowResult:
    """One attention row under Top-theta: threshold s >= theta, SDC, VMC."""
    s, _ = post_softmax(a)
    keep = s >= theta
    out, beta = row_output(s, keep, V, mu, vmc=vmc, renorm=renorm)
    return RowResult(out=out, keep=keep, kept_count=int(keep.sum()), beta=beta, s=s)


def prefix_mean(V) -> np.ndarray:
    """mu_p = mean of V rows 0..p for every p (Eq. 5 read causally): [L, d]."""
    V = _as64(V)
    L = V.shape[0]
    out = np.empty_like(V)
    acc = np.zeros(V.shape[1])
    for p in range(L):
        acc = acc + V[p]
        out[p] = acc / (p + 1)
    return out


# ---------------------------------------------------------------------------
# Prefill and decode built from the row rule
# ---------------------------------------------------------------------------
@dataclass
class PrefillResult:
    out: np.ndarray         # [B, Hq, L, d]
    kept_count: np.ndarray  # [B, Hq, L] int
    beta: np.ndarray        # [B, Hq, L]
    s: list                 # s[b][h][p] -> post-softmax row (length p+1), if kept
    keep: list              # keep[b][h][p] -> bool mask, if kept


def prefill(Q, K, V, theta, scale: float, *, vmc: bool, renorm: bool = False,
            rows=None, keep_rows: bool = False) -> PrefillResult:
    """Causal Top-theta prefill.  Q [B,Hq,L,d]; K, V [B,Hkv,L,d]; theta [Hq,R].

    ``rows`` optionally restricts the work to an iterable of (b, h, p); other
    entries of the result are left as NaN / -1.
    """
    Q = _as64(Q); K = _as64(K); V = _as64(V)
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    out = np.full((B, Hq, L, d), np.nan)
    kept = np.full((B, Hq, L), -1, dtype=np.int64)
    beta = np.full((B, Hq, L), np.nan)
    s_rows = [[[None] * L for _ in range(Hq)] for _ in range(B)]
    k_rows = [[[None] * L for _ in range(Hq)] for _ in range(B)]
    mu_cache = {}
    if rows is None:
        rows = [(b, h, p) for b in range(B) for h in range(Hq) for p in range(L)]
    for (b, h, p) in rows:
        kv = h // g
        if vmc and not renorm:
            if (b, kv) not in mu_cache:
                mu_cache[(b, kv)] = prefix_mean(V[b, kv])
            mu = mu_cache[(b, kv)][p]
        else:
            mu = np.zeros(d)
        a = scores(Q[b, h, p], K[b, kv, :p + 1], scale)
        r = topth_row(a, V[b, kv, :p + 1], theta_row(theta, h, p), mu, vmc=vmc, renorm=renorm)
        out[b, h, p] = r.out
        kept[b, h, p] = r.kept_count
        beta[b, h, p] = r.beta
        if keep_rows:
            s_rows[b][h][p] = r.s
            k_rows[b][h][p] = r.keep
    return PrefillResult(out, kept, beta, s_rows, k_rows)


@dataclass
class DecodeResult:
    out: np.ndarray         # [B, Hq, d]
    kept_count: np.ndarray  # [B, Hq]
    beta: np.ndarray        # [B, Hq]
    vrows_read: np.ndarray  # [B, Hkv]: size of the union of kept keys over the group
    s: list                 # s[b][h] -> post-softmax row (length n_b)
    keep: list              # keep[b][h] -> bool mask


def decode(q, K_cache, V_cache, seq_lens, theta, v_mean, scale: float, *, vmc: bool,
           renorm: bool = False) -> DecodeResult:
    """One generative-decoding step ([TT] §2.2 "Generative decoding phase").

    q [B,Hq,d]; caches [B,Hkv,Lmax,d] of which the first n_b = seq_lens[b] rows
    are valid (the current token included); the row id is n_b - 1; v_mean
    [B,Hkv,d] is mu (required when ``vmc``).
    """
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
            union = np.zeros(n, dtype=bool)
            for h in range(kv * g, (kv + 1) * g):
                mu = _as64(v_mean[b, kv]) if (vmc and v_mean is not None) else np.zeros(d)
                a = scores(q[b, h], K_cache[b, kv, :n], scale)
                r = topth_row(a, V_cache[b, kv, :n], theta_row(theta, h, n - 1), mu,
                              vmc=vmc, renorm=renorm)
                out[b, h] = r.out; kept[b, h] = r.kept_count; beta[b, h] = r.beta
                s_rows[b][h] = r.s; k_rows[b][h] = r.keep
                union |= r.keep
            vrows[b, kv] = int(union.sum())
    return DecodeResult(out, kept, beta, vrows, s_rows, k_rows)


# ---------------------------------------------------------------------------
# [TT] §3.1, Algorithm 1, adapted to post-softmax values
# ---------------------------------------------------------------------------
def calibration_samples(Q, K, ks, scale: float, q_pos0: int):
    """Per-sequence observations of Alg. 1 for one calibration sequence.

    Q [Hq,Lq,d], K [Hkv,Lk,d]; query row i sits at position p = q_pos0 + i and
    sees keys 0..p.  Returns ``{(ki, h, p): t}`` with t the k-th largest
    post-softmax value of the row, for every k = ks[ki] with p + 1 > k.
    Prefill-style calibration uses q_pos0 = 0 and Lq = Lk; decode-style uses
    q_pos0 = Lk - 1 and Lq = 1 (the decode branch of Alg. 1).
    """
    Q = _as64(Q); K = _as64(K)
    Hq, Lq, _ = Q.shape
    g = Hq // K.shape[0]
    obs = {}
    for h in range(Hq):
        for i in range(Lq):
            p = q_pos0 + i
            s, _ = post_softmax(scores(Q[h, i], K[h // g, :p + 1], scale))
            for ki, k in enumerate(ks):
                if p + 1 > k:
                    obs[(ki, h, p)] = kth_largest(s, k)
    return obs


class Calibrator:
    """Collects the observation sets Theta_r of Alg. 1 and returns
    theta_r = mean(Theta_r) + alpha * std(Theta_r) (population std)."""

    def __init__(self, ks, Hq: int, n_rows: int):
        self.ks = [int(k) for k in ks]
        self.Hq = Hq
        self.n_rows = n_rows
        self.sets = {}   # (ki, h, p) -> list of observed values

    def observe(self, Q, K, scale: float, q_pos0: int = 0):
        for key, t in calibration_samples(Q, K, self.ks, scale, q_pos0).items():
            if key[2] < self.n_rows:
                self.sets.setdefault(key, []).append(t)

    def counts(self) -> np.ndarray:
        c = np.zeros((len(self.ks), self.Hq, self.n_rows), dtype=np.int64)
        for (ki, h, p), v in self.sets.items():
            c[ki, h, p] = len(v)
        return c

    def finalize(self, alpha: float = 0.0) -> np.ndarray:
        """theta [n_k, Hq, n_rows]; -inf where p + 1 <= k; rows with no
        observation (and p + 1 > k) copy the nearest observed row."""
        nk = len(self.ks)
        th = np.full((nk, self.Hq, self.n_rows), -np.inf)
        for ki, k in enumerate(self.ks):
            for h in range(self.Hq):
                seen = []
                for p in range(self.n_rows):
                    vals = self.sets.get((ki, h, p))
                    if vals:
                        v = np.asarray(vals, dtype=np.float64)
                        th[ki, h, p] = v.mean() + alpha * v.std()
                        seen.append(p)
                if not seen:
                    continue
                seen_arr = np.asarray(seen)
                for p in range(k, self.n_rows):       # rows with p + 1 > k
                    if (ki, h, p) in self.sets:
                        continue
                    dist = np.abs(seen_arr - p)
                    th[ki, h, p] = th[ki, h, seen_arr[int(np.argmin(dist))]]
        return th
