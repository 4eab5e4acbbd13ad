"""Float64 reference of pre-softmax Top-theta with the three softmax-denominator
compensation estimates (test infrastructure only).

Source: "Top-Theta Attention: Sparsifying Transformers by Compensated
Thresholding" (arXiv 2502.08363), cited as [TT].  Algorithm 1 of [TT] §3.1 in
its printed form calibrates thresholds on the scores a themselves (pre-softmax);
§3.2.1 (Eq. 4) then approximates the post-softmax result from the pre-softmax
selection by the factor R / (R + E~), with three estimates of E~.

Readings of steps the paper leaves open (the shared ones -- 1/sqrt(d) and the
causal mask, k-th largest for the garbled quantile, ">=", row ids, nearest
calibrated row, GQA -- are those of ``oracle.topth``):

* Keep rule: a_j >= theta (theta in score units); theta = -inf keeps all.
* Eq. 4 frame: R = sum over kept j of exp(a_j - m) and E = the same sum over
  the discarded j, with m = max over all j of a_j (the maximum subtracted in
  softmax).  Kept weights are softmax over the kept scores times R / (R + E~),
  i.e. exp(a_j - m) / (R + E~).
* E~ estimates ([TT] §3.2.1 items 1-3):
    - "exact":   E~ = E;
    - "expth":   E~ = gamma * (n - k~) * exp(theta - m), n = keys of the row,
                 k~ = kept count, gamma = 0.05 in [TT];
    - "offline": E~ = a static value per (head, row) calibrated like theta:
                 the mean over calibration sequences of the discarded mass E of
                 the row's top-k selection (the set theta approximates), in the
                 same frame (relative to the row maximum);
    - "none":    E~ = 0 (plain softmax over the kept set, no compensation).
* VMC ([TT] §3.2.2 case (ii), pre-softmax followed by SDC): beta = 1 - sum of
  the kept weights = E~ / (R + E~); out += beta * mu.  With "none" the weights
  sum to one and beta = 0.
* A row whose denominator R + E~ is zero (nothing kept and E~ = 0) outputs zero
  with beta = 0; a row that keeps nothing but has E~ > 0 outputs beta * mu with
  beta = 1.
* Offline E~ for rows with p + 1 <= k is 0 (every element is kept, nothing is
  discarded); rows no calibration sequence reached copy the nearest calibrated
  row, as theta does.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .topth import Calibrator, _as64, kth_largest, prefix_mean, scores, theta_row

SDC_MODES = ("exact", "expth", "offline", "none")


@dataclass
class PreRowResult:
    out: np.ndarray       # [d]
    keep: np.ndarray      # [n] bool
    kept_count: int       # k~
    beta: float           # VMC mass (Eq. 6 with the SDC weights)
    a: np.ndarray         # [n] scores (for ambiguity bands)
    weights: np.ndarray   # [n] weights of the kept keys (0 elsewhere)


def pre_weights(a, theta: float, *, sdc: str, gamma: float = 0.05, e_tilde: float = 0.0):
    """Keep mask, weights and beta of one row under pre-softmax Top-theta:
    keep = a >= theta, then ``pre_weights_for_mask``."""
    a = _as64(a)
    keep = a >= theta
    w, beta = pre_weights_for_mask(a, keep, theta, sdc=sdc, gamma=gamma, e_tilde=e_tilde)
    return keep, w, beta


def pre_weights_for_mask(a, keep, theta: float, *, sdc: str, gamma: float = 0.05,
                         e_tilde: float = 0.0):
    """Weights and beta for a given kept set: Eq. 4, softmax over the kept
    scores times R / (R + E~), with E~ chosen by ``sdc`` (see the module notes)."""
    if sdc not in SDC_MODES:
        raise ValueError(f"unknown SDC estimate {sdc!r}")
    a = _as64(a)
    keep = np.asarray(keep, dtype=bool)
    n = a.size
    kt = int(keep.sum())
    m = float(a.max())
    e = np.exp(a - m)
    R = float(e[keep].sum())
    E = float(e[~keep].sum())
    if sdc == "exact":
        Et = E
    elif sdc == "expth":
        with np.errstate(over="ignore"):
            Et = float(gamma) * (n - kt) * float(np.exp(theta - m)) if n > kt else 0.0
    elif sdc == "offline":
        Et = float(e_tilde)
    else:
        Et = 0.0
    w = np.zeros(n)
    if R + Et > 0.0:
        if kt:
            w[keep] = (e[keep] / R) * (R / (R + Et))     # softmax(a~) * R / (R + E~)
        beta = 0.0 if sdc == "none" else 1.0 - R / (R + Et)   # = E~ / (R + E~)
    else:
        beta = 0.0
    return w, beta


def pre_row(a, V, theta: float, mu, *, sdc: str, vmc: bool, gamma: float = 0.05,
            e_tilde: float = 0.0) -> PreRowResult:
    """One attention row: threshold a >= theta, SDC estimate, VMC (Eq. 4-7)."""
    keep, w, beta = pre_weights(a, theta, sdc=sdc, gamma=gamma, e_tilde=e_tilde)
    out = w @ _as64(V)
    if vmc:
        out = out + beta * _as64(mu)
    return PreRowResult(out=out, keep=keep, kept_count=int(keep.sum()), beta=beta, a=_as64(a),
                        weights=w)


def table_row(table, h: int, p: int) -> float:
    """Entry of a [Hq, R] table at row p; rows past the table use its last row."""
    return theta_row(table, h, p)


@dataclass
class PrePrefillResult:
    out: np.ndarray
    kept_count: np.ndarray
    beta: np.ndarray
    a: list
    keep: list


def prefill_pre(Q, K, V, theta, scale: float, *, sdc: str, vmc: bool, gamma: float = 0.05,
                e_tilde=None, rows=None, keep_rows: bool = False) -> PrePrefillResult:
    """Causal pre-softmax Top-theta prefill.  Q [B,Hq,L,d]; K, V [B,Hkv,L,d];
    theta and e_tilde [Hq,R].  ``rows`` restricts the work to (b, h, p)."""
    Q = _as64(Q); K = _as64(K); V = _as64(V)
    B, Hq, L, d = Q.shape
    g = Hq // K.shape[1]
    out = np.full((B, Hq, L, d), np.nan)
    kept = np.full((B, Hq, L), -1, dtype=np.int64)
    beta = np.full((B, Hq, L), np.nan)
    a_rows = [[[None] * L for _ in range(Hq)] for _ in range(B)]
    k_rows = [[[None] * L for _ in range(Hq)] for _ in range(B)]
    mu_cache = {}
    if rows is None:
        rows = [(b, h, p) for b in range(B) for h in range(Hq) for p in range(L)]
    for (b, h, p) in rows:
        kv = h // g
        mu = np.zeros(d)
        if vmc:
            if (b, kv) not in mu_cache:
                mu_cache[(b, kv)] = prefix_mean(V[b, kv])
            mu = mu_cache[(b, kv)][p]
        a = scores(Q[b, h, p], K[b, kv, :p + 1], scale)
        et = table_row(e_tilde, h, p) if e_tilde is not None else 0.0
        r = pre_row(a, V[b, kv, :p + 1], table_row(theta, h, p), mu, sdc=sdc, vmc=vmc, gamma=gamma,
                    e_tilde=et)
        out[b, h, p] = r.out
        kept[b, h, p] = r.kept_count
        beta[b, h, p] = r.beta
        if keep_rows:
            a_rows[b][h][p] = r.a
            k_rows[b][h][p] = r.keep
    return PrePrefillResult(out, kept, beta, a_rows, k_rows)


@dataclass
class PreDecodeResult:
    out: np.ndarray
    kept_count: np.ndarray
    beta: np.ndarray
    vrows_read: np.ndarray
    a: list
    keep: list


def decode_pre(q, K_cache, V_cache, seq_lens, theta, v_mean, scale: float, *, sdc: str, vmc: bool,
               gamma: float = 0.05, e_tilde=None) -> PreDecodeResult:
    """One decoding step under pre-softmax Top-theta; row id n_b - 1."""
    q = _as64(q); K_cache = _as64(K_cache); V_cache = _as64(V_cache)
    B, Hq, d = q.shape
    Hkv = K_cache.shape[1]
    g = Hq // Hkv
    out = np.zeros((B, Hq, d)); kept = np.zeros((B, Hq), dtype=np.int64)
    beta = np.zeros((B, Hq)); vrows = np.zeros((B, Hkv), dtype=np.int64)
    a_rows = [[None] * Hq for _ in range(B)]
    k_rows = [[None] * Hq for _ in range(B)]
    for b in range(B):
        n = int(seq_lens[b])
        for kv in range(Hkv):
            union = np.zeros(n, dtype=bool)
            for h in range(kv * g, (kv + 1) * g):
                mu = _as64(v_mean[b, kv]) if vmc else np.zeros(d)
                a = scores(q[b, h], K_cache[b, kv, :n], scale)
                et = table_row(e_tilde, h, n - 1) if e_tilde is not None else 0.0
                r = pre_row(a, V_cache[b, kv, :n], table_row(theta, h, n - 1), mu, sdc=sdc, vmc=vmc,
                            gamma=gamma, e_tilde=et)
                out[b, h] = r.out; kept[b, h] = r.kept_count; beta[b, h] = r.beta
                a_rows[b][h] = r.a; k_rows[b][h] = r.keep
                union |= r.keep
            vrows[b, kv] = int(union.sum())
    return PreDecodeResult(out, kept, beta, vrows, a_rows, k_rows)


# ---------------------------------------------------------------------------
# Algorithm 1 in its printed (pre-softmax) form, plus the offline E~ estimate
# ---------------------------------------------------------------------------
def discarded_mass(a, k: int) -> float:
    """E of the top-k selection of one row: sum over the elements outside the k
    largest (counted with multiplicity) of exp(a - max a) ([TT] Eq. 4 frame)."""
    srt = np.sort(_as64(a))[::-1]
    return float(np.exp(srt[k:] - srt[0]).sum())


def calibration_samples_pre(Q, K, ks, scale: float, q_pos0: int):
    """Per-sequence observations for one calibration sequence: ``{(ki, h, p):
    (t, E)}`` with t the k-th largest score a of the row and E the discarded
    mass of its top-k, for every k = ks[ki] with p + 1 > k."""
    Q = _as64(Q); K = _as64(K)
    Hq, Lq, _ = Q.shape
    g = Hq // K.shape[0]
    obs = {}
    for h in range(Hq):
        for i in range(Lq):
            p = q_pos0 + i
            a = scores(Q[h, i], K[h // g, :p + 1], scale)
            for ki, k in enumerate(ks):
                if p + 1 > k:
                    obs[(ki, h, p)] = (kth_largest(a, k), discarded_mass(a, k))
    return obs


class PreCalibrator:
    """Alg. 1 on scores: theta_r = mean + alpha * std of the k-th largest score,
    and the offline E~_r = mean of the discarded mass, with the same row rules."""

    def __init__(self, ks, Hq: int, n_rows: int):
        self.theta = Calibrator(ks, Hq, n_rows)
        self.etilde = Calibrator(ks, Hq, n_rows)
        self.ks = self.theta.ks
        self.n_rows = n_rows

    def observe(self, Q, K, scale: float, q_pos0: int = 0):
        for key, (t, E) in calibration_samples_pre(Q, K, self.ks, scale, q_pos0).items():
            if key[2] < self.n_rows:
                self.theta.sets.setdefault(key, []).append(t)
                self.etilde.sets.setdefault(key, []).append(E)

    def counts(self) -> np.ndarray:
        return self.theta.counts()

    def finalize(self, alpha: float = 0.0) -> np.ndarray:
        """theta [n_k, Hq, n_rows] in score units (-inf where p + 1 <= k)."""
        return self.theta.finalize(alpha)

    def finalize_etilde(self) -> np.ndarray:
        """E~ [n_k, Hq, n_rows]: mean discarded mass; 0 where nothing is
        discarded (p + 1 <= k) or no row of the head was observed."""
        e = self.etilde.finalize(0.0)
        return np.where(np.isfinite(e), e, 0.0)
