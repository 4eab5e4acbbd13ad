"""The oracle's pins must catch plausible mistakes.  Each case below plants one
mistake in the oracle (on the CPU, for the duration of the case only) -- a
dropped scale, an off-by-one rank or row, a flipped sign, a wrong denominator
-- then runs every pin of the three pin modules and requires at least one of
them to fail.  A planted mistake that no pin notices would mean that the pins
do not fix that part of the oracle."""
import inspect

import numpy as np
import pytest

import oracle
import oracle.mkc as M
import oracle.presoftmax as P
import oracle.serving as S
import oracle.topth as T
import test_oracle_mkc_pins
import test_oracle_pins
import test_oracle_presoftmax_pins
import test_oracle_serving_pins

PIN_MODULES = (test_oracle_pins, test_oracle_presoftmax_pins, test_oracle_serving_pins, test_oracle_mkc_pins)


def _param_sets(fn):
    marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    if not marks:
        return [{}]
    out = [{}]
    for m in marks:
        names = [n.strip() for n in m.args[0].split(",")]
        vals = [v if len(names) > 1 else (v,) for v in m.args[1]]
        out = [dict(o, **dict(zip(names, v))) for o in out for v in vals]
    return out


def failing_pins():
    """Pin cases that fail by an assertion, and those that stop with another
    error (a planted mistake must be caught by the former: the latter would
    mean the mistake broke a call signature rather than a value)."""
    failed, errors = [], []
    for mod in PIN_MODULES:
        for name, fn in inspect.getmembers(mod, inspect.isfunction):
            if not name.startswith("test_") or fn.__module__ != mod.__name__:
                continue
            for kw in _param_sets(fn):
                try:
                    fn(**kw)
                except AssertionError:
                    failed.append(f"{mod.__name__}.{name}{kw or ''}")
                except Exception as e:          # noqa: BLE001
                    errors.append(f"{mod.__name__}.{name}{kw or ''}: {type(e).__name__}: {e}")
    return failed, errors


def _patch(monkeypatch, module, name, make):
    """Replace `name` in `module` and wherever the oracle re-exports the same object."""
    orig = getattr(module, name)
    new = make(orig)
    for mod in (oracle, T, P, S, M):
        if getattr(mod, name, None) is orig:
            monkeypatch.setattr(mod, name, new)


def _kth_off_by_one(orig):
    return lambda x, k: orig(x, k + 1) if k + 1 <= len(x) else -np.inf


def _softmax_with_padding(orig):
    def post_softmax(a):
        s, lse = orig(a)
        m = float(np.max(np.asarray(a, dtype=np.float64)))
        z, pad = np.exp(lse - m), np.exp(-m)
        return s * z / (z + pad), m + np.log(z + pad)
    return post_softmax


def _calib_n_minus_one(orig):
    def finalize(self, alpha=0.0):
        th = orig(self, alpha)
        c = self.counts()
        fin = np.isfinite(th) & (c > 1)
        out = th.copy()
        out[fin] = th[fin] * c[fin] / (c[fin] - 1)
        return out
    return finalize


def _kbar_strict(orig):
    # the intervals of Appendix D as printed, [v_i, v_{i+1}) with the count of
    # elements strictly greater than theta, in place of the >= reading
    def merged_kbar(sorted_samples, thetas):
        thetas = np.asarray(thetas, dtype=np.float64)
        total, cov = np.zeros(thetas.shape), np.zeros(thetas.shape)
        for v in sorted_samples:
            inside = (v[0] <= thetas) & (thetas < v[-1])
            total += np.where(inside, v.size - np.searchsorted(v, thetas, side="right"), 0)
            cov += inside
        return np.where(cov > 0, total / np.maximum(cov, 1), np.nan)
    return merged_kbar


def _kbar_every_sample(orig):
    # samples that do not cover theta counted with what they keep (0 above
    # their range, all below it) instead of being left out of Eq. 8's mean
    def merged_kbar(sorted_samples, thetas):
        thetas = np.asarray(thetas, dtype=np.float64)
        return sum(v.size - np.searchsorted(v, thetas, side="left") for v in sorted_samples) / len(sorted_samples)
    return merged_kbar


def _inverse_smallest(orig):
    # the smallest qualifying threshold instead of the largest
    def theta_of_ks(samples, ks):
        srt = [M.sample_intervals(s) for s in samples]
        cands = np.unique(np.concatenate(srt))
        kb = M.merged_kbar(srt, cands)
        out = np.full(len(ks), -np.inf)
        for t, k in enumerate(ks):
            ok = np.flatnonzero(kb >= k)
            if ok.size:
                out[t] = cands[ok[0]]
        return out
    return theta_of_ks


MUTANTS = {
    "MKC effective k counts elements above theta only": (M, "merged_kbar", _kbar_strict),
    "MKC mean over every sample, covering or not": (M, "merged_kbar", _kbar_every_sample),
    "MKC inverse takes the smallest qualifying theta": (M, "theta_of_ks", _inverse_smallest),
    "score scale dropped": (T, "scores", lambda o: (lambda q, K, scale: o(q, K, 1.0))),
    "softmax over one unmasked padding score of 0": (T, "post_softmax", _softmax_with_padding),
    "k-th largest off by one": (T, "kth_largest", _kth_off_by_one),
    "threshold read from the previous row": (
        T, "theta_row", lambda o: (lambda tbl, h, p: o(tbl, h, max(p - 1, 0)))),
    "exact SDC renormalised over the kept set": (
        T, "row_weights", lambda o: (lambda s, keep, renorm: o(s, keep, True))),
    "VMC term with the wrong sign": (
        T, "row_output", lambda o: (lambda s, keep, V, mu, **kw: o(s, keep, V, -np.asarray(mu, float), **kw))),
    "prefix mean divided by p + 2": (
        T, "prefix_mean",
        lambda o: (lambda V: o(V) * (np.arange(1, np.asarray(V).shape[-2] + 1)
                                     / np.arange(2, np.asarray(V).shape[-2] + 2))[:, None])),
    "pre-softmax exp-threshold estimate doubled": (
        P, "pre_weights", lambda o: (lambda a, theta, *, sdc, gamma=0.05, e_tilde=0.0:
                                     o(a, theta, sdc=sdc, gamma=2 * gamma, e_tilde=e_tilde))),
    "pre-softmax threshold read from the previous row": (
        P, "table_row", lambda o: (lambda tbl, h, p: o(tbl, h, max(p - 1, 0)))),
    "discarded mass counts the k-th element": (
        P, "discarded_mass", lambda o: (lambda a, k: o(a, k - 1) if k > 1 else o(a, k) + 1.0)),
    "running mean over one row too many": (
        S, "running_mean_append",
        lambda o: (lambda mu, n_old, V: o(mu, n_old, V) * (n_old + len(V)) / (n_old + len(V) + 1))),
    "fitted theta kept for rows p + 1 = k": (
        S, "eval_theta", lambda o: (lambda coef, k, n_out, log_domain: o(coef, k - 1, n_out, log_domain))),
}


def test_pins_pass_on_the_unchanged_oracle():
    assert failing_pins() == ([], [])


@pytest.mark.parametrize("name", list(MUTANTS))
def test_a_pin_catches_the_planted_mistake(name, monkeypatch):
    module, attr, make = MUTANTS[name]
    _patch(monkeypatch, module, attr, make)
    failed, errors = failing_pins()
    assert failed, f"no pin assertion fails with the planted mistake: {name} (errors: {errors[:3]})"


def test_a_pin_catches_calibration_mean_over_n_minus_one(monkeypatch):
    monkeypatch.setattr(T.Calibrator, "finalize", _calib_n_minus_one(T.Calibrator.finalize))
    failed, errors = failing_pins()
    assert failed, f"no pin assertion fails when the calibration mean divides by n - 1 (errors: {errors[:3]})"
