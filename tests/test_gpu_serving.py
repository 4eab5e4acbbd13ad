"""Decode-serving helpers on the GPU (through the C ABI) against the oracle:
the running V mean under KV-cache appends, and fitted thresholds."""
import numpy as np
import pytest
import torch

import calibrated_threshold_pruning_amd as tt
from oracle import serving
from synth import CONFIG_IDS, ROLE_TEST, attention_inputs, to_f64
from parity import device

pytestmark = pytest.mark.gpu

UNIT = CONFIG_IDS["unit"]


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_vmean_append_chain(dtype, d):
    """Append ragged blocks of rows step by step (one batch element starts
    empty, one gets nothing in some steps); after every step v_mean equals the
    mean of the cached rows (float32 storage between steps: 1e-5 relative)."""
    print(f"vmean_append {dtype} d={d}", flush=True)
    dev = device()
    B, Hkv, Lmax = 3, 2, 900
    _, _, v = attention_inputs(UNIT, ROLE_TEST, 7, 0, B=B, Hq=Hkv, Hkv=Hkv, Lq=1, Lk=Lmax, d=d, dtype=dtype)
    vd = v.to(dev)
    vf = to_f64(v)
    steps = [[5, 0, 1], [1, 17, 1], [300, 1, 0], [1, 1, 1], [200, 400, 7], [1, 0, 890]]
    lens = np.zeros(B, dtype=np.int64)
    mu = torch.zeros(B, Hkv, d, dtype=torch.float32, device=dev)
    mu_ref = [[None] * Hkv for _ in range(B)]
    for st in steps:
        new = lens + np.array(st)
        old_t = torch.tensor(lens, dtype=torch.int32, device=dev)
        new_t = torch.tensor(np.maximum(new, 1), dtype=torch.int32, device=dev)
        tt.topth_vmean_append(vd, old_t, new_t, mu)
        torch.cuda.synchronize()
        got = mu.cpu().numpy().astype(np.float64)
        for b in range(B):
            if new[b] == 0:
                continue
            for h in range(Hkv):
                mu_ref[b][h] = serving.running_mean_append(mu_ref[b][h], int(lens[b]),
                                                           vf[b, h, lens[b]:new[b]])
                exact = vf[b, h, :new[b]].mean(axis=0)
                np.testing.assert_allclose(mu_ref[b][h], exact, rtol=1e-12, atol=1e-14)
                np.testing.assert_allclose(got[b, h], exact, rtol=1e-5, atol=1e-6,
                                           err_msg=f"b{b} h{h} n{new[b]}")
        lens = new


def _noisy_table(rng, n_k, Hq, R, log_domain):
    x = np.log(np.arange(R) + 1.0)
    if log_domain:      # post-softmax: about a power of the row length
        th = np.exp(-1.1 * x[None, None, :] + 0.3 + 0.03 * rng.standard_normal((n_k, Hq, R)))
    else:               # pre-softmax: scores growing slowly with the row length
        th = 1.0 + 0.35 * x[None, None, :] + 0.02 * rng.standard_normal((n_k, Hq, R))
    return th.astype(np.float32)


@pytest.mark.parametrize("degree", [0, 1, 2, 3])
@pytest.mark.parametrize("log_domain", [True, False])
def test_theta_fit_and_eval(degree, log_domain):
    print(f"theta_fit degree={degree} log={log_domain}", flush=True)
    dev = device()
    rng = np.random.default_rng(degree + 10 * log_domain)
    n_k, Hq, R, n_out = 2, 5, 4096, 32768
    ks = [64, 256]
    th = _noisy_table(rng, n_k, Hq, R, log_domain)
    cnt = np.zeros((n_k, Hq, R), dtype=np.int32)
    probes = np.unique(np.round(np.geomspace(300, R - 1, 24)).astype(int))
    cnt[:, :, probes] = 3
    cnt[:, 4, :] = 0
    cnt[:, 4, probes[:degree]] = 1          # too few rows for the degree: NaN coefficients
    if log_domain:
        th[0, 1, probes[3]] = -1.0          # not usable in the log domain
    coef = torch.empty(n_k, Hq, degree + 1, dtype=torch.float64, device=dev)
    tt.topth_theta_fit(torch.tensor(th, device=dev), torch.tensor(cnt, device=dev), coef, degree=degree,
                       log_domain=log_domain)
    out = torch.empty(n_k, Hq, n_out, dtype=torch.float32, device=dev)
    tt.topth_theta_eval(coef, ks, out, log_domain=log_domain)
    torch.cuda.synchronize()
    cg, og = coef.cpu().numpy(), out.cpu().numpy().astype(np.float64)
    for t in range(n_k):
        cr = serving.fit_theta(th[t], cnt[t] > 0, degree, log_domain)
        ref = serving.eval_theta(cr, ks[t], n_out, log_domain)
        for h in range(Hq):
            if h == 4:
                assert np.isnan(cg[t, h]).all() and np.isnan(cr[h]).all()
                continue
            if degree <= 2:      # a cubic in ln(p + 1) over one decade is ill-conditioned: values only
                np.testing.assert_allclose(cg[t, h], cr[h], rtol=1e-6, atol=1e-9, err_msg=f"t{t} h{h}")
            assert np.isneginf(og[t, h, :ks[t]]).all()
            np.testing.assert_allclose(og[t, h, ks[t]:], ref[h, ks[t]:], rtol=1e-5, atol=1e-30)
