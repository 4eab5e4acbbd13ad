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


@pytest.mark.parametrize("degree,min_len", [(0, 0), (1, 0), (2, 0), (3, 0), (1, 4), (2, 4)])
@pytest.mark.parametrize("log_domain", [True, False])
def test_theta_fit_and_eval(degree, min_len, log_domain):
    print(f"theta_fit degree={degree} log={log_domain} min_len_over_k={min_len}", flush=True)
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
    tt.topth_theta_fit(torch.tensor(th, device=dev), torch.tensor(cnt, device=dev), coef, ks, degree=degree,
                       log_domain=log_domain, min_len_over_k=min_len)
    out = torch.empty(n_k, Hq, n_out, dtype=torch.float32, device=dev)
    tt.topth_theta_eval(coef, ks, out, log_domain=log_domain)
    torch.cuda.synchronize()
    cg, og = coef.cpu().numpy(), out.cpu().numpy().astype(np.float64)
    for t in range(n_k):
        cr = serving.fit_theta(th[t], cnt[t] > 0, degree, log_domain, min_row=max(min_len * ks[t] - 1, 0))
        ref = serving.eval_theta(cr, ks[t], n_out, log_domain)
        for h in range(Hq):
            if h == 4:
                assert np.isnan(cg[t, h]).all() and np.isnan(cr[h]).all()
                continue
            if degree <= 2:      # a cubic in ln(p + 1) over one decade is ill-conditioned: values only
                np.testing.assert_allclose(cg[t, h], cr[h], rtol=1e-6, atol=1e-9, err_msg=f"t{t} h{h}")
            assert np.isneginf(og[t, h, :ks[t]]).all()
            np.testing.assert_allclose(og[t, h, ks[t]:], ref[h, ks[t]:], rtol=1e-5, atol=1e-30)



@pytest.mark.parametrize("dtype,Hq,Hkv,d,Lmax,lens", [
    (torch.bfloat16, 8, 2, 128, 1000, [1000, 537, 1]),       # g = 4, a single-key row
    (torch.bfloat16, 16, 2, 128, 4100, [4100, 2049]),        # g = 8, several chunks per group
    (torch.bfloat16, 16, 1, 64, 600, [600, 90]),             # g = 16 (FMA accumulation)
    (torch.float32, 8, 2, 64, 500, [500, 77]),               # row kernels: update kernel first
])
def test_decode_append_fused(dtype, Hq, Hkv, d, Lmax, lens):
    """topth_decode_append appends row n - 1 to the running mean and decodes
    with it.  Over two steps (n, then n + 1 where the cache has room; a row at
    the end of the cache starts again from the mean of its first n - 1 rows)
    the updated mean and the output equal, bit for bit, the stand-alone update
    followed by topth_decode; the mean is that of the cached rows (1e-5
    relative) and masks, counts and outputs match the oracle."""
    print(f"decode_append {dtype} Hq={Hq} Hkv={Hkv} d={d} lens={lens}", flush=True)
    from test_gpu_decode import compare_decode, decode_theta
    dev = device()
    B = len(lens)
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 11, 0, B=B, Hq=Hq, Hkv=Hkv, Lq=1, Lk=Lmax, d=d, dtype=dtype)
    q = q[:, :, 0].contiguous()
    vf = to_f64(v)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    scale = 1.0 / np.sqrt(d)
    ws_a = tt.workspace(tt.TOPTH_OP_DECODE, B, Hq, Hkv, 1, Lmax, d)
    ws_b = tt.workspace(tt.TOPTH_OP_DECODE, B, Hq, Hkv, 1, Lmax, d)

    def mean_before(b, h, n):           # rows 0..n-2; for n = 1 a value the update must ignore
        return vf[b, h, :n - 1].mean(0) if n > 1 else np.full(d, 123.0)

    mu_a = torch.tensor(np.stack([[mean_before(b, h, lens[b]) for h in range(Hkv)] for b in range(B)]),
                        dtype=torch.float32, device=dev)
    mu_b = mu_a.clone()
    steps = [lens, [min(n + 1, Lmax) for n in lens]]
    for step, lens_s in enumerate(steps):
        if step == 1:
            for b in range(B):
                if lens_s[b] == steps[0][b]:
                    for h in range(Hkv):
                        mu_a[b, h] = torch.tensor(mean_before(b, h, lens_s[b]), dtype=torch.float32)
                        mu_b[b, h] = mu_a[b, h]
        theta = decode_theta(UNIT, Hq, Hkv, d, lens_s, 24, 3, dtype, 1, n_rows=Lmax)
        th = torch.tensor(theta, dtype=torch.float32, device=dev)
        ln = torch.tensor(lens_s, dtype=torch.int32, device=dev)
        out_a = torch.empty(B, Hq, d, dtype=dtype, device=dev)
        out_b = torch.empty_like(out_a)
        kc = torch.full((B, Hq), -7, dtype=torch.int32, device=dev)
        bt = torch.full((B, Hq), -7.0, dtype=torch.float32, device=dev)
        vr = torch.full((B, Hkv), -7, dtype=torch.int32, device=dev)
        km = torch.zeros((B, Hq, Lmax), dtype=torch.uint8, device=dev)
        tt.topth_decode_append(qd, kd, vd, ln, th, out_a, ws_a, mu_a, scale=scale, flags=tt.TOPTH_VMC,
                               kept_count=kc, beta=bt, vrows_read=vr, kept_mask=km)
        old = torch.tensor([n - 1 for n in lens_s], dtype=torch.int32, device=dev)
        tt.topth_vmean_append(vd, old, ln, mu_b)
        tt.topth_decode(qd, kd, vd, ln, th, out_b, ws_b, scale=scale, flags=tt.TOPTH_VMC, v_mean=mu_b)
        torch.cuda.synchronize()
        assert int(ws_a[:4].view(torch.int32)[0].item()) == 0, "exchange wait timed out"
        assert torch.equal(mu_a, mu_b), "fused and stand-alone running means differ"
        assert torch.equal(out_a, out_b), "fused and two-call outputs differ"
        exact = np.stack([[vf[b, h, :lens_s[b]].mean(0) for h in range(Hkv)] for b in range(B)])
        mu_g = mu_a.cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(mu_g, exact, rtol=1e-5, atol=1e-6)
        g = dict(out=out_a.float().cpu().numpy(), kc=kc.cpu().numpy(), beta=bt.cpu().numpy(),
                 vr=vr.cpu().numpy(), mask=km.cpu().numpy().astype(bool))
        compare_decode(g, q, k, v, lens_s, theta, mu_g, tt.TOPTH_VMC, dtype)


def test_decode_append_steps_in_a_graph():
    """Three generation steps (n, n + 1, n + 2 cached rows) of
    topth_decode_append captured in one HIP graph: every replay (the running
    mean reset eagerly before each, with synchronisations between) gives the
    same outputs and the same running mean, bit for bit, as the steps run
    eagerly; the workspace slots left empty by each step serve the next."""
    print("decode_append graph", flush=True)
    from test_gpu_decode import decode_theta
    dev = device()
    Hq, Hkv, d, Lmax, B = 8, 2, 128, 700, 2
    base = [600, 333]
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 12, 0, B=B, Hq=Hq, Hkv=Hkv, Lq=1, Lk=Lmax, d=d,
                               dtype=torch.bfloat16)
    q = q[:, :, 0].contiguous()
    vf = to_f64(v)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    steps = [[n + s for n in base] for s in range(3)]
    theta = torch.tensor(decode_theta(UNIT, Hq, Hkv, d, sum(steps, []), 24, 2, torch.bfloat16, 1, n_rows=Lmax),
                         dtype=torch.float32, device=dev)
    lens = [torch.tensor(st, dtype=torch.int32, device=dev) for st in steps]
    mu0 = torch.tensor(np.stack([[vf[b, h, :base[b] - 1].mean(0) for h in range(Hkv)] for b in range(B)]),
                       dtype=torch.float32, device=dev)
    mu = mu0.clone()
    outs = [torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev) for _ in steps]
    ws = tt.workspace(tt.TOPTH_OP_DECODE, B, Hq, Hkv, 1, Lmax, d)

    def run():
        for s in range(len(steps)):
            tt.topth_decode_append(qd, kd, vd, lens[s], theta, outs[s], ws, mu, scale=1.0 / np.sqrt(d),
                                   flags=tt.TOPTH_VMC)

    run()                                      # eager reference
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32)[0].item()) == 0, "exchange wait timed out"
    mu_e, out_e = mu.clone(), [o.clone() for o in outs]
    exact = np.stack([[vf[b, h, :steps[-1][b]].mean(0) for h in range(Hkv)] for b in range(B)])
    np.testing.assert_allclose(mu_e.cpu().numpy().astype(np.float64), exact, rtol=1e-5, atol=1e-6)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        mu.copy_(mu0)
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32)[0].item()) == 0, "exchange wait timed out"
        assert torch.equal(mu, mu_e), f"replay {rep}: running mean"
        for s in range(len(steps)):
            assert torch.equal(outs[s], out_e[s]), f"replay {rep} step {s}"
