"""Pre-softmax Top-theta parity: HIP path (through the C ABI) against the CPU
oracle (``oracle.presoftmax``), for calibration (k-th largest score and the
discarded mass E of the top-k), prefill and decode with the exact,
exp-threshold, offline-calibrated and no-compensation estimates of E~.

Protocol (scores instead of post-softmax values):
* an element is ambiguous when |a - theta| <= 1e-5 * max(1, |theta|): a score
  error of 1e-5 is a relative error of 1e-5 in exp(a - lse), the band the
  post-softmax compare uses; masks and counts agree exactly elsewhere, and the
  oracle output is re-evaluated with the GPU's decisions on ambiguous elements;
* outputs: bf16 1e-2 max-abs beyond the output's own rounding, f32 1e-5
  relative per row; beta to 1e-5;
* calibrated thresholds to 1e-5 * max(1, |theta|) (same score-error argument);
  the E~ table to 1e-4 relative: each term exp(a - max) carries the score error
  (1e-5 relative at most) and float32 sums of up to a few thousand terms add
  about 1e-5 more.
"""
import numpy as np
import pytest
import torch

import calibrated_threshold_pruning_amd as tt
from oracle import presoftmax as pre
from synth import CONFIG_IDS, ROLE_CALIB, ROLE_TEST, attention_inputs, batch_of_sequences, to_f64
from parity import check_out, device

pytestmark = pytest.mark.gpu

UNIT = CONFIG_IDS["unit"]
GAMMA = 0.05
MODES = {"exact": 0, "expth": tt.TOPTH_SDC_EXPTH, "offline": tt.TOPTH_SDC_OFFLINE,
         "none": tt.TOPTH_SDC_NONE}


def ambiguous(a, theta):
    a = np.asarray(a, dtype=np.float64)
    if not np.isfinite(theta):
        return np.zeros(a.shape, dtype=bool)
    return np.abs(a - theta) <= 1e-5 * max(1.0, abs(theta))


def check_pre_row(gk, a, theta, V, mu, sdc, et, vmc, out_g, beta_g, dtype, where):
    """Mask parity outside the band, then output and beta against the oracle
    evaluated on the GPU's kept set."""
    gk = np.asarray(gk, dtype=bool)
    amb = ambiguous(a, theta)
    bad = (gk != (a >= theta)) & ~amb
    assert not bad.any(), f"mask mismatch {where}: {np.flatnonzero(bad)[:10]}"
    w, beta = pre.pre_weights_for_mask(a, gk, theta, sdc=sdc, gamma=GAMMA, e_tilde=et)
    ref = w @ V + (beta * mu if vmc else 0.0)
    check_out(out_g, ref, dtype, where)
    assert abs(beta_g - beta) <= 1e-5, (where, beta_g, beta)
    return int(amb.sum())


def calib_tables(cfg, Hq, Hkv, L, d, k, n_seq, dtype, q_pos0=0, Lq=None):
    """Oracle theta and E~ [Hq, L] from n_seq calibration sequences."""
    Lq = L if Lq is None else Lq
    cal = pre.PreCalibrator([k], Hq, L)
    q, kk, _ = batch_of_sequences(cfg, ROLE_CALIB, 3, 0, n_seq, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d,
                                  dtype=dtype)
    for s in range(n_seq):
        cal.observe(to_f64(q[s][:, q_pos0:q_pos0 + Lq]), to_f64(kk[s]), 1.0 / np.sqrt(d), q_pos0)
    return cal.finalize()[0], cal.finalize_etilde()[0]


# --------------------------------------------------------------- calibration
@pytest.mark.parametrize("dtype,Hq,Hkv,L,d,ks,q_pos0,Lq", [
    (torch.bfloat16, 4, 2, 300, 128, [8, 32, 100], 0, 300),   # column kernel, prefill-style
    (torch.bfloat16, 8, 2, 1500, 64, [64], 1499, 1),          # column kernel, decode-style
    (torch.float32, 2, 1, 200, 64, [16, 199], 0, 200),        # row kernel
    (torch.bfloat16, 2, 1, 2100, 64, [64, 700], 0, 2100),    # 8 columns of 2 waves each
    (torch.bfloat16, 4, 1, 5000, 128, [64, 300], 4999, 1),   # 4 columns of 4 waves each
])
def test_calibrate_pre_parity(dtype, Hq, Hkv, L, d, ks, q_pos0, Lq):
    print(f"calibrate_pre {dtype} Hq={Hq} L={L} ks={ks} q_pos0={q_pos0}", flush=True)
    dev = device()
    S = 3
    q, kk, _ = batch_of_sequences(UNIT, ROLE_CALIB, 5, 0, S, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d, dtype=dtype)
    q = q[:, :, q_pos0:q_pos0 + Lq].contiguous()
    scale = 1.0 / np.sqrt(d)
    nk = len(ks)
    s1 = torch.zeros(nk, Hq, L, dtype=torch.float64, device=dev)
    s2 = torch.zeros_like(s1)
    es = torch.zeros_like(s1)
    cnt = torch.zeros(nk, Hq, L, dtype=torch.int32, device=dev)
    ws = tt.workspace(tt.TOPTH_OP_CALIBRATE_PRE_E, S, Hq, Hkv, Lq, L, d, nk)
    tt.topth_calibrate_pre(q.to(dev), kk.to(dev), ks, s1, s2, cnt, ws, scale=scale, q_pos0=q_pos0, esum=es)
    th = torch.empty(nk, Hq, L, dtype=torch.float32, device=dev)
    et = torch.empty_like(th)
    tt.topth_calibrate_finalize(s1, s2, cnt, ks, th)
    tt.topth_calibrate_finalize_etilde(es, cnt, ks, et)
    torch.cuda.synchronize()
    cal = pre.PreCalibrator(ks, Hq, L)
    for s in range(S):
        cal.observe(to_f64(q[s]), to_f64(kk[s]), scale, q_pos0)
    th_ref, et_ref = cal.finalize(), cal.finalize_etilde()
    assert np.array_equal(cnt.cpu().numpy(), cal.counts())
    thg = th.cpu().numpy().astype(np.float64)
    etg = et.cpu().numpy().astype(np.float64)
    fin = np.isfinite(th_ref)
    assert np.array_equal(np.isfinite(thg), fin)
    err = np.abs(thg[fin] - th_ref[fin]) / np.maximum(1.0, np.abs(th_ref[fin]))
    assert err.max() <= 1e-5, err.max()
    assert (etg[~fin] == 0).all()
    rel = np.abs(etg - et_ref) / np.maximum(np.abs(et_ref), 1e-30)
    assert rel[et_ref > 0].max() <= 1e-4, rel[et_ref > 0].max()
    assert (etg[et_ref == 0] == 0).all()


@pytest.mark.parametrize("Hq,Hkv,L,d,ks", [(4, 2, 300, 128, [1, 8, 100, 299]), (16, 1, 200, 64, [16, 64])])
def test_calibrate_pre_tiled(Hq, Hkv, L, d, ks):
    """Pre-softmax calibration of whole causal prefills without the discarded
    mass takes the tiled kernel (the k-th largest scores): four targets, from
    the row maximum to L - 1, and 16 query heads per KV head."""
    print(f"calibrate_pre tiled Hq={Hq} Hkv={Hkv} L={L} ks={ks}", flush=True)
    dev = device()
    S = 3
    q, kk, _ = batch_of_sequences(UNIT, ROLE_CALIB, 6, 0, S, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    scale = 1.0 / np.sqrt(d)
    nk = len(ks)
    s1 = torch.zeros(nk, Hq, L, dtype=torch.float64, device=dev)
    s2 = torch.zeros_like(s1)
    cnt = torch.zeros(nk, Hq, L, dtype=torch.int32, device=dev)
    ws = tt.workspace(tt.TOPTH_OP_CALIBRATE, S, Hq, Hkv, L, L, d, nk)
    tt.topth_calibrate_pre(q.to(dev), kk.to(dev), ks, s1, s2, cnt, ws, scale=scale, q_pos0=0)
    th = torch.empty(nk, Hq, L, dtype=torch.float32, device=dev)
    tt.topth_calibrate_finalize(s1, s2, cnt, ks, th)
    torch.cuda.synchronize()
    cal = pre.PreCalibrator(ks, Hq, L)
    for s in range(S):
        cal.observe(to_f64(q[s]), to_f64(kk[s]), scale, 0)
    th_ref = cal.finalize()
    assert np.array_equal(cnt.cpu().numpy(), cal.counts())
    thg = th.cpu().numpy().astype(np.float64)
    fin = np.isfinite(th_ref)
    assert np.array_equal(np.isfinite(thg), fin)
    err = np.abs(thg[fin] - th_ref[fin]) / np.maximum(1.0, np.abs(th_ref[fin]))
    assert err.max() <= 1e-5, err.max()


# ------------------------------------------------------------------ prefill
def run_prefill_pre(q, k, v, theta, et, flags, dev):
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    out = torch.empty(B, Hq, L, d, dtype=q.dtype, device=dev)
    kc = torch.full((B, Hq, L), -7, dtype=torch.int32, device=dev)
    bt = torch.full((B, Hq, L), -7.0, dtype=torch.float32, device=dev)
    km = torch.zeros((B, Hq, L, L), dtype=torch.uint8, device=dev) if L <= 1024 else None
    ws = tt.workspace(tt.TOPTH_OP_PREFILL, B, Hq, Hkv, L, L, d) if flags & tt.TOPTH_VMC else None
    tt.topth_prefill_pre(q.to(dev), k.to(dev), v.to(dev),
                         torch.tensor(theta, dtype=torch.float32, device=dev), out,
                         scale=1.0 / np.sqrt(d), flags=flags, gamma=GAMMA,
                         e_tilde=torch.tensor(et, dtype=torch.float32, device=dev),
                         kept_count=kc, beta=bt, kept_mask=km, ws=ws)
    torch.cuda.synchronize()
    return (out.float().cpu().numpy(), kc.cpu().numpy(), bt.cpu().numpy(),
            None if km is None else km.cpu().numpy().astype(bool))


def compare_prefill_pre(q, k, v, theta, et, sdc, vmc, g, dtype, rows):
    out_g, kc_g, bt_g, km_g = g
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    B, Hq, L, d = qf.shape
    G = Hq // kf.shape[1]
    scale = 1.0 / np.sqrt(d)
    mu_cache = {}
    for (b, h, p) in rows:
        kv = h // G
        a = (kf[b, kv, :p + 1] @ qf[b, h, p]) * scale
        thv = pre.table_row(theta, h, p)
        if km_g is not None:
            gk = km_g[b, h, p, :p + 1]
        else:                        # no byte mask at this size: the count must match exactly
            gk = a >= thv
            assert not ambiguous(a, thv).any()
        assert kc_g[b, h, p] == gk.sum(), (b, h, p)
        mu = np.zeros(d)
        if vmc:
            if (b, kv) not in mu_cache:
                mu_cache[(b, kv)] = pre.prefix_mean(vf[b, kv])
            mu = mu_cache[(b, kv)][p]
        check_pre_row(gk, a, thv, vf[b, kv, :p + 1], mu, sdc, pre.table_row(et, h, p), vmc,
                      out_g[b, h, p], bt_g[b, h, p], dtype, f"b{b} h{h} p{p}")


@pytest.mark.parametrize("sdc", list(MODES))
@pytest.mark.parametrize("vmc", [False, True])
def test_prefill_pre_bf16_modes(sdc, vmc):
    print(f"prefill_pre bf16 sdc={sdc} vmc={vmc}", flush=True)
    dev = device()
    Hq, Hkv, L, d = 8, 2, 300, 128
    theta, et = calib_tables(UNIT, Hq, Hkv, L, d, 24, 3, torch.bfloat16)
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 3, 0, B=2, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d,
                               dtype=torch.bfloat16)
    flags = MODES[sdc] | (tt.TOPTH_VMC if vmc else 0)
    g = run_prefill_pre(q, k, v, theta, et, flags, dev)
    rows = [(b, h, p) for b in range(2) for h in range(Hq) for p in range(L)]
    compare_prefill_pre(q, k, v, theta, et, sdc, vmc and sdc != "none", g, torch.bfloat16, rows)


@pytest.mark.parametrize("Hq,Hkv,L,d", [(2, 1, 257, 64), (8, 8, 97, 128), (16, 2, 130, 128), (4, 2, 64, 64)])
def test_prefill_pre_bf16_shapes(Hq, Hkv, L, d):
    print(f"prefill_pre bf16 Hq={Hq} Hkv={Hkv} L={L} d={d}", flush=True)
    dev = device()
    theta, et = calib_tables(UNIT, Hq, Hkv, L, d, 16, 2, torch.bfloat16)
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 3, 1, B=1, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d,
                               dtype=torch.bfloat16)
    for sdc in ("expth", "offline"):
        flags = MODES[sdc] | tt.TOPTH_VMC
        g = run_prefill_pre(q, k, v, theta, et, flags, dev)
        rows = [(0, h, p) for h in range(Hq) for p in range(L)]
        compare_prefill_pre(q, k, v, theta, et, sdc, True, g, torch.bfloat16, rows)


@pytest.mark.parametrize("Hq,Hkv,L,d", [(8, 2, 300, 128), (4, 1, 200, 64)])
def test_prefill_pre_benchmark_form_all_rows(Hq, Hkv, L, d):
    """The kernel form the benchmark times: float16 P V (workspace given), no
    byte mask, no VMC.  Every row with no element in the ambiguity band is
    checked element by element against the oracle; the others by their count,
    which must lie between the strict and the banded count."""
    print(f"prefill_pre benchmark form Hq={Hq} Hkv={Hkv} L={L} d={d}", flush=True)
    dev = device()
    theta, et = calib_tables(UNIT, Hq, Hkv, L, d, 16, 2, torch.bfloat16)
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 3, 5, B=1, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d,
                               dtype=torch.bfloat16)
    qf, kf = to_f64(q), to_f64(k)
    for sdc in ("expth", "exact"):
        out = torch.empty(1, Hq, L, d, dtype=q.dtype, device=dev)
        kc = torch.full((1, Hq, L), -7, dtype=torch.int32, device=dev)
        bt = torch.full((1, Hq, L), -7.0, dtype=torch.float32, device=dev)
        ws = tt.workspace(tt.TOPTH_OP_PREFILL, 1, Hq, Hkv, L, L, d)
        tt.topth_prefill_pre(q.to(dev), k.to(dev), v.to(dev), torch.tensor(theta, dtype=torch.float32, device=dev),
                             out, scale=1.0 / np.sqrt(d), flags=MODES[sdc], gamma=GAMMA,
                             e_tilde=torch.tensor(et, dtype=torch.float32, device=dev), kept_count=kc, beta=bt,
                             ws=ws)
        torch.cuda.synchronize()
        g = (out.float().cpu().numpy(), kc.cpu().numpy(), bt.cpu().numpy(), None)
        ok = []
        for h in range(Hq):
            for p in range(L):
                a = (kf[0, h // (Hq // Hkv), :p + 1] @ qf[0, h, p]) / np.sqrt(d)
                thv = pre.table_row(theta, h, p)
                amb = ambiguous(a, thv)
                if amb.any():
                    lo = int(((a >= thv) & ~amb).sum())
                    assert lo <= g[1][0, h, p] <= lo + int(amb.sum()), (h, p)
                else:
                    ok.append((0, h, p))
        assert len(ok) >= 0.9 * Hq * L
        compare_prefill_pre(q, k, v, theta, et, sdc, False, g, torch.bfloat16, ok)


@pytest.mark.parametrize("sdc", list(MODES))
def test_prefill_pre_f32(sdc):
    print(f"prefill_pre f32 sdc={sdc}", flush=True)
    dev = device()
    Hq, Hkv, L, d = 2, 1, 256, 64
    theta, et = calib_tables(UNIT, Hq, Hkv, L, d, 32, 4, torch.float32)
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 3, 2, B=2, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d,
                               dtype=torch.float32)
    flags = MODES[sdc] | tt.TOPTH_VMC
    g = run_prefill_pre(q, k, v, theta, et, flags, dev)
    rows = [(b, h, p) for b in range(2) for h in range(Hq) for p in range(L)]
    compare_prefill_pre(q, k, v, theta, et, sdc, sdc != "none", g, torch.float32, rows)


@pytest.mark.parametrize("sdc", ["exact", "expth", "offline", "none"])
def test_prefill_pre_edge_thresholds(sdc):
    """theta = -inf keeps everything (dense for exact, exp-threshold and none);
    a threshold above every score keeps nothing (beta = 1 where E~ > 0)."""
    print(f"prefill_pre edges sdc={sdc}", flush=True)
    dev = device()
    Hq, Hkv, L, d = 4, 2, 130, 128
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 3, 3, B=1, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d,
                               dtype=torch.bfloat16)
    theta = np.full((Hq, L), -np.inf)
    theta[2:] = 1e4                                     # heads 2, 3 keep nothing
    et = np.full((Hq, L), 0.25)
    et[3] = 0.0                                         # offline with E~ = 0: denominator 0
    flags = MODES[sdc] | tt.TOPTH_VMC
    g = run_prefill_pre(q, k, v, theta, et, flags, dev)
    rows = [(0, h, p) for h in range(Hq) for p in range(L)]
    compare_prefill_pre(q, k, v, theta, et, sdc, sdc != "none", g, torch.bfloat16, rows)
    assert (g[1][0, :2] == np.arange(1, L + 1)).all() and (g[1][0, 2:] == 0).all()


def test_prefill_pre_8k_full_size_sampled_rows():
    """Full prefill size (32/8 heads, d=128, L=8192, bf16): sampled rows of every
    head against the oracle; theta from a 512-row calibration, clamped past it."""
    print("prefill_pre 8k sampled rows", flush=True)
    dev = device()
    Hq, Hkv, L, d = 32, 8, 8192, 128
    theta, et = calib_tables(UNIT, Hq, Hkv, 512, d, 128, 1, torch.bfloat16)
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 3, 4, B=1, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d,
                               dtype=torch.bfloat16)
    rng = np.random.default_rng(7)
    for sdc in ("expth", "exact"):
        g = run_prefill_pre(q, k, v, theta, et, MODES[sdc], dev)
        rows = [(0, h, int(p)) for h in range(Hq) for p in rng.choice(L, 6, replace=False)]
        rows += [(0, h, L - 1) for h in (0, 31)] + [(0, 5, 0), (0, 6, 511), (0, 7, 512)]
        # without a byte mask at this size, a row with elements in the ambiguity
        # band is checked by its count only (between the strict and the banded count)
        qf, kf = to_f64(q), to_f64(k)
        ok = []
        for (b, h, p) in rows:
            a = (kf[b, h // 4, :p + 1] @ qf[b, h, p]) / np.sqrt(d)
            thv = pre.table_row(theta, h, p)
            amb = ambiguous(a, thv)
            if amb.any():
                lo = int(((a >= thv) & ~amb).sum())
                assert lo <= g[1][b, h, p] <= lo + int(amb.sum()), (b, h, p)
            else:
                ok.append((b, h, p))
        assert len(ok) >= 0.9 * len(rows)
        compare_prefill_pre(q, k, v, theta, et, sdc, False, g, torch.bfloat16, ok)
    # the same launch with the byte mask (2 GiB at this size): every sampled
    # row, ambiguous elements included, element by element against the oracle
    # re-evaluated with the GPU's decisions
    print("prefill_pre 8k sampled rows with the kept mask", flush=True)
    km = torch.zeros((1, Hq, L, L), dtype=torch.uint8, device=dev)
    out = torch.empty(1, Hq, L, d, dtype=q.dtype, device=dev)
    kc = torch.full((1, Hq, L), -7, dtype=torch.int32, device=dev)
    bt = torch.full((1, Hq, L), -7.0, dtype=torch.float32, device=dev)
    tt.topth_prefill_pre(q.to(dev), k.to(dev), v.to(dev), torch.tensor(theta, dtype=torch.float32, device=dev), out,
                         scale=1.0 / np.sqrt(d), flags=MODES["expth"], gamma=GAMMA,
                         e_tilde=torch.tensor(et, dtype=torch.float32, device=dev),
                         kept_count=kc, beta=bt, kept_mask=km)
    torch.cuda.synchronize()

    class SampledRowMasks:
        """kept_mask[b, h, p, :p + 1] of the sampled rows only, copied to the host."""
        def __init__(self, rows):
            self.m = {(b, h, p): km[b, h, p, :p + 1].cpu().numpy().astype(bool) for (b, h, p) in rows}

        def __getitem__(self, idx):
            b, h, p, sl = idx
            return self.m[(b, h, p)][sl]

    g = (out.float().cpu().numpy(), kc.cpu().numpy(), bt.cpu().numpy(), SampledRowMasks(rows))
    del km
    compare_prefill_pre(q, k, v, theta, et, "expth", False, g, torch.bfloat16, rows)


# ------------------------------------------------------------------- decode
def run_decode_pre(q, k, v, lens, theta, et, vm, flags, dev):
    B, Hq, d = q.shape
    Hkv, Lmax = k.shape[1], k.shape[2]
    out = torch.empty(B, Hq, d, dtype=q.dtype, device=dev)
    kc = torch.full((B, Hq), -7, dtype=torch.int32, device=dev)
    bt = torch.full((B, Hq), -7.0, dtype=torch.float32, device=dev)
    vr = torch.full((B, Hkv), -7, dtype=torch.int32, device=dev)
    km = torch.zeros((B, Hq, Lmax), dtype=torch.uint8, device=dev)
    ws = tt.workspace(tt.TOPTH_OP_DECODE, B, Hq, Hkv, 1, Lmax, d)
    tt.topth_decode_pre(q.to(dev), k.to(dev), v.to(dev), torch.tensor(lens, dtype=torch.int32, device=dev),
                        torch.tensor(theta, dtype=torch.float32, device=dev), out, ws,
                        scale=1.0 / np.sqrt(d), flags=flags, gamma=GAMMA,
                        e_tilde=torch.tensor(et, dtype=torch.float32, device=dev),
                        v_mean=torch.tensor(vm, dtype=torch.float32, device=dev),
                        kept_count=kc, beta=bt, vrows_read=vr, kept_mask=km)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32)[0].item()) == 0, "exchange wait timed out"
    return (out.float().cpu().numpy(), kc.cpu().numpy(), bt.cpu().numpy(), vr.cpu().numpy(),
            km.cpu().numpy().astype(bool))


def decode_case(Hq, Hkv, d, Lmax, lens, dtype, seed_index, k=32, n_cal=3):
    q, kk, v = attention_inputs(UNIT, ROLE_TEST, 4, seed_index, B=len(lens), Hq=Hq, Hkv=Hkv, Lq=1,
                                Lk=Lmax, d=d, dtype=dtype)
    q = q[:, :, 0].contiguous()
    # decode-style calibration at the longest row; shorter rows use the table's nearest rows
    R = max(lens)
    cal = pre.PreCalibrator([k], Hq, R)
    for i in range(n_cal):
        for n in sorted(set(lens)):
            qc, kc, _ = attention_inputs(UNIT, ROLE_CALIB, 4, i * 16 + lens.index(n), B=1, Hq=Hq, Hkv=Hkv,
                                         Lq=1, Lk=n, d=d, dtype=dtype, with_v=False)
            cal.observe(to_f64(qc[0]), to_f64(kc[0]), 1.0 / np.sqrt(d), q_pos0=n - 1)
    theta, et = cal.finalize()[0], cal.finalize_etilde()[0]
    vf = to_f64(v)
    vm = np.stack([[vf[b, h, :lens[b]].mean(0) for h in range(Hkv)] for b in range(len(lens))])
    return q, kk, v, theta, et, vm.astype(np.float32).astype(np.float64)


def compare_decode_pre(q, k, v, lens, theta, et, vm, sdc, vmc, g, dtype):
    out_g, kc_g, bt_g, vr_g, km_g = g
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    B, Hq, d = qf.shape
    Hkv = kf.shape[1]
    G = Hq // Hkv
    for b in range(B):
        n = int(lens[b])
        for kv in range(Hkv):
            union = np.zeros(n, dtype=bool)
            for h in range(kv * G, (kv + 1) * G):
                a = (kf[b, kv, :n] @ qf[b, h]) / np.sqrt(d)
                gk = km_g[b, h, :n]
                assert kc_g[b, h] == gk.sum()
                check_pre_row(gk, a, pre.table_row(theta, h, n - 1), vf[b, kv, :n],
                              vm[b, kv] if vmc else 0.0, sdc, pre.table_row(et, h, n - 1), vmc,
                              out_g[b, h], bt_g[b, h], dtype, f"b{b} h{h}")
                union |= gk
            assert vr_g[b, kv] == union.sum(), (b, kv)


@pytest.mark.parametrize("sdc", list(MODES))
@pytest.mark.parametrize("Hq,Hkv,d,Lmax,lens", [
    (8, 2, 128, 1000, [1000, 537, 1]),        # g=4, ragged, single-key row
    (16, 2, 128, 4100, [4100, 2049]),         # g=8, several chunks
    (4, 4, 64, 300, [300, 129]),              # g=1, d=64
    (16, 1, 64, 600, [600, 90]),              # g=16 (FMA accumulate), d=64
])
def test_decode_pre_bf16(sdc, Hq, Hkv, d, Lmax, lens):
    print(f"decode_pre bf16 sdc={sdc} Hq={Hq} Hkv={Hkv} d={d} lens={lens}", flush=True)
    dev = device()
    q, k, v, theta, et, vm = decode_case(Hq, Hkv, d, Lmax, lens, torch.bfloat16, 0)
    vmc = sdc != "none"
    g = run_decode_pre(q, k, v, lens, theta, et, vm, MODES[sdc] | tt.TOPTH_VMC, dev)
    compare_decode_pre(q, k, v, lens, theta, et, vm, sdc, vmc, g, torch.bfloat16)


@pytest.mark.parametrize("sdc", list(MODES))
def test_decode_pre_f32(sdc):
    print(f"decode_pre f32 sdc={sdc}", flush=True)
    dev = device()
    lens = [700, 64]
    q, k, v, theta, et, vm = decode_case(8, 2, 64, 700, lens, torch.float32, 1)
    g = run_decode_pre(q, k, v, lens, theta, et, vm, MODES[sdc] | tt.TOPTH_VMC, dev)
    compare_decode_pre(q, k, v, lens, theta, et, vm, sdc, sdc != "none", g, torch.float32)


@pytest.mark.parametrize("sdc", list(MODES))
def test_decode_pre_edge_thresholds(sdc):
    print(f"decode_pre edges sdc={sdc}", flush=True)
    dev = device()
    Hq, Hkv, d, Lmax, lens = 8, 2, 128, 600, [600, 333]
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 4, 5, B=2, Hq=Hq, Hkv=Hkv, Lq=1, Lk=Lmax, d=d,
                               dtype=torch.bfloat16)
    q = q[:, :, 0].contiguous()
    theta = np.full((Hq, Lmax), -np.inf)
    theta[4:] = 1e4                                     # group 1 keeps nothing
    et = np.full((Hq, Lmax), 0.5)
    et[6:] = 0.0
    vf = to_f64(v)
    vm = np.stack([[vf[b, h, :lens[b]].mean(0) for h in range(Hkv)] for b in range(2)])
    vm = vm.astype(np.float32).astype(np.float64)
    g = run_decode_pre(q, k, v, lens, theta, et, vm, MODES[sdc] | tt.TOPTH_VMC, dev)
    compare_decode_pre(q, k, v, lens, theta, et, vm, sdc, sdc != "none", g, torch.bfloat16)
    assert (g[3][:, 1] == 0).all() and (g[3][:, 0] == np.array(lens)).all()


@pytest.mark.parametrize("sdc", ["expth", "offline"])
def test_decode_pre_bf16_without_optional_outputs(sdc):
    """The launch a server makes: no kept mask, counts, beta or union size."""
    print(f"decode_pre bf16 bare sdc={sdc}", flush=True)
    dev = device()
    Hq, Hkv, d, Lmax, lens = 16, 2, 128, 4100, [4100, 2049]
    q, k, v, theta, et, vm = decode_case(Hq, Hkv, d, Lmax, lens, torch.bfloat16, 2)
    full = run_decode_pre(q, k, v, lens, theta, et, vm, MODES[sdc] | tt.TOPTH_VMC, dev)
    out = torch.empty(len(lens), Hq, d, dtype=torch.bfloat16, device=dev)
    ws = tt.workspace(tt.TOPTH_OP_DECODE, len(lens), Hq, Hkv, 1, Lmax, d)
    tt.topth_decode_pre(q.to(dev), k.to(dev), v.to(dev), torch.tensor(lens, dtype=torch.int32, device=dev),
                        torch.tensor(theta, dtype=torch.float32, device=dev), out, ws,
                        scale=1.0 / np.sqrt(d), flags=MODES[sdc] | tt.TOPTH_VMC, gamma=GAMMA,
                        e_tilde=torch.tensor(et, dtype=torch.float32, device=dev),
                        v_mean=torch.tensor(vm, dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32)[0].item()) == 0, "exchange wait timed out"
    # the same kernels with and without the optional outputs give the same bits
    assert np.array_equal(out.float().cpu().numpy(), full[0])
    compare_decode_pre(q, k, v, lens, theta, et, vm, sdc, True, full, torch.bfloat16)
