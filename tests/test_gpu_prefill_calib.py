"""Prefill and calibration parity: HIP path (through the C ABI) against the oracle."""
import numpy as np
import pytest
import torch

import calibrated_threshold_pruning_amd as tt
import oracle
from synth import CONFIG_IDS, ROLE_CALIB, ROLE_TEST, attention_inputs, batch_of_sequences, to_f64
from parity import check_out, check_row_mask, device, theta_of

pytestmark = pytest.mark.gpu

UNIT = CONFIG_IDS["unit"]


# ------------------------------------------------------------------ helpers
def gpu_calibrate(q, k, ks, n_rows, q_pos0=0, alpha=0.0, chunks=1):
    """theta [n_k, Hq, n_rows] from the HIP calibration, fed in `chunks` calls."""
    dev = device()
    S, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    n_k = len(ks)
    s1 = torch.zeros(n_k, Hq, n_rows, dtype=torch.float64, device=dev)
    s2 = torch.zeros_like(s1)
    cnt = torch.zeros(n_k, Hq, n_rows, dtype=torch.int32, device=dev)
    per = (S + chunks - 1) // chunks
    ws = tt.workspace(tt.TOPTH_OP_CALIBRATE, per, Hq, Hkv, Lq, Lk, d, n_k)
    for c0 in range(0, S, per):
        tt.topth_calibrate(q[c0:c0 + per].to(dev).contiguous(), k[c0:c0 + per].to(dev).contiguous(),
                           ks, s1, s2, cnt, ws, scale=1.0 / np.sqrt(d), q_pos0=q_pos0)
    th = torch.empty(n_k, Hq, n_rows, dtype=torch.float32, device=dev)
    tt.topth_calibrate_finalize(s1, s2, cnt, ks, th, alpha=alpha)
    torch.cuda.synchronize()
    return th.cpu().numpy().astype(np.float64), cnt.cpu().numpy()


def oracle_calibrate(q, k, ks, n_rows, q_pos0=0, alpha=0.0):
    S, Hq = q.shape[0], q.shape[1]
    d = q.shape[-1]
    cal = oracle.Calibrator(ks, Hq, n_rows)
    qf, kf = to_f64(q), to_f64(k)
    for s in range(S):
        cal.observe(qf[s], kf[s], 1.0 / np.sqrt(d), q_pos0=q_pos0)
    return cal.finalize(alpha=alpha), cal.counts()


def check_theta(gpu, ref):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(gpu), fin)
    assert (np.isneginf(gpu) == np.isneginf(ref)).all()
    rel = np.abs(gpu[fin] - ref[fin]) / np.abs(ref[fin])
    assert rel.max() <= 1e-5, rel.max()


def run_prefill(q, k, v, theta, flags, with_ws=True, with_beta=True):
    """with_ws: the full prefill workspace (bf16: P V in float16 when every V
    element is within 16 in magnitude); False: none (bf16 high/low split).
    with_beta False: no beta output (with neither VMC nor SDC_NONE the kernel
    then skips the kept-mass sum); beta is returned as NaN."""
    dev = device()
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    out = torch.empty_like(q, device=dev)
    kc = torch.full((B, Hq, L), -7, dtype=torch.int32, device=dev)
    bt = torch.full((B, Hq, L), -7.0, dtype=torch.float32, device=dev)
    km = torch.zeros((B, Hq, L, L), dtype=torch.uint8, device=dev)
    ws = tt.workspace(tt.TOPTH_OP_PREFILL, B, Hq, Hkv, L, L, d) if with_ws else None
    tt.topth_prefill(q.to(dev), k.to(dev), v.to(dev),
                     torch.tensor(theta, dtype=torch.float32, device=dev).contiguous(), out,
                     scale=1.0 / np.sqrt(d), flags=flags, kept_count=kc, beta=bt if with_beta else None,
                     kept_mask=km, ws=ws)
    torch.cuda.synchronize()
    beta = bt.cpu().numpy() if with_beta else np.full(bt.shape, np.nan)
    return dict(out=out.float().cpu().numpy(), kc=kc.cpu().numpy(), beta=beta,
                mask=km.cpu().numpy().astype(bool))


def compare_prefill(g, q, k, v, theta, flags, dtype, rows=None):
    vmc = bool(flags & tt.TOPTH_VMC)
    renorm = bool(flags & tt.TOPTH_SDC_NONE)
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    B, Hq, L, d = qf.shape
    G = Hq // kf.shape[1]
    ref = oracle.prefill(qf, kf, vf, theta, 1.0 / np.sqrt(d), vmc=vmc, renorm=renorm, rows=rows,
                         keep_rows=True)
    if rows is None:
        rows = [(b, h, p) for b in range(B) for h in range(Hq) for p in range(L)]
    mu_cache = {}
    n_amb = 0
    for (b, h, p) in rows:
        kv = h // G
        gk = g["mask"][b, h, p, :p + 1]
        assert not g["mask"][b, h, p, p + 1:].any()
        th = theta_of(theta, h, p)
        amb = check_row_mask(gk, ref.s[b][h][p], th, f"b{b} h{h} p{p}")
        n_amb += amb
        assert g["kc"][b, h, p] == gk.sum()
        if amb == 0:
            assert g["kc"][b, h, p] == ref.kept_count[b, h, p]
        if (b, kv) not in mu_cache:
            mu_cache[(b, kv)] = oracle.prefix_mean(vf[b, kv])
        ro, rb = oracle.row_output(ref.s[b][h][p], gk, vf[b, kv, :p + 1], mu_cache[(b, kv)][p],
                                   vmc=vmc, renorm=renorm)
        check_out(g["out"][b, h, p], ro, dtype, f"b{b} h{h} p{p}")
        if not np.isnan(g["beta"][b, h, p]):
            assert abs(g["beta"][b, h, p] - rb) <= 1e-5
    return n_amb


# --------------------------------------------------- tiny fp32 prefill workload
def test_tiny_prefill_f32_calibrate_and_apply():
    """1 head, d=64, L=256, fp32, causal; theta for k=32 from 64 calibration
    sequences, applied to 8 test sequences with SDC + VMC."""
    cfg = CONFIG_IDS["tiny_prefill_f32"]
    print("tiny prefill f32", flush=True)
    qc, kc, _ = batch_of_sequences(cfg, ROLE_CALIB, 0, 0, 64, Hq=1, Hkv=1, Lq=256, Lk=256, d=64,
                                   dtype=torch.float32)
    th_gpu, cnt_gpu = gpu_calibrate(qc, kc, [32], 256, chunks=4)
    th_ref, cnt_ref = oracle_calibrate(qc, kc, [32], 256)
    assert np.array_equal(cnt_gpu, cnt_ref)
    check_theta(th_gpu, th_ref)
    theta = th_ref[0]
    q, k, v = attention_inputs(cfg, ROLE_TEST, 0, 0, B=8, Hq=1, Hkv=1, Lq=256, Lk=256, d=64,
                               dtype=torch.float32)
    g = run_prefill(q, k, v, theta, tt.TOPTH_VMC)
    compare_prefill(g, q, k, v, theta, tt.TOPTH_VMC, torch.float32)
    kept = g["kc"][:, 0, 32:]
    ratio = kept.mean() / 32
    assert 0.3 < ratio < 3.0


@pytest.mark.parametrize("flags", [tt.TOPTH_VMC, 0, tt.TOPTH_SDC_NONE])
def test_prefill_bf16_gqa(flags):
    Hq, Hkv, L, d = 8, 2, 300, 128
    qc, kc, _ = batch_of_sequences(UNIT, ROLE_CALIB, 3, 0, 4, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    theta = oracle_calibrate(qc, kc, [24], L)[0][0]
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 3, 0, B=2, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    g = run_prefill(q, k, v, theta, flags)
    compare_prefill(g, q, k, v, theta, flags, torch.bfloat16)


def test_prefill_dense_theta_bf16_d64():
    Hq, Hkv, L, d = 4, 4, 130, 64
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 4, 0, B=1, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    theta = np.full((Hq, 1), -np.inf)
    g = run_prefill(q, k, v, theta, tt.TOPTH_VMC)
    compare_prefill(g, q, k, v, theta, tt.TOPTH_VMC, torch.bfloat16)
    assert (g["kc"] == np.arange(1, L + 1)).all()


@pytest.mark.parametrize("L", [1, 2, 64, 65])
def test_prefill_bf16_edge_lengths(L):
    """Sequences of one row, one full key tile and one tile plus a key, with
    theta from calibration (k=1) and VMC."""
    Hq, Hkv, d = 4, 2, 128
    qc, kc, _ = batch_of_sequences(UNIT, ROLE_CALIB, 9, 0, 3, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    theta = oracle_calibrate(qc, kc, [1], L)[0][0]
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 9, L, B=2, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    g = run_prefill(q, k, v, theta, tt.TOPTH_VMC)
    compare_prefill(g, q, k, v, theta, tt.TOPTH_VMC, torch.bfloat16)


@pytest.mark.parametrize("flags", [tt.TOPTH_VMC, 0, tt.TOPTH_SDC_NONE])
def test_prefill_keeps_nothing(flags):
    """theta above every probability: k~ = 0 on every row, beta = 1; the output
    is mu (VMC), 0 (exact SDC without VMC) or 0 (SDC_NONE, beta 0)."""
    Hq, Hkv, L, d = 4, 1, 150, 128
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 10, 0, B=1, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    theta = np.full((Hq, L), 1.5)
    g = run_prefill(q, k, v, theta, flags)
    compare_prefill(g, q, k, v, theta, flags, torch.bfloat16)
    assert (g["kc"] == 0).all()


# ----------------------------------------------------------------- calibration
def test_calibrate_bf16_extreme_k():
    """Eight targets at once, from k = 1 (the row maximum) to k >= L (no row
    reaches it: no samples, theta = -inf on every row)."""
    Hq, L, d = 2, 100, 128
    q, k, _ = batch_of_sequences(UNIT, ROLE_CALIB, 11, 0, 3, Hq=Hq, Hkv=Hq, Lq=L, Lk=L, d=d)
    ks = [1, 2, 3, 50, 99, 100, 150, 7]
    th_gpu, cnt_gpu = gpu_calibrate(q, k, ks, L)
    th_ref, cnt_ref = oracle_calibrate(q, k, ks, L)
    assert np.array_equal(cnt_gpu, cnt_ref)
    check_theta(th_gpu, th_ref)
    assert np.isneginf(th_gpu[5]).all() and np.isneginf(th_gpu[6]).all()
    assert (cnt_gpu[5] == 0).all() and (cnt_gpu[6] == 0).all()


def test_calibrate_bf16_multi_k_prefill_style():
    Hq, L, d = 4, 300, 128
    q, k, _ = batch_of_sequences(UNIT, ROLE_CALIB, 5, 0, 6, Hq=Hq, Hkv=Hq, Lq=L, Lk=L, d=d)
    ks = [8, 32, 100]
    th_gpu, cnt_gpu = gpu_calibrate(q, k, ks, 320, chunks=2)
    th_ref, cnt_ref = oracle_calibrate(q, k, ks, 320)
    assert np.array_equal(cnt_gpu, cnt_ref)
    check_theta(th_gpu, th_ref)


def test_calibrate_decode_style_and_alpha():
    Hq, Hkv, L, d = 8, 2, 1000, 64
    q, k, _ = batch_of_sequences(UNIT, ROLE_CALIB, 6, 0, 5, Hq=Hq, Hkv=Hkv, Lq=1, Lk=L, d=d)
    q = q[:, :, :1].contiguous()
    for alpha in (0.0, 0.5):
        th_gpu, _ = gpu_calibrate(q, k, [64], 1024, q_pos0=L - 1, alpha=alpha)
        th_ref, _ = oracle_calibrate(q, k, [64], 1024, q_pos0=L - 1, alpha=alpha)
        check_theta(th_gpu, th_ref)
        assert np.isneginf(th_gpu[0, :, :64]).all()
        assert (th_gpu[0, :, 64:] == th_gpu[0, :, L - 1:L]).all()   # nearest-row fill


# Shapes that reach every score-column variant of the tiled bf16 calibration
# (16 columns up to 2048 keys, then 8, 4, 2, 1 as the longest row doubles) and
# both head/row mappings of a workgroup (several heads of a KV group, several
# rows of one head).
CALIB_SHAPES = [
    # name, Hq, Hkv, Lq, Lk, q_pos0, S, ks, d
    ("c16_gqa_rows", 8, 2, 300, 300, 0, 3, [16, 64], 128),
    ("c16_chunk", 2, 1, 100, 400, 300, 2, [32, 200], 64),
    ("c8_prefill", 1, 1, 2500, 2500, 0, 1, [128], 64),
    ("c4_decode", 8, 2, 1, 6000, 5999, 3, [64, 256], 128),
    ("c2_decode", 8, 1, 1, 12000, 11999, 2, [256], 128),
    ("c1_decode", 2, 2, 1, 30000, 29999, 2, [256, 1000], 64),
]


@pytest.mark.parametrize("name,Hq,Hkv,Lq,Lk,q_pos0,S,ks,d", CALIB_SHAPES,
                         ids=[c[0] for c in CALIB_SHAPES])
def test_calibrate_bf16_column_variants(name, Hq, Hkv, Lq, Lk, q_pos0, S, ks, d):
    print("calibrate", name, flush=True)
    q, k, _ = batch_of_sequences(UNIT, ROLE_CALIB, 7, 0, S, Hq=Hq, Hkv=Hkv, Lq=Lq, Lk=Lk, d=d)
    n_rows = q_pos0 + Lq
    th_gpu, cnt_gpu = gpu_calibrate(q, k, ks, n_rows, q_pos0=q_pos0)
    th_ref, cnt_ref = oracle_calibrate(q, k, ks, n_rows, q_pos0=q_pos0)
    assert np.array_equal(cnt_gpu, cnt_ref)
    check_theta(th_gpu, th_ref)


@pytest.mark.parametrize("Hq,Hkv,L,d", [(16, 2, 333, 128), (16, 1, 200, 64), (2, 1, 257, 64)])
def test_calibrate_tiled_group_sizes(Hq, Hkv, L, d):
    """Whole causal prefills through the tiled calibration at 8, 16 and 2
    query heads per KV head: every mapping of heads and 32-row blocks onto
    its workgroups (several head blocks per KV head, several row blocks of
    two heads)."""
    print(f"calibrate tiled Hq={Hq} Hkv={Hkv} L={L} d={d}", flush=True)
    q, k, _ = batch_of_sequences(UNIT, ROLE_CALIB, 14, 0, 2, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    ks = [16, 100]
    th_gpu, cnt_gpu = gpu_calibrate(q, k, ks, L)
    th_ref, cnt_ref = oracle_calibrate(q, k, ks, L)
    assert np.array_equal(cnt_gpu, cnt_ref)
    check_theta(th_gpu, th_ref)


@pytest.mark.parametrize("ks", [[7], [12, 90], [5, 40, 90], [3, 40, 90, 250]], ids=["1k", "2k", "3k", "4k"])
def test_calibrate_tiled_target_counts(ks):
    """Whole causal prefills through the tiled calibration with one to four
    targets: the member sweep is compiled once per target count, and each
    form has to find every row's k-th largest exactly."""
    Hq, Hkv, L, d = 8, 2, 700, 128
    print(f"calibrate tiled ks={ks}", flush=True)
    q, k, _ = batch_of_sequences(UNIT, ROLE_CALIB, 15, 0, 2, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    th_gpu, cnt_gpu = gpu_calibrate(q, k, ks, L)
    th_ref, cnt_ref = oracle_calibrate(q, k, ks, L)
    assert np.array_equal(cnt_gpu, cnt_ref)
    check_theta(th_gpu, th_ref)


def test_calibrate_bf16_ties():
    """Keys drawn from three distinct rows: every score row holds long runs of
    equal values, so the bin of the k-th largest overflows the copy space and
    the restricted radix select decides (ties count with multiplicity)."""
    Hq, L, d = 2, 600, 128
    q, k, _ = batch_of_sequences(UNIT, ROLE_CALIB, 8, 0, 2, Hq=Hq, Hkv=Hq, Lq=L, Lk=L, d=d)
    k = k[:, :, torch.arange(L) % 3].contiguous()
    ks = [50, 300]
    th_gpu, cnt_gpu = gpu_calibrate(q, k, ks, L)
    th_ref, cnt_ref = oracle_calibrate(q, k, ks, L)
    assert np.array_equal(cnt_gpu, cnt_ref)
    check_theta(th_gpu, th_ref)


def test_calibrate_tiled_longest_rows_with_ties():
    """The longest rows of the tiled calibration (16384 keys) with keys drawn
    from three distinct rows, so every score row is three long runs of equal
    values: the rows go to the exact fixup, whose row of scores then needs more
    than 48 KiB of LDS.  Counts on every row, theta on sampled rows (one
    sequence: theta is the k-th largest value itself)."""
    Hq, L, d = 2, 16384, 64
    print("calibrate 16384-key rows with ties", flush=True)
    q, k, _ = batch_of_sequences(UNIT, ROLE_CALIB, 15, 0, 1, Hq=Hq, Hkv=1, Lq=L, Lk=L, d=d)
    k = k[:, :, torch.arange(L) % 3].contiguous()
    ks = [50, 3000]
    th_gpu, cnt_gpu = gpu_calibrate(q, k, ks, L)
    for ki, kk in enumerate(ks):
        assert (cnt_gpu[ki, :, :kk] == 0).all() and (cnt_gpu[ki, :, kk:] == 1).all()
    qf, kf = to_f64(q), to_f64(k)
    for i in [50, 51, 2999, 3000, 12287, 12288, 16000, 16383]:
        for (ki, h, p), t in oracle.calibration_samples(qf[0][:, i:i + 1], kf[0], ks, 1.0 / np.sqrt(d),
                                                        q_pos0=i).items():
            assert abs(th_gpu[ki, h, p] - t) <= 1e-5 * abs(t), (ki, h, p)


def test_calibrate_sweep_shape_sampled_rows():
    """Calibration-sweep shape (8 independent heads, d=128, L=2048, k in
    {64, 128, 256}) on a few sequences: counts on every row, theta on sampled
    rows against the oracle's mean of per-sequence k-th largest values."""
    Hq, L, d, S = 8, 2048, 128, 2
    ks = [64, 128, 256]
    q, k, _ = batch_of_sequences(CONFIG_IDS["calib_sweep"], ROLE_CALIB, 0, 0, S, Hq=Hq, Hkv=Hq,
                                 Lq=L, Lk=L, d=d)
    th_gpu, cnt_gpu = gpu_calibrate(q, k, ks, L)
    for ki, kk in enumerate(ks):
        assert (cnt_gpu[ki, :, :kk] == 0).all() and (cnt_gpu[ki, :, kk:] == S).all()
        assert np.isneginf(th_gpu[ki, :, :kk]).all()
    rows = [64, 127, 128, 255, 256, 257, 700, 1023, 1500, 2046, 2047]
    qf, kf = to_f64(q), to_f64(k)
    for i in rows:
        obs = {}
        for s in range(S):
            for key, t in oracle.calibration_samples(qf[s][:, i:i + 1], kf[s], ks, 1.0 / np.sqrt(d),
                                                     q_pos0=i).items():
                obs.setdefault(key, []).append(t)
        for (ki, h, p), vals in obs.items():
            ref = float(np.mean(vals))
            assert abs(th_gpu[ki, h, p] - ref) <= 1e-5 * abs(ref), (ki, h, p)


def test_decode_matches_prefill_row():
    """Decode with n = p + 1 keys equals prefill row p (both on the GPU): kept
    masks agree outside the 1e-5 band around theta (the two kernels accumulate
    q.k in different orders), outputs within the bf16 tolerance."""
    dev = device()
    Hq, Hkv, L, d = 8, 2, 400, 128
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 7, 0, B=1, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    theta = np.exp(np.random.default_rng(0).uniform(-6, -2, size=(Hq, L)))
    g = run_prefill(q, k, v, theta, tt.TOPTH_VMC)
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    for p in (0, 63, 64, 255, 399):
        vm = torch.tensor(vf[:, :, :p + 1].mean(2), dtype=torch.float32, device=dev)
        out = torch.empty(1, Hq, d, dtype=torch.bfloat16, device=dev)
        km = torch.zeros(1, Hq, L, dtype=torch.uint8, device=dev)
        ws = tt.workspace(tt.TOPTH_OP_DECODE, 1, Hq, Hkv, 1, L, d)
        tt.topth_decode(q[:, :, p].contiguous().to(dev), k.to(dev), v.to(dev),
                        torch.tensor([p + 1], dtype=torch.int32, device=dev),
                        torch.tensor(theta, dtype=torch.float32, device=dev), out, ws,
                        scale=1.0 / np.sqrt(d), flags=tt.TOPTH_VMC, v_mean=vm, kept_mask=km)
        torch.cuda.synchronize()
        dm = km.cpu().numpy()[0, :, :p + 1].astype(bool)
        for h in range(Hq):
            s_row, _ = oracle.post_softmax(oracle.scores(qf[0, h, p], kf[0, h // 4, :p + 1], 1.0 / np.sqrt(d)))
            th = theta_of(theta, h, p)
            diff = dm[h] != g["mask"][0, h, p, :p + 1]
            assert not (diff & ~(np.abs(s_row - th) <= 1e-5 * abs(th))).any(), (p, h)
        assert np.abs(out.float().cpu().numpy()[0] - g["out"][0, :, p]).max() <= 1e-2


@pytest.mark.parametrize("Hq,Hkv,L,d", [(16, 2, 333, 128), (16, 1, 200, 128), (2, 1, 257, 64), (8, 8, 97, 128)])
def test_prefill_bf16_group_sizes(Hq, Hkv, L, d):
    """g = 8, 16, 2, 1 with lengths that leave ragged query and key tiles."""
    print(f"prefill bf16 Hq={Hq} Hkv={Hkv} L={L} d={d}", flush=True)
    qc, kc, _ = batch_of_sequences(UNIT, ROLE_CALIB, 8, 0, 2, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    theta = oracle_calibrate(qc, kc, [16], L)[0][0]
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 8, Hq, B=2, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    g = run_prefill(q, k, v, theta, tt.TOPTH_VMC)
    compare_prefill(g, q, k, v, theta, tt.TOPTH_VMC, torch.bfloat16)


def test_calibrate_long_prefill_sampled_rows():
    """Whole causal prefills of 8192 keys (4 query heads per KV head, d=128,
    k = 128 and 512) through the tiled calibration: counts on every row, theta
    on sampled rows (both sides of 4096 and of each k) against the oracle."""
    Hq, Hkv, L, d, S = 4, 1, 8192, 128, 2
    ks = [128, 512]
    print("calibrate 8192-key prefills", flush=True)
    q, k, _ = batch_of_sequences(CONFIG_IDS["prefill_8k"], ROLE_CALIB, 1, 0, S, Hq=Hq, Hkv=Hkv,
                                 Lq=L, Lk=L, d=d)
    th_gpu, cnt_gpu = gpu_calibrate(q, k, ks, L)
    for ki, kk in enumerate(ks):
        assert (cnt_gpu[ki, :, :kk] == 0).all() and (cnt_gpu[ki, :, kk:] == S).all()
        assert np.isneginf(th_gpu[ki, :, :kk]).all()
    rows = [128, 129, 511, 512, 513, 2000, 4095, 4096, 4097, 6000, 8190, 8191]
    qf, kf = to_f64(q), to_f64(k)
    for i in rows:
        obs = {}
        for s in range(S):
            for key, t in oracle.calibration_samples(qf[s][:, i:i + 1], kf[s], ks, 1.0 / np.sqrt(d),
                                                     q_pos0=i).items():
                obs.setdefault(key, []).append(t)
        for (ki, h, p), vals in obs.items():
            ref = float(np.mean(vals))
            assert abs(th_gpu[ki, h, p] - ref) <= 1e-5 * abs(ref), (ki, h, p)


def test_prefill_8k_full_size_sampled_rows():
    """One layer of the 8k prefill workload (32/8 heads, d=128, L=8192, k=128,
    SDC, no VMC), checked on sampled rows that span the whole causal range."""
    dev = device()
    cfg = CONFIG_IDS["prefill_8k"]
    Hq, Hkv, L, d, k = 32, 8, 8192, 128, 128
    print("prefill 8k full size", flush=True)
    # theta from the oracle: decode-style calibration at 24 rows, nearest-row fill between them
    probe_rows = sorted(set(int(x) for x in np.geomspace(k + 1, L, 24).round()) | {L - 1})
    cal = oracle.Calibrator([k], Hq, L)
    scale = 1.0 / np.sqrt(d)
    for i in range(2):
        qc, kc, _ = attention_inputs(cfg, ROLE_CALIB, 2, i, B=1, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d, with_v=False)
        qf, kf = to_f64(qc[0]), to_f64(kc[0])
        for p in probe_rows:
            cal.observe(qf[:, p:p + 1], kf[:, :p + 1], scale, q_pos0=p)
    theta = cal.finalize()[0]
    q, kk, v = attention_inputs(cfg, ROLE_TEST, 2, 0, B=1, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    rng = np.random.default_rng(0)
    rows = [(0, int(h), int(p)) for h, p in zip(rng.integers(0, Hq, 48), rng.integers(0, L, 48))]
    rows += [(0, 0, 0), (0, 31, L - 1), (0, 5, 127), (0, 6, 128), (0, 7, 4095)]
    ref = oracle.prefill(to_f64(q), to_f64(kk), to_f64(v), theta, scale, vmc=False, rows=rows, keep_rows=True)
    vf = to_f64(v)
    # no workspace with the beta output (bf16 split P V, kept mass summed), then
    # the benchmark's launch: full workspace, no beta (float16 P V, no mass sum)
    for with_ws in (False, True):
        print(f"prefill 8k full size, workspace={with_ws}", flush=True)
        out = torch.empty(1, Hq, L, d, dtype=torch.bfloat16, device=dev)
        kc_ = torch.empty(1, Hq, L, dtype=torch.int32, device=dev)
        bt = None if with_ws else torch.empty(1, Hq, L, dtype=torch.float32, device=dev)
        ws = tt.workspace(tt.TOPTH_OP_PREFILL, 1, Hq, Hkv, L, L, d) if with_ws else None
        tt.topth_prefill(q.to(dev), kk.to(dev), v.to(dev), torch.tensor(theta, dtype=torch.float32, device=dev),
                         out, scale=scale, flags=0, kept_count=kc_, beta=bt, ws=ws)
        torch.cuda.synchronize()
        go, gk = out.float().cpu().numpy(), kc_.cpu().numpy()
        gb = None if bt is None else bt.cpu().numpy()
        for (b, h, p) in rows:
            th = theta_of(theta, h, p)
            sv = ref.s[b][h][p]
            amb = int((np.abs(sv - th) <= 1e-5 * abs(th)).sum()) if np.isfinite(th) else 0
            if amb == 0:
                assert gk[b, h, p] == ref.kept_count[b, h, p], (h, p)
            else:
                assert abs(gk[b, h, p] - ref.kept_count[b, h, p]) <= amb
            check_out(go[b, h, p], ref.out[b, h, p], torch.bfloat16, f"h{h} p{p}")
            if gb is not None:
                assert abs(gb[b, h, p] - ref.beta[b, h, p]) <= 1e-4, (h, p)
        del out, kc_, ws


@pytest.mark.parametrize("case", ["f16", "large_v", "no_ws"])
def test_prefill_bf16_pv_forms(case):
    """The P V product runs in float16 when the workspace holds a float16 copy
    of V and every V element is within 16 in magnitude; a larger element (here
    one of 40 and one of -1000) or no workspace selects the bfloat16 high/low
    split.  Every form meets the bf16 tolerance against the oracle."""
    print(f"prefill bf16 P V form {case}", flush=True)
    Hq, Hkv, L, d = 8, 2, 200, 128
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 0, 9, B=1, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    if case == "large_v":
        v[0, 1, 0, 3] = 40.0
        v[0, 0, 150, 7] = -1000.0
    theta = oracle_calibrate(*batch_of_sequences(UNIT, ROLE_CALIB, 0, 20, 2, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)[:2],
                             [16], L)[0][0]
    for flags, with_beta in ((0, True), (0, False), (tt.TOPTH_VMC, True)):
        if case == "no_ws" and flags & tt.TOPTH_VMC:
            continue                     # VMC needs the workspace
        g = run_prefill(q, k, v, theta, flags, with_ws=case != "no_ws", with_beta=with_beta)
        compare_prefill(g, q, k, v, theta, flags, torch.bfloat16)


@pytest.mark.parametrize("Hq,Hkv,L,d", [(8, 2, 300, 128), (4, 1, 200, 64), (16, 2, 333, 128), (2, 2, 65, 128)])
def test_prefill_benchmark_form_all_rows(Hq, Hkv, L, d):
    """The kernel form the benchmark times: float16 P V (workspace given), no
    byte mask, no beta, exact SDC without VMC.  Every row: the kept count equals
    the oracle's outside the 1e-5 band around theta (and differs by at most the
    band's element count inside it); outputs within the bf16 tolerance."""
    print(f"prefill benchmark form Hq={Hq} Hkv={Hkv} L={L} d={d}", flush=True)
    dev = device()
    qc, kc, _ = batch_of_sequences(UNIT, ROLE_CALIB, 11, 0, 2, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    theta = oracle_calibrate(qc, kc, [16], L)[0][0]
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 11, L, B=2, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    scale = 1.0 / np.sqrt(d)
    out = torch.empty(2, Hq, L, d, dtype=torch.bfloat16, device=dev)
    kc_ = torch.empty(2, Hq, L, dtype=torch.int32, device=dev)
    ws = tt.workspace(tt.TOPTH_OP_PREFILL, 2, Hq, Hkv, L, L, d)
    tt.topth_prefill(q.to(dev), k.to(dev), v.to(dev), torch.tensor(theta, dtype=torch.float32, device=dev), out,
                     scale=scale, flags=0, kept_count=kc_, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.prefill(to_f64(q), to_f64(k), to_f64(v), theta, scale, vmc=False, keep_rows=True)
    go, gk = out.float().cpu().numpy(), kc_.cpu().numpy()
    for b in range(2):
        for h in range(Hq):
            for p in range(L):
                th = theta_of(theta, h, p)
                sv = ref.s[b][h][p]
                amb = int((np.abs(sv - th) <= 1e-5 * abs(th)).sum()) if np.isfinite(th) else 0
                assert abs(int(gk[b, h, p]) - int(ref.kept_count[b, h, p])) <= amb, (b, h, p)
                check_out(go[b, h, p], ref.out[b, h, p], torch.bfloat16, f"b{b} h{h} p{p}")


def test_prefill_f16_pv_long_keep_all_rows_large_v():
    """The float16 P V form on its worst case: rows of up to 8192 keys that keep
    every element, a peaked softmax (most weights far below the float16 normal
    range) and every V element at +-15.875, just inside the float16 form's bound
    of 16.  Sampled rows against the oracle at the bf16 tolerance."""
    dev = device()
    L, d = 8192, 128
    print("prefill float16 P V, keep-all rows of 8192 keys, |V| = 15.875", flush=True)
    q, k, _ = attention_inputs(UNIT, ROLE_TEST, 21, 0, B=1, Hq=1, Hkv=1, Lq=L, Lk=L, d=d, with_v=False)
    q = (q.float() * 6.0).to(torch.bfloat16)          # wide score spread: many tiny weights
    sign = torch.from_numpy(np.random.default_rng(3).integers(0, 2, size=(1, 1, L, d)) * 2 - 1)
    v = (15.875 * sign).to(torch.bfloat16)
    theta = np.full((1, 1), -np.inf)
    out = torch.empty(1, 1, L, d, dtype=torch.bfloat16, device=dev)
    ws = tt.workspace(tt.TOPTH_OP_PREFILL, 1, 1, 1, L, L, d)
    tt.topth_prefill(q.to(dev), k.to(dev), v.to(dev), torch.tensor(theta, dtype=torch.float32, device=dev), out,
                     scale=1.0 / np.sqrt(d), flags=0, ws=ws)
    torch.cuda.synchronize()
    rows = [(0, 0, p) for p in (8191, 6000, 4096, 100)]
    ref = oracle.prefill(to_f64(q), to_f64(k), to_f64(v), theta, 1.0 / np.sqrt(d), vmc=False, rows=rows)
    g = out.float().cpu().numpy()
    for (_, _, p) in rows:
        s = oracle.post_softmax(oracle.scores(to_f64(q)[0, 0, p], to_f64(k)[0, 0, :p + 1], 1.0 / np.sqrt(d)))[0]
        assert (s < 2.0 ** -14).sum() > p // 2            # most weights are float16 subnormals unscaled
        check_out(g[0, 0, p], ref.out[0, 0, p], torch.bfloat16, f"row {p}")
