"""Multi-k cumulative calibration (Appendix D, Algorithm 2, Eq. 8): the HIP
path through the C ABI against oracle/mkc.py.

* Integer-valued inputs with a power-of-two score scale give scores that
  float32 computes exactly, so the pre-softmax thresholds must equal the oracle's bit
  for bit (with many ties within and across samples).
* Post-softmax thresholds are compared to 1e-5 relative (float32 values
  against the float64 oracle); -inf (keep all) must match exactly.
"""
import numpy as np
import pytest
import torch

import calibrated_threshold_pruning_amd as tt
from oracle import mkc
from synth import CONFIG_IDS, ROLE_CALIB, attention_inputs, attention_inputs_device, to_f64
from parity import device

pytestmark = pytest.mark.gpu

UNIT = CONFIG_IDS["unit"]


def run_mkc(q, k, ks, q_pos0, pre, n_rows=None, fill=123.0, scale=None):
    dev = device()
    S, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    n_rows = n_rows or (q_pos0 + Lq)
    theta = torch.full((len(ks), Hq, n_rows), fill, dtype=torch.float32, device=dev)
    ws = torch.empty(tt.topth_workspace_size(tt.TOPTH_OP_CALIBRATE_MKC, S, Hq, Hkv, Lq, Lk, d, 0),
                     dtype=torch.uint8, device=dev)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    tt.topth_calibrate_mkc(q.to(dev), k.to(dev), ks, theta, ws, scale=scale, q_pos0=q_pos0, pre=pre)
    torch.cuda.synchronize()
    return theta.cpu().numpy().astype(np.float64)


def compare(got, ref, rel, where):
    inf_r, inf_g = np.isneginf(ref), np.isneginf(got)
    assert np.array_equal(inf_r, inf_g), f"-inf pattern differs {where}: {np.argwhere(inf_r != inf_g)[:5]}"
    fin = ~inf_r
    if rel == 0:
        assert np.array_equal(got[fin], ref[fin]), where
    else:
        err = np.abs(got[fin] - ref[fin]) / np.abs(ref[fin])
        assert err.max(initial=0.0) <= rel, f"rel error {err.max():.3g} {where}"


@pytest.mark.parametrize("dtype,d", [(torch.float32, 64), (torch.bfloat16, 128)])
def test_mkc_exact_on_integer_scores(dtype, d):
    print(f"mkc exact integer scores {dtype} d={d}", flush=True)
    rng = np.random.default_rng(5 + d)
    S, Hq, Hkv, L = 5, 4, 2, 40
    q = torch.tensor(rng.integers(-2, 3, size=(S, Hq, L, d)), dtype=dtype)
    k = torch.tensor(rng.integers(-1, 2, size=(S, Hkv, L, d)), dtype=dtype)
    ks = [1, 2, 3, 5, 8, 13, 39, 40, 41]
    scale = 0.125                     # a power of two: every score is exact in float32
    got = run_mkc(q, k, ks, 0, pre=True, scale=scale)
    ref = mkc.mkc_calibrate(to_f64(q), to_f64(k), scale, 0, ks, pre=True)
    compare(got, ref, 0, "pre-softmax, integer scores")
    assert np.isfinite(got).sum() > got.size // 3


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_mkc_post_softmax_prefill_rows(dtype):
    # the tiny prefill workload's shape: 1 head, d = 64, 256 rows
    print(f"mkc post-softmax prefill rows {dtype}", flush=True)
    S, L, d = 16, 256, 64
    q, k, _ = attention_inputs(UNIT, ROLE_CALIB, 3, 0, B=S, Hq=1, Hkv=1, Lq=L, Lk=L, d=d, n_sinks=1,
                               dtype=dtype, with_v=False)
    ks = [32, 1, 8, 64, 255, 256]
    got = run_mkc(q, k, ks, 0, pre=False)
    ref = mkc.mkc_calibrate(to_f64(q), to_f64(k), 1.0 / np.sqrt(d), 0, ks, pre=False)
    compare(got, ref, 1e-5, "post-softmax prefill")


def test_mkc_decode_rows_gqa_and_row_slice():
    # decode-style rows (one query row at p = Lk - 1) with 4 query heads per KV
    # head, then a slice of prefill rows that starts at q_pos0 = 100 and runs
    # past n_rows (rows p >= n_rows are left untouched)
    print("mkc decode rows, g = 4", flush=True)
    S, Hq, Hkv, d, Lk = 48, 8, 2, 128, 2000
    q, k, _ = attention_inputs(UNIT, ROLE_CALIB, 4, 0, B=S, Hq=Hq, Hkv=Hkv, Lq=1, Lk=Lk, d=d, n_sinks=1,
                               with_v=False)
    ks = [1, 16, 64, 128, 500, 1999, 2000]
    got = run_mkc(q, k, ks, Lk - 1, pre=False)
    ref = mkc.mkc_calibrate(to_f64(q), to_f64(k), 1.0 / np.sqrt(d), Lk - 1, ks, pre=False)
    compare(got[:, :, Lk - 1:], ref, 1e-5, "decode rows")
    assert (got[:, :, :Lk - 1] == 123.0).all()          # only row Lk - 1 is written
    got = run_mkc(q[:8], k[:8], [4, 30], Lk - 1, pre=True)    # pre-softmax on the same draws
    ref = mkc.mkc_calibrate(to_f64(q[:8]), to_f64(k[:8]), 1.0 / np.sqrt(d), Lk - 1, [4, 30], pre=True)
    compare(got[:, :, Lk - 1:], ref, 1e-5, "decode rows, pre-softmax")

    print("mkc row slice past n_rows", flush=True)
    S, Lq, Lk, q0 = 6, 40, 150, 100
    q, k, _ = attention_inputs(UNIT, ROLE_CALIB, 5, 0, B=S, Hq=2, Hkv=1, Lq=Lq, Lk=Lk, d=64, n_sinks=1,
                               dtype=torch.float32, with_v=False)
    got = run_mkc(q, k, [2, 50], q0, pre=False, n_rows=120)
    ref = mkc.mkc_calibrate(to_f64(q), to_f64(k), 1.0 / 8.0, q0, [2, 50], pre=False)
    compare(got[:, :, q0:], ref[:, :, :120 - q0], 1e-5, "row slice")
    assert (got[:, :, :q0] == 123.0).all()


def test_mkc_single_sample_is_the_kth_largest_and_edges():
    print("mkc single sample and edge rows", flush=True)
    rng = np.random.default_rng(8)
    L, d = 70, 64
    q = torch.tensor(rng.standard_normal((1, 1, L, d)), dtype=torch.float32)
    k = torch.tensor(rng.standard_normal((1, 1, L, d)), dtype=torch.float32)
    ks = [1, 2, 7, 69, 70]
    got = run_mkc(q, k, ks, 0, pre=True)
    a = (to_f64(k)[0, 0] @ to_f64(q)[0, 0].T).T / 8.0          # a[p, j] = q_p . k_j / sqrt(d)
    for p in range(L):
        row = np.sort(a[p, :p + 1])[::-1]
        for t, kk in enumerate(ks):
            want = row[kk - 1] if kk < p + 1 else -np.inf        # row 0 and k >= p + 1: keep all
            if np.isfinite(want):
                assert abs(got[t, 0, p] - want) <= 1e-5 * abs(want) + 1e-6, (p, kk)
            else:
                assert got[t, 0, p] == -np.inf, (p, kk)


def test_mkc_decode_8b_calibration_size_sampled_heads():
    # the decode_8b calibration: 256 sequences, 32/8 heads, 4096 keys, row 4095;
    # the oracle checks two heads of different KV groups
    print("mkc at the decode_8b calibration size", flush=True)
    cfg = CONFIG_IDS["decode_8b"]
    S, Hq, Hkv, d, n = 256, 32, 8, 128, 4096
    q, k, _ = attention_inputs_device(cfg, ROLE_CALIB, 7, 0, B=S, Hq=Hq, Hkv=Hkv, Lq=1, Lk=n, d=d, n_sinks=1,
                                      device=device(), with_v=False)
    q, k = q.cpu(), k.cpu()
    ks = [8, 64, 128, 256, 1024]
    got = run_mkc(q, k, ks, n - 1, pre=False)
    for h in (0, 17):
        ref = mkc.mkc_calibrate(to_f64(q[:, h:h + 1]), to_f64(k[:, h // 4:h // 4 + 1]), 1.0 / np.sqrt(d), n - 1,
                                ks, pre=False)
        compare(got[:, h:h + 1, n - 1:], ref, 1e-5, f"decode_8b calibration, head {h}")


@pytest.mark.parametrize("dtype,d,Lk", [(torch.bfloat16, 64, 300), (torch.float32, 128, 9000)])
def test_mkc_eight_query_heads_per_kv_head(dtype, d, Lk):
    # one KV head shared by 8 query heads: short rows put the scores of all 8
    # heads in one workgroup's LDS, a 9000-key row only those of 2
    print(f"mkc g = 8 {dtype} d={d} Lk={Lk}", flush=True)
    S, Hq, Hkv = 6, 8, 1
    q, k, _ = attention_inputs(UNIT, ROLE_CALIB, 9, 0, B=S, Hq=Hq, Hkv=Hkv, Lq=1, Lk=Lk, d=d, n_sinks=1,
                               dtype=dtype, with_v=False)
    ks = [1, 8, 100, Lk - 1]
    for pre in (False, True):
        got = run_mkc(q, k, ks, Lk - 1, pre=pre)
        ref = mkc.mkc_calibrate(to_f64(q), to_f64(k), 1.0 / np.sqrt(d), Lk - 1, ks, pre=pre)
        compare(got[:, :, Lk - 1:], ref, 1e-5, f"g = 8, Lk = {Lk}, pre = {pre}")


def test_mkc_bound_and_compaction_exact_with_ties():
    # decode rows of 3000 keys from 300 samples (900k pooled values: several
    # compaction and sort chunks) with integer-valued scores, so values repeat
    # everywhere, also at the bound below which values are left unsorted;
    # pre-softmax thresholds must match bit for bit
    print("mkc bound and compaction, 300 x 3000 integer scores", flush=True)
    rng = np.random.default_rng(12)
    S, Hq, Hkv, d, Lk = 300, 2, 1, 64, 3000
    q = torch.tensor(rng.integers(-2, 3, size=(S, Hq, 1, d)), dtype=torch.float32)
    k = torch.tensor(rng.integers(-1, 2, size=(S, Hkv, Lk, d)), dtype=torch.float32)
    # with k = 2999 the bound sits near the bottom; with k <= 50 it prunes hard
    for ks in ([1, 50, 300, 2999, 3000], [3, 50]):
        got = run_mkc(q, k, ks, Lk - 1, pre=True, scale=0.125)
        ref = mkc.mkc_calibrate(to_f64(q), to_f64(k), 0.125, Lk - 1, ks, pre=True)
        compare(got[:, :, Lk - 1:], ref, 0, f"pre-softmax, 300 x 3000 integer scores, ks {ks}")
        got = run_mkc(q, k, ks, Lk - 1, pre=False, scale=0.125)
        ref = mkc.mkc_calibrate(to_f64(q), to_f64(k), 0.125, Lk - 1, ks, pre=False)
        compare(got[:, :, Lk - 1:], ref, 1e-5, f"post-softmax, 300 x 3000 integer scores, ks {ks}")


def test_mkc_most_samples():
    # the largest sample count one call takes (4096: the maxima and minima
    # sorted in one workgroup, the bound tested against all of them), on
    # 20-key decode rows
    print("mkc 4096 samples", flush=True)
    rng = np.random.default_rng(13)
    S, Hq, Hkv, d, Lk = tt.TOPTH_MKC_MAX_SAMPLES, 2, 1, 64, 20
    q = torch.tensor(rng.standard_normal((S, Hq, 1, d)), dtype=torch.float32)
    k = torch.tensor(rng.standard_normal((S, Hkv, Lk, d)), dtype=torch.float32)
    ks = [1, 5, 19, 20]
    got = run_mkc(q, k, ks, Lk - 1, pre=False, scale=0.125)
    ref = mkc.mkc_calibrate(to_f64(q), to_f64(k), 0.125, Lk - 1, ks, pre=False)
    compare(got[:, :, Lk - 1:], ref, 1e-5, "4096 samples")


def test_mkc_rows_spanning_several_chunks():
    # 24 query rows at positions 500..523 of 64 samples: every (head, row)
    # pools 32k-34k values, so each spans several sort chunks, with a ragged
    # last chunk that differs from row to row
    print("mkc 24 rows of ~33k pooled values", flush=True)
    S, Hq, Hkv, d, Lq, q0 = 64, 2, 1, 64, 24, 500
    q, k, _ = attention_inputs(UNIT, ROLE_CALIB, 16, 0, B=S, Hq=Hq, Hkv=Hkv, Lq=Lq, Lk=q0 + Lq, d=d,
                               n_sinks=1, dtype=torch.float32, with_v=False)
    ks = [4, 40, 200]
    for pre in (False, True):
        got = run_mkc(q, k, ks, q0, pre=pre)
        ref = mkc.mkc_calibrate(to_f64(q), to_f64(k), 1.0 / np.sqrt(d), q0, ks, pre=pre)
        compare(got[:, :, q0:], ref, 1e-5, f"24 rows, pre = {pre}")
