"""Float32 output of the bfloat16 paths (TOPTH_OUT_F32).

* The float32 output, rounded to bfloat16 (round to nearest even), equals the
  plain bfloat16 call's output bit for bit: both store the same float32 value.
* Against the oracle, re-evaluated with the GPU's own decisions on elements
  within 1e-5 relative of theta, every output is within a flat 1e-2 (bfloat16
  inputs, float32 accumulation) with no allowance for output rounding.
"""
import numpy as np
import pytest
import torch

import calibrated_threshold_pruning_amd as tt
import oracle
from synth import CONFIG_IDS, ROLE_CALIB, ROLE_TEST, attention_inputs, batch_of_sequences, to_f64
from parity import ambiguous, check_row_mask, device, theta_of

pytestmark = pytest.mark.gpu

UNIT = CONFIG_IDS["unit"]
FLAT = 1e-2


def flat_check(gpu, ref, where):
    err = np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64)).max()
    assert err <= FLAT, f"max-abs error {err:.3g} beyond the flat 1e-2 {where}"


def bf16_bits(t):
    return t.contiguous().view(torch.int16).cpu()


def prefill_pair(q, k, v, theta, flags, with_ws):
    """The same prefill twice: bfloat16 output, then float32 output."""
    dev = device()
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    th = torch.tensor(theta, dtype=torch.float32, device=dev).contiguous()
    ws = tt.workspace(tt.TOPTH_OP_PREFILL, B, Hq, Hkv, L, L, d) if with_ws else None
    res = []
    for f32 in (False, True):
        out = torch.full((B, Hq, L, d), 7.0, dtype=torch.float32 if f32 else torch.bfloat16, device=dev)
        km = torch.zeros((B, Hq, L, L), dtype=torch.uint8, device=dev)
        tt.topth_prefill(qd, kd, vd, th, out, scale=1.0 / np.sqrt(d),
                         flags=flags | (tt.TOPTH_OUT_F32 if f32 else 0), kept_mask=km, ws=ws)
        torch.cuda.synchronize()
        res.append((out, km.cpu().numpy().astype(bool)))
    return res


@pytest.mark.parametrize("with_ws", [True, False], ids=["f16_pv", "bf16_split_pv"])
@pytest.mark.parametrize("flags", [tt.TOPTH_VMC, 0, tt.TOPTH_SDC_NONE])
def test_prefill_out_f32(flags, with_ws):
    if flags & tt.TOPTH_VMC and not with_ws:
        pytest.skip("VMC needs the workspace")
    print(f"prefill out f32 flags={flags} ws={with_ws}", flush=True)
    Hq, Hkv, L, d = 8, 2, 300, 128
    qc, kc, _ = batch_of_sequences(UNIT, ROLE_CALIB, 3, 0, 4, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    cal = oracle.Calibrator([24], Hq, L)
    for s in range(qc.shape[0]):
        cal.observe(to_f64(qc[s]), to_f64(kc[s]), 1.0 / np.sqrt(d))
    theta = cal.finalize()[0]
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 3, 0, B=2, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    (ob, mb), (of, mf) = prefill_pair(q, k, v, theta, flags, with_ws)
    assert np.array_equal(mb, mf)
    assert torch.equal(bf16_bits(of.to(torch.bfloat16)), bf16_bits(ob)), "f32 output does not round to the bf16 one"
    vmc, renorm = bool(flags & tt.TOPTH_VMC), bool(flags & tt.TOPTH_SDC_NONE)
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    ref = oracle.prefill(qf, kf, vf, theta, 1.0 / np.sqrt(d), vmc=vmc, renorm=renorm, keep_rows=True)
    g = of.cpu().numpy()
    for b in range(2):
        for h in range(Hq):
            kv = h // (Hq // Hkv)
            mu = oracle.prefix_mean(vf[b, kv])
            for p in range(L):
                gk = mf[b, h, p, :p + 1]
                check_row_mask(gk, ref.s[b][h][p], theta_of(theta, h, p), f"b{b} h{h} p{p}")
                ro, _ = oracle.row_output(ref.s[b][h][p], gk, vf[b, kv, :p + 1], mu[p], vmc=vmc, renorm=renorm)
                flat_check(g[b, h, p], ro, f"b{b} h{h} p{p}")


def test_prefill_pre_out_f32():
    """The pre-softmax prefill (exact E, Eq. 4) with thresholds in score units."""
    dev = device()
    Hq, Hkv, L, d = 4, 2, 200, 128
    print("prefill_pre out f32", flush=True)
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 5, 0, B=1, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d)
    theta = np.full((Hq, L), 1.5)
    th = torch.tensor(theta, dtype=torch.float32, device=dev)
    ws = tt.workspace(tt.TOPTH_OP_PREFILL, 1, Hq, Hkv, L, L, d)
    res = []
    for f32 in (False, True):
        out = torch.full((1, Hq, L, d), 7.0, dtype=torch.float32 if f32 else torch.bfloat16, device=dev)
        km = torch.zeros((1, Hq, L, L), dtype=torch.uint8, device=dev)
        tt.topth_prefill_pre(q.to(dev), k.to(dev), v.to(dev), th, out, scale=1.0 / np.sqrt(d),
                             flags=tt.TOPTH_OUT_F32 if f32 else 0, kept_mask=km, ws=ws)
        torch.cuda.synchronize()
        res.append((out, km.cpu().numpy().astype(bool)))
    (ob, mb), (of, mf) = res
    assert np.array_equal(mb, mf)
    assert torch.equal(bf16_bits(of.to(torch.bfloat16)), bf16_bits(ob)), "f32 output does not round to the bf16 one"
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    g = of.cpu().numpy()
    for h in range(Hq):
        kv = h // (Hq // Hkv)
        for p in range(L):
            a = oracle.scores(qf[0, h, p], kf[0, kv, :p + 1], 1.0 / np.sqrt(d))
            gk = mf[0, h, p, :p + 1]
            assert not ((gk != (a >= 1.5)) & ~ambiguous(a, 1.5)).any(), f"mask mismatch h{h} p{p}"
            w, _ = oracle.presoftmax.pre_weights_for_mask(a, gk, 1.5, sdc="exact")
            flat_check(g[0, h, p], w @ vf[0, kv, :p + 1], f"h{h} p{p}")


def test_prefill_out_f32_long_rows_large_v():
    """Keep-all rows of 8192 keys with |V| = 15.875 and a peaked softmax: the
    float16 P V form at its bound, checked without output rounding."""
    dev = device()
    L, d = 8192, 128
    print("prefill out f32, keep-all rows of 8192 keys", flush=True)
    q, k, _ = attention_inputs(UNIT, ROLE_TEST, 21, 0, B=1, Hq=1, Hkv=1, Lq=L, Lk=L, d=d, with_v=False)
    q = (q.float() * 6.0).to(torch.bfloat16)
    sign = torch.from_numpy(np.random.default_rng(3).integers(0, 2, size=(1, 1, L, d)) * 2 - 1)
    v = (15.875 * sign).to(torch.bfloat16)
    out = torch.empty(1, 1, L, d, dtype=torch.float32, device=dev)
    ws = tt.workspace(tt.TOPTH_OP_PREFILL, 1, 1, 1, L, L, d)
    tt.topth_prefill(q.to(dev), k.to(dev), v.to(dev), torch.full((1, 1), -float("inf"), device=dev), out,
                     scale=1.0 / np.sqrt(d), flags=tt.TOPTH_OUT_F32, ws=ws)
    torch.cuda.synchronize()
    rows = [(0, 0, p) for p in (8191, 6000, 4096, 100)]
    ref = oracle.prefill(to_f64(q), to_f64(k), to_f64(v), np.full((1, 1), -np.inf), 1.0 / np.sqrt(d), vmc=False,
                         rows=rows)
    g = out.cpu().numpy()
    for (_, _, p) in rows:
        flat_check(g[0, 0, p], ref.out[0, 0, p], f"row {p}")


def decode_case(Hq, Hkv, d, Lmax, lens, seed_index, cfg=UNIT):
    q, k, v = attention_inputs(cfg, ROLE_TEST, 0, seed_index, B=len(lens), Hq=Hq, Hkv=Hkv, Lq=1, Lk=Lmax, d=d,
                               n_sinks=1)
    q = q[:, :, 0].contiguous()
    p = np.arange(Lmax, dtype=np.float64)
    theta = np.broadcast_to(0.6 / (p + 1.0), (Hq, Lmax)).astype(np.float32).astype(np.float64).copy()
    theta[:, :16] = -np.inf
    vf = to_f64(v)
    vm = np.stack([[vf[b, h, :lens[b]].mean(0) for h in range(Hkv)] for b in range(len(lens))])
    return q, k, v, theta, vm.astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("entry", ["decode", "decode_pre", "decode_noalloc"])
@pytest.mark.parametrize("Hq,Hkv,d,Lmax,lens", [
    (8, 2, 128, 1000, [1000, 537, 1]),
    (32, 8, 128, 4096, [4096, 3000]),        # the decode_8b head layout, two sequences
    (16, 1, 64, 2500, [2500, 65]),
])
def test_decode_out_f32(entry, Hq, Hkv, d, Lmax, lens):
    print(f"{entry} out f32 Hq={Hq} Hkv={Hkv} d={d} Lmax={Lmax} lens={lens}", flush=True)
    dev = device()
    q, k, v, theta, vm = decode_case(Hq, Hkv, d, Lmax, lens, seed_index=30 + d)
    B = len(lens)
    pre = entry == "decode_pre"
    if pre:                                  # pre-softmax thresholds in score units
        theta = np.where(np.isfinite(theta), 1.5, -np.inf)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=dev)
    th = torch.tensor(theta, dtype=torch.float32, device=dev).contiguous()
    vmd = torch.tensor(vm, dtype=torch.float32, device=dev).contiguous()
    ws = tt.workspace(tt.TOPTH_OP_DECODE, B, Hq, Hkv, 1, Lmax, d)
    res = []
    for f32 in (False, True):
        out = torch.full((B, Hq, d), 7.0, dtype=torch.float32 if f32 else torch.bfloat16, device=dev)
        km = torch.zeros((B, Hq, Lmax), dtype=torch.uint8, device=dev)
        flags = tt.TOPTH_VMC | (tt.TOPTH_OUT_F32 if f32 else 0)
        kw = dict(scale=1.0 / np.sqrt(d), flags=flags, v_mean=vmd, kept_mask=km)
        if entry == "decode":
            tt.topth_decode(qd, kd, vd, lens_d, th, out, ws, **kw)
        elif entry == "decode_pre":
            tt.topth_decode_pre(qd, kd, vd, lens_d, th, out, ws, **kw)
        else:
            tt.topth_decode_noalloc(qd, kd, vd, lens_d, th, out, **kw)
        torch.cuda.synchronize()
        res.append((out, km.cpu().numpy().astype(bool)))
    assert tt.topth_workspace_status(ws) == 0
    (ob, mb), (of, mf) = res
    assert np.array_equal(mb, mf)
    assert torch.equal(bf16_bits(of.to(torch.bfloat16)), bf16_bits(ob)), "f32 output does not round to the bf16 one"
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    g = of.cpu().numpy()
    G = Hq // Hkv
    sc = 1.0 / np.sqrt(d)
    for b in range(B):
        n = lens[b]
        for h in range(Hq):
            kv = h // G
            a = oracle.scores(qf[b, h], kf[b, kv, :n], sc)
            gk = mf[b, h, :n]
            if pre:                          # exact E, Eq. 4, on the GPU's kept set
                thv = oracle.presoftmax.table_row(theta, h, n - 1)
                assert not ((gk != (a >= thv)) & ~ambiguous(a, thv)).any(), f"mask mismatch b{b} h{h}"
                w, beta = oracle.presoftmax.pre_weights_for_mask(a, gk, thv, sdc="exact")
                ro = w @ vf[b, kv, :n] + beta * vm[b, kv]
            else:
                s = oracle.post_softmax(a)[0]
                check_row_mask(gk, s, theta_of(theta, h, n - 1), f"b{b} h{h}")
                ro, _ = oracle.row_output(s, gk, vf[b, kv, :n], vm[b, kv], vmc=True, renorm=False)
            flat_check(g[b, h], ro, f"b{b} h{h}")


@pytest.mark.parametrize("dtype,L,d", [(torch.bfloat16, 4133, 128), (torch.bfloat16, 191, 64),
                                       (torch.bfloat16, 127, 128), (torch.float32, 300, 64)])
def test_prefill_vmc_keeps_nothing_is_prefix_mean(dtype, L, d):
    """theta above every probability, with VMC: nothing is kept, beta = 1, and
    the float32 output of row p is the causal mean of V rows 0..p.  Every row
    is checked against the oracle's prefix mean, at lengths whose running sums
    span one chunk of 64 rows (127), three with a longer last one (191) and 64
    with a ragged last one (4133)."""
    print(f"prefill vmc prefix mean {dtype} L={L} d={d}", flush=True)
    dev = device()
    Hq, Hkv = 2, 2
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 12, L, B=1, Hq=Hq, Hkv=Hkv, Lq=L, Lk=L, d=d, dtype=dtype)
    th = torch.full((Hq, L), 1.5, dtype=torch.float32, device=dev)
    out = torch.full((1, Hq, L, d), 7.0, dtype=torch.float32, device=dev)
    kc = torch.full((1, Hq, L), -7, dtype=torch.int32, device=dev)
    bt = torch.full((1, Hq, L), -7.0, dtype=torch.float32, device=dev)
    ws = tt.workspace(tt.TOPTH_OP_PREFILL, 1, Hq, Hkv, L, L, d)
    tt.topth_prefill(q.to(dev), k.to(dev), v.to(dev), th, out, scale=1.0 / np.sqrt(d),
                     flags=tt.TOPTH_VMC | tt.TOPTH_OUT_F32, kept_count=kc, beta=bt, ws=ws)
    torch.cuda.synchronize()
    assert (kc.cpu().numpy() == 0).all()
    assert (bt.cpu().numpy() == 1.0).all()
    g = out.cpu().numpy()[0]
    vf = to_f64(v)
    for h in range(Hq):
        mu = oracle.prefix_mean(vf[0, h])
        err = np.abs(g[h] - mu) / np.maximum(np.abs(mu), 1e-30)
        assert (np.abs(g[h] - mu) <= 2.0 ** -23 * np.abs(mu) + 1e-30).all(), (h, float(err.max()))
