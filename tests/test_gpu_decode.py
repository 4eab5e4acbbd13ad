"""Decode parity: HIP path (through the C ABI) against the CPU oracle."""
import numpy as np
import pytest
import torch

import calibrated_threshold_pruning_amd as tt
import oracle
from synth import CONFIG_IDS, ROLE_CALIB, ROLE_TEST, attention_inputs, to_f64
from parity import check_out, check_row_mask, device, theta_of

pytestmark = pytest.mark.gpu

UNIT = CONFIG_IDS["unit"]


def decode_theta(cfg, Hq, Hkv, d, lens, k, n_seq, dtype, n_sinks, n_rows=None):
    """Oracle theta [Hq, n_rows] from decode-style calibration at rows n-1."""
    scale = 1.0 / np.sqrt(d)
    rows = sorted(set(int(n) - 1 for n in lens))
    R = n_rows or (max(rows) + 1)
    cal = oracle.Calibrator([k], Hq, R)
    for i in range(n_seq):
        for r in rows:
            q, kk, _ = attention_inputs(cfg, ROLE_CALIB, 0, i * 64 + rows.index(r), B=1, Hq=Hq,
                                        Hkv=Hkv, Lq=1, Lk=r + 1, d=d, n_sinks=n_sinks, dtype=dtype,
                                        with_v=False)
            cal.observe(to_f64(q[0]), to_f64(kk[0]), scale, q_pos0=r)
    return cal.finalize()[0]


def run_decode(q, k, v, lens, theta, vm, flags, ws=None):
    dev = device()
    B, Hq, d = q.shape
    Hkv, Lmax = k.shape[1], k.shape[2]
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=dev)
    th = torch.tensor(theta, dtype=torch.float32, device=dev).contiguous()
    vmd = torch.tensor(vm, dtype=torch.float32, device=dev).contiguous()
    out = torch.empty_like(qd)
    kc = torch.full((B, Hq), -7, dtype=torch.int32, device=dev)
    bt = torch.full((B, Hq), -7.0, dtype=torch.float32, device=dev)
    vr = torch.full((B, Hkv), -7, dtype=torch.int32, device=dev)
    km = torch.zeros((B, Hq, Lmax), dtype=torch.uint8, device=dev)
    if ws is None:
        ws = tt.workspace(tt.TOPTH_OP_DECODE, B, Hq, Hkv, 1, Lmax, d)
    tt.topth_decode(qd, kd, vd, lens_d, th, out, ws, scale=1.0 / np.sqrt(d), flags=flags,
                    v_mean=vmd, kept_count=kc, beta=bt, vrows_read=vr, kept_mask=km)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32)[0].item()) == 0, "exchange wait timed out"
    return dict(out=out.float().cpu().numpy(), kc=kc.cpu().numpy(), beta=bt.cpu().numpy(),
                vr=vr.cpu().numpy(), mask=km.cpu().numpy().astype(bool))


def compare_decode(g, q, k, v, lens, theta, vm, flags, dtype):
    """Oracle on the same inputs; masks, counts, union, beta and outputs."""
    vmc = bool(flags & tt.TOPTH_VMC)
    renorm = bool(flags & tt.TOPTH_SDC_NONE)
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    B, Hq, d = qf.shape
    Hkv = kf.shape[1]
    G = Hq // Hkv
    ref = oracle.decode(qf, kf, vf, lens, theta, vm, 1.0 / np.sqrt(d), vmc=vmc, renorm=renorm)
    n_amb = 0
    for b in range(B):
        n = int(lens[b])
        for kv in range(Hkv):
            union = np.zeros(n, dtype=bool)
            for h in range(kv * G, (kv + 1) * G):
                gk = g["mask"][b, h, :n]
                th = theta_of(theta, h, n - 1)
                amb = check_row_mask(gk, ref.s[b][h], th, f"b{b} h{h}")
                n_amb += amb
                assert g["kc"][b, h] == gk.sum()
                if amb == 0:
                    assert g["kc"][b, h] == ref.kept_count[b, h]
                ro, rb = oracle.row_output(ref.s[b][h], gk, vf[b, kv, :n], vm[b, kv],
                                                 vmc=vmc, renorm=renorm)
                check_out(g["out"][b, h], ro, dtype, f"b{b} h{h}")
                assert abs(g["beta"][b, h] - rb) <= 1e-5, (b, h, g["beta"][b, h], rb)
                union |= gk
            assert g["vr"][b, kv] == union.sum(), (b, kv)
    return ref, n_amb


def make_case(Hq, Hkv, d, Lmax, lens, k=32, dtype=torch.bfloat16, n_sinks=1, seed_index=0,
              n_cal=6, cfg=UNIT):
    q, kk, v = attention_inputs(cfg, ROLE_TEST, 0, seed_index, B=len(lens), Hq=Hq, Hkv=Hkv, Lq=1,
                                Lk=Lmax, d=d, n_sinks=n_sinks, dtype=dtype)
    q = q[:, :, 0].contiguous()
    theta = decode_theta(cfg, Hq, Hkv, d, lens, k, n_cal, dtype, n_sinks)
    vf = to_f64(v)
    vm = np.stack([[vf[b, h, :lens[b]].mean(0) for h in range(Hkv)] for b in range(len(lens))])
    vm = vm.astype(np.float32).astype(np.float64)    # the float32 values the GPU receives
    return q, kk, v, theta, vm


@pytest.mark.parametrize("Hq,Hkv,d,Lmax,lens", [
    (8, 2, 128, 1000, [1000, 537, 1]),        # g=4, ragged, single-key row
    (16, 2, 128, 700, [700, 65]),             # g=8
    (4, 4, 128, 300, [300, 129]),             # g=1
    (8, 4, 64, 520, [520, 17]),               # g=2, d=64
    (16, 1, 128, 400, [400, 200]),            # g=16
    (8, 2, 64, 2500, [2500, 2499, 1024]),     # g=4, d=64, several chunks
    (8, 2, 128, 4100, [4100, 2049, 2048, 2047]),  # lengths at and around chunk boundaries
    (16, 1, 64, 300, [300, 33]),              # g=16, d=64
    # one KV head, 10 chunks of 2048 keys per group: the exchange and the combine
    # poll in several batches, and the short row leaves most of its chunks empty
    (4, 1, 128, 20000, [20000, 100]),
])
def test_decode_bf16_parity(Hq, Hkv, d, Lmax, lens):
    print(f"decode bf16 Hq={Hq} Hkv={Hkv} d={d} Lmax={Lmax} lens={lens}", flush=True)
    q, k, v, theta, vm = make_case(Hq, Hkv, d, Lmax, lens)
    g = run_decode(q, k, v, lens, theta, vm, tt.TOPTH_VMC)
    compare_decode(g, q, k, v, lens, theta, vm, tt.TOPTH_VMC, torch.bfloat16)


@pytest.mark.parametrize("flags", [0, tt.TOPTH_SDC_NONE, tt.TOPTH_VMC | tt.TOPTH_SDC_NONE])
def test_decode_bf16_flags(flags):
    lens = [900, 300]
    q, k, v, theta, vm = make_case(8, 2, 128, 900, lens, seed_index=1)
    g = run_decode(q, k, v, lens, theta, vm, flags)
    compare_decode(g, q, k, v, lens, theta, vm, flags, torch.bfloat16)


def test_decode_dense_and_empty_thresholds():
    lens = [640, 77]
    q, k, v, theta, vm = make_case(8, 2, 128, 640, lens, seed_index=2)
    dense = np.full_like(theta, -np.inf)
    g = run_decode(q, k, v, lens, dense, vm, tt.TOPTH_VMC)
    compare_decode(g, q, k, v, lens, dense, vm, tt.TOPTH_VMC, torch.bfloat16)
    assert (g["vr"] == np.array(lens)[:, None]).all()
    assert np.abs(g["beta"]).max() < 1e-5
    none = np.full_like(theta, 2.0)               # above every probability: nothing kept
    g = run_decode(q, k, v, lens, none, vm, tt.TOPTH_VMC)
    assert (g["kc"] == 0).all() and (g["vr"] == 0).all()
    np.testing.assert_allclose(g["beta"], 1.0)
    vmb = np.repeat(vm, 4, axis=1)                # out = mu for every head of the group
    assert np.abs(g["out"] - vmb).max() <= 1e-2
    g = run_decode(q, k, v, lens, none, vm, tt.TOPTH_SDC_NONE)
    assert np.abs(g["out"]).max() == 0.0


@pytest.mark.parametrize("B,Hq,Hkv,d,Lmax", [
    # g=8, d=128: 64 groups x 5 chunks of the 8-tile variant exceed 256 workgroups,
    # so the 16-tile variant runs (512 keys per wave, 256 in the LDS list)
    (8, 64, 8, 128, 8200),
    # g=4, d=64: 128 groups x 3 chunks of the 4-tile variant exceed 256, so the
    # 8-tile variant runs (512 keys per wave, 256 in the LDS list)
    (64, 8, 2, 64, 4200),
])
def test_decode_dense_overflow(B, Hq, Hkv, d, Lmax):
    """theta = -inf keeps every key: each wave's kept list outgrows its LDS room and
    the rest of its weights go through the workspace on the MFMA accumulate path."""
    print(f"decode dense overflow B={B} Hq={Hq} Hkv={Hkv} d={d} Lmax={Lmax}", flush=True)
    base = [Lmax, Lmax - 1, Lmax // 2 + 1, Lmax // 2, 1000, 257, 33, 1]
    lens = [base[i % len(base)] for i in range(B)]
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 0, 7, B=B, Hq=Hq, Hkv=Hkv, Lq=1, Lk=Lmax, d=d,
                               n_sinks=1, dtype=torch.bfloat16)
    q = q[:, :, 0].contiguous()
    vf = to_f64(v)
    vm = np.stack([[vf[b, h, :lens[b]].mean(0) for h in range(Hkv)] for b in range(B)])
    vm = vm.astype(np.float32).astype(np.float64)
    dense = np.full((Hq, Lmax), -np.inf)
    g = run_decode(q, k, v, lens, dense, vm, tt.TOPTH_VMC)
    assert (g["vr"] == np.array(lens)[:, None]).all()
    assert (g["kc"] == np.array(lens)[:, None]).all()
    compare_decode(g, q, k, v, lens, dense, vm, tt.TOPTH_VMC, torch.bfloat16)


def test_decode_workspace_shared_by_f32_and_bf16_calls():
    """An fp32 decode call (row kernels, kept-key masks in the workspace) between
    bf16 calls on the same workspace: the bf16 result is bit-identical to the one
    on a fresh workspace, so the fp32 call leaves the exchange slots empty."""
    lens = [4100, 2049]                            # several key chunks per group
    qb, kb, vb, thb, vmb = make_case(8, 2, 128, 4100, lens, seed_index=8)
    qf, kf, vf, thf, vmf = make_case(8, 2, 128, 4100, lens, dtype=torch.float32, seed_index=9)
    fresh = run_decode(qb, kb, vb, lens, thb, vmb, tt.TOPTH_VMC)
    ws = tt.workspace(tt.TOPTH_OP_DECODE, 2, 8, 2, 1, 4100, 128)
    gb1 = run_decode(qb, kb, vb, lens, thb, vmb, tt.TOPTH_VMC, ws=ws)
    gf = run_decode(qf, kf, vf, lens, thf, vmf, tt.TOPTH_VMC, ws=ws)
    gb2 = run_decode(qb, kb, vb, lens, thb, vmb, tt.TOPTH_VMC, ws=ws)
    for key in fresh:
        assert np.array_equal(fresh[key], gb1[key]), key
        assert np.array_equal(fresh[key], gb2[key]), key
    compare_decode(gf, qf, kf, vf, lens, thf, vmf, tt.TOPTH_VMC, torch.float32)
    compare_decode(gb2, qb, kb, vb, lens, thb, vmb, tt.TOPTH_VMC, torch.bfloat16)


def test_decode_f32_parity():
    lens = [333, 100, 1]
    q, k, v, theta, vm = make_case(8, 2, 64, 333, lens, dtype=torch.float32, seed_index=3)
    for flags in (tt.TOPTH_VMC, tt.TOPTH_SDC_NONE):
        g = run_decode(q, k, v, lens, theta, vm, flags)
        compare_decode(g, q, k, v, lens, theta, vm, flags, torch.float32)


def test_decode_deterministic_and_workspace_reuse():
    lens = [1500, 1499]
    q, k, v, theta, vm = make_case(16, 2, 128, 1500, lens, seed_index=4)
    ws = tt.workspace(tt.TOPTH_OP_DECODE, 2, 16, 2, 1, 1500, 128)
    g1 = run_decode(q, k, v, lens, theta, vm, tt.TOPTH_VMC, ws=ws)
    # a smaller call on the same workspace, then the first call again
    q2, k2, v2, th2, vm2 = make_case(8, 2, 64, 300, [300], seed_index=5)
    g2 = run_decode(q2, k2, v2, [300], th2, vm2, tt.TOPTH_VMC, ws=ws)
    compare_decode(g2, q2, k2, v2, [300], th2, vm2, tt.TOPTH_VMC, torch.bfloat16)
    g3 = run_decode(q, k, v, lens, theta, vm, tt.TOPTH_VMC, ws=ws)
    for key in g1:
        assert np.array_equal(g1[key], g3[key]), key
    compare_decode(g1, q, k, v, lens, theta, vm, tt.TOPTH_VMC, torch.bfloat16)


def test_vmean_kernel():
    dev = device()
    _, _, v = attention_inputs(UNIT, ROLE_TEST, 1, 0, B=2, Hq=2, Hkv=2, Lq=1, Lk=257, d=128)
    lens = [257, 30]
    out = torch.empty(2, 2, 128, dtype=torch.float32, device=dev)
    tt.topth_vmean(v.to(dev), torch.tensor(lens, dtype=torch.int32, device=dev), out)
    torch.cuda.synchronize()
    vf = to_f64(v)
    ref = np.stack([[vf[b, h, :lens[b]].mean(0) for h in range(2)] for b in range(2)])
    np.testing.assert_allclose(out.cpu().numpy(), ref, rtol=1e-6, atol=1e-7)


# ----------------------------------------------------------------- full sizes
def test_decode_8b_full_size():
    """LLaMA-3-8B-like decode step: B16, 32/8 heads, d128, n=4096, k=128, VMC."""
    cfg = CONFIG_IDS["decode_8b"]
    lens = [4096] * 16
    print("decode_8b full size", flush=True)
    q, k, v, theta, vm = make_case(32, 8, 128, 4096, lens, k=128, n_cal=16, cfg=cfg)
    g = run_decode(q, k, v, lens, theta, vm, tt.TOPTH_VMC)
    ref, n_amb = compare_decode(g, q, k, v, lens, theta, vm, tt.TOPTH_VMC, torch.bfloat16)
    assert n_amb < 50


def test_decode_70b_32k_full_size():
    """LLaMA-3-70B-like decode step: B8, 64/8 heads, d128, n=32768, sinks 0-3, k=256."""
    cfg = CONFIG_IDS["decode_70b_32k"]
    lens = [32768] * 8
    print("decode_70b_32k full size", flush=True)
    q, k, v, theta, vm = make_case(64, 8, 128, 32768, lens, k=256, n_cal=4, cfg=cfg, n_sinks=4)
    g = run_decode(q, k, v, lens, theta, vm, tt.TOPTH_VMC)
    compare_decode(g, q, k, v, lens, theta, vm, tt.TOPTH_VMC, torch.bfloat16)


def test_decode_graph_replay_matches_eager():
    """Several decode steps captured in one HIP graph: every replay (with eager
    work and synchronisations in between) reproduces the eager results."""
    dev = device()
    Hq, Hkv, d, n = 16, 2, 128, 1200
    cases = [make_case(Hq, Hkv, d, n, [n, 700], seed_index=10 + i) for i in range(3)]
    lens = torch.tensor([n, 700], dtype=torch.int32, device=dev)
    ws = tt.workspace(tt.TOPTH_OP_DECODE, 2, Hq, Hkv, 1, n, d)
    ins, outs = [], []
    for q, k, v, theta, vm in cases:
        ins.append((q.to(dev), k.to(dev), v.to(dev), torch.tensor(theta, dtype=torch.float32, device=dev),
                    torch.tensor(vm, dtype=torch.float32, device=dev)))
        outs.append((torch.empty(2, Hq, d, dtype=torch.bfloat16, device=dev),
                     torch.empty(2, Hq, dtype=torch.int32, device=dev)))

    def run_all():
        for (q, k, v, th, vm), (o, kc) in zip(ins, outs):
            tt.topth_decode(q, k, v, lens, th, o, ws, scale=1.0 / np.sqrt(d), flags=tt.TOPTH_VMC,
                            v_mean=vm, kept_count=kc)

    run_all()
    torch.cuda.synchronize()
    eager = [(o.clone(), kc.clone()) for o, kc in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_all()
    for rep in range(4):
        for o, kc in outs:
            o.zero_(); kc.zero_()
        junk = torch.randn(1 << 20, device=dev).sum()      # unrelated eager work in between
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for (o, kc), (eo, ekc) in zip(outs, eager):
            assert torch.equal(o, eo), f"replay {rep}: output differs"
            assert torch.equal(kc, ekc), f"replay {rep}: kept counts differ"
    assert int(ws[:4].view(torch.int32)[0].item()) == 0
