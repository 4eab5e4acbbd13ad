"""GQA selection variants of decode (load a key when at least min_votes heads of
the group keep it; optionally give every head all loaded keys) on the GPU,
through the C ABI, against the oracle (``oracle.serving.decode_gqa``).

The cases are chosen with no element inside the 1e-5 ambiguity band of its
threshold (checked on the oracle side first), so loaded sets, per-head masks
and counts must agree exactly; outputs to the bf16 / f32 output tolerances."""
import numpy as np
import pytest
import torch

import calibrated_threshold_pruning_amd as tt
from oracle import serving
from synth import CONFIG_IDS, ROLE_TEST, attention_inputs, to_f64
from parity import ambiguous, check_out, device, theta_of

from test_gpu_decode import decode_theta

pytestmark = pytest.mark.gpu

UNIT = CONFIG_IDS["unit"]


def _case(Hq, Hkv, d, Lmax, lens, dtype, seed_index):
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 9, seed_index, B=len(lens), Hq=Hq, Hkv=Hkv, Lq=1, Lk=Lmax,
                               d=d, dtype=dtype)
    q = q[:, :, 0].contiguous()
    theta = decode_theta(UNIT, Hq, Hkv, d, lens, 32, 3, dtype, 1)
    vf = to_f64(v)
    vm = np.stack([[vf[b, h, :lens[b]].mean(0) for h in range(Hkv)] for b in range(len(lens))])
    return q, k, v, theta, vm.astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("dtype,Hq,Hkv,d,Lmax,lens,seed", [
    (torch.bfloat16, 8, 2, 128, 1000, [1000, 537], 0),      # g = 4
    (torch.bfloat16, 16, 2, 128, 4100, [4100, 700], 1),     # g = 8, several chunks
    (torch.bfloat16, 16, 1, 64, 600, [600, 90], 0),         # g = 16
    (torch.bfloat16, 4, 2, 128, 300, [300, 129], 0),        # g = 2
    (torch.float32, 8, 2, 64, 500, [500, 77], 0),           # row kernels, two passes
])
@pytest.mark.parametrize("min_votes,augment", [(2, False), (2, True), (1, True), ("g", False)])
def test_decode_gqa_variants(dtype, Hq, Hkv, d, Lmax, lens, seed, min_votes, augment):
    g = Hq // Hkv
    m = g if min_votes == "g" else min_votes
    print(f"decode_gqa {dtype} Hq={Hq} Hkv={Hkv} d={d} lens={lens} min_votes={m} augment={augment}", flush=True)
    dev = device()
    q, k, v, theta, vm = _case(Hq, Hkv, d, Lmax, lens, dtype, seed)
    ref = serving.decode_gqa(to_f64(q), to_f64(k), to_f64(v), lens, theta, vm, 1.0 / np.sqrt(d), vmc=True,
                             min_votes=m, augment=augment)
    for b in range(len(lens)):
        for h in range(Hq):
            assert not ambiguous(ref.s[b][h], theta_of(theta, h, lens[b] - 1)).any(), "case has ambiguous elements"
    B = len(lens)
    out = torch.empty(B, Hq, d, dtype=dtype, device=dev)
    kc = torch.full((B, Hq), -7, dtype=torch.int32, device=dev)
    bt = torch.full((B, Hq), -7.0, dtype=torch.float32, device=dev)
    vr = torch.full((B, Hkv), -7, dtype=torch.int32, device=dev)
    km = torch.zeros((B, Hq, Lmax), dtype=torch.uint8, device=dev)
    ws = tt.workspace(tt.TOPTH_OP_DECODE, B, Hq, Hkv, 1, Lmax, d)
    for rep in range(2):                 # the second call reuses the workspace the first left prepared
        tt.topth_decode_gqa(q.to(dev), k.to(dev), v.to(dev), torch.tensor(lens, dtype=torch.int32, device=dev),
                            torch.tensor(theta, dtype=torch.float32, device=dev), out, ws,
                            scale=1.0 / np.sqrt(d), flags=tt.TOPTH_VMC, min_votes=m, augment=augment,
                            v_mean=torch.tensor(vm, dtype=torch.float32, device=dev), kept_count=kc, beta=bt,
                            vrows_read=vr, kept_mask=km)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32)[0].item()) == 0, "exchange wait timed out"
        og, kcg, btg = out.float().cpu().numpy(), kc.cpu().numpy(), bt.cpu().numpy()
        vrg, kmg = vr.cpu().numpy(), km.cpu().numpy().astype(bool)
        assert (vrg == ref.vrows_read).all(), (vrg, ref.vrows_read)
        assert (kcg == ref.kept_count).all()
        for b in range(B):
            for h in range(Hq):
                assert (kmg[b, h, :lens[b]] == ref.keep[b][h]).all(), (b, h)
                check_out(og[b, h], ref.out[b, h], dtype, f"b{b} h{h}")
                assert abs(btg[b, h] - ref.beta[b, h]) <= 1e-5


def test_decode_gqa_without_optional_outputs():
    """No kept mask, counts, beta or union size: same output bits as with them."""
    print("decode_gqa bare", flush=True)
    dev = device()
    Hq, Hkv, d, Lmax, lens = 16, 2, 128, 4100, [4100, 700]
    q, k, v, theta, vm = _case(Hq, Hkv, d, Lmax, lens, torch.bfloat16, 1)
    outs = []
    for full in (True, False):
        B = len(lens)
        out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)
        extra = dict(kept_count=torch.empty(B, Hq, dtype=torch.int32, device=dev),
                     beta=torch.empty(B, Hq, dtype=torch.float32, device=dev),
                     vrows_read=torch.empty(B, Hkv, dtype=torch.int32, device=dev),
                     kept_mask=torch.zeros(B, Hq, Lmax, dtype=torch.uint8, device=dev)) if full else {}
        ws = tt.workspace(tt.TOPTH_OP_DECODE, B, Hq, Hkv, 1, Lmax, d)
        tt.topth_decode_gqa(q.to(dev), k.to(dev), v.to(dev), torch.tensor(lens, dtype=torch.int32, device=dev),
                            torch.tensor(theta, dtype=torch.float32, device=dev), out, ws,
                            scale=1.0 / np.sqrt(d), flags=tt.TOPTH_VMC, min_votes=3, augment=True,
                            v_mean=torch.tensor(vm, dtype=torch.float32, device=dev), **extra)
        torch.cuda.synchronize()
        outs.append(out.float().cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    ref = serving.decode_gqa(to_f64(q), to_f64(k), to_f64(v), lens, theta, vm, 1.0 / np.sqrt(d), vmc=True,
                             min_votes=3, augment=True)
    for b in range(len(lens)):
        for h in range(Hq):
            check_out(outs[1][b, h], ref.out[b, h], torch.bfloat16, f"b{b} h{h}")
