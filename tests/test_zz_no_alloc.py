"""topth_decode_noalloc (the decode step for callers that cannot allocate)
against topth_decode on the same inputs: both run the same kernels, so every
output must agree bit for bit.  Two calls in a row share the library's static
scratch, the second on a smaller input; a shape beyond the scratch is refused
before anything runs."""
import numpy as np
import pytest
import torch

import calibrated_threshold_pruning_amd as tt
from synth import CONFIG_IDS, ROLE_TEST, attention_inputs
from parity import device

pytestmark = pytest.mark.gpu

UNIT = CONFIG_IDS["unit"]


def _inputs(dev, B, Hq, Hkv, d, Lmax, lens, dtype, index):
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 0, index, B=B, Hq=Hq, Hkv=Hkv, Lq=1, Lk=Lmax, d=d,
                               n_sinks=1, dtype=dtype)
    q = q[:, :, 0].contiguous().to(dev)
    k, v = k.to(dev), v.to(dev)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=dev)
    # thresholds a little under 1/n keep tens to hundreds of keys per row
    n_rows = Lmax
    p = torch.arange(n_rows, dtype=torch.float32, device=dev)
    theta = (0.6 / (p + 1.0)).expand(Hq, n_rows).contiguous()
    theta[:, :16] = -float("inf")
    vm = torch.empty(B, Hkv, d, dtype=torch.float32, device=dev)
    tt.topth_vmean(v, lens_d, vm)
    return q, k, v, lens_d, theta, vm


def _outputs(q, k, dev):
    B, Hq, d = q.shape
    Hkv, Lmax = k.shape[1], k.shape[2]
    return dict(out=torch.full_like(q, 7.0), kc=torch.full((B, Hq), -7, dtype=torch.int32, device=dev),
                bt=torch.full((B, Hq), -7.0, dtype=torch.float32, device=dev),
                vr=torch.full((B, Hkv), -7, dtype=torch.int32, device=dev),
                km=torch.zeros((B, Hq, Lmax), dtype=torch.uint8, device=dev))


def _compare(case, dev, flags):
    q, k, v, lens_d, theta, vm = case
    B, Hq, d = q.shape
    Hkv, Lmax = k.shape[1], k.shape[2]
    ref = _outputs(q, k, dev)
    ws = tt.workspace(tt.TOPTH_OP_DECODE, B, Hq, Hkv, 1, Lmax, d)
    tt.topth_decode(q, k, v, lens_d, theta, ref["out"], ws, scale=1.0 / np.sqrt(d), flags=flags, v_mean=vm,
                    kept_count=ref["kc"], beta=ref["bt"], vrows_read=ref["vr"], kept_mask=ref["km"])
    got = _outputs(q, k, dev)
    tt.topth_decode_noalloc(q, k, v, lens_d, theta, got["out"], scale=1.0 / np.sqrt(d), flags=flags, v_mean=vm,
                            kept_count=got["kc"], beta=got["bt"], vrows_read=got["vr"], kept_mask=got["km"])
    torch.cuda.synchronize()
    assert tt.topth_workspace_status(ws) == 0
    for name in ("out", "kc", "bt", "vr", "km"):
        a, b = ref[name], got[name]
        if a.dtype.is_floating_point:
            a, b = a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32), \
                b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)
        assert torch.equal(a, b), name
    assert (ref["kc"] >= 0).all() and (ref["vr"] >= 0).all()
    return ref


def test_noalloc_matches_decode_on_two_calls():
    dev = device()
    print("noalloc: call 1, batch 4, 32/8 heads, 4096 keys", flush=True)
    big = _inputs(dev, 4, 32, 8, 128, 4096, [4096, 3000, 1, 2049], torch.bfloat16, 31)
    r = _compare(big, dev, tt.TOPTH_VMC)
    assert r["kc"].max() > 16
    print("noalloc: call 2, batch 2, 8/2 heads, 700 keys", flush=True)
    small = _inputs(dev, 2, 8, 2, 128, 700, [700, 65], torch.bfloat16, 32)
    _compare(small, dev, tt.TOPTH_VMC)
    print("noalloc: call 3, group size 8, SDC none", flush=True)
    g8 = _inputs(dev, 2, 16, 2, 64, 2500, [2500, 1000], torch.bfloat16, 33)
    _compare(g8, dev, tt.TOPTH_SDC_NONE)


def test_noalloc_float32_path():
    dev = device()
    print("noalloc: float32, 8/2 heads, d 64, 300 keys", flush=True)
    case = _inputs(dev, 2, 8, 2, 64, 300, [300, 129], torch.float32, 34)
    _compare(case, dev, tt.TOPTH_VMC)


def test_noalloc_refuses_shapes_beyond_scratch():
    dev = device()
    # batch 16 x 8 KV heads x 32768 keys at group size 8: 128 MiB of overflow
    # weights alone, more than the 80 MiB scratch; refused before any launch
    B, Hq, Hkv, d, Lmax = 16, 64, 8, 128, 32768
    q = torch.zeros(B, Hq, d, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(B, Hkv, Lmax, d, dtype=torch.bfloat16, device=dev)
    lens = torch.full((B,), Lmax, dtype=torch.int32, device=dev)
    theta = torch.full((Hq, Lmax), -float("inf"), dtype=torch.float32, device=dev)
    out = torch.full_like(q, 3.0)
    with pytest.raises(tt.TopthError) as ei:
        tt.topth_decode_noalloc(q, k, k, lens, theta, out, scale=1.0 / np.sqrt(d), flags=0)
    assert ei.value.status == tt.TOPTH_ESCRATCH
    torch.cuda.synchronize()
    assert (out.float() == 3.0).all()                 # nothing ran
