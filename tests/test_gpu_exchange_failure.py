"""The decode exchange's failure path, forced from the host.

The key chunks of one (batch, KV head) group exchange partial results through
workspace slots with bounded waits.  A spin limit of one poll makes a wait give
up whenever one chunk runs ahead of another; every kernel still ends normally.
The contract checked here (include/topth.h, "Exchange failures"):
  * the status word reports the timeout;
  * each group either matches the undisturbed result bit for bit or is
    poisoned (NaN outputs and beta, -1 counts), never partial;
  * while the status is set, every later call poisons all of its outputs (the
    running mean of topth_decode_append is still updated);
  * topth_workspace_init restores the undisturbed results bit for bit.
"""
import numpy as np
import pytest
import torch

import calibrated_threshold_pruning_amd as tt
from synth import CONFIG_IDS, ROLE_TEST, attention_inputs
from parity import device

pytestmark = pytest.mark.gpu

UNIT = CONFIG_IDS["unit"]


def _case(dev):
    # 4 query heads per KV head; 20000 keys give ten key chunks per group
    B, Hq, Hkv, d, Lmax = 4, 8, 2, 128, 20000
    lens = [20000, 15000, 9000, 3000]
    q, k, v = attention_inputs(UNIT, ROLE_TEST, 0, 21, B=B, Hq=Hq, Hkv=Hkv, Lq=1, Lk=Lmax, d=d, n_sinks=1,
                               dtype=torch.bfloat16)
    q = q[:, :, 0].contiguous().to(dev)
    k, v = k.to(dev), v.to(dev)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=dev)
    theta = torch.full((Hq, Lmax), 2e-4, dtype=torch.float32, device=dev)
    vm = torch.empty(B, Hkv, d, dtype=torch.float32, device=dev)
    tt.topth_vmean(v, lens_d, vm)
    return q, k, v, lens_d, theta, vm


def _run(case, ws, append_mean=None):
    q, k, v, lens_d, theta, vm = case
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    out = torch.zeros_like(q)
    kc = torch.full((B, Hq), -7, dtype=torch.int32, device=q.device)
    bt = torch.full((B, Hq), -7.0, dtype=torch.float32, device=q.device)
    vr = torch.full((B, Hkv), -7, dtype=torch.int32, device=q.device)
    if append_mean is None:
        tt.topth_decode(q, k, v, lens_d, theta, out, ws, scale=1.0 / np.sqrt(d), flags=tt.TOPTH_VMC,
                        v_mean=vm, kept_count=kc, beta=bt, vrows_read=vr)
    else:
        tt.topth_decode_append(q, k, v, lens_d, theta, out, ws, append_mean, scale=1.0 / np.sqrt(d),
                               flags=tt.TOPTH_VMC, kept_count=kc, beta=bt, vrows_read=vr)
    torch.cuda.synchronize()
    return dict(out=out.view(torch.int16).cpu().numpy(), kc=kc.cpu().numpy(), beta=bt.cpu().numpy(),
                vr=vr.cpu().numpy())


def _group_state(r, ref, b, kv, G):
    """'ok' when the group's outputs equal the reference bit for bit,
    'poisoned' when all of them carry the poison values, else 'partial'."""
    hs = slice(kv * G, (kv + 1) * G)
    same = (np.array_equal(r["out"][b, hs], ref["out"][b, hs]) and np.array_equal(r["kc"][b, hs], ref["kc"][b, hs])
            and np.array_equal(r["beta"][b, hs].view(np.int32), ref["beta"][b, hs].view(np.int32))
            and r["vr"][b, kv] == ref["vr"][b, kv])
    if same:
        return "ok"
    out_nan = (r["out"][b, hs].view(np.uint16) & 0x7FFF) > 0x7F80       # bfloat16 NaN bit patterns
    poisoned = (out_nan.all() and (r["kc"][b, hs] == -1).all() and np.isnan(r["beta"][b, hs]).all()
                and r["vr"][b, kv] == -1)
    return "poisoned" if poisoned else "partial"


def test_exchange_give_up_is_reported_and_recoverable():
    dev = device()
    case = _case(dev)
    q, k, _, _, _, vm = case
    B, Hq = q.shape[0], q.shape[1]
    Hkv = k.shape[1]
    G = Hq // Hkv
    ws = tt.workspace(tt.TOPTH_OP_DECODE, B, Hq, Hkv, 1, k.shape[2], q.shape[2])
    print("exchange failure: undisturbed reference", flush=True)
    ref = _run(case, ws)
    assert tt.topth_workspace_status(ws) == 0
    assert (ref["kc"] > 0).all() and (ref["vr"] > 0).all()

    print("exchange failure: spin limit 1", flush=True)
    tt.topth_workspace_set_spin_limit(ws, 1)
    r = _run(case, ws)
    status = tt.topth_workspace_status(ws)
    states = [_group_state(r, ref, b, kv, G) for b in range(B) for kv in range(Hkv)]
    assert "partial" not in states, states
    assert status == tt.TOPTH_STATUS_EXCHANGE_TIMEOUT, (status, states)
    assert "poisoned" in states, states

    print("exchange failure: status set, default spin limit restored", flush=True)
    tt.topth_workspace_set_spin_limit(ws, 0)
    r = _run(case, ws)
    assert all(_group_state(r, ref, b, kv, G) == "poisoned" for b in range(B) for kv in range(Hkv))
    assert tt.topth_workspace_status(ws) == tt.TOPTH_STATUS_EXCHANGE_TIMEOUT

    # the running mean is updated even by a poisoned call: the same as in a
    # call on a prepared workspace
    print("exchange failure: running mean under a set status", flush=True)
    lens = case[3].cpu().tolist()
    old = torch.tensor([n - 1 for n in lens], dtype=torch.int32, device=dev)
    mu_prev = torch.empty_like(vm)
    tt.topth_vmean(case[2], old, mu_prev)
    mu_bad = mu_prev.clone()
    _run(case, ws, append_mean=mu_bad)
    ws2 = tt.workspace(tt.TOPTH_OP_DECODE, B, Hq, Hkv, 1, k.shape[2], q.shape[2])
    mu_good = mu_prev.clone()
    _run(case, ws2, append_mean=mu_good)
    assert torch.equal(mu_bad, mu_good)

    print("exchange failure: re-initialised workspace", flush=True)
    tt.topth_workspace_init(ws)
    r = _run(case, ws)
    assert tt.topth_workspace_status(ws) == 0
    assert all(_group_state(r, ref, b, kv, G) == "ok" for b in range(B) for kv in range(Hkv))
    # and the workspace stays prepared for the next call
    r = _run(case, ws)
    assert tt.topth_workspace_status(ws) == 0
    assert all(_group_state(r, ref, b, kv, G) == "ok" for b in range(B) for kv in range(Hkv))
