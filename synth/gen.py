"""Seeded generator for the synthetic attention workloads.

Recipe (one call = one seed = one group of tensors):

* ``u = ones(d) / sqrt(d)`` is a fixed unit vector.
* Keys: ``K ~ N(0, 1)``; every key row (per batch element, KV head and
  position) is multiplied by ``lambda = exp(0.5 * z)``, ``z ~ N(0, 1)``
  (a lognormal(0, 0.5) scale); afterwards the first ``n_sinks`` key rows get
  ``+3u`` added.
* Queries: ``Q ~ N(0, 1) + u`` (``u`` added once to every query row).
* Values: ``V ~ N(0, 1)``, unscaled.
* Draw order inside one seed: K normals, lambda normals, Q normals, V normals,
  all from ``numpy.random.Generator(Philox(seed))`` in float64, then cast to
  float32 and, for bf16 workloads, rounded to bfloat16 (round-to-nearest-even,
  done by torch).

Seeds are ``(config_id << 40) | (role << 32) | (layer << 20) | index`` so that
calibration, test and probe draws never share a stream.

Every tensor is returned on the CPU; callers move it to the GPU.  ``to_f64``
gives the exact float64 up-cast of a (possibly bf16) tensor for the oracle.
"""
from __future__ import annotations

import numpy as np
import torch

# Workload ids (one per synthetic configuration, see the bench and tests).
CONFIG_IDS = {
    "tiny_prefill_f32": 0,       # 1 head, d=64, L=256, fp32
    "decode_8b": 1,              # B16, 32/8 heads, d=128, n=4096, bf16
    "prefill_8k": 2,             # 32/8 heads, d=128, L=8192, bf16, 4 layers
    "decode_70b_32k": 3,         # B8, 64/8 heads, d=128, n=32768, bf16
    "calib_sweep": 4,            # 32 layers x 8 heads, d=128, L=2048, bf16
    "unit": 15,                  # small shapes used only by unit tests
}
ROLE_TEST, ROLE_CALIB, ROLE_PROBE = 0, 1, 2


def seed_of(config_id: int, role: int, layer: int, index: int) -> int:
    if not (0 <= role < 256 and 0 <= layer < 4096 and 0 <= index < (1 << 20)):
        raise ValueError("seed field out of range")
    return (int(config_id) << 40) | (int(role) << 32) | (int(layer) << 20) | int(index)


def _cast(x64: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x64.astype(np.float32)))
    return t if dtype == torch.float32 else t.to(dtype)


def attention_inputs(config_id: int, role: int, layer: int, index: int, *,
                     B: int, Hq: int, Hkv: int, Lq: int, Lk: int, d: int,
                     n_sinks: int = 1, dtype: torch.dtype = torch.bfloat16,
                     with_v: bool = True):
    """Return ``(q, k, v)`` CPU tensors of shapes ``[B,Hq,Lq,d]``,
    ``[B,Hkv,Lk,d]``, ``[B,Hkv,Lk,d]`` (``v`` is None if ``with_v`` is False)."""
    if dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("dtype must be float32 or bfloat16")
    rng = np.random.Generator(np.random.Philox(seed_of(config_id, role, layer, index)))
    u = np.ones(d) / np.sqrt(d)
    k = rng.standard_normal((B, Hkv, Lk, d))
    lam = np.exp(0.5 * rng.standard_normal((B, Hkv, Lk, 1)))
    k = k * lam
    ns = min(n_sinks, Lk)
    if ns > 0:
        k[:, :, :ns, :] += 3.0 * u
    q = rng.standard_normal((B, Hq, Lq, d)) + u
    v = rng.standard_normal((B, Hkv, Lk, d)) if with_v else None
    return (_cast(q, dtype), _cast(k, dtype), None if v is None else _cast(v, dtype))


def batch_of_sequences(config_id: int, role: int, layer: int, first: int, count: int, *,
                       Hq: int, Hkv: int, Lq: int, Lk: int, d: int, n_sinks: int = 1,
                       dtype: torch.dtype = torch.bfloat16, with_v: bool = False):
    """Stack ``count`` independently seeded sequences (indices ``first..first+count-1``)
    along a leading batch axis: ``q [count,Hq,Lq,d]``, ``k [count,Hkv,Lk,d]``."""
    qs, ks, vs = [], [], []
    for i in range(first, first + count):
        q, k, v = attention_inputs(config_id, role, layer, i, B=1, Hq=Hq, Hkv=Hkv, Lq=Lq,
                                   Lk=Lk, d=d, n_sinks=n_sinks, dtype=dtype, with_v=with_v)
        qs.append(q[0]); ks.append(k[0])
        if with_v:
            vs.append(v[0])
    q = torch.stack(qs); k = torch.stack(ks)
    v = torch.stack(vs) if with_v else None
    return q, k, v


def attention_inputs_device(config_id: int, role: int, layer: int, index: int, *,
                            B: int, Hq: int, Hkv: int, Lq: int, Lk: int, d: int,
                            n_sinks: int = 1, dtype: torch.dtype = torch.bfloat16,
                            device="cuda", with_v: bool = True):
    """Same recipe as ``attention_inputs`` drawn on the GPU with torch's device
    generator (float32 draws, so the values differ from the CPU stream; the
    distribution is the same).  Used where the CPU draw would dominate set-up
    time (large calibration sets)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(config_id, role, layer, index))
    u = torch.full((d,), 1.0 / float(np.sqrt(d)), device=device)
    k = torch.randn((B, Hkv, Lk, d), generator=g, device=device)
    lam = torch.exp(0.5 * torch.randn((B, Hkv, Lk, 1), generator=g, device=device))
    k = k * lam
    ns = min(n_sinks, Lk)
    if ns > 0:
        k[:, :, :ns, :] += 3.0 * u
    q = torch.randn((B, Hq, Lq, d), generator=g, device=device) + u
    v = torch.randn((B, Hkv, Lk, d), generator=g, device=device) if with_v else None
    cast = (lambda t: t) if dtype == torch.float32 else (lambda t: t.to(dtype))
    return cast(q).contiguous(), cast(k).contiguous(), None if v is None else cast(v).contiguous()


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a float32/bfloat16 CPU tensor."""
    return t.detach().to(torch.float64).cpu().numpy()
