"""ctypes binding of libtopth (argument marshalling only).

Every function has the name of the C entry point it calls and takes torch
tensors for device buffers: it checks dtype, shape, contiguity and device,
passes ``data_ptr()`` and the current HIP stream of torch, and raises
``TopthError`` when the library returns a negative status.  All computation
happens in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtopth.so")

TOPTH_F32, TOPTH_BF16 = 0, 1
TOPTH_VMC, TOPTH_SDC_NONE = 0x1, 0x2
TOPTH_SDC_EXPTH, TOPTH_SDC_OFFLINE = 0x4, 0x8
TOPTH_OUT_F32 = 0x10
TOPTH_OP_CALIBRATE, TOPTH_OP_PREFILL, TOPTH_OP_DECODE, TOPTH_OP_CALIBRATE_PRE_E = 0, 1, 2, 3
TOPTH_OP_CALIBRATE_MKC = 4
TOPTH_MKC_MAX_TARGETS, TOPTH_MKC_MAX_SAMPLES, TOPTH_MKC_MAX_KEYS = 64, 4096, 32768
TOPTH_MAX_NK = 8
TOPTH_WS_HEADER_BYTES = 65536
TOPTH_STATUS_EXCHANGE_TIMEOUT = 0x1
TOPTH_ESCRATCH = -5
TOPTH_NOALLOC_SCRATCH_BYTES = 80 << 20

EXPORTS = ("topth_strerror", "topth_workspace_size", "topth_workspace_init", "topth_calibrate",
           "topth_calibrate_finalize", "topth_prefill", "topth_decode", "topth_vmean",
           "topth_calibrate_pre", "topth_calibrate_finalize_etilde", "topth_prefill_pre",
           "topth_decode_pre", "topth_vmean_append", "topth_theta_fit", "topth_theta_eval",
           "topth_decode_gqa", "topth_decode_append", "topth_workspace_status",
           "topth_workspace_set_spin_limit", "topth_decode_noalloc", "topth_calibrate_mkc")


class TopthError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libtopth.so; raise if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m calibrated_threshold_pruning_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, i, f, sz, u = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_uint
    lib.topth_strerror.restype = ctypes.c_char_p
    lib.topth_strerror.argtypes = [i]
    lib.topth_workspace_size.restype = sz
    lib.topth_workspace_size.argtypes = [i] * 8
    lib.topth_workspace_init.restype = i
    lib.topth_workspace_init.argtypes = [vp, sz, vp]
    lib.topth_workspace_status.restype = i
    lib.topth_workspace_status.argtypes = [vp, sz, ctypes.POINTER(ctypes.c_int), vp]
    lib.topth_workspace_set_spin_limit.restype = i
    lib.topth_workspace_set_spin_limit.argtypes = [vp, sz, u, vp]
    lib.topth_calibrate.restype = i
    lib.topth_calibrate.argtypes = [vp, vp, i, i, i, i, i, i, i, f, i, vp, i, vp, vp, vp, i, vp, sz, vp]
    lib.topth_calibrate_mkc.restype = i
    lib.topth_calibrate_mkc.argtypes = [vp, vp, i, i, i, i, i, i, i, f, i, i, vp, i, vp, i, vp, sz, vp]
    lib.topth_calibrate_finalize.restype = i
    lib.topth_calibrate_finalize.argtypes = [vp, vp, vp, vp, i, i, i, f, vp, vp]
    lib.topth_prefill.restype = i
    lib.topth_prefill.argtypes = [vp, vp, vp, i, i, i, i, i, i, f, vp, i, u, vp, vp, vp, vp, vp, sz, vp]
    lib.topth_decode.restype = i
    lib.topth_decode.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, vp, i, vp, u, vp, vp, vp, vp,
                                 vp, vp, sz, vp]
    lib.topth_decode_noalloc.restype = i
    lib.topth_decode_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, vp, i, vp, u, vp, vp, vp, vp,
                                         vp, vp]
    lib.topth_decode_append.restype = i
    lib.topth_decode_append.argtypes = list(lib.topth_decode.argtypes)
    lib.topth_vmean.restype = i
    lib.topth_vmean.argtypes = [vp, vp, i, i, i, i, i, vp, vp]
    lib.topth_calibrate_pre.restype = i
    lib.topth_calibrate_pre.argtypes = [vp, vp, i, i, i, i, i, i, i, f, i, vp, i, vp, vp, vp, vp, i, vp,
                                        sz, vp]
    lib.topth_calibrate_finalize_etilde.restype = i
    lib.topth_calibrate_finalize_etilde.argtypes = [vp, vp, vp, i, i, i, vp, vp]
    lib.topth_prefill_pre.restype = i
    lib.topth_prefill_pre.argtypes = [vp, vp, vp, i, i, i, i, i, i, f, vp, vp, i, u, f, vp, vp, vp, vp,
                                      vp, sz, vp]
    lib.topth_vmean_append.restype = i
    lib.topth_vmean_append.argtypes = [vp, vp, vp, i, i, i, i, i, vp, vp]
    lib.topth_theta_fit.restype = i
    lib.topth_theta_fit.argtypes = [vp, vp, vp, i, i, i, i, i, i, vp, vp]
    lib.topth_theta_eval.restype = i
    lib.topth_theta_eval.argtypes = [vp, vp, i, i, i, i, i, vp, vp]
    lib.topth_decode_gqa.restype = i
    lib.topth_decode_gqa.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, vp, i, vp, u, i, i, vp, vp, vp,
                                     vp, vp, vp, sz, vp]
    lib.topth_decode_pre.restype = i
    lib.topth_decode_pre.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, vp, vp, i, vp, u, f, vp, vp,
                                     vp, vp, vp, vp, sz, vp]
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        raise TopthError(fn, status, load_library().topth_strerror(status).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TOPTH_F32
    if t.dtype == torch.bfloat16:
        return TOPTH_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _out_dtype(q: torch.Tensor, flags: int):
    """dtype of the output: float32 with TOPTH_OUT_F32, else the input dtype"""
    return torch.float32 if int(flags) & TOPTH_OUT_F32 else q.dtype


def _dev(t, name, dtype=None, shape=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def topth_strerror(status: int) -> str:
    return load_library().topth_strerror(status).decode()


def topth_workspace_size(op: int, B: int, Hq: int, Hkv: int, Lq: int, Lk: int, d: int,
                         n_k: int = 1) -> int:
    return int(load_library().topth_workspace_size(op, B, Hq, Hkv, Lq, Lk, d, n_k))


def topth_workspace_init(ws: torch.Tensor, stream=None):
    _dev(ws, "ws", torch.uint8)
    _check("topth_workspace_init", load_library().topth_workspace_init(
        ws.data_ptr(), ws.numel(), _stream(stream)))


def topth_workspace_status(ws: torch.Tensor, stream=None) -> int:
    """Status word of a decode workspace after the work enqueued so far (the
    call synchronises the stream): 0 or TOPTH_STATUS_EXCHANGE_TIMEOUT."""
    _dev(ws, "ws", torch.uint8)
    out = ctypes.c_int(0)
    _check("topth_workspace_status", load_library().topth_workspace_status(
        ws.data_ptr(), ws.numel(), ctypes.byref(out), _stream(stream)))
    return int(out.value)


def topth_workspace_set_spin_limit(ws: torch.Tensor, limit: int, stream=None):
    """Polls an exchange wait of later decode calls on ``ws`` makes before it
    gives up (0: the default)."""
    _dev(ws, "ws", torch.uint8)
    _check("topth_workspace_set_spin_limit", load_library().topth_workspace_set_spin_limit(
        ws.data_ptr(), ws.numel(), int(limit), _stream(stream)))


def workspace(op: int, B: int, Hq: int, Hkv: int, Lq: int, Lk: int, d: int, n_k: int = 1,
              device="cuda") -> torch.Tensor:
    """Allocate a workspace tensor of the size the library asks for, prepared by
    topth_workspace_init (header zeroed, decode exchange slots empty)."""
    n = topth_workspace_size(op, B, Hq, Hkv, Lq, Lk, d, n_k)
    if n == 0:
        raise ValueError("no workspace size for these arguments")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    topth_workspace_init(ws)
    return ws


def topth_calibrate(q, k, ks, sum_, sumsq, count, ws, *, scale: float, q_pos0: int = 0,
                    stream=None):
    """Accumulate Algorithm-1 samples of S sequences. q [S,Hq,Lq,d], k [S,Hkv,Lk,d];
    sum_/sumsq float64 and count int32 of shape [n_k,Hq,n_rows]."""
    S, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    dt = _dtype_code(q)
    _dev(q, "q"); _dev(k, "k", q.dtype, (S, Hkv, Lk, d))
    n_k = len(ks)
    n_rows = sum_.shape[-1]
    _dev(sum_, "sum", torch.float64, (n_k, Hq, n_rows))
    _dev(sumsq, "sumsq", torch.float64, (n_k, Hq, n_rows))
    _dev(count, "count", torch.int32, (n_k, Hq, n_rows))
    _dev(ws, "ws", torch.uint8)
    karr = (ctypes.c_int * max(n_k, 1))(*[int(x) for x in ks])
    _check("topth_calibrate", load_library().topth_calibrate(
        q.data_ptr(), k.data_ptr(), S, Hq, Hkv, Lq, Lk, d, dt, float(scale), int(q_pos0),
        ctypes.cast(karr, ctypes.c_void_p), n_k, sum_.data_ptr(), sumsq.data_ptr(),
        count.data_ptr(), n_rows, ws.data_ptr(), ws.numel(), _stream(stream)))


def topth_calibrate_mkc(q, k, ks, theta, ws, *, scale: float, q_pos0: int = 0, pre: bool = False,
                        stream=None):
    """Multi-k cumulative calibration of all S sequences at once: q [S,Hq,Lq,d],
    k [S,Hkv,Lk,d]; theta [n_k,Hq,n_rows] float32 gets theta_p(ks[t]) at rows
    p = q_pos0 .. q_pos0 + Lq - 1."""
    S, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    dt = _dtype_code(q)
    _dev(q, "q"); _dev(k, "k", q.dtype, (S, Hkv, Lk, d))
    n_k = len(ks)
    _dev(theta, "theta", torch.float32)
    if theta.dim() != 3 or tuple(theta.shape[:2]) != (n_k, Hq):
        raise ValueError("theta must be [n_k, Hq, n_rows]")
    _dev(ws, "ws", torch.uint8)
    karr = (ctypes.c_int * max(n_k, 1))(*[int(x) for x in ks])
    _check("topth_calibrate_mkc", load_library().topth_calibrate_mkc(
        q.data_ptr(), k.data_ptr(), S, Hq, Hkv, Lq, Lk, d, dt, float(scale), int(q_pos0), int(bool(pre)),
        ctypes.cast(karr, ctypes.c_void_p), n_k, theta.data_ptr(), theta.shape[2], ws.data_ptr(), ws.numel(),
        _stream(stream)))


def topth_calibrate_finalize(sum_, sumsq, count, ks, theta, *, alpha: float = 0.0, stream=None):
    n_k, Hq, n_rows = sum_.shape
    _dev(sum_, "sum", torch.float64); _dev(sumsq, "sumsq", torch.float64, sum_.shape)
    _dev(count, "count", torch.int32, sum_.shape); _dev(theta, "theta", torch.float32, sum_.shape)
    karr = (ctypes.c_int * max(len(ks), 1))(*[int(x) for x in ks])
    _check("topth_calibrate_finalize", load_library().topth_calibrate_finalize(
        sum_.data_ptr(), sumsq.data_ptr(), count.data_ptr(), ctypes.cast(karr, ctypes.c_void_p),
        len(ks), Hq, n_rows, float(alpha), theta.data_ptr(), _stream(stream)))


def topth_prefill(q, k, v, theta, out, *, scale: float, flags: int, kept_count=None, beta=None,
                  kept_mask=None, ws=None, stream=None):
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    dt = _dtype_code(q)
    _dev(q, "q"); _dev(k, "k", q.dtype, (B, Hkv, L, d)); _dev(v, "v", q.dtype, (B, Hkv, L, d))
    _dev(theta, "theta", torch.float32)
    if theta.dim() != 2 or theta.shape[0] != Hq:
        raise ValueError("theta must be [Hq, n_rows]")
    _dev(out, "out", _out_dtype(q, flags), (B, Hq, L, d))
    kc = _dev(kept_count, "kept_count", torch.int32, (B, Hq, L), optional=True)
    bt = _dev(beta, "beta", torch.float32, (B, Hq, L), optional=True)
    km = _dev(kept_mask, "kept_mask", torch.uint8, (B, Hq, L, L), optional=True)
    wp = _dev(ws, "ws", torch.uint8, optional=True)
    _check("topth_prefill", load_library().topth_prefill(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), B, Hq, Hkv, L, d, dt, float(scale),
        theta.data_ptr(), theta.shape[1], int(flags), out.data_ptr(), kc, bt, km, wp,
        0 if ws is None else ws.numel(), _stream(stream)))


def topth_decode(q, k_cache, v_cache, seq_lens, theta, out, ws, *, scale: float, flags: int,
                 v_mean=None, kept_count=None, beta=None, vrows_read=None, kept_mask=None,
                 stream=None):
    B, Hq, d = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    dt = _dtype_code(q)
    _dev(q, "q"); _dev(k_cache, "k_cache", q.dtype, (B, Hkv, Lmax, d))
    _dev(v_cache, "v_cache", q.dtype, (B, Hkv, Lmax, d))
    _dev(seq_lens, "seq_lens", torch.int32, (B,))
    _dev(theta, "theta", torch.float32)
    if theta.dim() != 2 or theta.shape[0] != Hq:
        raise ValueError("theta must be [Hq, n_rows]")
    _dev(out, "out", _out_dtype(q, flags), (B, Hq, d))
    vm = _dev(v_mean, "v_mean", torch.float32, (B, Hkv, d), optional=True)
    kc = _dev(kept_count, "kept_count", torch.int32, (B, Hq), optional=True)
    bt = _dev(beta, "beta", torch.float32, (B, Hq), optional=True)
    vr = _dev(vrows_read, "vrows_read", torch.int32, (B, Hkv), optional=True)
    km = _dev(kept_mask, "kept_mask", torch.uint8, (B, Hq, Lmax), optional=True)
    _dev(ws, "ws", torch.uint8)
    _check("topth_decode", load_library().topth_decode(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv,
        Lmax, d, dt, float(scale), theta.data_ptr(), theta.shape[1], vm, int(flags),
        out.data_ptr(), kc, bt, vr, km, ws.data_ptr(), ws.numel(), _stream(stream)))


def topth_decode_noalloc(q, k_cache, v_cache, seq_lens, theta, out, *, scale: float, flags: int,
                         v_mean=None, kept_count=None, beta=None, vrows_read=None, kept_mask=None,
                         stream=None):
    """topth_decode without a workspace: the library's static per-GPU scratch
    serves instead (calls that overlap on one GPU race)."""
    B, Hq, d = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    dt = _dtype_code(q)
    _dev(q, "q"); _dev(k_cache, "k_cache", q.dtype, (B, Hkv, Lmax, d))
    _dev(v_cache, "v_cache", q.dtype, (B, Hkv, Lmax, d))
    _dev(seq_lens, "seq_lens", torch.int32, (B,))
    _table(theta, "theta", Hq)
    _dev(out, "out", _out_dtype(q, flags), (B, Hq, d))
    vm = _dev(v_mean, "v_mean", torch.float32, (B, Hkv, d), optional=True)
    kc = _dev(kept_count, "kept_count", torch.int32, (B, Hq), optional=True)
    bt = _dev(beta, "beta", torch.float32, (B, Hq), optional=True)
    vr = _dev(vrows_read, "vrows_read", torch.int32, (B, Hkv), optional=True)
    km = _dev(kept_mask, "kept_mask", torch.uint8, (B, Hq, Lmax), optional=True)
    _check("topth_decode_noalloc", load_library().topth_decode_noalloc(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv,
        Lmax, d, dt, float(scale), theta.data_ptr(), theta.shape[1], vm, int(flags),
        out.data_ptr(), kc, bt, vr, km, _stream(stream)))


def topth_decode_append(q, k_cache, v_cache, seq_lens, theta, out, ws, v_mean, *, scale: float, flags: int,
                        kept_count=None, beta=None, vrows_read=None, kept_mask=None, stream=None):
    """topth_decode that first appends row n - 1 to the running mean v_mean
    [B,Hkv,d] (mean of rows 0..n-2 on entry, of rows 0..n-1 on return) and
    uses the updated mean for VMC."""
    B, Hq, d = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    dt = _dtype_code(q)
    _dev(q, "q"); _dev(k_cache, "k_cache", q.dtype, (B, Hkv, Lmax, d))
    _dev(v_cache, "v_cache", q.dtype, (B, Hkv, Lmax, d))
    _dev(seq_lens, "seq_lens", torch.int32, (B,))
    _dev(theta, "theta", torch.float32)
    if theta.dim() != 2 or theta.shape[0] != Hq:
        raise ValueError("theta must be [Hq, n_rows]")
    _dev(out, "out", _out_dtype(q, flags), (B, Hq, d))
    _dev(v_mean, "v_mean", torch.float32, (B, Hkv, d))
    kc = _dev(kept_count, "kept_count", torch.int32, (B, Hq), optional=True)
    bt = _dev(beta, "beta", torch.float32, (B, Hq), optional=True)
    vr = _dev(vrows_read, "vrows_read", torch.int32, (B, Hkv), optional=True)
    km = _dev(kept_mask, "kept_mask", torch.uint8, (B, Hq, Lmax), optional=True)
    _dev(ws, "ws", torch.uint8)
    _check("topth_decode_append", load_library().topth_decode_append(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv,
        Lmax, d, dt, float(scale), theta.data_ptr(), theta.shape[1], v_mean.data_ptr(), int(flags),
        out.data_ptr(), kc, bt, vr, km, ws.data_ptr(), ws.numel(), _stream(stream)))


def topth_vmean(v, seq_lens, v_mean, stream=None):
    B, Hkv, Lmax, d = v.shape
    dt = _dtype_code(v)
    _dev(v, "v"); _dev(seq_lens, "seq_lens", torch.int32, (B,))
    _dev(v_mean, "v_mean", torch.float32, (B, Hkv, d))
    _check("topth_vmean", load_library().topth_vmean(
        v.data_ptr(), seq_lens.data_ptr(), B, Hkv, Lmax, d, dt, v_mean.data_ptr(), _stream(stream)))


# --------------------------------------------------------------- pre-softmax
def topth_calibrate_pre(q, k, ks, sum_, sumsq, count, ws, *, scale: float, q_pos0: int = 0,
                        esum=None, stream=None):
    """Algorithm 1 on the scores (k-th largest score per row); with ``esum``
    [n_k,Hq,n_rows] float64 also the discarded mass of each row's top-k."""
    S, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    dt = _dtype_code(q)
    _dev(q, "q"); _dev(k, "k", q.dtype, (S, Hkv, Lk, d))
    n_k = len(ks)
    n_rows = sum_.shape[-1]
    _dev(sum_, "sum", torch.float64, (n_k, Hq, n_rows))
    _dev(sumsq, "sumsq", torch.float64, (n_k, Hq, n_rows))
    _dev(count, "count", torch.int32, (n_k, Hq, n_rows))
    ep = _dev(esum, "esum", torch.float64, (n_k, Hq, n_rows), optional=True)
    _dev(ws, "ws", torch.uint8)
    karr = (ctypes.c_int * max(n_k, 1))(*[int(x) for x in ks])
    _check("topth_calibrate_pre", load_library().topth_calibrate_pre(
        q.data_ptr(), k.data_ptr(), S, Hq, Hkv, Lq, Lk, d, dt, float(scale), int(q_pos0),
        ctypes.cast(karr, ctypes.c_void_p), n_k, sum_.data_ptr(), sumsq.data_ptr(),
        count.data_ptr(), ep, n_rows, ws.data_ptr(), ws.numel(), _stream(stream)))


def topth_calibrate_finalize_etilde(esum, count, ks, e_tilde, *, stream=None):
    n_k, Hq, n_rows = esum.shape
    _dev(esum, "esum", torch.float64); _dev(count, "count", torch.int32, esum.shape)
    _dev(e_tilde, "e_tilde", torch.float32, esum.shape)
    karr = (ctypes.c_int * max(len(ks), 1))(*[int(x) for x in ks])
    _check("topth_calibrate_finalize_etilde", load_library().topth_calibrate_finalize_etilde(
        esum.data_ptr(), count.data_ptr(), ctypes.cast(karr, ctypes.c_void_p), len(ks), Hq, n_rows,
        e_tilde.data_ptr(), _stream(stream)))


def _table(t, name, Hq, n_rows=None, optional=False):
    p = _dev(t, name, torch.float32, optional=optional)
    if p is not None and (t.dim() != 2 or t.shape[0] != Hq or (n_rows is not None and t.shape[1] != n_rows)):
        raise ValueError(f"{name} must be [Hq, n_rows]")
    return p


def topth_prefill_pre(q, k, v, theta, out, *, scale: float, flags: int, gamma: float = 0.05,
                      e_tilde=None, kept_count=None, beta=None, kept_mask=None, ws=None, stream=None):
    """Pre-softmax prefill: theta [Hq,n_rows] in score units; e_tilde [Hq,n_rows]
    for TOPTH_SDC_OFFLINE."""
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    dt = _dtype_code(q)
    _dev(q, "q"); _dev(k, "k", q.dtype, (B, Hkv, L, d)); _dev(v, "v", q.dtype, (B, Hkv, L, d))
    _table(theta, "theta", Hq)
    et = _table(e_tilde, "e_tilde", Hq, theta.shape[1], optional=True)
    _dev(out, "out", _out_dtype(q, flags), (B, Hq, L, d))
    kc = _dev(kept_count, "kept_count", torch.int32, (B, Hq, L), optional=True)
    bt = _dev(beta, "beta", torch.float32, (B, Hq, L), optional=True)
    km = _dev(kept_mask, "kept_mask", torch.uint8, (B, Hq, L, L), optional=True)
    wp = _dev(ws, "ws", torch.uint8, optional=True)
    _check("topth_prefill_pre", load_library().topth_prefill_pre(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), B, Hq, Hkv, L, d, dt, float(scale),
        theta.data_ptr(), et, theta.shape[1], int(flags), float(gamma), out.data_ptr(), kc, bt, km, wp,
        0 if ws is None else ws.numel(), _stream(stream)))


def topth_decode_pre(q, k_cache, v_cache, seq_lens, theta, out, ws, *, scale: float, flags: int,
                     gamma: float = 0.05, e_tilde=None, v_mean=None, kept_count=None, beta=None,
                     vrows_read=None, kept_mask=None, stream=None):
    """Pre-softmax decoding step: theta [Hq,n_rows] in score units."""
    B, Hq, d = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    dt = _dtype_code(q)
    _dev(q, "q"); _dev(k_cache, "k_cache", q.dtype, (B, Hkv, Lmax, d))
    _dev(v_cache, "v_cache", q.dtype, (B, Hkv, Lmax, d))
    _dev(seq_lens, "seq_lens", torch.int32, (B,))
    _table(theta, "theta", Hq)
    et = _table(e_tilde, "e_tilde", Hq, theta.shape[1], optional=True)
    _dev(out, "out", _out_dtype(q, flags), (B, Hq, d))
    vm = _dev(v_mean, "v_mean", torch.float32, (B, Hkv, d), optional=True)
    kc = _dev(kept_count, "kept_count", torch.int32, (B, Hq), optional=True)
    bt = _dev(beta, "beta", torch.float32, (B, Hq), optional=True)
    vr = _dev(vrows_read, "vrows_read", torch.int32, (B, Hkv), optional=True)
    km = _dev(kept_mask, "kept_mask", torch.uint8, (B, Hq, Lmax), optional=True)
    _dev(ws, "ws", torch.uint8)
    _check("topth_decode_pre", load_library().topth_decode_pre(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv,
        Lmax, d, dt, float(scale), theta.data_ptr(), et, theta.shape[1], vm, int(flags), float(gamma),
        out.data_ptr(), kc, bt, vr, km, ws.data_ptr(), ws.numel(), _stream(stream)))


# ----------------------------------------------------------- serving helpers
def topth_vmean_append(v_cache, old_lens, new_lens, v_mean, stream=None):
    """v_mean [B,Hkv,d] (mean of the first old_lens rows) becomes the mean of the
    first new_lens rows of v_cache [B,Hkv,Lmax,d]."""
    B, Hkv, Lmax, d = v_cache.shape
    dt = _dtype_code(v_cache)
    _dev(v_cache, "v_cache"); _dev(old_lens, "old_lens", torch.int32, (B,))
    _dev(new_lens, "new_lens", torch.int32, (B,)); _dev(v_mean, "v_mean", torch.float32, (B, Hkv, d))
    _check("topth_vmean_append", load_library().topth_vmean_append(
        v_cache.data_ptr(), old_lens.data_ptr(), new_lens.data_ptr(), B, Hkv, Lmax, d, dt,
        v_mean.data_ptr(), _stream(stream)))


def topth_theta_fit(theta, count, coef, ks, *, degree: int, log_domain: bool, min_len_over_k: int = 4,
                    stream=None):
    """Fit coef [n_k,Hq,degree+1] (float64) to the observed rows of theta/count
    [n_k,Hq,n_rows] with p + 1 >= min_len_over_k * ks[t] (0: every observed row)."""
    n_k, Hq, n_rows = theta.shape
    _dev(theta, "theta", torch.float32); _dev(count, "count", torch.int32, theta.shape)
    _dev(coef, "coef", torch.float64, (n_k, Hq, degree + 1))
    if len(ks) != n_k:
        raise ValueError("ks must have one k per slab")
    karr = (ctypes.c_int * max(n_k, 1))(*[int(x) for x in ks])
    _check("topth_theta_fit", load_library().topth_theta_fit(
        theta.data_ptr(), count.data_ptr(), ctypes.cast(karr, ctypes.c_void_p), n_k, Hq, n_rows, int(degree),
        int(bool(log_domain)), int(min_len_over_k), coef.data_ptr(), _stream(stream)))


def topth_theta_eval(coef, ks, theta_out, *, log_domain: bool, stream=None):
    """theta_out [n_k,Hq,n_out] from fitted coefficients coef [n_k,Hq,degree+1]."""
    n_k, Hq, m = coef.shape
    _dev(coef, "coef", torch.float64)
    _dev(theta_out, "theta_out", torch.float32)
    if theta_out.dim() != 3 or tuple(theta_out.shape[:2]) != (n_k, Hq) or len(ks) != n_k:
        raise ValueError("theta_out must be [n_k, Hq, n_out] and ks of length n_k")
    karr = (ctypes.c_int * max(n_k, 1))(*[int(x) for x in ks])
    _check("topth_theta_eval", load_library().topth_theta_eval(
        coef.data_ptr(), ctypes.cast(karr, ctypes.c_void_p), n_k, Hq, m - 1, int(bool(log_domain)),
        theta_out.shape[2], theta_out.data_ptr(), _stream(stream)))


def topth_decode_gqa(q, k_cache, v_cache, seq_lens, theta, out, ws, *, scale: float, flags: int,
                     min_votes: int = 1, augment: bool = False, v_mean=None, kept_count=None, beta=None,
                     vrows_read=None, kept_mask=None, stream=None):
    """Decoding step with the GQA selection variants: load keys kept by at least
    ``min_votes`` heads of the group; ``augment`` gives every head all of them."""
    B, Hq, d = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    dt = _dtype_code(q)
    _dev(q, "q"); _dev(k_cache, "k_cache", q.dtype, (B, Hkv, Lmax, d))
    _dev(v_cache, "v_cache", q.dtype, (B, Hkv, Lmax, d))
    _dev(seq_lens, "seq_lens", torch.int32, (B,))
    _table(theta, "theta", Hq)
    _dev(out, "out", _out_dtype(q, flags), (B, Hq, d))
    vm = _dev(v_mean, "v_mean", torch.float32, (B, Hkv, d), optional=True)
    kc = _dev(kept_count, "kept_count", torch.int32, (B, Hq), optional=True)
    bt = _dev(beta, "beta", torch.float32, (B, Hq), optional=True)
    vr = _dev(vrows_read, "vrows_read", torch.int32, (B, Hkv), optional=True)
    km = _dev(kept_mask, "kept_mask", torch.uint8, (B, Hq, Lmax), optional=True)
    _dev(ws, "ws", torch.uint8)
    _check("topth_decode_gqa", load_library().topth_decode_gqa(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv,
        Lmax, d, dt, float(scale), theta.data_ptr(), theta.shape[1], vm, int(flags), int(min_votes),
        int(bool(augment)), out.data_ptr(), kc, bt, vr, km, ws.data_ptr(), ws.numel(), _stream(stream)))
