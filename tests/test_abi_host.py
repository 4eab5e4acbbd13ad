"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import calibrated_threshold_pruning_amd as tt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "topth.h")

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(topth_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tt.LIB_PATH):
        pytest.fail("libtopth.so is not built; run `python -m calibrated_threshold_pruning_amd.build`")
    return tt.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 8
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(tt.EXPORTS)


def test_binding_constants_match_the_header():
    """Every #define of the header that the binding mirrors has the same value."""
    text = open(HEADER).read()
    macros = {}
    for name, val in re.findall(r"#define\s+(TOPTH_[A-Z0-9_]+)\s+(\(?[0-9xXa-fA-Fu <()]+\)?)", text):
        macros[name] = eval(val.replace("u", ""), {})
    mirrored = [n for n in macros if hasattr(tt._lib, n)]
    assert {"TOPTH_VMC", "TOPTH_SDC_NONE", "TOPTH_SDC_EXPTH", "TOPTH_SDC_OFFLINE", "TOPTH_OUT_F32",
            "TOPTH_WS_HEADER_BYTES", "TOPTH_NOALLOC_SCRATCH_BYTES", "TOPTH_MAX_NK"} <= set(mirrored)
    for n in mirrored:
        assert getattr(tt._lib, n) == macros[n], n


def test_strerror(lib):
    assert tt.topth_strerror(0) == "success"
    assert "invalid" in tt.topth_strerror(-1)
    assert "workspace" in tt.topth_strerror(-3)
    assert tt.topth_strerror(12345) == "unknown status"


def test_workspace_size(lib):
    ws = tt.topth_workspace_size
    assert ws(tt.TOPTH_OP_DECODE, 16, 32, 8, 1, 4096, 128) > 65536
    assert ws(tt.TOPTH_OP_DECODE, 16, 32, 8, 1, 4096, 96) == 0          # d not supported
    assert ws(tt.TOPTH_OP_DECODE, 16, 30, 8, 1, 4096, 128) == 0         # Hq % Hkv != 0
    # prefix means (fp32) and the float16 copy of V
    assert ws(tt.TOPTH_OP_PREFILL, 1, 32, 8, 8192, 8192, 128) >= 8 * 8192 * 128 * (4 + 2)
    assert ws(tt.TOPTH_OP_CALIBRATE, 4, 8, 8, 2048, 2048, 128, 3) >= 4 * 3 * 8 * 2048 * 4
    assert ws(tt.TOPTH_OP_CALIBRATE, 4, 8, 8, 2048, 2048, 128, 9) == 0  # too many k
    assert ws(7, 1, 1, 1, 1, 1, 64) == 0
    # monotone in the cache length
    assert ws(tt.TOPTH_OP_DECODE, 8, 64, 8, 1, 32768, 128) > ws(tt.TOPTH_OP_DECODE, 8, 64, 8, 1, 4096, 128)


def _decode(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, lens=FAKE, B=2, Hq=8, Hkv=2, Lmax=64, d=128, dt=1, scale=0.1,
             theta=FAKE, n_rows=64, vm=FAKE, flags=1, out=FAKE, kc=None, bt=None, vr=None, km=None,
             ws=FAKE, wsb=1 << 30)
    a.update(over)
    return lib.topth_decode(a["q"], a["k"], a["v"], a["lens"], a["B"], a["Hq"], a["Hkv"], a["Lmax"],
                            a["d"], a["dt"], a["scale"], a["theta"], a["n_rows"], a["vm"], a["flags"],
                            a["out"], a["kc"], a["bt"], a["vr"], a["km"], a["ws"], a["wsb"], None)


def test_decode_argument_errors(lib):
    assert _decode(lib, q=None) == -1
    assert _decode(lib, lens=None) == -1
    assert _decode(lib, Hq=6, Hkv=4) == -1
    assert _decode(lib, d=96) == -1
    assert _decode(lib, dt=7) == -1
    assert _decode(lib, B=0) == -1
    assert _decode(lib, n_rows=0) == -1
    assert _decode(lib, flags=8) == -1
    assert _decode(lib, vm=None) == -1                   # VMC needs the running mean
    assert _decode(lib, scale=float("nan")) == -1
    assert _decode(lib, scale=0.0) == -1
    assert _decode(lib, scale=-0.1) == -1
    assert _decode(lib, ws=None) == -3
    assert _decode(lib, wsb=100) == -3
    assert _decode(lib, Hq=24, Hkv=8) == -2              # g = 3: no kernel
    assert _decode(lib, dt=0, Lmax=40000, wsb=1 << 40) == -2  # float32 rows longer than LDS


def test_prefill_argument_errors(lib):
    def call(**over):
        a = dict(q=FAKE, k=FAKE, v=FAKE, B=1, Hq=4, Hkv=2, L=32, d=64, dt=0, scale=0.1, theta=FAKE,
                 n_rows=32, flags=1, out=FAKE, ws=FAKE, wsb=1 << 30)
        a.update(over)
        return lib.topth_prefill(a["q"], a["k"], a["v"], a["B"], a["Hq"], a["Hkv"], a["L"], a["d"],
                                 a["dt"], a["scale"], a["theta"], a["n_rows"], a["flags"], a["out"],
                                 None, None, None, a["ws"], a["wsb"], None)
    assert call(v=None) == -1
    assert call(theta=None) == -1
    assert call(L=0) == -1
    assert call(Hkv=3) == -1
    assert call(flags=0x20) == -1
    assert call(ws=None) == -3           # VMC needs the prefix-mean workspace
    assert call(wsb=16) == -3


def test_calibrate_argument_errors(lib):
    ks = (ctypes.c_int * 3)(64, 128, 256)
    bad = (ctypes.c_int * 2)(64, 0)

    def call(**over):
        a = dict(q=FAKE, k=FAKE, S=2, Hq=8, Hkv=8, Lq=256, Lk=256, d=128, dt=1, scale=0.1, qp=0,
                 ks=ctypes.cast(ks, ctypes.c_void_p), nk=3, sum=FAKE, sumsq=FAKE, count=FAKE,
                 n_rows=256, ws=FAKE, wsb=1 << 30)
        a.update(over)
        return lib.topth_calibrate(a["q"], a["k"], a["S"], a["Hq"], a["Hkv"], a["Lq"], a["Lk"], a["d"],
                                   a["dt"], a["scale"], a["qp"], a["ks"], a["nk"], a["sum"],
                                   a["sumsq"], a["count"], a["n_rows"], a["ws"], a["wsb"], None)
    assert call(ks=None) == -1
    assert call(nk=0) == -1
    assert call(nk=9) == -1
    assert call(ks=ctypes.cast(bad, ctypes.c_void_p), nk=2) == -1
    assert call(qp=1) == -1                        # q_pos0 + Lq > Lk
    assert call(sum=None) == -1
    assert call(ws=None) == -3
    assert call(wsb=8) == -3


def test_finalize_argument_errors(lib):
    ks = (ctypes.c_int * 1)(4)
    kp = ctypes.cast(ks, ctypes.c_void_p)
    assert lib.topth_calibrate_finalize(None, FAKE, FAKE, kp, 1, 2, 8, 0.0, FAKE, None) == -1
    assert lib.topth_calibrate_finalize(FAKE, FAKE, FAKE, kp, 0, 2, 8, 0.0, FAKE, None) == -1
    assert lib.topth_calibrate_finalize(FAKE, FAKE, FAKE, kp, 1, 2, 8, float("inf"), FAKE, None) == -1


def test_vmean_and_ws_init_argument_errors(lib):
    assert lib.topth_vmean(None, FAKE, 1, 1, 8, 64, 0, FAKE, None) == -1
    assert lib.topth_vmean(FAKE, FAKE, 1, 1, 8, 63, 0, FAKE, None) == -1
    assert lib.topth_workspace_init(None, 16, None) == -1
    assert lib.topth_workspace_init(FAKE, 0, None) == -1


def test_binding_rejects_cpu_tensors(lib):
    import torch
    q = torch.zeros(1, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tt.topth_vmean(torch.zeros(1, 1, 4, 64), torch.ones(1, dtype=torch.int32),
                       torch.zeros(1, 1, 64))
    with pytest.raises(ValueError):
        tt.topth_decode(q, q, q, None, None, None, None, scale=0.1, flags=0)


# ------------------------------------------------------------- pre-softmax calls
def _decode_pre(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, lens=FAKE, B=2, Hq=8, Hkv=2, Lmax=64, d=128, dt=1, scale=0.1,
             theta=FAKE, et=None, n_rows=64, vm=FAKE, flags=1, gamma=0.05, out=FAKE, kc=None, bt=None,
             vr=None, km=None, ws=FAKE, wsb=1 << 30)
    a.update(over)
    return lib.topth_decode_pre(a["q"], a["k"], a["v"], a["lens"], a["B"], a["Hq"], a["Hkv"], a["Lmax"],
                                a["d"], a["dt"], a["scale"], a["theta"], a["et"], a["n_rows"], a["vm"],
                                a["flags"], a["gamma"], a["out"], a["kc"], a["bt"], a["vr"], a["km"],
                                a["ws"], a["wsb"], None)


def _prefill_pre(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, B=1, Hq=8, Hkv=2, L=64, d=128, dt=1, scale=0.1, theta=FAKE,
             et=None, n_rows=64, flags=0, gamma=0.05, out=FAKE, kc=None, bt=None, km=None, ws=None, wsb=0)
    a.update(over)
    return lib.topth_prefill_pre(a["q"], a["k"], a["v"], a["B"], a["Hq"], a["Hkv"], a["L"], a["d"], a["dt"],
                                 a["scale"], a["theta"], a["et"], a["n_rows"], a["flags"], a["gamma"],
                                 a["out"], a["kc"], a["bt"], a["km"], a["ws"], a["wsb"], None)


def test_pre_flag_errors(lib):
    E, O, N = tt.TOPTH_SDC_EXPTH, tt.TOPTH_SDC_OFFLINE, tt.TOPTH_SDC_NONE
    for call in (_decode_pre, _prefill_pre):
        assert call(lib, flags=E | O) == -1                 # two estimates
        assert call(lib, flags=E | N) == -1
        assert call(lib, flags=O) == -1                     # offline needs the E~ table
        assert call(lib, flags=E, gamma=float("nan")) == -1
        assert call(lib, flags=E, gamma=-0.5) == -1
        assert call(lib, flags=0x20) == -1
        assert call(lib, theta=None) == -1
        assert call(lib, scale=0.0) == -1
    assert _decode_pre(lib, flags=tt.TOPTH_VMC, vm=None) == -1   # VMC needs the running mean
    assert _decode_pre(lib, ws=None) == -3
    assert _prefill_pre(lib, flags=tt.TOPTH_VMC) == -3            # VMC needs the prefix-mean workspace
    # the post-softmax calls take no estimate flags
    assert _decode(lib, flags=tt.TOPTH_VMC | E) == -1


def test_calibrate_pre_errors_and_workspace(lib):
    ws = tt.topth_workspace_size
    base = ws(tt.TOPTH_OP_CALIBRATE, 4, 8, 8, 2048, 2048, 128, 3)
    assert ws(tt.TOPTH_OP_CALIBRATE_PRE_E, 4, 8, 8, 2048, 2048, 128, 3) == 2 * base
    karr = (ctypes.c_int * 1)(32)
    kp = ctypes.cast(karr, ctypes.c_void_p)

    def cal(esum, wsb):
        return lib.topth_calibrate_pre(FAKE, FAKE, 4, 8, 8, 2048, 2048, 128, 1, 0.1, 0, kp, 1,
                                       FAKE, FAKE, FAKE, esum, 2048, FAKE, wsb, None)
    one = ws(tt.TOPTH_OP_CALIBRATE, 4, 8, 8, 2048, 2048, 128, 1)
    assert cal(FAKE, one) == -3                            # the E~ samples need twice the room
    assert lib.topth_calibrate_pre(None, FAKE, 4, 8, 8, 2048, 2048, 128, 1, 0.1, 0, kp, 1,
                                   FAKE, FAKE, FAKE, None, 2048, FAKE, one, None) == -1
    assert lib.topth_calibrate_finalize_etilde(None, FAKE, kp, 1, 8, 2048, FAKE, None) == -1
    assert lib.topth_calibrate_finalize_etilde(FAKE, FAKE, kp, 0, 8, 2048, FAKE, None) == -1


def test_serving_helper_errors(lib):
    karr = (ctypes.c_int * 1)(32)
    kp = ctypes.cast(karr, ctypes.c_void_p)
    assert lib.topth_vmean_append(None, FAKE, FAKE, 2, 8, 64, 128, 1, FAKE, None) == -1
    assert lib.topth_vmean_append(FAKE, FAKE, FAKE, 2, 8, 64, 96, 1, FAKE, None) == -1     # d
    assert lib.topth_vmean_append(FAKE, FAKE, FAKE, 2, 8, 64, 128, 5, FAKE, None) == -1    # dtype
    ks1 = ctypes.cast((ctypes.c_int * 1)(64), ctypes.c_void_p)
    assert lib.topth_theta_fit(FAKE, FAKE, ks1, 1, 8, 64, 4, 1, 4, FAKE, None) == -1            # degree > 3
    assert lib.topth_theta_fit(FAKE, FAKE, ks1, 1, 8, 64, -1, 1, 4, FAKE, None) == -1
    assert lib.topth_theta_fit(FAKE, None, ks1, 1, 8, 64, 1, 1, 4, FAKE, None) == -1
    assert lib.topth_theta_fit(FAKE, FAKE, None, 1, 8, 64, 1, 1, 4, FAKE, None) == -1
    assert lib.topth_theta_fit(FAKE, FAKE, ks1, 1, 8, 64, 1, 1, -1, FAKE, None) == -1         # negative factor
    assert lib.topth_theta_eval(FAKE, kp, 1, 8, 2, 1, 0, FAKE, None) == -1                 # n_out
    assert lib.topth_theta_eval(FAKE, None, 1, 8, 2, 1, 100, FAKE, None) == -1
    assert lib.topth_theta_eval(FAKE, kp, 9, 8, 2, 1, 100, FAKE, None) == -1               # n_k


def test_decode_gqa_errors(lib):
    def call(mv, aug, Hq=8, Hkv=2):
        return lib.topth_decode_gqa(FAKE, FAKE, FAKE, FAKE, 2, Hq, Hkv, 64, 128, 1, 0.1, FAKE, 64, FAKE, 1,
                                    mv, aug, FAKE, None, None, None, None, FAKE, 1 << 30, None)
    assert call(0, 0) == -1          # min_votes below 1
    assert call(5, 0) == -1          # more votes than heads in the group (g = 4)
    assert call(2, 2) == -1          # augment is 0 or 1
    assert call(2, 0, Hq=6, Hkv=4) == -1


def test_decode_append_errors(lib):
    def call(vm=FAKE, flags=1, d=128, ws=FAKE):
        return lib.topth_decode_append(FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 64, d, 1, 0.1, FAKE, 64, vm, flags,
                                       FAKE, None, None, None, None, ws, 1 << 30, None)
    assert call(vm=None) == -1              # the running mean is always read and updated
    assert call(vm=None, flags=0) == -1
    assert call(flags=0x20) == -1           # unknown flag
    assert call(d=96) == -1
    assert call(ws=None) == -3


def test_workspace_status_and_spin_limit_errors(lib):
    st = ctypes.c_int(5)
    assert lib.topth_workspace_status(None, 1 << 20, ctypes.byref(st), None) == -1
    assert lib.topth_workspace_status(FAKE, 1 << 20, None, None) == -1
    assert lib.topth_workspace_status(FAKE, 1024, ctypes.byref(st), None) == -1   # smaller than the header
    assert st.value == 5                                                          # untouched on error
    assert lib.topth_workspace_set_spin_limit(None, 1 << 20, 1, None) == -1
    assert lib.topth_workspace_set_spin_limit(FAKE, 100, 1, None) == -1
    assert tt.TOPTH_WS_HEADER_BYTES == 65536 and tt.TOPTH_STATUS_EXCHANGE_TIMEOUT == 1


def _mkc(lib, **over):
    ks = (ctypes.c_int * 3)(1, 8, 64)
    a = dict(q=FAKE, k=FAKE, S=4, Hq=8, Hkv=2, Lq=1, Lk=512, d=128, dt=1, scale=0.1, q0=511, pre=0,
             ks=ctypes.cast(ks, ctypes.c_void_p), n_k=3, theta=FAKE, n_rows=512, ws=FAKE, wsb=1 << 40)
    a.update(over)
    return lib.topth_calibrate_mkc(a["q"], a["k"], a["S"], a["Hq"], a["Hkv"], a["Lq"], a["Lk"], a["d"], a["dt"],
                                   a["scale"], a["q0"], a["pre"], a["ks"], a["n_k"], a["theta"], a["n_rows"],
                                   a["ws"], a["wsb"], None)


def test_calibrate_mkc_argument_errors(lib):
    assert _mkc(lib, q=None) == -1
    assert _mkc(lib, ks=None) == -1
    assert _mkc(lib, theta=None) == -1
    assert _mkc(lib, q0=512) == -1                           # q_pos0 + Lq > Lk
    assert _mkc(lib, pre=2) == -1
    assert _mkc(lib, n_k=0) == -1 and _mkc(lib, n_k=65) == -1
    bad = (ctypes.c_int * 1)(0)
    assert _mkc(lib, ks=ctypes.cast(bad, ctypes.c_void_p), n_k=1) == -1
    assert _mkc(lib, S=4097) == -2                           # more samples than one call merges
    assert _mkc(lib, Lk=40000, q0=39999, n_rows=40000) == -2 # more keys than the LDS score row
    assert _mkc(lib, ws=None) == -3
    need = tt.topth_workspace_size(tt.TOPTH_OP_CALIBRATE_MKC, 4, 8, 2, 1, 512, 128, 0)
    assert need >= 2 * 4 * 8 * 512 * 4
    assert _mkc(lib, wsb=need - 1) == -3
    assert tt.topth_workspace_size(tt.TOPTH_OP_CALIBRATE_MKC, 4097, 8, 2, 1, 512, 128, 0) == 0
