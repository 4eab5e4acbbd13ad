"""Top-theta attention for AMD Instinct MI355X (gfx950).

The compute lives in ``libtopth.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/topth.h``); this package only loads it and marshals torch
tensors into its calls.  Build the library with
``python -m calibrated_threshold_pruning_amd.build``.
"""
from ._lib import (  # noqa: F401
    TOPTH_F32, TOPTH_BF16, TOPTH_VMC, TOPTH_SDC_NONE, TOPTH_OP_CALIBRATE, TOPTH_OP_PREFILL,
    TOPTH_OP_DECODE, TOPTH_MAX_NK, EXPORTS, LIB_PATH, TopthError, load_library,
    topth_strerror, topth_workspace_size, topth_workspace_init, workspace, topth_calibrate,
    topth_calibrate_finalize, topth_prefill, topth_decode, topth_vmean,
    TOPTH_SDC_EXPTH, TOPTH_SDC_OFFLINE, TOPTH_OP_CALIBRATE_PRE_E, topth_calibrate_pre,
    topth_calibrate_finalize_etilde, topth_prefill_pre, topth_decode_pre,
    topth_vmean_append, topth_theta_fit, topth_theta_eval, topth_decode_gqa, topth_decode_append,
    TOPTH_WS_HEADER_BYTES, TOPTH_STATUS_EXCHANGE_TIMEOUT, topth_workspace_status,
    topth_workspace_set_spin_limit, TOPTH_ESCRATCH, TOPTH_NOALLOC_SCRATCH_BYTES, topth_decode_noalloc,
    TOPTH_OP_CALIBRATE_MKC, TOPTH_MKC_MAX_TARGETS, TOPTH_MKC_MAX_SAMPLES, TOPTH_MKC_MAX_KEYS,
    topth_calibrate_mkc, TOPTH_OUT_F32,
)
