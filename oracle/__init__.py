"""CPU oracle for Top-theta attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy code that states what the hot path computes, step by
step, in the notation of "Top-Theta Attention: Sparsifying Transformers by
Compensated Thresholding" (arXiv 2502.08363).  Only the test-suite, the smoke
check and the benchmark's CPU-baseline leg may import it.  The HIP library never
calls into it and shares no code, tables or helpers with it.

Every function is pinned by ``tests/test_oracle_pins.py`` against closed forms,
library routines it does not itself call, brute force on tiny inputs and
invariants of the method.  One reading is not pinned by anything the pages fix:
the causal prefix mean used for VMC in prefill (the paper's Eq. 5 averages all n
rows in non-causal notation) -- parity unpinned for that choice of mu; every
other step is pinned.

``oracle.presoftmax`` holds the pre-softmax variant (thresholds on the scores,
Algorithm 1 in its printed form) with the three estimates of the discarded
softmax mass of Sec. 3.2.1 (exact, exp-threshold, offline-calibrated); it is
pinned by ``tests/test_oracle_presoftmax_pins.py``.

``oracle.serving`` holds the decode-serving helpers (running V mean under
KV-cache appends, thresholds fitted to the row position) and the GQA selection
variants of Sec. 4.6, pinned by ``tests/test_oracle_serving_pins.py``; the
fitted function's form is a reading the pages do not fix (parity unpinned for
that choice).

``oracle.mkc`` holds multi-k cumulative calibration (Appendix D, Algorithm 2,
Eq. 8), pinned by ``tests/test_oracle_mkc_pins.py``: single-sample and
identical-copy closed forms, the pooled-quantile closed form where every
sample covers theta, and brute force over explicit interval lists.
"""
from .topth import (  # noqa: F401
    scores, post_softmax, kth_largest, theta_row, row_weights, row_output, topth_row,
    prefix_mean, prefill, decode, Calibrator, calibration_samples,
    PrefillResult, DecodeResult, RowResult,
)
from . import presoftmax  # noqa: F401,E402
from . import serving  # noqa: F401,E402
from . import mkc  # noqa: F401,E402
