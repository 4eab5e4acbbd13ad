"""Seeded synthetic attention inputs shared by the tests, the benchmark and smoke().

This package draws random Q/K/V tensors only.  It holds none of the attention
arithmetic (no scores, softmax, thresholds or compensation), so the CPU oracle
and the HIP path can both be fed from it without sharing any of the method.
"""
from .gen import (  # noqa: F401
    CONFIG_IDS, ROLE_TEST, ROLE_CALIB, ROLE_PROBE, seed_of, attention_inputs,
    batch_of_sequences, attention_inputs_device, to_f64,
)
