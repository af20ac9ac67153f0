"""Seeded synthetic inputs for the ReaDy state reader.

Serves both the HIP path's tests/benchmark and the CPU oracle: it draws the
verify-step state buffers (by running the fp32 gated delta rule in C), the
accept indices, the draft representations and the reader weights.  It holds
none of the reader's own arithmetic.
"""
from .gen import CONFIGS, Inputs, VerifyInputs, build, make, make_readers, make_shape, make_verify, philox4x32_10  # noqa: F401
