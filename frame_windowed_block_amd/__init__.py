"""Frame-windowed sparse attention for AMD Instinct MI355X (gfx950).

Python face of the C-ABI library ``libfsa.so`` (declared in ``include/fsa.h``):
``plan`` (frame-aligned active-block list), ``bounds`` (norm array and per-head
eligibility for the Cauchy-Schwarz softmax bound), ``attention`` (one pass
of q, k, v -> o) and ``pre_attention`` (normalisation, projection, rotary
embedding and head packing of the attention inputs in one kernel). torch
provides device memory and streams; all computation happens in the library's
HIP kernels.
"""
from ._abi import (  # noqa: F401
    FSA_ERR_BUFFER_TOO_SMALL, FSA_ERR_HIP, FSA_ERR_INVALID_ARG, FSA_ERR_UNALIGNED,
    FSA_ERR_UNSUPPORTED, FSA_OK, DevicePlan, FsaError, PlanInfo, attention, bounds, forward,
    header_symbols, lib, plan, pre_attention, version,
)

__all__ = [
    "plan", "bounds", "attention", "forward", "pre_attention", "DevicePlan", "PlanInfo", "FsaError", "lib",
    "version", "header_symbols",
]
