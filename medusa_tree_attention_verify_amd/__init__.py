"""Medusa single-pass tree verification on MI355X (gfx950).

The compute lives in the HIP library ``libmedusa_verify.so`` (C ABI in
include/medusa_verify.h).  ``ops`` holds thin PyTorch wrappers of its entry points,
``workloads`` the seeded synthetic inputs, ``step`` one whole verify step.
"""
__all__ = ["ops", "workloads", "step"]
