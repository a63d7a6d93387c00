"""Exact FP32 row-wise Top-K for MI355X (gfx950): a sample-guided exact selector.

The selector itself lives in the HIP library built from `csrc/` and is reached
through the ctypes binding in `topkf` (importing it raises if the library has
not been built).  `workloads` draws the seeded synthetic score rows.
"""
__all__ = ["topkf", "workloads"]
