"""Exact widening of stored element bits to float64 (oracle side).

Storage types: fp32 (IEEE binary32), fp16 (IEEE binary16) and bf16 (the top 16
bits of a binary32).  Widening is exact for all three.
"""
import numpy as np

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Return the float64 values held by raw storage ``bits`` of ``dtype``."""
    bits = np.asarray(bits)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype}")


def bits_dtype(dtype: str):
    return np.uint32 if dtype == "f32" else np.uint16
