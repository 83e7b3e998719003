"""W4A16 consumer of the packed format: float64 CPU oracle.

TEST INFRASTRUCTURE ONLY -- imported by ``tests/``, by the smoke check and by
the benchmark's ``cpu_baseline`` leg, never by the product path.  It shares no
code with the HIP library.

What it computes.  "INT4/INT8 量化推理：从 GPTQ 到 AWQ 的取舍", section 六: the
weight-only setting (W4A16) keeps activations in 16-bit floating point and
quantizes only the weights; it cuts memory and memory traffic while the
multiply still runs on 16-bit matrix units.  Section 一 of the same page fixes
the stored form of a group: 4-bit codes, an fp16 scale and a 4-bit zero.  So
a layer's output for activations X (M tokens x d_in) is

    Y[m, n] = sum_c X[m, c] * Q[n, c],   Q[n, c] = s[n, g(c)] (q[n, c] - z[n, g(c)]),

with q read back from the packed bytes (low nibble = even column) and g(c)
the group of input channel c.  This is the plain definition, written out: an
unpack, a dequantization and one library matmul in float64.
"""
from __future__ import annotations

import numpy as np

from .gptq import dequantize, unpack_int4

__all__ = ["w4a16_matmul"]


def w4a16_matmul(X: np.ndarray, packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                 g_idx: np.ndarray) -> np.ndarray:
    """Y = X Q^T in float64.

    X: (M, d_in) activations (any float dtype, taken exactly); packed: (d_out,
    d_in / 2) uint8; scales: (d_out, ng) fp16 values; zeros: (d_out, ng)
    integers; g_idx: (d_in,) group of each input channel.  Returns (M, d_out).
    """
    codes = unpack_int4(packed)
    if codes.shape[1] != len(g_idx):
        raise ValueError("packed width does not match g_idx")
    Q = dequantize(codes, scales, zeros, g_idx)
    return np.asarray(X, dtype=np.float64) @ Q.T

