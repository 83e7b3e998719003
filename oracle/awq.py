"""Activation-aware per-channel scaling as a pre-pass to GPTQ: float64 CPU oracle.

TEST INFRASTRUCTURE ONLY -- imported by ``tests/``, by the smoke check and by
the benchmark's ``cpu_baseline`` leg, never by the product path.  It shares no
code with the HIP library.

What the pages say.  ipipp.com, section 二 (AWQ): the weights of input
channels that meet large activations matter most; before quantizing, each
input channel's weights are multiplied by a scale and the scale is divided
back out afterwards (folded into the previous layer, so the layer's output is
unchanged before rounding); the scales come from activation statistics (the
per-channel mean of |x| in its listing) and, more directly, from a search
that evaluates a few candidate scales and keeps the one with the smallest
output error; AWQ scaling can precede GPTQ.  "INT4/INT8 量化推理：从 GPTQ 到 AWQ
的取舍", section 四: the transform is exact (X W^T = (X diag(s)^-1)(W diag(s))^T)
and s follows the activations' magnitude, not the weights'.

Readings taken (the pages fix no formula for the candidates, the error or
dead channels):

R20 statistic: a_c = mean over the calibration tokens of |x_tc| (the
    listing's act_abs), accumulated in float64.
R21 candidates: s_c(alpha) = max(a_c, 1e-6) ** alpha for alpha in a grid the
    caller gives (alpha = 0: no scaling), evaluated in float64 and rounded to
    float32; the floor keeps a dead channel's scale finite.  alpha is the
    float32 value of the grid point (the form in which a caller hands it to
    the library).
R22 search: E(alpha) = ||(W - Q(alpha)) Xs^T||_F^2 on a sample Xs of
    calibration tokens, where Q(alpha) = RTN(W diag(s)) diag(s)^-1 is
    group-wise round-to-nearest with the path's own quantizer (R4-R8, R12, R18
    for the symmetric variant) applied to the scaled weights fp32(w * s_c)
    and each dequantized value divided back by s_c in float32; alpha* is the
    grid's argmin (the first on ties).
R23 application: W' = fp32(W * s*) column by column, and the Hessian of the
    scaled inputs X diag(s*)^-1, i.e. S'_ij = S_ij / (s*_i s*_j); then GPTQ
    runs unchanged on (W', S').  The codes, scales and zeros describe W'; the
    layer's input must be divided by s* (folded into the previous layer).
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .gptq import dequantize, gptq_layer, group_params, quantize_values

__all__ = ["channel_abs_mean", "awq_scales", "awq_rtn_error", "awq_search", "awq_apply", "awq_gptq_layer"]

F32 = np.float32
SCALE_FLOOR = 1e-6


def channel_abs_mean(chunks) -> np.ndarray:
    """R20: a_c = sum_t |x_tc| / N over all chunks, float64."""
    tot = None
    n = 0
    for X in chunks:
        X = np.asarray(X, dtype=np.float64)
        s = np.abs(X).sum(axis=0)
        tot = s if tot is None else tot + s
        n += X.shape[0]
    return tot / n


def awq_scales(a: np.ndarray, alpha: float) -> np.ndarray:
    """R21: fp32(max(a, 1e-6) ** alpha), alpha as float32, the power in float64."""
    al = float(np.float32(alpha))
    return (np.maximum(np.asarray(a, dtype=np.float64), SCALE_FLOOR) ** al).astype(F32)


def _rtn_scaled(W: np.ndarray, s: np.ndarray, bits: int, group_size: int, sym: bool) -> np.ndarray:
    """Q(alpha) of R22: group-wise RTN of fp32(w * s), divided back by s in fp32."""
    maxq = (1 << bits) - 1
    Ws = np.asarray(W, dtype=F32) * s[None, :]          # one fp32 rounding per weight
    rows, d = Ws.shape
    Q = np.empty((rows, d), dtype=F32)
    g = group_size
    for j in range(d // g):
        blk = Ws[:, j * g:(j + 1) * g]
        sc, z = group_params(blk, maxq, sym)
        _, dq = quantize_values(blk, sc[:, None], z[:, None], maxq)
        Q[:, j * g:(j + 1) * g] = dq.astype(F32) / s[None, j * g:(j + 1) * g]
    return Q


def awq_rtn_error(W: np.ndarray, Xs: np.ndarray, s: np.ndarray, bits: int = 4, group_size: int = 128,
                  sym: bool = False) -> float:
    """R22: ||(W - Q) Xs^T||_F^2 in float64 for one candidate s."""
    W64 = np.asarray(W, dtype=np.float64)
    Q = _rtn_scaled(W, s, bits, group_size, sym).astype(np.float64)
    Y = (W64 - Q) @ np.asarray(Xs, dtype=np.float64).T
    return float(np.sum(Y * Y))


def awq_search(W: np.ndarray, Xs: np.ndarray, a: np.ndarray, alphas: Sequence[float], bits: int = 4,
               group_size: int = 128, sym: bool = False) -> Dict[str, np.ndarray]:
    """R22: the error of every candidate and the grid's argmin (first on ties)."""
    errs = np.array([awq_rtn_error(W, Xs, awq_scales(a, al), bits, group_size, sym) for al in alphas])
    best = int(np.argmin(errs))
    return dict(errors=errs, best=best, alpha=float(alphas[best]), s=awq_scales(a, alphas[best]))


def awq_apply(W: np.ndarray, S: np.ndarray, s: np.ndarray):
    """R23: W' = fp32(W * s) and S' = S / (s s^T) (float64)."""
    Wp = (np.asarray(W, dtype=F32) * s[None, :]).astype(np.float64)
    s64 = s.astype(np.float64)
    Sp = np.asarray(S, dtype=np.float64) / np.outer(s64, s64)
    return Wp, Sp


def awq_gptq_layer(W: np.ndarray, S: np.ndarray, n: int, s: np.ndarray, **kw) -> Dict[str, np.ndarray]:
    """GPTQ on the scaled problem (R23); also returns Q_eff = Q' / s, the
    weights the unscaled inputs effectively meet."""
    Wp, Sp = awq_apply(W, S, s)
    r = gptq_layer(Wp, Sp, n, **kw)
    r["W_scaled"] = Wp
    r["S_scaled"] = Sp
    r["Q_eff"] = r["Q"] / s.astype(np.float64)[None, :]
    return r
