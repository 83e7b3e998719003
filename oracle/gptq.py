"""GPTQ layer-wise weight quantization: float64 CPU oracle.

TEST INFRASTRUCTURE ONLY -- imported by ``tests/``, by the smoke check and by
the benchmark's ``cpu_baseline`` leg, never by the product path.  It shares no
code, table or helper with the HIP library.

What it computes, step by step, in the order the pages give it.  Sources are
cited by page title and section:

[A] "3. 模型量化技术(下)：权重量化与激活量化、KL散度校准、GPTQ/AWQ量化方法",
    section "GPTQ：基于二阶信息的后训练量化" and its pseudocode block: per
    layer, collect the layer's calibration inputs, build H from them, walk the
    columns, quantize, push a compensation onto the later columns.
[B] "INT4/INT8 量化推理：从 GPTQ 到 AWQ 的取舍": section 一 (every 128
    consecutive weights share one scale and one zero-point; fp16 scale, 4-bit
    zero, 66.5 bytes per 128 weights) and section 三 "GPTQ：逐列纠错" (the
    column loop: err = (w_j - q_j) / Hinv[j, j]; w[j+1:] -= err * Hinv[j, j+1:]).
[C] ipipp.com, section 一 "GPTQ：在每一列权重上做二阶误差补偿": the output
    error is ||dW X^T||_F^2; H = 2 X^T X / N; damping H + eps I; inverse;
    column loop with round() (half-to-even) and the row update divided by the
    inverse's diagonal; blocks or an approximate decomposition of the inverse
    to save memory; columns optionally ordered by importance.
[D] "1. 项目概述：大模型量化的“校准”艺术": section 2.1 (min-max maps the
    range [min, max] linearly onto the integer range) and section 2.2 (the five
    GPTQ steps; an efficient approximation of the inverse Hessian).
[E] "大模型量化实战（上）：从显存焦虑到算法本质", section 算法本质: RTN rounds every
    weight the same way, without compensation.

Readings taken where the pages are silent, garbled or disagree:

R1  H = 2 X^T X / N with X token-major ([C]); codes do not depend on the
    scaling of H because damping is relative.
R2  damping lam = damp_rel * mean(diag H), damp_rel = 0.01 (the workloads'
    constant; [C] prints an absolute 1e-6).
R3  the "approximate decomposition" of the inverse ([C], [D] step 4) is the
    upper Cholesky factor U of Hd^-1 (U^T U = Hd^-1): row k of U scaled by
    U[k,k] equals row k of the inverse of the still-unquantized sub-Hessian,
    which is the exact OBS update.  The listings' single static inverse is
    not the optimum beyond the first column (a negative control in the pins
    feeds its rows to ``gptq_quantize`` and shows the difference).
R4  quantizer: asymmetric min-max per (row, group of g consecutive columns in
    quantization order), fp16 scale, integer zero in [0, maxq] ([B] §一, [D]
    §2.1).
R5  the range always contains 0: xmin = min(0, min w), xmax = max(0, max w),
    so the stored zero lies in [0, maxq] and 0.0 is representable.
R6  s = fp16_rne((xmax - xmin) / maxq); if that is 0 (all-zero group, or a
    range below fp16's smallest subnormal) s = 1, which makes every code of
    the group equal to z = 0 and its dequantized value exactly 0; an fp16
    overflow saturates to 65504.
R7  rounding is half-to-even everywhere (torch.round in [C]).
R8  the loop quantizes and dequantizes with the fp16-rounded scale.
R9  a group's scale and zero are fixed from the group's *current* values when
    its first column is reached (after all earlier feedback): [C]'s loop
    quantizes W[:, j] as it stands when column j comes up.  No page prints a
    worked example; the pins compare this loop with one written from the
    definition (a fresh inverse of the remaining sub-Hessian per column).
R10 groups run along the input dimension, in quantization order.
R11 act-order: perm = stable argsort of -diag(H) (descending importance,
    ties to the lower index); groups are formed after the permutation and
    results return to the original column order with g_idx.
R12 decisions that turn floats into integers (scale, zero, code) are taken
    in float32, the precision of the working copy in [C] (``.float()``); the
    rest is float64.
R18 symmetric variant (``sym``): [C]'s listing takes the scale from the
    largest magnitude, s = max|w| / (2^(bits-1) - 1), and clamps the signed
    code round(w / s) to [-2^(bits-1), 2^(bits-1) - 1]; its text says real
    frameworks do this per group.  So per group: amax = max(-xmin, xmax) over
    the R5 range, s = fp16_rne(amax / (2^(bits-1) - 1)) with R6's zero and
    overflow rules, and the stored (unsigned) code is the signed code plus
    the fixed zero z = 2^(bits-1).
R19 static groups (``static_groups``; the pages are silent, the variant is
    named only as a quantizer option): every group's scale and zero are fixed
    before the column loop, from the layer's weights as given (no error
    feedback yet), over g consecutive ORIGINAL columns; with act-order a
    column is quantized in permuted order but with its original group's
    parameters, so g_idx = column // g.  Everything else (U, the loop, the
    feedback) is unchanged.

Pins that tie this code to something other than itself live in
``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional

import numpy as np
import scipy.linalg

__all__ = [
    "hessian_sum", "hessian", "damping", "act_order_perm", "inverse_factor",
    "group_params", "quantize_values", "gptq_quantize", "gptq_quantize_elimination",
    "rtn_quantize", "gptq_layer", "dequantize",
    "pack_int4", "unpack_int4", "pack_bits", "unpack_bits", "recon_error",
    "recon_error_direct", "storage_bytes", "FP16_MAX", "group_range", "decision_margins",
    "static_group_params",
]

F32 = np.float32
FP16_MAX = 65504.0


# ----------------------------------------------------------------------------
# Hessian: [C] H = 2 * (X^T X) / N ; [A] H from the layer's calibration inputs
# ----------------------------------------------------------------------------
def hessian_sum(chunks: Iterable[np.ndarray]):
    """S = sum over chunks of X_c^T X_c (float64), N = total rows.

    The sum is kept separate from the 1/N so that calibration data can be fed
    chunk by chunk; H = 2 S / N is formed once at the end (R1).
    """
    S = None
    n = 0
    for X in chunks:
        X = np.asarray(X, dtype=np.float64)
        if S is None:
            S = np.zeros((X.shape[1], X.shape[1]))
        S += X.T @ X
        n += X.shape[0]
    if S is None:
        raise ValueError("no calibration rows")
    return S, n


def hessian(S: np.ndarray, n: int) -> np.ndarray:
    """H0 = 2 S / N ([C]; R1)."""
    if n <= 0:
        raise ValueError("N must be positive")
    return 2.0 * np.asarray(S, dtype=np.float64) / float(n)


def damping(H0: np.ndarray, damp_rel: float):
    """lam = damp_rel * mean(diag H0); Hd = H0 + lam I  ([C] damping; R2)."""
    lam = float(damp_rel) * float(np.mean(np.diag(H0)))
    return lam, H0 + lam * np.eye(H0.shape[0])


def act_order_perm(H0: np.ndarray) -> np.ndarray:
    """Quantization order by importance ([C], last paragraph before the
    listing): perm[k] = original column quantized k-th; descending diag(H0),
    ties to the lower original index (R11)."""
    return np.argsort(-np.diag(H0), kind="stable").astype(np.int64)


def inverse_factor(Hd: np.ndarray) -> np.ndarray:
    """Upper triangular U with U^T U = Hd^-1 (R3).

    Hd^-1 comes from a Cholesky solve against the identity; its lower Cholesky
    factor L (L L^T = Hd^-1) gives U = L^T.  Raises numpy/scipy LinAlgError
    when Hd is not positive definite.
    """
    d = Hd.shape[0]
    c = scipy.linalg.cho_factor(Hd, lower=True, check_finite=True)
    Hinv = scipy.linalg.cho_solve(c, np.eye(d))
    L = np.linalg.cholesky(Hinv)
    return np.triu(L.T)


# ----------------------------------------------------------------------------
# Quantizer ([B] §一, [D] §2.1; readings R4-R8, R12)
# ----------------------------------------------------------------------------
def group_range(Wg: np.ndarray):
    """(xmin, xmax) of each row of a group in float32, widened to contain 0 (R5)."""
    w32 = np.asarray(Wg).astype(F32)
    return np.minimum(w32.min(axis=1), F32(0.0)), np.maximum(w32.max(axis=1), F32(0.0))


def group_params(Wg: np.ndarray, maxq: int, sym: bool = False):
    """Scale and zero of each row of a group.

    Wg: (rows, g) current values (any float dtype).  Returns (s, z) with s the
    fp16-rounded scale held as float32 (rows,) and z int64 (rows,).
    Arithmetic in float32 (R12); ``sym``: R18.
    """
    xmin, xmax = group_range(Wg)
    if sym:
        half = (maxq + 1) // 2
        t = np.maximum(-xmin, xmax) / F32(half - 1)
        with np.errstate(over="ignore"):
            s16 = t.astype(np.float16)
        s16 = np.where(np.isinf(s16), np.float16(FP16_MAX), s16)
        s = s16.astype(F32)
        s = np.where(s == F32(0.0), F32(1.0), s)
        return s, np.full(s.shape, half, dtype=np.int64)
    t = (xmax - xmin) / F32(maxq)
    with np.errstate(over="ignore"):
        s16 = t.astype(np.float16)
    s16 = np.where(np.isinf(s16), np.float16(FP16_MAX), s16)
    s = s16.astype(F32)
    s = np.where(s == F32(0.0), F32(1.0), s)
    z = np.clip(np.rint(-xmin / s), 0, maxq).astype(np.int64)
    return s, z


def quantize_values(w: np.ndarray, s: np.ndarray, z: np.ndarray, maxq: int):
    """q = clamp(round(w / s) + z, 0, maxq); dq = s (q - z).

    The division and the rounding are float32 (R12, R7); dq is exact in float64
    because s is an fp16 value and q - z a small integer.
    """
    v = np.asarray(w).astype(F32) / s
    q = np.clip(np.rint(v).astype(np.float64) + z, 0, maxq)
    dq = s.astype(np.float64) * (q - z)
    return q.astype(np.int64), dq


# ----------------------------------------------------------------------------
# Column loop with error feedback ([B] §三, [C] listing, [A] pseudocode)
# ----------------------------------------------------------------------------
def _check_shapes(d: int, group_size: int, block_size: int):
    if d % group_size:
        raise ValueError("group_size must divide the number of columns")
    if group_size % block_size and block_size % group_size:
        raise ValueError("one of group_size and block_size must divide the other")


def static_group_params(W: np.ndarray, bits: int, group_size: int, sym: bool = False) -> Dict[str, np.ndarray]:
    """R19: scale, zero and range of each group of g consecutive original
    columns of W, from W as given.  Arrays (rows, d / g)."""
    W = np.asarray(W)
    rows, d = W.shape
    g = int(group_size)
    if d % g:
        raise ValueError("group_size must divide the number of columns")
    maxq = (1 << bits) - 1
    ng = d // g
    out = dict(s=np.zeros((rows, ng), dtype=F32), z=np.zeros((rows, ng), dtype=np.int64),
               gmin=np.zeros((rows, ng), dtype=F32), gmax=np.zeros((rows, ng), dtype=F32))
    for j in range(ng):
        blk = W[:, j * g:(j + 1) * g]
        out["s"][:, j], out["z"][:, j] = group_params(blk, maxq, sym)
        out["gmin"][:, j], out["gmax"][:, j] = group_range(blk)
    return out


def gptq_quantize(Wp: np.ndarray, U: np.ndarray, bits: int = 4, group_size: int = 128,
                  block_size: int = 128, trace: bool = False,
                  force: Optional[Dict[int, dict]] = None, sym: bool = False,
                  static: Optional[Dict[str, np.ndarray]] = None) -> Dict[str, np.ndarray]:
    """Quantize the columns of Wp in order 0..d-1 with error feedback.

    Wp: (rows, d) weights already in quantization order; U: upper factor of
    the damped inverse Hessian in the same order (R3).  For column k:
      group start (k % g == 0): s, z from the group's current values (R9);
      q, dq from the current w[:, k];
      e = (w[:, k] - dq) / U[k, k];
      w[:, j] -= e * U[k, j] for every later column j   ([B] §三 / [C]).
    ``block_size`` B only regroups the later-column updates ([C] "按块处理"):
    inside a block they are applied at once, to the columns beyond the block
    they are applied together after the block as  w[:, rest] -= Err @ U[blk,
    rest].  B = 1 is the plain column loop.

    Returns codes, scales (fp16 values as float32), zeros, Q (dequantized),
    pre (each column's value just before it was quantized), Err (all e), and
    with ``trace`` a list of snapshots of the working copy after each column.

    ``force`` (a test hook for following the other side of a rounding tie)
    maps a column k to {"q": code} or {"s": scale, "z": zero}; the given
    decision replaces the computed one for every row at that column.

    ``static`` (R19): the output of ``static_group_params`` plus "col_group",
    the group of each column in the order given; column k then takes the
    parameters of group col_group[k] instead of computing them at a group
    start, and scales/zeros/gmin/gmax are returned as given.
    """
    if trace and block_size != 1:
        raise ValueError("trace needs the unblocked loop (block_size=1)")
    W = np.array(Wp, dtype=np.float64, copy=True)
    if not np.all(np.isfinite(W)) or not np.all(np.isfinite(U)):
        raise ValueError("non-finite input")
    rows, d = W.shape
    g, B = int(group_size), int(block_size)
    _check_shapes(d, g, B)
    maxq = (1 << bits) - 1
    ng = d // g
    codes = np.zeros((rows, d), dtype=np.int64)
    scales = np.zeros((rows, ng), dtype=F32)
    zeros = np.zeros((rows, ng), dtype=np.int64)
    Q = np.zeros((rows, d))
    pre = np.zeros((rows, d))
    err_all = np.zeros((rows, d))
    gmin = np.zeros((rows, ng), dtype=F32)
    gmax = np.zeros((rows, ng), dtype=F32)
    snaps = []
    s = z = None
    for b0 in range(0, d, B):
        b1 = min(b0 + B, d)
        Err = np.zeros((rows, b1 - b0))
        for k in range(b0, b1):
            fk = force.get(k) if force else None
            if static is not None:
                s = static["s"][:, static["col_group"][k]]
                z = static["z"][:, static["col_group"][k]]
            elif k % g == 0:
                s, z = group_params(W[:, k:k + g], maxq, sym)
                if fk is not None and "s" in fk:
                    s = np.full(rows, fk["s"], dtype=F32)
                    z = np.full(rows, fk["z"], dtype=np.int64)
                scales[:, k // g] = s
                zeros[:, k // g] = z
                gmin[:, k // g], gmax[:, k // g] = group_range(W[:, k:k + g])
            pre[:, k] = W[:, k]
            q, dq = quantize_values(W[:, k], s, z, maxq)
            if fk is not None and "q" in fk:
                q = np.full(rows, int(fk["q"]), dtype=np.int64)
                dq = s.astype(np.float64) * (q - z)
            codes[:, k] = q
            Q[:, k] = dq
            e = (W[:, k] - dq) / U[k, k]
            W[:, k + 1:b1] -= np.outer(e, U[k, k + 1:b1])
            W[:, k] = dq
            Err[:, k - b0] = e
        if b1 < d:
            W[:, b1:] -= Err @ U[b0:b1, b1:]
        err_all[:, b0:b1] = Err
        if trace:
            snaps.append(W.copy())
    if static is not None:
        scales, zeros = static["s"].copy(), static["z"].copy()
        gmin, gmax = static["gmin"].copy(), static["gmax"].copy()
    out = dict(codes=codes, scales=scales, zeros=zeros, Q=Q, pre=pre, Err=err_all, gmin=gmin, gmax=gmax)
    if trace:
        out["trace"] = snaps
    return out


def gptq_quantize_elimination(Wp: np.ndarray, Hd: np.ndarray, bits: int = 4,
                              group_size: int = 128, trace: bool = False):
    """Same loop, written with the explicitly updated inverse (OBS form).

    Keeps F = inverse of the still-unquantized sub-Hessian (as a full matrix
    whose eliminated rows/columns are zero).  Column k uses
    e = (w_k - dq_k) / F[k,k] and w[:, k+1:] -= e * F[k, k+1:], then removes
    index k from F by the rank-1 elimination F -= F[:,k] F[k,:] / F[k,k].
    Mathematically identical to ``gptq_quantize`` (R3); kept as a self-check.
    """
    W = np.array(Wp, dtype=np.float64, copy=True)
    rows, d = W.shape
    g = int(group_size)
    _check_shapes(d, g, 1)
    maxq = (1 << bits) - 1
    c = scipy.linalg.cho_factor(Hd, lower=True)
    F = scipy.linalg.cho_solve(c, np.eye(d))
    codes = np.zeros((rows, d), dtype=np.int64)
    scales = np.zeros((rows, d // g), dtype=F32)
    zeros = np.zeros((rows, d // g), dtype=np.int64)
    Q = np.zeros((rows, d))
    pre = np.zeros((rows, d))
    snaps = []
    for k in range(d):
        if k % g == 0:
            s, z = group_params(W[:, k:k + g], maxq)
            scales[:, k // g] = s
            zeros[:, k // g] = z
        pre[:, k] = W[:, k]
        q, dq = quantize_values(W[:, k], s, z, maxq)
        codes[:, k] = q
        Q[:, k] = dq
        fkk = F[k, k]
        e = (W[:, k] - dq) / fkk
        W[:, k + 1:] -= np.outer(e, F[k, k + 1:])
        W[:, k] = dq
        F = F - np.outer(F[:, k], F[k, :]) / fkk
        if trace:
            snaps.append(W.copy())
    out = dict(codes=codes, scales=scales, zeros=zeros, Q=Q, pre=pre)
    if trace:
        out["trace"] = snaps
    return out


def rtn_quantize(W: np.ndarray, bits: int = 4, group_size: int = 128, sym: bool = False):
    """Round-to-nearest with the same group quantizer and no compensation
    ([E]; the baseline GPTQ improves on)."""
    W = np.asarray(W, dtype=np.float64)
    rows, d = W.shape
    g = int(group_size)
    maxq = (1 << bits) - 1
    ng = d // g
    codes = np.zeros((rows, d), dtype=np.int64)
    scales = np.zeros((rows, ng), dtype=F32)
    zeros = np.zeros((rows, ng), dtype=np.int64)
    Q = np.zeros((rows, d))
    for j in range(ng):
        sl = slice(j * g, (j + 1) * g)
        s, z = group_params(W[:, sl], maxq, sym)
        scales[:, j] = s
        zeros[:, j] = z
        v = W[:, sl].astype(F32) / s[:, None]
        q = np.clip(np.rint(v).astype(np.float64) + z[:, None], 0, maxq)
        codes[:, sl] = q.astype(np.int64)
        Q[:, sl] = s[:, None].astype(np.float64) * (q - z[:, None])
    return dict(codes=codes, scales=scales, zeros=zeros, Q=Q)


# ----------------------------------------------------------------------------
# One whole layer ([A]: per layer, H from its calibration inputs, then the loop)
# ----------------------------------------------------------------------------
def gptq_layer(W: np.ndarray, S: np.ndarray, n: int, bits: int = 4, group_size: int = 128,
               block_size: int = 128, damp_rel: float = 0.01, act_order: bool = False,
               perm: Optional[np.ndarray] = None, sym: bool = False,
               static_groups: bool = False) -> Dict[str, np.ndarray]:
    """H0 = 2S/N -> damping -> (act-order perm) -> U -> column loop, with
    every result returned in the ORIGINAL column order:
      codes[:, perm[k]] = q_k; Q likewise; g_idx[perm[k]] = k // g;
      scales/zeros are indexed [row][group] with groups in quantization order.
    With ``static_groups`` (R19) groups are original columns: g_idx[c] = c // g
    and scales/zeros are in original group order; the static parameters are
    returned under "static" (with "col_group" in quantization order).
    """
    W = np.asarray(W, dtype=np.float64)
    d = W.shape[1]
    H0 = hessian(S, n)
    lam, Hd = damping(H0, damp_rel)
    if perm is None:
        perm = act_order_perm(H0) if act_order else np.arange(d, dtype=np.int64)
    perm = np.asarray(perm, dtype=np.int64)
    Hp = Hd[np.ix_(perm, perm)]
    U = inverse_factor(Hp)
    st = None
    if static_groups:
        st = static_group_params(W, bits, group_size, sym)
        st["col_group"] = perm // group_size
    r = gptq_quantize(W[:, perm], U, bits=bits, group_size=group_size, block_size=block_size, sym=sym,
                      static=st)
    out = {}
    for key in ("codes", "Q", "pre"):
        a = np.empty_like(r[key])
        a[:, perm] = r[key]
        out[key] = a
    g_idx = np.empty(d, dtype=np.int64)
    if static_groups:
        g_idx[:] = np.arange(d) // group_size
        out["static"] = st
    else:
        g_idx[perm] = np.arange(d) // group_size
    out.update(scales=r["scales"], zeros=r["zeros"], g_idx=g_idx, perm=perm, U=U, H0=H0,
               lam=lam, gmin=r["gmin"], gmax=r["gmax"])
    return out


# ----------------------------------------------------------------------------
# How close each integer decision of a run was to flipping (for judging ties)
# ----------------------------------------------------------------------------
def _half_integer_distance(v: np.ndarray) -> np.ndarray:
    """Distance of v to the nearest rounding midpoint (k + 1/2)."""
    v = np.asarray(v, dtype=np.float64)
    return np.abs(v - (np.floor(v) + 0.5))


def decision_margins(res: Dict[str, np.ndarray], bits: int, group_size: int,
                     sym: bool = False) -> Dict[str, np.ndarray]:
    """Margins of the rounding decisions of a ``gptq_layer`` result.

    code[r, c]:   distance of fp32(pre)/s to the nearest half-integer, in
                  quantization steps (a mismatch of +-1 can only come from a
                  value this close to a midpoint, up to the other side's
                  rounding differences);
    zero[r, g]:   distance of -xmin/s to the nearest half-integer, in steps;
    scale[r, g]:  relative distance of (xmax - xmin)/maxq (sym: amax /
                  (2^(bits-1) - 1)) to the nearest midpoint between two fp16
                  values.
    Arrays are in the result's original column order (codes) and group
    order (zeros, scales).  Under ``sym`` the zero is fixed (margin inf).
    """
    maxq = (1 << bits) - 1
    s = res["scales"].astype(F32)
    gi = res["g_idx"]
    v = res["pre"].astype(F32) / s[:, gi]
    code = _half_integer_distance(v.astype(np.float64))
    if sym:
        zero = np.full(s.shape, np.inf)
        t = (np.maximum(-res["gmin"], res["gmax"]) / F32((maxq + 1) // 2 - 1)).astype(np.float64)
    else:
        zero = _half_integer_distance((-res["gmin"] / s).astype(np.float64))
        t = ((res["gmax"] - res["gmin"]) / F32(maxq)).astype(np.float64)
    t16 = t.astype(np.float16).astype(np.float64)
    # the neighbouring fp16 value on the other side of t
    up = np.nextafter(t.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(t.astype(np.float16), np.float16(-np.inf)).astype(np.float64)
    other = np.where(t >= t16, up, dn)
    mid = 0.5 * (t16 + other)
    with np.errstate(divide="ignore", invalid="ignore"):
        scale = np.where(t > 0, np.abs(t - mid) / t, np.inf)
    return dict(code=code, zero=zero, scale=scale)


def dequantize(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
               g_idx: np.ndarray) -> np.ndarray:
    """Q[r, c] = s[r, g_idx[c]] * (codes[r, c] - z[r, g_idx[c]])."""
    s = np.asarray(scales, dtype=np.float64)[:, g_idx]
    z = np.asarray(zeros, dtype=np.int64)[:, g_idx]
    return s * (np.asarray(codes, dtype=np.int64) - z)


# ----------------------------------------------------------------------------
# Storage ([B] §一: 128 x 4-bit codes + fp16 scale + 4-bit zero = 66.5 bytes)
# ----------------------------------------------------------------------------
def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte along a row: low nibble = even column."""
    c = np.asarray(codes, dtype=np.int64)
    if c.shape[-1] % 2:
        raise ValueError("need an even number of columns")
    if c.min(initial=0) < 0 or c.max(initial=0) > 15:
        raise ValueError("codes out of 4-bit range")
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.int64)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int64)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def pack_bits(codes: np.ndarray, bits: int) -> np.ndarray:
    """Dense little-endian bit stream per row: code j occupies stream bits
    j*bits .. j*bits+bits-1 (its least significant bit first); stream bit i
    is bit (i mod 8) of byte i div 8.  Needs cols*bits to be a multiple of 8."""
    c = np.asarray(codes, dtype=np.int64)
    rows, cols = c.shape
    if (cols * bits) % 8:
        raise ValueError("cols * bits must be a multiple of 8")
    stream = np.zeros((rows, cols * bits), dtype=np.uint8)
    for b in range(bits):
        stream[:, b::bits] = (c >> b) & 1
    return np.packbits(stream, axis=1, bitorder="little")


def unpack_bits(packed: np.ndarray, bits: int, cols: int) -> np.ndarray:
    stream = np.unpackbits(np.asarray(packed, dtype=np.uint8), axis=1,
                           bitorder="little")[:, : cols * bits].astype(np.int64)
    out = np.zeros((stream.shape[0], cols), dtype=np.int64)
    for b in range(bits):
        out |= stream[:, b::bits] << b
    return out


def storage_bytes(rows: int, cols: int, bits: int = 4, group_size: int = 128,
                  scale_bytes: int = 2, zero_bits: Optional[int] = None) -> float:
    """Bytes of the packed format: per group g*bits/8 code bytes + one scale +
    one zero of ``zero_bits`` (default: ``bits``) bits ([B] §一)."""
    zb = bits if zero_bits is None else zero_bits
    per_group = group_size * bits / 8.0 + scale_bytes + zb / 8.0
    return rows * (cols // group_size) * per_group


# ----------------------------------------------------------------------------
# Objective ([C]: output error = ||dW X^T||_F^2)
# ----------------------------------------------------------------------------
def recon_error(W: np.ndarray, Q: np.ndarray, S: np.ndarray) -> float:
    """tr(dW S dW^T) with the undamped S = X^T X; equals ||(W-Q) X^T||_F^2."""
    D = np.asarray(W, dtype=np.float64) - np.asarray(Q, dtype=np.float64)
    return float(np.sum((D @ S) * D))


def recon_error_direct(W: np.ndarray, Q: np.ndarray, X: np.ndarray) -> float:
    D = np.asarray(W, dtype=np.float64) - np.asarray(Q, dtype=np.float64)
    R = D @ np.asarray(X, dtype=np.float64).T
    return float(np.sum(R * R))
