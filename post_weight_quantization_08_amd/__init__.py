"""MI355X (gfx950) GPTQ layer-wise weight quantization.

A thin ctypes binding over ``libgptq.so`` (built from ``csrc/`` by
``post_weight_quantization_08_amd.build``).  Every numeric step runs in the
library's HIP kernels; this module only marshals arguments.  PyTorch provides
device memory and streams.  There is no CPU fallback: importing the binding
without the built library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch  # loads the process's HIP runtime before libgptq.so binds to it

__all__ = [
    "GptqError", "GptqParams", "lib", "gptq_abi_version", "gptq_status_string",
    "gptq_workspace_size", "gptq_hessian_accumulate", "gptq_prepare_hinv",
    "gptq_quantize_layer", "gptq_pack_int4", "gptq_pack_bits", "gptq_timing_enable",
    "gptq_timing_reset", "gptq_timing_read", "gptq_pack_int4_permuted", "gptq_w4a16_matmul",
    "gptq_abs_accumulate", "gptq_awq_search", "gptq_awq_apply", "gptq_layer_forward",
    "gptq_probe_mfma", "gptq_probe_copy", "gptq_probe_sink_bytes", "gptq_w4a16_matmul_noalloc",
    "ACT_NONE", "ACT_RELU", "ACT_SILU",
    "OP_HESSIAN", "OP_PREPARE", "OP_QUANTIZE", "OP_W4A16", "OP_ABS", "OP_AWQ_SEARCH", "OP_FORWARD",
    "TIME_SYRK", "TIME_DIAG", "TIME_FACTOR", "TIME_BLOCK_QUANT", "TIME_TRAILING",
    "TIME_PACK", "TIME_PREP", "TIME_SYRK_REDUCE", "TIME_W4_STAGE", "TIME_W4_MAIN", "TIME_ABS",
    "TIME_AWQ_SEARCH", "TIME_AWQ_APPLY", "TIME_FORWARD", "dtype_code", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgptq.so")

OK, EINVAL, ENOTPD, EHIP, EUNSUPPORTED, ENOMEM = range(6)
F32, F16, BF16 = 0, 1, 2
OP_HESSIAN, OP_PREPARE, OP_QUANTIZE, OP_W4A16, OP_ABS, OP_AWQ_SEARCH, OP_FORWARD = 0, 1, 2, 3, 4, 5, 6
ACT_NONE, ACT_RELU, ACT_SILU = 0, 1, 2
(TIME_SYRK, TIME_DIAG, TIME_FACTOR, TIME_BLOCK_QUANT, TIME_TRAILING, TIME_PACK, TIME_PREP,
 TIME_SYRK_REDUCE, TIME_W4_STAGE, TIME_W4_MAIN, TIME_ABS, TIME_AWQ_SEARCH, TIME_AWQ_APPLY, TIME_FORWARD) = range(14)


class GptqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {gptq_status_string(status)} ({status})")


class GptqParams(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("damp_rel", ctypes.c_float),
                ("act_order", ctypes.c_int32), ("sym", ctypes.c_int32), ("static_groups", ctypes.c_int32)]

    @classmethod
    def make(cls, bits=4, group_size=128, block_size=128, damp_rel=0.01, act_order=False, sym=False,
             static_groups=False):
        return cls(int(bits), int(group_size), int(block_size), float(damp_rel), int(bool(act_order)),
                   int(bool(sym)), int(bool(static_groups)))


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m post_weight_quantization_08_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER
    L.gptq_abi_version.restype = i32
    L.gptq_status_string.restype = ctypes.c_char_p
    L.gptq_status_string.argtypes = [i32]
    L.gptq_workspace_size.restype = i32
    L.gptq_workspace_size.argtypes = [i32, P(GptqParams), i64, i64, i64, i64, P(sz)]
    L.gptq_hessian_accumulate.restype = i32
    L.gptq_hessian_accumulate.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, vp, P(i64), i64, vp, sz, vp]
    L.gptq_prepare_hinv.restype = i32
    L.gptq_prepare_hinv.argtypes = [vp, vp, vp, i64, i64, P(GptqParams), vp, vp, vp, vp, sz, vp]
    L.gptq_quantize_layer.restype = i32
    L.gptq_quantize_layer.argtypes = [vp, i32, i64, i64, i64, i64, vp, vp, P(GptqParams), vp, vp, vp, vp, vp,
                                      vp, sz, vp]
    L.gptq_pack_int4.restype = i32
    L.gptq_pack_int4.argtypes = [vp, i64, i64, vp, vp]
    L.gptq_pack_bits.restype = i32
    L.gptq_pack_bits.argtypes = [vp, i64, i64, i32, vp, vp]
    L.gptq_pack_int4_permuted.restype = i32
    L.gptq_pack_int4_permuted.argtypes = [vp, i64, i64, vp, vp, vp]
    L.gptq_abs_accumulate.restype = i32
    L.gptq_abs_accumulate.argtypes = [vp, vp, i32, i64, i64, i64, vp, P(i64), i64, vp, sz, vp]
    L.gptq_awq_search.restype = i32
    L.gptq_awq_search.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, i32, i64, i64, P(GptqParams),
                                  P(ctypes.c_float), i32, vp, vp, vp, vp, sz, vp]
    L.gptq_awq_apply.restype = i32
    L.gptq_awq_apply.argtypes = [vp, vp, i64, vp, vp, i32, i64, i64, vp, vp]
    L.gptq_layer_forward.restype = i32
    L.gptq_layer_forward.argtypes = [vp, i32, i64, i64, i64, vp, i64, i64, i32, vp, i64, vp, sz, vp]
    L.gptq_w4a16_matmul.restype = i32
    L.gptq_w4a16_matmul.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp, i64, i32, vp, i64, vp, sz, vp]
    L.gptq_probe_sink_bytes.restype = sz
    L.gptq_probe_mfma.restype = i32
    L.gptq_probe_mfma.argtypes = [i32, i32, vp, P(ctypes.c_double), vp]
    L.gptq_probe_copy.restype = i32
    L.gptq_probe_copy.argtypes = [vp, vp, sz, P(ctypes.c_double), P(ctypes.c_double), vp]
    L.gptq_w4a16_matmul_noalloc.restype = i32
    L.gptq_w4a16_matmul_noalloc.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp, i64, i32, vp, i64, vp]
    L.gptq_timing_enable.restype = i32
    L.gptq_timing_enable.argtypes = [i32]
    L.gptq_timing_reset.restype = i32
    L.gptq_timing_read.restype = i32
    L.gptq_timing_read.argtypes = [i32, P(ctypes.c_double), P(i64)]
    return L


lib = _load()


# ---------------------------------------------------------------- marshalling helpers
def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dtype_code(dt) -> int:
    if dt == torch.float32:
        return F32
    if dt == torch.float16:
        return F16
    if dt == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported dtype {dt}")


def _check(status: int, what: str) -> None:
    if status != OK:
        raise GptqError(status, what)


def _i64_array(vals) -> "ctypes.Array":
    arr = (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])
    return arr


# ---------------------------------------------------------------- the C entry points
def gptq_abi_version() -> int:
    return int(lib.gptq_abi_version())


def gptq_status_string(status: int) -> str:
    return lib.gptq_status_string(int(status)).decode()


def gptq_workspace_size(op: int, params: Optional[GptqParams] = None, d_out: int = 1, d_in: int = 1,
                        n_rows: int = 0, batch: int = 1) -> int:
    out = ctypes.c_size_t(0)
    pp = ctypes.byref(params) if params is not None else None
    _check(lib.gptq_workspace_size(op, pp, d_out, d_in, n_rows, batch, ctypes.byref(out)), "gptq_workspace_size")
    return int(out.value)


def gptq_hessian_accumulate(S, D, n_tokens, X, d_in: int, n_rows: int, ld_x: Optional[int] = None,
                            x_dtype: Optional[int] = None, row_idx=None, row_ptr: Optional[Sequence[int]] = None,
                            batch: int = 1, workspace=None, ws_bytes: int = 0, stream=None) -> None:
    """S += X^T X (lower), D += diag in fp64, n_tokens[b] += rows used (a device int64 tensor)."""
    rp = _i64_array(row_ptr) if row_ptr is not None else None
    if x_dtype is None:
        x_dtype = dtype_code(X.dtype)
    if ld_x is None:
        ld_x = d_in
    st = lib.gptq_hessian_accumulate(_ptr(S), _ptr(D), _ptr(n_tokens), _ptr(X), x_dtype, n_rows, d_in, ld_x,
                                     _ptr(row_idx), rp, batch, _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "gptq_hessian_accumulate")


def gptq_prepare_hinv(S, D, n_tokens, d_in: int, batch: int, params: GptqParams, U, perm, info,
                      workspace, ws_bytes: int, stream=None) -> None:
    st = lib.gptq_prepare_hinv(_ptr(S), _ptr(D), _ptr(n_tokens), d_in, batch, ctypes.byref(params), _ptr(U), _ptr(perm),
                               _ptr(info), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "gptq_prepare_hinv")


def gptq_quantize_layer(W, w_dtype: int, d_out: int, d_in: int, ld_w: int, batch: int, U, perm,
                        params: GptqParams, codes, scales, zeros, g_idx, Q_opt, workspace, ws_bytes: int,
                        stream=None) -> None:
    st = lib.gptq_quantize_layer(_ptr(W), w_dtype, d_out, d_in, ld_w, batch, _ptr(U), _ptr(perm),
                                 ctypes.byref(params), _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(g_idx),
                                 _ptr(Q_opt), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "gptq_quantize_layer")


def gptq_pack_int4(codes, rows: int, cols: int, packed, stream=None) -> None:
    _check(lib.gptq_pack_int4(_ptr(codes), rows, cols, _ptr(packed), _stream(stream)), "gptq_pack_int4")


def gptq_pack_bits(codes, rows: int, cols: int, bits: int, packed, stream=None) -> None:
    _check(lib.gptq_pack_bits(_ptr(codes), rows, cols, bits, _ptr(packed), _stream(stream)), "gptq_pack_bits")


def gptq_pack_int4_permuted(codes, rows: int, cols: int, perm, packed, stream=None) -> None:
    _check(lib.gptq_pack_int4_permuted(_ptr(codes), rows, cols, _ptr(perm), _ptr(packed), _stream(stream)),
           "gptq_pack_int4_permuted")


def gptq_w4a16_matmul(X, x_dtype: int, M: int, d_in: int, ld_x: int, qweight, scales, zeros, perm, d_out: int,
                      group_size: int, Y, ld_y: int, workspace, ws_bytes: int, stream=None) -> None:
    st = lib.gptq_w4a16_matmul(_ptr(X), x_dtype, M, d_in, ld_x, _ptr(qweight), _ptr(scales), _ptr(zeros),
                               _ptr(perm), d_out, group_size, _ptr(Y), ld_y, _ptr(workspace), ws_bytes,
                               _stream(stream))
    _check(st, "gptq_w4a16_matmul")


def gptq_abs_accumulate(A, X, x_dtype: int, n_rows: int, d_in: int, ld_x: int, row_idx=None,
                        row_ptr: Optional[Sequence[int]] = None, batch: int = 1, workspace=None, ws_bytes: int = 0,
                        stream=None) -> None:
    rp = _i64_array(row_ptr) if row_ptr is not None else None
    _check(lib.gptq_abs_accumulate(_ptr(A), _ptr(X), x_dtype, n_rows, d_in, ld_x, _ptr(row_idx), rp, batch,
                                   _ptr(workspace), ws_bytes, _stream(stream)), "gptq_abs_accumulate")


def gptq_awq_search(W, w_dtype: int, d_out: int, d_in: int, ld_w: int, A, n_tokens, Xs, xs_dtype: int,
                    n_s: int, ld_xs: int, params: GptqParams, alphas: Sequence[float], err_out, s_out, best_out,
                    workspace, ws_bytes: int, stream=None) -> None:
    al = (ctypes.c_float * len(alphas))(*[float(a) for a in alphas])
    _check(lib.gptq_awq_search(_ptr(W), w_dtype, d_out, d_in, ld_w, _ptr(A), _ptr(n_tokens), _ptr(Xs), xs_dtype, n_s,
                               ld_xs, ctypes.byref(params), al, len(alphas), _ptr(err_out), _ptr(s_out),
                               _ptr(best_out), _ptr(workspace), ws_bytes, _stream(stream)), "gptq_awq_search")


def gptq_w4a16_matmul_noalloc(X, x_dtype: int, M: int, d_in: int, ld_x: int, qweight, scales, zeros, perm,
                              d_out: int, group_size: int, Y, ld_y: int, stream=None) -> None:
    st = lib.gptq_w4a16_matmul_noalloc(_ptr(X), x_dtype, M, d_in, ld_x, _ptr(qweight), _ptr(scales), _ptr(zeros),
                                       _ptr(perm), d_out, group_size, _ptr(Y), ld_y, _stream(stream))
    _check(st, "gptq_w4a16_matmul_noalloc")


def gptq_probe_mfma(kind: int, iters: int, sink, stream=None) -> float:
    """Sustained MFMA rate (TFLOP/s) of a register-only loop: kind 0 fp16, 1 bf16, 2 fp64 (one operand
    set), 3 fp16, 4 bf16 (new operands for every MFMA)."""
    out = ctypes.c_double(0.0)
    _check(lib.gptq_probe_mfma(kind, iters, _ptr(sink), ctypes.byref(out), _stream(stream)), "gptq_probe_mfma")
    return float(out.value)


def gptq_probe_copy(src, dst, nbytes: int, stream=None):
    """(GB/s counting read + write, ms) of a plain device copy of nbytes."""
    gbs, ms = ctypes.c_double(0.0), ctypes.c_double(0.0)
    _check(lib.gptq_probe_copy(_ptr(src), _ptr(dst), nbytes, ctypes.byref(gbs), ctypes.byref(ms), _stream(stream)),
           "gptq_probe_copy")
    return float(gbs.value), float(ms.value)


def gptq_probe_sink_bytes() -> int:
    return int(lib.gptq_probe_sink_bytes())


def gptq_awq_apply(S, D, d_in: int, s, W, w_dtype: int, d_out: int, ld_w: int, W_out, stream=None) -> None:
    _check(lib.gptq_awq_apply(_ptr(S), _ptr(D), d_in, _ptr(s), _ptr(W), w_dtype, d_out, ld_w, _ptr(W_out),
                              _stream(stream)), "gptq_awq_apply")


def gptq_layer_forward(X, x_dtype: int, n_tok: int, d_in: int, ld_x: int, Q, d_out: int, ld_q: int, act: int, Y,
                       ld_y: int, workspace, ws_bytes: int, stream=None) -> None:
    _check(lib.gptq_layer_forward(_ptr(X), x_dtype, n_tok, d_in, ld_x, _ptr(Q), d_out, ld_q, act, _ptr(Y), ld_y,
                                  _ptr(workspace), ws_bytes, _stream(stream)), "gptq_layer_forward")


def gptq_timing_enable(on: bool) -> None:
    _check(lib.gptq_timing_enable(int(bool(on))), "gptq_timing_enable")


def gptq_timing_reset() -> None:
    _check(lib.gptq_timing_reset(), "gptq_timing_reset")


def gptq_timing_read(kind: int):
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check(lib.gptq_timing_read(kind, ctypes.byref(ms), ctypes.byref(n)), "gptq_timing_read")
    return float(ms.value), int(n.value)
