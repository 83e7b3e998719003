"""Sequencing of the four library calls for one layer (or a batch of experts).

Allocation of outputs and workspaces goes through torch; every computation is
one of the library's entry points.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np
import torch

from . import (F32, GptqError, GptqParams, OP_ABS, OP_AWQ_SEARCH, OP_FORWARD, OP_HESSIAN, OP_PREPARE, OP_QUANTIZE, OP_W4A16,
               ENOTPD, dtype_code, gptq_abs_accumulate, gptq_awq_apply, gptq_awq_search, gptq_hessian_accumulate,
               gptq_layer_forward, gptq_pack_bits, gptq_pack_int4, gptq_pack_int4_permuted, gptq_prepare_hinv,
               gptq_quantize_layer, gptq_w4a16_matmul, gptq_workspace_size)


def to_device(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Host array in storage form ('f32', 'f16', or 'bf16' as uint16 bits) -> device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


class HessianState:
    """The running accumulator (S, D, N) of one layer or of a batch of experts,
    all in device memory (N: int64 rows used per entry)."""

    def __init__(self, d_in: int, batch: int = 1, device="cuda", track_abs: bool = False):
        self.d_in, self.batch, self.device = int(d_in), int(batch), device
        self.S = torch.zeros(batch, d_in, d_in, dtype=torch.float32, device=device)
        self.D = torch.zeros(batch, d_in, dtype=torch.float64, device=device)
        # per-channel sum of |x| (activation-aware scaling), when asked for
        self.A = torch.zeros(batch, d_in, dtype=torch.float64, device=device) if track_abs else None
        self.n = torch.zeros(batch, dtype=torch.int64, device=device)
        self._ws = None

    def workspace(self, n_rows: int) -> torch.Tensor:
        need = gptq_workspace_size(OP_HESSIAN, None, 1, self.d_in, n_rows, self.batch)
        if self._ws is None or self._ws.numel() < need:
            self._ws = _ws(need, self.device)
        return self._ws

    def zero(self) -> None:
        self.S.zero_()
        self.D.zero_()
        if self.A is not None:
            self.A.zero_()
        self.n.zero_()

    def add(self, X: torch.Tensor, row_idx: Optional[torch.Tensor] = None,
            row_ptr: Optional[Sequence[int]] = None, stream=None) -> None:
        n_rows = X.shape[0]
        rows_for_ws = n_rows if row_idx is None else int(np.max(np.diff(np.asarray(row_ptr))))
        ws = self.workspace(rows_for_ws)
        nb = self.batch if row_idx is not None else 1
        if self.A is not None:
            need = gptq_workspace_size(OP_ABS, None, 1, self.d_in, rows_for_ws, nb)
            if ws.numel() < need:
                ws = self._ws = _ws(need, self.device)
            gptq_abs_accumulate(self.A, X, dtype_code(X.dtype), n_rows, self.d_in, X.stride(0), row_idx, row_ptr,
                                nb, ws, ws.numel(), stream)
        gptq_hessian_accumulate(self.S, self.D, self.n, X, self.d_in, n_rows, X.stride(0), dtype_code(X.dtype),
                                row_idx, row_ptr, nb, ws, ws.numel(), stream)


class Prepared:
    def __init__(self, U, perm, info):
        self.U, self.perm, self.info = U, perm, info


def prepare(state: HessianState, params: GptqParams, ws: Optional[torch.Tensor] = None, stream=None,
            check: bool = True) -> Prepared:
    d, b, dev = state.d_in, state.batch, state.device
    U = torch.empty(b, d, d, dtype=torch.float32, device=dev)
    perm = torch.empty(b, d, dtype=torch.int32, device=dev) if params.act_order else None
    info = torch.empty(b, dtype=torch.int32, device=dev)
    need = gptq_workspace_size(OP_PREPARE, None, 1, d, 0, b)
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    gptq_prepare_hinv(state.S, state.D, state.n, d, b, params, U, perm, info, ws, ws.numel(), stream)
    out = Prepared(U, perm, info)
    if check:
        bad = info.cpu().numpy()
        if np.any(bad != 0):
            raise GptqError(ENOTPD, f"gptq_prepare_hinv (info={bad.tolist()})")
    return out


def quantize(W: torch.Tensor, prep: Prepared, params: GptqParams, want_q: bool = False,
             ws: Optional[torch.Tensor] = None, stream=None) -> Dict[str, torch.Tensor]:
    """W: (batch, d_out, d_in) or (d_out, d_in) tensor of fp32/fp16/bf16."""
    if W.dim() == 2:
        W = W.unsqueeze(0)
    b, d_out, d_in = W.shape
    dev = W.device
    ng = d_in // params.group_size
    codes = torch.empty(b, d_out, d_in, dtype=torch.uint8, device=dev)
    scales = torch.empty(b, d_out, ng, dtype=torch.int16, device=dev)
    zeros = torch.empty(b, d_out, ng, dtype=torch.uint8, device=dev)
    g_idx = torch.empty(b, d_in, dtype=torch.int32, device=dev)
    Q = torch.empty(b, d_out, d_in, dtype=torch.float32, device=dev) if want_q else None
    need = gptq_workspace_size(OP_QUANTIZE, params, d_out, d_in, 0, b)
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    gptq_quantize_layer(W, dtype_code(W.dtype), d_out, d_in, W.stride(1), b, prep.U, prep.perm, params, codes,
                        scales, zeros, g_idx, Q, ws, ws.numel(), stream)
    return dict(codes=codes, scales=scales, zeros=zeros, g_idx=g_idx, Q=Q)


def pack(codes: torch.Tensor, bits: int, stream=None) -> torch.Tensor:
    """Pack the last dimension of a uint8 code tensor (4-bit nibbles or a dense bit stream)."""
    shape = codes.shape
    rows = int(np.prod(shape[:-1]))
    cols = shape[-1]
    out = torch.empty(*shape[:-1], cols * bits // 8, dtype=torch.uint8, device=codes.device)
    if bits == 4:
        gptq_pack_int4(codes, rows, cols, out, stream)
    else:
        gptq_pack_bits(codes, rows, cols, bits, out, stream)
    return out


def pack_int4_permuted(codes: torch.Tensor, perm: torch.Tensor, stream=None) -> torch.Tensor:
    """4-bit packing of a (rows, cols) code matrix with its columns taken in the order perm."""
    rows, cols = codes.shape
    out = torch.empty(rows, cols // 2, dtype=torch.uint8, device=codes.device)
    gptq_pack_int4_permuted(codes, rows, cols, perm, out, stream)
    return out


def w4a16_matmul(X: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                 group_size: int, perm: Optional[torch.Tensor] = None, Y: Optional[torch.Tensor] = None,
                 ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Y = X Q^T (fp32) from the packed 4-bit weights; X is (M, d_in) fp16 or bf16."""
    M, d_in = X.shape
    d_out = qweight.shape[0]
    if Y is None:
        Y = torch.empty(M, d_out, dtype=torch.float32, device=X.device)
    need = gptq_workspace_size(OP_W4A16, None, d_out, d_in, M, 1)
    if ws is None or ws.numel() < need:
        ws = _ws(need, X.device)
    gptq_w4a16_matmul(X, dtype_code(X.dtype), M, d_in, X.stride(0), qweight, scales, zeros, perm, d_out,
                      group_size, Y, Y.stride(0), ws, ws.numel(), stream)
    return Y


def awq_search(W: torch.Tensor, state: HessianState, Xs: torch.Tensor, params: GptqParams,
               alphas: Sequence[float], entry: int = 0, stream=None) -> Dict[str, object]:
    """Candidate errors, the chosen index and its per-channel scales for one
    layer W (d_out, d_in), from the state's |x| sums and a token sample Xs."""
    d_out, d_in = W.shape
    dev = W.device
    err = torch.empty(len(alphas), dtype=torch.float64, device=dev)
    s = torch.empty(d_in, dtype=torch.float32, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    need = gptq_workspace_size(OP_AWQ_SEARCH, None, d_out, d_in, Xs.shape[0], len(alphas))
    ws = _ws(need, dev)
    gptq_awq_search(W, dtype_code(W.dtype), d_out, d_in, W.stride(0), state.A[entry], state.n[entry:entry + 1], Xs,
                    dtype_code(Xs.dtype), Xs.shape[0], Xs.stride(0), params, alphas, err, s, best, ws, ws.numel(),
                    stream)
    return dict(err=err, s=s, best=best)


def awq_apply(W: torch.Tensor, state: HessianState, s: torch.Tensor, entry: int = 0, stream=None) -> torch.Tensor:
    """Scale the state's Hessian in place and return W' = fp32(W s)."""
    d_out, d_in = W.shape
    Wp = torch.empty(d_out, d_in, dtype=torch.float32, device=W.device)
    gptq_awq_apply(state.S[entry], state.D[entry], d_in, s, W, dtype_code(W.dtype), d_out, W.stride(0), Wp, stream)
    return Wp


def layer_forward(X: torch.Tensor, Q: torch.Tensor, act: int, Y: Optional[torch.Tensor] = None,
                  ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Y = round(act(X Q^T)) in X's format; Q (d_out, d_in) fp32 dequantized weights."""
    n, d_in = X.shape
    d_out = Q.shape[0]
    if Y is None:
        Y = torch.empty(n, d_out, dtype=X.dtype, device=X.device)
    need = gptq_workspace_size(OP_FORWARD, None, d_out, d_in, n, 1)
    if ws is None or ws.numel() < need:
        ws = _ws(need, X.device)
    gptq_layer_forward(X, dtype_code(X.dtype), n, d_in, X.stride(0), Q, d_out, Q.stride(0), act, Y, Y.stride(0),
                       ws, ws.numel(), stream)
    return Y


def calibrate_block(chunks: Sequence[torch.Tensor], W1: torch.Tensor, W2: torch.Tensor, params: GptqParams,
                    act: int, stream=None) -> Dict[str, object]:
    """Sequential calibration of y = act(x W1^T) W2^T: layer 1 on the chunks,
    layer 2 on the rounded activations of the quantized layer 1, produced
    chunk by chunk with layer_forward."""
    d_in, h = W1.shape[1], W1.shape[0]
    st1 = HessianState(d_in, 1, W1.device)
    for X in chunks:
        st1.add(X, stream=stream)
    p1 = prepare(st1, params, stream=stream)
    r1 = quantize(W1, p1, params, want_q=True, stream=stream)
    del st1
    Q1 = r1["Q"][0]
    st2 = HessianState(h, 1, W1.device)
    n_max = max(X.shape[0] for X in chunks)
    ws = _ws(gptq_workspace_size(OP_FORWARD, None, h, d_in, n_max, 1), W1.device)
    for X in chunks:
        st2.add(layer_forward(X, Q1, act, ws=ws, stream=stream), stream=stream)
    del ws
    p2 = prepare(st2, params, stream=stream)
    r2 = quantize(W2, p2, params, want_q=True, stream=stream)
    return dict(layer1=r1, layer2=r2, prep1=p1, prep2=p2, state2=st2)
