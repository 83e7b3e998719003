"""Sequential calibration of a two-layer block: float64 CPU oracle.

TEST INFRASTRUCTURE ONLY -- imported by ``tests/``, by the smoke check and by
the benchmark's ``cpu_baseline`` leg, never by the product path.  It shares no
code with the HIP library.

What it computes.  "3. 模型量化技术(下)", section "GPTQ：基于二阶信息的后训练量化",
pseudocode: for each layer, collect that layer's inputs, build H from them,
quantize the layer.  Readings (the pages fix neither the block nor where the
later layers' inputs come from):

R24 block: y = act(x W1^T) W2^T, two linear layers with an elementwise
    activation between them (none, ReLU or SiLU x / (1 + e^-x)).
R25 sequence: layer 1 is calibrated on the block's inputs; layer 2 on
    act(X Q1^T), the output of the already quantized layer 1 (Q1 its
    dequantized weights), rounded to the activations' 16-bit format
    (round to nearest even), as the next layer would receive it.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .gptq import gptq_layer, hessian_sum

__all__ = ["ACT_NONE", "ACT_RELU", "ACT_SILU", "activation", "round_to", "layer_forward", "calibrate_block"]

ACT_NONE, ACT_RELU, ACT_SILU = 0, 1, 2


def activation(v: np.ndarray, act: int) -> np.ndarray:
    """R24, in float64."""
    v = np.asarray(v, dtype=np.float64)
    if act == ACT_NONE:
        return v
    if act == ACT_RELU:
        return np.maximum(v, 0.0)
    if act == ACT_SILU:
        return v / (1.0 + np.exp(-v))
    raise ValueError(act)


def round_to(v: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to fp16 / bf16 (nearest, ties to even) and back.

    bf16: the float32 value's top 16 bits after adding 0x7FFF plus the lowest
    kept bit (nearest-even on the 16 dropped bits); the float64 -> float32
    step rounds first, which can only matter at exact double-rounding ties."""
    if dtype == "f32":
        return np.asarray(v, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(v, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def layer_forward(X: np.ndarray, Q: np.ndarray, act: int, dtype: str) -> np.ndarray:
    """R25: round(act(X Q^T)) to the activation format."""
    return round_to(activation(np.asarray(X, dtype=np.float64) @ np.asarray(Q, dtype=np.float64).T, act), dtype)


def calibrate_block(X: np.ndarray, W1: np.ndarray, W2: np.ndarray, act: int, dtype: str,
                    **gptq_kw) -> Dict[str, object]:
    """R25: quantize W1 on X, form layer 2's inputs from the quantized layer 1,
    quantize W2 on them.  Returns both layers' results, X2 and the block's
    output with quantized and with float weights."""
    S1, N1 = hessian_sum([X])
    r1 = gptq_layer(W1, S1, N1, **gptq_kw)
    X2 = layer_forward(X, r1["Q"], act, dtype)
    S2, N2 = hessian_sum([X2])
    r2 = gptq_layer(W2, S2, N2, **gptq_kw)
    Xf = np.asarray(X, dtype=np.float64)
    y_ref = activation(Xf @ np.asarray(W1, dtype=np.float64).T, act) @ np.asarray(W2, dtype=np.float64).T
    y_q = X2 @ r2["Q"].T
    return dict(layer1=r1, layer2=r2, X2=X2, S2=S2, y_ref=y_ref, y_q=y_q)
