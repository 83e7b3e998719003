"""Pins of the sequential block calibration oracle: activations and rounding
against closed forms and numpy's own fp16, the forward step against a loop,
and the chain against its pieces called by hand."""
import numpy as np
import pytest

import oracle as O


def _rng(i):
    return np.random.default_rng([960, i])


def test_activation_closed_forms():
    v = np.array([-2.0, -0.5, 0.0, 0.5, 3.0])
    np.testing.assert_array_equal(O.activation(v, O.ACT_RELU), [0.0, 0.0, 0.0, 0.5, 3.0])
    np.testing.assert_array_equal(O.activation(v, O.ACT_NONE), v)
    # SiLU: x sigmoid(x); SiLU(0) = 0, SiLU(x) - SiLU(-x) = x
    s = O.activation(v, O.ACT_SILU)
    assert s[2] == 0.0
    assert O.activation(np.array([3.0]), O.ACT_SILU)[0] - O.activation(np.array([-3.0]), O.ACT_SILU)[0] == pytest.approx(3.0, rel=1e-15)
    assert s[4] == pytest.approx(3.0 / (1.0 + np.exp(-3.0)), rel=1e-15)


def test_bf16_rounding_hand_values():
    """1 + 2^-8 is the midpoint between bf16 1 and 1 + 2^-7: ties to even
    gives 1; 1 + 3 * 2^-8 ties up to 1 + 2^-6; a value just above the first
    midpoint rounds up."""
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -(1.0 + 2.0 ** -8)])
    np.testing.assert_array_equal(O.round_to(v, "bf16"), [1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -1.0])
    w = _rng(1).standard_normal(1000)
    np.testing.assert_array_equal(O.round_to(w, "f16"), w.astype(np.float16).astype(np.float64))


def test_layer_forward_loop():
    r = _rng(2)
    X = r.standard_normal((3, 5))
    Q = r.standard_normal((4, 5))
    Y = O.layer_forward(X, Q, O.ACT_RELU, "f32")
    for t in range(3):
        for n in range(4):
            v = sum(float(X[t, k]) * float(Q[n, k]) for k in range(5))
            assert Y[t, n] == float(np.float32(max(v, 0.0)))


def test_chain_is_its_pieces():
    """Layer 2 is calibrated on the rounded activations of the quantized
    layer 1 (not of the float one): the pieces called by hand agree, and the
    float-layer-1 variant gives a different layer-2 Hessian."""
    r = _rng(3)
    X = (r.standard_normal((400, 128))).astype(np.float16).astype(np.float64)
    W1 = (r.standard_normal((256, 128)) * 0.05).astype(np.float16).astype(np.float64)
    W2 = (r.standard_normal((64, 256)) * 0.05).astype(np.float16).astype(np.float64)
    out = O.calibrate_block(X, W1, W2, O.ACT_SILU, "f16")
    S1, N1 = O.hessian_sum([X])
    r1 = O.gptq_layer(W1, S1, N1)
    np.testing.assert_array_equal(out["layer1"]["codes"], r1["codes"])
    X2 = O.round_to(O.activation(X @ r1["Q"].T, O.ACT_SILU), "f16")
    np.testing.assert_array_equal(out["X2"], X2)
    S2, N2 = O.hessian_sum([X2])
    np.testing.assert_array_equal(out["S2"], S2)
    r2 = O.gptq_layer(W2, S2, N2)
    np.testing.assert_array_equal(out["layer2"]["codes"], r2["codes"])
    X2f = O.round_to(O.activation(X @ W1.T, O.ACT_SILU), "f16")
    assert not np.array_equal(O.hessian_sum([X2f])[0], S2)
    # quantization error of the block stays small against its float output
    rel = np.linalg.norm(out["y_q"] - out["y_ref"]) / np.linalg.norm(out["y_ref"])
    assert 0.0 < rel < 0.2
