"""Pins of the AWQ pre-pass oracle: brute-force statistics and errors, the
exactness of the channel scaling, its reduction to plain rounding at alpha = 0,
and GPTQ's invariance under a uniform power-of-two scaling."""
import numpy as np
import pytest

import oracle as O

F32 = np.float32


def _rng(i):
    return np.random.default_rng([950, i])


def _layer(rows=12, d=256, n=300, seed=1, outliers=(5, 77, 200)):
    r = _rng(seed)
    X = r.standard_normal((n, d))
    X[:, list(outliers)] *= 30.0
    X = X.astype(np.float16).astype(np.float64)           # 16-bit activations, exact in float64
    W = (r.standard_normal((rows, d)) * 0.02).astype(np.float16).astype(np.float64)
    return X, W


def test_channel_abs_mean_brute_force():
    X = _rng(2).standard_normal((9, 6))
    a = O.channel_abs_mean([X[:4], X[4:]])
    for c in range(6):
        assert a[c] == pytest.approx(sum(abs(float(X[t, c])) for t in range(9)) / 9, rel=1e-15)


def test_scales_closed_forms():
    a = np.array([4.0, 0.25, 0.0, 9.0])
    np.testing.assert_array_equal(O.awq_scales(a, 0.0), np.ones(4, F32))
    np.testing.assert_array_equal(O.awq_scales(a, 0.5), np.array([2.0, 0.5, 1e-3, 3.0], F32))
    np.testing.assert_array_equal(O.awq_scales(a, 1.0), np.array([4.0, 0.25, 1e-6, 9.0], F32))


def test_alpha_zero_is_plain_group_rounding():
    """s = 1: the candidate's error is the error of the path's group-wise
    round-to-nearest (catches a scale applied twice or not divided back)."""
    X, W = _layer(seed=3)
    e0 = O.awq_rtn_error(W, X, np.ones(256, F32))
    for sym in (False, True):
        Q = O.rtn_quantize(W, 4, 128, sym=sym)["Q"]
        want = float(np.sum(((W - Q) @ X.T) ** 2))
        assert O.awq_rtn_error(W, X, np.ones(256, F32), sym=sym) == pytest.approx(want, rel=1e-12)
    assert e0 > 0


def test_error_brute_force_tiny():
    """Two rows, eight channels, groups of four, explicit loops for the
    scaled rounding and the output error."""
    r = _rng(4)
    W = (r.standard_normal((2, 8)) * 0.1).astype(F32).astype(np.float64)
    Xs = r.standard_normal((3, 8))
    s = np.array([1.5, 0.5, 2.0, 1.0, 3.0, 0.25, 1.0, 4.0], F32)
    Q = np.zeros((2, 8))
    for i in range(2):
        for g0 in (0, 4):
            v = [F32(W[i, c]) * s[c] for c in range(g0, g0 + 4)]
            lo, hi = min(min(v), F32(0)), max(max(v), F32(0))
            sc = float(np.float16((hi - lo) / F32(15)))
            z = min(max(round(float(-lo / F32(sc))), 0), 15)   # no exact .5 ties in this draw
            for k, c in enumerate(range(g0, g0 + 4)):
                q = min(max(round(float(v[k] / F32(sc))) + z, 0), 15)
                Q[i, c] = float(F32(F32(sc * (q - z)) / s[c]))
    want = sum(sum((W[i, c] - Q[i, c]) * Xs[t, c] for c in range(8)) ** 2 for i in range(2) for t in range(3))
    assert O.awq_rtn_error(W, Xs, s, group_size=4) == pytest.approx(want, rel=1e-12)


def test_scaled_hessian_is_the_hessian_of_the_scaled_inputs():
    """S' = S / (s s^T) equals (X diag(1/s))^T (X diag(1/s)) (catches s_i^2 or
    a product instead of a quotient)."""
    X, W = _layer(seed=5)
    s = O.awq_scales(O.channel_abs_mean([X]), 0.5)
    S, _ = O.hessian_sum([X])
    Wp, Sp = O.awq_apply(W, S, s)
    Xp = X / s.astype(np.float64)[None, :]
    np.testing.assert_allclose(Sp, Xp.T @ Xp, rtol=1e-12, atol=1e-12)
    # the layer's output is unchanged before rounding: (X / s) (W s)^T = X W^T
    np.testing.assert_allclose(Xp @ Wp.T, X @ W.T, rtol=0, atol=1e-6)   # W' carries one fp32 rounding


def test_uniform_power_of_two_scaling_leaves_gptq_codes_unchanged():
    X, W = _layer(rows=16, d=256, n=500, seed=6)
    S, N = O.hessian_sum([X])
    base = O.gptq_layer(W, S, N)
    r = O.awq_gptq_layer(W, S, N, np.full(256, 4.0, F32))
    np.testing.assert_array_equal(r["codes"], base["codes"])
    np.testing.assert_array_equal(r["scales"], 4.0 * base["scales"])
    np.testing.assert_allclose(r["Q_eff"], base["Q"], rtol=0, atol=0)


def test_search_prefers_scaling_when_channels_are_outliers():
    """With a few channels 30x louder the search moves away from alpha = 0 and
    lowers the output error (the pages' claim for activation-aware scaling);
    alpha = 0 stays a candidate, so the search is never worse than rounding."""
    X, W = _layer(rows=32, d=512, n=400, seed=7, outliers=(3, 100, 257, 400, 511))
    a = O.channel_abs_mean([X])
    alphas = [i / 10 for i in range(10)]
    res = O.awq_search(W, X[:256], a, alphas)
    assert res["best"] > 0
    assert res["errors"][res["best"]] < 0.9 * res["errors"][0]
    assert res["errors"][res["best"]] == res["errors"].min()
    np.testing.assert_array_equal(res["s"], O.awq_scales(a, res["alpha"]))
