"""Pins of the float64 oracle against facts fixed by the pages and by
mathematics (closed forms, brute force, worked examples), never against a
retyping of the oracle's own formulas.

Each test names the mistake it is there to catch.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _rng(seed):
    return np.random.default_rng([900, seed])


def _correlated_x(n, d, seed, strength=0.8):
    r = _rng(seed)
    A = np.eye(d) + strength * r.standard_normal((d, d)) / math.sqrt(d)
    return r.standard_normal((n, d)) @ A


# ---------------------------------------------------------------- Hessian
def test_hessian_sum_matches_outer_product_loop():
    """S = sum_t x_t x_t^T by an explicit per-token, per-entry loop (brute force)."""
    X = _rng(1).standard_normal((7, 5))
    S, n = O.hessian_sum([X[:3], X[3:]])
    brute = [[0.0] * 5 for _ in range(5)]
    for t in range(7):
        for i in range(5):
            for j in range(5):
                brute[i][j] += float(X[t, i]) * float(X[t, j])
    assert n == 7
    np.testing.assert_allclose(S, np.array(brute), rtol=1e-14, atol=1e-14)


def test_hessian_is_second_derivative_of_mean_output_error():
    """H0 must be the Hessian of the per-token output error
    L(w) = (1/N) sum_t ((w - w0) . x_t)^2  (the loss whose second derivative the
    pages call H).  Central second differences of a quadratic are exact up to
    rounding, so this catches a dropped factor 2 or a missing 1/N."""
    X = _rng(2).standard_normal((40, 4))
    S, n = O.hessian_sum([X])
    H = O.hessian(S, n)
    w0 = _rng(3).standard_normal(4)

    def loss(w):
        r = X @ (w - w0)
        return float(np.sum(r * r)) / X.shape[0]

    h = 0.5
    I = np.eye(4)
    fd = np.zeros((4, 4))
    for i in range(4):
        for j in range(4):
            fd[i, j] = (loss(w0 + h * I[i] + h * I[j]) - loss(w0 + h * I[i] - h * I[j])
                        - loss(w0 - h * I[i] + h * I[j]) + loss(w0 - h * I[i] - h * I[j])) / (4 * h * h)
    np.testing.assert_allclose(H, fd, rtol=1e-12, atol=1e-12)


def test_chunk_invariance_of_hessian():
    X = _rng(4).standard_normal((4096, 48))
    S1, n1 = O.hessian_sum([X])
    S16, n16 = O.hessian_sum(np.array_split(X, 16))
    assert n1 == n16 == 4096
    assert np.linalg.norm(S1 - S16) / np.linalg.norm(S1) < 1e-13


# ---------------------------------------------------------------- damping / order / factor
def test_damping_closed_form():
    """diag(1..d): mean = (d+1)/2, so lam = 0.01 (d+1)/2."""
    d = 9
    H0 = np.diag(np.arange(1.0, d + 1))
    lam, Hd = O.damping(H0, 0.01)
    assert lam == pytest.approx(0.01 * (d + 1) / 2, rel=1e-15)
    np.testing.assert_array_equal(np.diag(Hd), np.arange(1.0, d + 1) + lam)


def test_act_order_descending_with_stable_ties():
    H0 = np.diag([3.0, 5.0, 1.0, 5.0, 0.0, 3.0])
    assert O.act_order_perm(H0).tolist() == [1, 3, 0, 5, 2, 4]


def test_inverse_factor_definition():
    """U upper, positive diagonal, and U^T U is the inverse of Hd."""
    X = _correlated_x(300, 24, 5)
    S, n = O.hessian_sum([X])
    _, Hd = O.damping(O.hessian(S, n), 0.01)
    U = O.inverse_factor(Hd)
    assert np.all(np.tril(U, -1) == 0)
    assert np.all(np.diag(U) > 0)
    np.testing.assert_allclose(U.T @ U @ Hd, np.eye(24), atol=1e-10)


def test_inverse_factor_2x2_closed_form():
    """Hd = [[a, b], [b, c]]: U00 = sqrt(c/det), U01 = -b/(det U00), U11 = 1/sqrt(c)."""
    a, b, c = 3.0, 1.2, 2.0
    det = a * c - b * b
    U = O.inverse_factor(np.array([[a, b], [b, c]]))
    u00 = math.sqrt(c / det)
    np.testing.assert_allclose(U, [[u00, -b / (det * u00)], [0.0, 1 / math.sqrt(c)]], rtol=1e-14)


def test_inverse_factor_diagonal():
    h = np.array([0.5, 2.0, 9.0, 1e3])
    np.testing.assert_allclose(O.inverse_factor(np.diag(h)), np.diag(1 / np.sqrt(h)), rtol=1e-15)


# ---------------------------------------------------------------- quantizer
def test_quantizer_worked_example():
    """Min-max mapping of [min, max] onto [0, 15] (the linear range mapping of
    the Min-Max section), worked by hand: range 0.75 -> 0.75/15 = 0.05 ->
    fp16 0.049987793 (0x2A66); zero = round(0.3/s) = 6; codes of
    [-0.3, 0, 0.15, 0.45] are round(w/s) + 6 = [0, 6, 9, 15]."""
    w = np.array([[-0.3, 0.0, 0.15, 0.45]])
    s, z = O.group_params(w, 15)
    assert np.float16(s[0]).view(np.uint16) == 0x2A66
    assert z[0] == 6
    q, dq = O.quantize_values(w[0], np.repeat(s, 4), np.repeat(z, 4), 15)
    assert q.tolist() == [0, 6, 9, 15]
    assert dq[1] == 0.0
    np.testing.assert_allclose(dq, float(s[0]) * (np.array([0, 6, 9, 15]) - 6), rtol=0)


def test_quantizer_range_includes_zero_and_degenerate_group():
    """All-positive group: xmin is taken as 0, so z = 0; all-zero group: s = 1,
    every code 0 and dq exactly 0."""
    s, z = O.group_params(np.array([[0.2, 0.4, 0.8, 0.6]]), 15)
    assert z[0] == 0
    assert float(s[0]) == float(np.float16(F32(0.8) / F32(15)))
    s0, z0 = O.group_params(np.zeros((1, 8)), 15)
    assert s0[0] == 1.0 and z0[0] == 0
    q, dq = O.quantize_values(np.zeros(8), np.repeat(s0, 8), np.repeat(z0, 8), 15)
    assert q.tolist() == [0] * 8 and np.all(dq == 0.0)


def test_quantizer_half_to_even_and_clamp():
    s = np.array([F32(0.25)])
    z = np.array([3])
    w = np.array([0.625, 0.875, 100.0, -100.0])      # /s = 2.5, 3.5, 400, -400
    q, _ = O.quantize_values(w, np.repeat(s, 4), np.repeat(z, 4), 15)
    assert q.tolist() == [2 + 3, 4 + 3, 15, 0]


def test_quantizer_grid_roundtrip_and_half_step_bound():
    r = _rng(6)
    for bits in (3, 4):
        maxq = (1 << bits) - 1
        W = r.normal(0, 0.02, (50, 128))
        s, z = O.group_params(W, maxq)
        q, dq = O.quantize_values(W, s[:, None], z[:, None], maxq)
        assert np.all(np.abs(W - dq) <= s[:, None].astype(np.float64) * (0.5 + 1e-6))
        # values already on the grid come back unchanged
        q2, dq2 = O.quantize_values(dq, s[:, None], z[:, None], maxq)
        np.testing.assert_array_equal(q2, q)
        np.testing.assert_array_equal(dq2, dq)


def _listing_sym_rtn(W, bits, g):
    """The symmetric rule of the GPTQ listing on the ipipp page (scale from
    the largest magnitude over 2^(b-1) - 1, round, clamp to the signed range),
    applied per group of g columns as its text says frameworks do; written
    with signed codes and no zero point."""
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    rows, d = W.shape
    signed = np.zeros((rows, d), dtype=np.int64)
    scale = np.zeros((rows, d // g), dtype=F32)
    for j in range(d // g):
        blk = W[:, j * g:(j + 1) * g].astype(F32)
        amax = np.abs(blk).max(axis=1)
        sc = (amax / F32(hi)).astype(np.float16).astype(F32)
        sc[sc == 0] = 1.0
        scale[:, j] = sc
        signed[:, j * g:(j + 1) * g] = np.clip(np.rint(blk / sc[:, None]), lo, hi)
    return signed, scale


def test_sym_quantizer_worked_example():
    """Largest magnitude 0.7 -> s = 0.7/7 = 0.1 -> fp16 0.099975586 (0x2E66);
    w/s for [-0.35, 0, 0.1, 0.7] is [-3.5009, 0, 1.0002, 7.0017], rounded
    [-4, 0, 1, 7]; stored with the fixed zero 8 as [4, 8, 9, 15].  Catches an
    asymmetric range or a zero that moves with the data."""
    w = np.array([[-0.35, 0.0, 0.1, 0.7]])
    s, z = O.group_params(w, 15, sym=True)
    assert np.float16(s[0]).view(np.uint16) == 0x2E66
    assert z[0] == 8
    q, dq = O.quantize_values(w[0], np.repeat(s, 4), np.repeat(z, 4), 15)
    assert q.tolist() == [4, 8, 9, 15]
    np.testing.assert_allclose(dq, float(s[0]) * np.array([-4, 0, 1, 7]), rtol=0)


def test_sym_degenerate_and_overflowing_groups():
    """All-zero group: s = 1, every code the zero, dq = 0.  A magnitude past
    fp16's range saturates the scale at 65504 like the asymmetric rule."""
    s0, z0 = O.group_params(np.zeros((1, 8)), 15, sym=True)
    assert s0[0] == 1.0 and z0[0] == 8
    s1, z1 = O.group_params(np.array([[-1e9, 3.0]]), 7, sym=True)
    assert s1[0] == 65504.0 and z1[0] == 4


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_sym_rtn_matches_listing_rule(bits):
    """With no feedback (diagonal H) symmetric GPTQ is the listing's rule per
    group, bit for bit: signed code = stored code - 2^(b-1), Q = s * signed."""
    W = _rng(20 + bits).normal(0, 0.02, (24, 256))
    W[3, 5] = 0.3                                           # an outlier sets one group's scale
    W[7, 128:] = 0.0                                        # an all-zero group
    signed, scale = _listing_sym_rtn(W, bits, 64)
    _, Hd = O.damping(np.diag(_rng(30).uniform(0.5, 4.0, 256)), 0.01)
    r = O.gptq_quantize(W, O.inverse_factor(Hd), bits=bits, group_size=64, block_size=128, sym=True)
    np.testing.assert_array_equal(r["codes"] - (1 << (bits - 1)), signed)
    np.testing.assert_array_equal(r["scales"], scale)
    np.testing.assert_array_equal(r["zeros"], np.full(scale.shape, 1 << (bits - 1)))
    np.testing.assert_array_equal(r["Q"], signed * np.repeat(scale, 64, axis=1).astype(np.float64))


def test_sym_grid_is_odd_symmetric():
    """Negating the weights negates the symmetric round-to-nearest result
    exactly, and a group's largest magnitude lands on code 2^b - 1 or 1 (the
    end of the grid): a wrong divisor, 2^(b-1) or 2^b - 1, breaks the second."""
    W = _rng(25).normal(0, 0.02, (16, 256))
    a = O.rtn_quantize(W, sym=True)
    b = O.rtn_quantize(-W, sym=True)
    np.testing.assert_array_equal(b["Q"], -a["Q"])
    for j in range(2):
        blk = W[:, j * 128:(j + 1) * 128]
        at = np.abs(blk).argmax(axis=1)
        c = a["codes"][np.arange(16), j * 128 + at]
        assert np.all(np.where(blk[np.arange(16), at] > 0, c == 15, c == 1))


def test_sym_gptq_feedback_and_margins():
    """On a correlated layer symmetric GPTQ still beats symmetric rounding, its
    codes stay in [0, 2^b - 1], and decision_margins reports no zero margin."""
    X, S, N, W = _layer_inputs(48, 256, 2048, 84)
    g = O.gptq_layer(W, S, N, sym=True)
    r = O.rtn_quantize(W, sym=True)
    assert O.recon_error(W, g["Q"], S) < 0.8 * O.recon_error(W, r["Q"], S)
    assert g["codes"].min() >= 0 and g["codes"].max() <= 15
    m = O.decision_margins(g, 4, 128, sym=True)
    assert np.all(np.isinf(m["zero"])) and np.all(m["scale"] >= 0)


# ---------------------------------------------------------------- feedback
def _tiny_problem(rows, d, seed, n=64, damp=0.01):
    X = _correlated_x(n, d, seed, strength=1.5)
    S, N = O.hessian_sum([X])
    H0 = O.hessian(S, N)
    lam, Hd = O.damping(H0, damp)
    W = _rng(seed + 100).normal(0, 0.02, (rows, d))
    return X, N, lam, Hd, W


def _lstsq_remaining(W0_row, dq_fixed, k, X, N, lam):
    """argmin over the free columns of ||(w - w0) Xt^T||^2 with columns 0..k
    fixed to dq, where Xt = [X; sqrt(N lam / 2) I] so that 2 Xt^T Xt / N = Hd.
    Solved with an SVD least-squares routine: independent of Cholesky and of
    any inverse."""
    d = W0_row.shape[0]
    Xt = np.vstack([X, math.sqrt(N * lam / 2.0) * np.eye(d)])
    P = slice(0, k + 1)
    F = slice(k + 1, d)
    rhs = -Xt[:, P] @ (dq_fixed - W0_row[P])
    delta, *_ = np.linalg.lstsq(Xt[:, F], rhs, rcond=None)
    return W0_row[F] + delta


@pytest.mark.parametrize("g", [4, 8])
def test_feedback_equals_least_squares_optimum(g):
    """After each column k the still-free columns must equal the least-squares
    optimum given the quantized ones (the OBS property the pages' update
    implements).  Catches a wrong sign, a wrong row of U, a transposed factor,
    or the static inverse."""
    rows, d = 4, 8
    X, N, lam, Hd, W = _tiny_problem(rows, d, 10 + g)
    U = O.inverse_factor(Hd)
    r = O.gptq_quantize(W, U, bits=3, group_size=g, block_size=1, trace=True)
    for k in range(d - 1):
        snap = r["trace"][k]
        for row in range(rows):
            want = _lstsq_remaining(W[row], r["Q"][row, :k + 1], k, X, N, lam)
            got = snap[row, k + 1:]
            np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-12 * np.abs(W).max())


def _static_inverse_rows(Hd):
    """The listings' single inverse as a factor the column loop can take:
    V = triu(A) / sqrt(diag A), A = Hd^-1, so that e = (w - dq) / V[k, k] and
    e V[k, j] = (w - dq) A[k, j] / A[k, k], the update the listings print with
    an inverse that is never updated."""
    A = np.linalg.inv(Hd)
    return np.triu(A) / np.sqrt(np.diag(A))[:, None]


def test_static_inverse_fails_least_squares_pin():
    """Negative control: feedback through the rows of the static inverse (the
    listings read literally) is the optimum only for the first column; on a
    correlated layer the pin rejects it at every later column."""
    rows, d = 4, 8
    X, N, lam, Hd, W = _tiny_problem(rows, d, 31)
    r = O.gptq_quantize(W, _static_inverse_rows(Hd), bits=3, group_size=8, block_size=1, trace=True)
    # the first column's update is exact in both forms
    want0 = _lstsq_remaining(W[0], r["trace"][0][0, :1], 0, X, N, lam)
    np.testing.assert_allclose(r["trace"][0][0, 1:], want0, rtol=1e-9)
    failed = 0
    for k in range(1, d - 1):
        snap = r["trace"][k]
        row_fail = False
        for row in range(rows):
            dq = snap[row, :k + 1]
            want = _lstsq_remaining(W[row], dq, k, X, N, lam)
            if not np.allclose(snap[row, k + 1:], want, rtol=1e-6, atol=0):
                row_fail = True
        failed += row_fail
    assert failed == d - 2


def test_wrong_factor_row_fails_least_squares_pin():
    """Negative control: one row of U taken from the wrong position (rows 2
    and 5 swapped, upper part kept) breaks the optimum from the first column
    whose feedback uses it."""
    rows, d = 4, 8
    X, N, lam, Hd, W = _tiny_problem(rows, d, 32)
    U = O.inverse_factor(Hd)
    V = U.copy()
    V[2, 3:], V[5, 3:] = U[5, 3:], U[2, 3:]
    V = np.triu(V)
    r = O.gptq_quantize(W, V, bits=3, group_size=8, block_size=1, trace=True)
    for k in range(d - 1):
        snap = r["trace"][k]
        ok = all(np.allclose(snap[row, k + 1:], _lstsq_remaining(W[row], snap[row, :k + 1], k, X, N, lam),
                             rtol=1e-6, atol=0) for row in range(rows))
        assert ok == (k < 2), k


def test_two_column_closed_form():
    """After column 0: w1' = w1 + (w0 - q0) Hd01 / Hd11."""
    X, N, lam, Hd, W = _tiny_problem(3, 2, 40)
    U = O.inverse_factor(Hd)
    r = O.gptq_quantize(W, U, bits=4, group_size=2, block_size=1, trace=True)
    w1p = r["trace"][0][:, 1]
    want = W[:, 1] + (W[:, 0] - r["Q"][:, 0]) * Hd[0, 1] / Hd[1, 1]
    np.testing.assert_allclose(w1p, want, rtol=1e-12)


def test_diagonal_hessian_reduces_to_rtn_bitwise():
    """H = I (or any diagonal H) gives no feedback: GPTQ must equal group-wise
    round-to-nearest bit for bit."""
    W = _rng(7).normal(0, 0.02, (32, 256))
    for h in (np.ones(256), _rng(8).uniform(0.1, 10.0, 256)):
        _, Hd = O.damping(np.diag(h), 0.01)
        r = O.gptq_quantize(W, O.inverse_factor(Hd), bits=4, group_size=128, block_size=128)
        t = O.rtn_quantize(W, bits=4, group_size=128)
        for key in ("codes", "scales", "zeros", "Q"):
            np.testing.assert_array_equal(r[key], t[key])


def _layer_inputs(rows, d, n, seed):
    X = _correlated_x(n, d, seed)
    S, N = O.hessian_sum([X])
    W = _rng(seed + 1).normal(0, 0.02, (rows, d))
    return X, S, N, W


def test_elimination_form_equals_cholesky_form():
    cfg = synth.CONFIGS["tiny"]
    cases = [(synth.to_f64(synth.weights(cfg), "f32"),
              O.hessian_sum([synth.to_f64(c, "f32") for c in synth.x_chunks(cfg)]))]
    for seed in (60, 61):
        _, S, N, W = _layer_inputs(64, 512, 2048, seed)
        cases.append((W, (S, N)))
    for W, (S, N) in cases:
        _, Hd = O.damping(O.hessian(S, N), 0.01)
        a = O.gptq_quantize(W, O.inverse_factor(Hd), bits=4, group_size=128, block_size=1)
        b = O.gptq_quantize_elimination(W, Hd, bits=4, group_size=128)
        np.testing.assert_array_equal(a["codes"], b["codes"])
        np.testing.assert_allclose(a["pre"], b["pre"], rtol=1e-10, atol=1e-10 * np.abs(W).max())


def test_block_size_invariance():
    _, S, N, W = _layer_inputs(48, 512, 2048, 70)
    _, Hd = O.damping(O.hessian(S, N), 0.01)
    U = O.inverse_factor(Hd)
    outs = [O.gptq_quantize(W, U, bits=4, group_size=128, block_size=B) for B in (1, 32, 128)]
    for o in outs[1:]:
        np.testing.assert_array_equal(o["codes"], outs[0]["codes"])
        np.testing.assert_allclose(o["pre"], outs[0]["pre"], rtol=1e-12, atol=1e-15)


def test_group_256_block_128_and_group_64_block_128():
    _, S, N, W = _layer_inputs(16, 512, 2048, 71)
    _, Hd = O.damping(O.hessian(S, N), 0.01)
    U = O.inverse_factor(Hd)
    for g in (64, 256):
        a = O.gptq_quantize(W, U, bits=4, group_size=g, block_size=1)
        b = O.gptq_quantize(W, U, bits=4, group_size=g, block_size=128)
        np.testing.assert_array_equal(a["codes"], b["codes"])


def test_x_scale_invariance_and_row_independence():
    X, S, N, W = _layer_inputs(40, 256, 1024, 80)
    base = O.gptq_layer(W, S, N)
    S2, N2 = O.hessian_sum([3.7 * X])
    scaled = O.gptq_layer(W, S2, N2)
    np.testing.assert_array_equal(base["codes"], scaled["codes"])
    top = O.gptq_layer(W[:17], S, N)
    bot = O.gptq_layer(W[17:], S, N)
    np.testing.assert_array_equal(np.vstack([top["codes"], bot["codes"]]), base["codes"])
    np.testing.assert_array_equal(np.vstack([top["scales"], bot["scales"]]), base["scales"])


def test_act_order_identity_perm_is_natural_order_and_gidx_roundtrip():
    X, S, N, W = _layer_inputs(20, 256, 1024, 81)
    nat = O.gptq_layer(W, S, N)
    ident = O.gptq_layer(W, S, N, perm=np.arange(256))
    for key in ("codes", "scales", "zeros", "Q"):
        np.testing.assert_array_equal(nat[key], ident[key])
    Xs = X * np.linspace(0.2, 3.0, 256)[None, :]
    S3, N3 = O.hessian_sum([Xs])
    ao = O.gptq_layer(W, S3, N3, act_order=True)
    assert ao["perm"].tolist() == np.argsort(-np.diag(S3), kind="stable").tolist()
    # dequantizing the original-order codes through g_idx gives back Q
    np.testing.assert_array_equal(O.dequantize(ao["codes"], ao["scales"], ao["zeros"], ao["g_idx"]), ao["Q"])
    # every group holds exactly g consecutive positions of the quantization order
    assert np.bincount(ao["g_idx"]).tolist() == [128, 128]


def test_act_order_hand_example():
    """Four columns, g = 2: importance order 2, 0, 3, 1 puts columns {2, 0} in
    group 0 and {3, 1} in group 1."""
    S = np.diag([2.0, 0.5, 9.0, 1.0])
    W = _rng(9).normal(0, 0.02, (3, 4))
    r = O.gptq_layer(W, S, 1, group_size=2, block_size=2, act_order=True)
    assert r["perm"].tolist() == [2, 0, 3, 1]
    assert r["g_idx"].tolist() == [0, 1, 0, 1]
    # a diagonal H has no feedback: group 0 is RTN of columns (2, 0)
    t = O.rtn_quantize(W[:, [2, 0, 3, 1]], bits=4, group_size=2)
    np.testing.assert_array_equal(r["codes"][:, [2, 0, 3, 1]], t["codes"])


def test_gptq_not_worse_than_rtn_on_correlated_layer():
    """Soft quality check (GPTQ is greedy): it should beat plain rounding on
    the output-error objective."""
    X, S, N, W = _layer_inputs(64, 512, 4096, 82)
    g = O.gptq_layer(W, S, N)
    r = O.rtn_quantize(W)
    assert O.recon_error(W, g["Q"], S) < 0.8 * O.recon_error(W, r["Q"], S)


def test_reconstruction_identity():
    X, S, N, W = _layer_inputs(16, 128, 500, 83)
    g = O.gptq_layer(W, S, N)
    a = O.recon_error(W, g["Q"], S)
    b = O.recon_error_direct(W, g["Q"], X)
    assert a == pytest.approx(b, rel=1e-11)


# ---------------------------------------------------------------- static groups
def test_static_groups_diagonal_h_is_rtn_of_original_columns():
    """No feedback (diagonal H): static groups give group-wise rounding of the
    ORIGINAL columns even under act-order, whereas dynamic groups round the
    permuted columns.  Catches groups formed in quantization order or
    parameters looked up through the wrong index."""
    W = _rng(40).normal(0, 0.02, (20, 256))
    h = _rng(41).uniform(0.5, 5.0, 256)                     # a non-trivial act-order permutation
    S = np.diag(h)
    for sym in (False, True):
        t = O.rtn_quantize(W, bits=4, group_size=64, sym=sym)
        r = O.gptq_layer(W, S, 1, group_size=64, act_order=True, static_groups=True, sym=sym)
        assert not np.array_equal(r["perm"], np.arange(256))
        np.testing.assert_array_equal(r["g_idx"], np.arange(256) // 64)
        for key in ("codes", "scales", "zeros", "Q"):
            np.testing.assert_array_equal(r[key], t[key])
        dyn = O.gptq_layer(W, S, 1, group_size=64, act_order=True, sym=sym)
        assert not np.array_equal(dyn["codes"], t["codes"])


def _brute_static_gptq(W, Hd, perm, bits, g):
    """Column loop written from the OBS form with a fresh inverse of the
    still-unquantized sub-Hessian at every step (no factor, no blocks), with
    every group's scale and zero taken from the weights before the loop."""
    maxq = (1 << bits) - 1
    W0 = np.asarray(W, dtype=np.float64)
    W = W0.copy()
    rows, d = W.shape
    codes = np.zeros((rows, d), dtype=np.int64)
    for k in range(d):
        c = perm[k]
        grp = (c // g) * g
        blk = W0[:, grp:grp + g].astype(F32)
        lo = np.minimum(blk.min(axis=1), F32(0))
        hi = np.maximum(blk.max(axis=1), F32(0))
        sc = ((hi - lo) / F32(maxq)).astype(np.float16).astype(F32)
        sc[sc == 0] = 1.0
        z = np.clip(np.rint(-lo / sc), 0, maxq)
        q = np.clip(np.rint(W[:, c].astype(F32) / sc) + z, 0, maxq)
        dq = sc.astype(np.float64) * (q - z)
        codes[:, c] = q
        rest = perm[k:]
        F = np.linalg.inv(Hd[np.ix_(rest, rest)])
        e = (W[:, c] - dq) / F[0, 0]
        W[:, rest[1:]] -= np.outer(e, F[0, 1:])
        W[:, c] = dq
    return codes


def test_static_groups_match_brute_force_obs_loop():
    """Act-order with static groups against the loop above on a 6 x 16 layer:
    catches parameters taken after feedback, a wrong group of a permuted
    column, or a feedback term that skips columns."""
    X, S, N, W = _layer_inputs(6, 16, 200, 85)
    W[2, :4] *= 8.0                                        # a wide group
    r = O.gptq_layer(W, S, N, group_size=4, block_size=4, act_order=True, static_groups=True)
    _, Hd = O.damping(O.hessian(S, N), 0.01)
    want = _brute_static_gptq(W, Hd, r["perm"], 4, 4)
    np.testing.assert_array_equal(r["codes"], want)


def _brute_dynamic_gptq(W, Hd, perm, bits, g, params_from="current"):
    """Column loop from its definition, for dynamic groups: at every column a
    fresh inverse of the sub-Hessian of the columns not yet quantized (no
    factor, no blocks); a group's scale and zero are set when its first
    column (in quantization order) is reached, from the values its columns
    hold at that moment.  ``params_from="original"`` takes them from the
    weights before any feedback instead (a wrong timing, kept to show that
    the pin tells the two apart)."""
    maxq = (1 << bits) - 1
    W0 = np.asarray(W, dtype=np.float64)
    W = W0.copy()
    rows, d = W.shape
    codes = np.zeros((rows, d), dtype=np.int64)
    scales = np.zeros((rows, d // g), dtype=F32)
    zeros = np.zeros((rows, d // g), dtype=np.int64)
    for k in range(d):
        c = perm[k]
        if k % g == 0:
            src = W if params_from == "current" else W0
            blk = src[:, perm[k:k + g]].astype(F32)
            lo = np.minimum(blk.min(axis=1), F32(0))
            hi = np.maximum(blk.max(axis=1), F32(0))
            sc = ((hi - lo) / F32(maxq)).astype(np.float16).astype(F32)
            sc[sc == 0] = 1.0
            z = np.clip(np.rint(-lo / sc), 0, maxq)
            scales[:, k // g], zeros[:, k // g] = sc, z
        q = np.clip(np.rint(W[:, c].astype(F32) / sc) + z, 0, maxq)
        dq = sc.astype(np.float64) * (q - z)
        codes[:, c] = q
        rest = perm[k:]
        F = np.linalg.inv(Hd[np.ix_(rest, rest)])
        e = (W[:, c] - dq) / F[0, 0]
        W[:, rest[1:]] -= np.outer(e, F[0, 1:])
        W[:, c] = dq
    return dict(codes=codes, scales=scales, zeros=zeros)


@pytest.mark.parametrize("act_order", [False, True])
@pytest.mark.parametrize("block", [4, 8])
def test_dynamic_group_timing_matches_brute_force_obs_loop(act_order, block):
    """Reading R9 (a group's scale and zero come from its current values when
    its first column is reached) against the loop above on a 6 x 16 layer
    with g = 4: codes, scales and zeros bit-equal, natural and act-order,
    blocks of 4 and 8.  Catches parameters taken before the earlier groups'
    feedback, after feedback from inside the group, or from the wrong
    columns of a permuted layer."""
    X, S, N, W = _layer_inputs(6, 16, 200, 87)
    W[1, 4:8] *= 6.0                                       # groups of different widths
    W[4, :] *= 0.25
    r = O.gptq_layer(W, S, N, group_size=4, block_size=block, act_order=act_order)
    _, Hd = O.damping(O.hessian(S, N), 0.01)
    if act_order:
        assert not np.array_equal(r["perm"], np.arange(16))
    want = _brute_dynamic_gptq(W, Hd, r["perm"], 4, 4)
    np.testing.assert_array_equal(r["codes"], want["codes"])
    np.testing.assert_array_equal(r["scales"], want["scales"])
    np.testing.assert_array_equal(r["zeros"], want["zeros"])
    # the pin has teeth: parameters from the weights before any feedback
    # differ on this layer
    early = _brute_dynamic_gptq(W, Hd, r["perm"], 4, 4, params_from="original")
    assert not np.array_equal(early["scales"][:, 1:], want["scales"][:, 1:])


def test_static_groups_first_group_equals_dynamic_and_beats_rtn():
    """Natural order: the first group sees no feedback before it starts, so its
    parameters equal the dynamic ones; later ones come from the original
    weights (RTN's), not the updated ones.  Static GPTQ still beats RTN."""
    X, S, N, W = _layer_inputs(48, 512, 4096, 86)
    st = O.gptq_layer(W, S, N, static_groups=True)
    dy = O.gptq_layer(W, S, N)
    rt = O.rtn_quantize(W)
    np.testing.assert_array_equal(st["scales"][:, 0], dy["scales"][:, 0])
    np.testing.assert_array_equal(st["scales"], rt["scales"])
    np.testing.assert_array_equal(st["zeros"], rt["zeros"])
    assert not np.array_equal(st["scales"][:, 1:], dy["scales"][:, 1:])
    assert O.recon_error(W, st["Q"], S) < 0.8 * O.recon_error(W, rt["Q"], S)


# ---------------------------------------------------------------- storage / packing
def test_storage_arithmetic_matches_page():
    gold = json.load(open(os.path.join(GOLDEN, "storage_arithmetic.json")))
    per_group = O.storage_bytes(1, 128, bits=4, group_size=128)
    assert per_group == gold["total_bytes_per_group"]
    assert round(per_group * 8 / 128, 2) == gold["bits_per_weight_rounded"]
    g64 = O.storage_bytes(1, 64, bits=4, group_size=64) * 8 / 64
    assert round(g64, 1) == gold["g64_bits_per_weight_rounded"]
    # a 28672 x 8192 layer: 234881024 weights -> 122028032 bytes
    assert O.storage_bytes(28672, 8192) == 28672 * 8192 * 66.5 / 128 == 122028032


def test_pack_int4_layout_and_roundtrip():
    assert O.pack_int4(np.array([[1, 2, 3, 4]])).tolist() == [[0x21, 0x43]]
    c = _rng(10).integers(0, 16, (7, 64))
    p = O.pack_int4(c)
    assert p.shape == (7, 32) and p.dtype == np.uint8
    np.testing.assert_array_equal(O.unpack_int4(p), c)


def test_pack_3bit_layout_and_roundtrip():
    # sum_j code_j << 3j = 0x1F58D1 -> little-endian bytes D1 58 1F
    assert O.pack_bits(np.array([[1, 2, 3, 4, 5, 6, 7, 0]]), 3).tolist() == [[0xD1, 0x58, 0x1F]]
    c = _rng(11).integers(0, 8, (5, 128))
    p = O.pack_bits(c, 3)
    assert p.shape == (5, 48)
    np.testing.assert_array_equal(O.unpack_bits(p, 3, 128), c)
    c4 = _rng(12).integers(0, 16, (3, 64))
    np.testing.assert_array_equal(O.pack_bits(c4, 4), O.pack_int4(c4))
