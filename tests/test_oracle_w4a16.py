"""Pins of the W4A16 oracle (Y = X Q^T from packed 4-bit codes) against a hand
example and a brute-force loop that reads the packed bytes itself."""
import numpy as np

import oracle as O


def test_hand_example():
    """Bytes 0x21 0x43 hold codes 1, 2, 3, 4 (low nibble first); with s = 0.5
    and z = 2 the weights are -0.5, 0, 0.5, 1, so x = (1, 2, 3, 4) gives
    -0.5 + 0 + 1.5 + 4 = 5.  Catches a swapped nibble order (which gives 4)
    or a zero added instead of subtracted."""
    packed = np.array([[0x21, 0x43]], dtype=np.uint8)
    Y = O.w4a16_matmul(np.array([[1.0, 2.0, 3.0, 4.0]]), packed, np.array([[0.5]], np.float32),
                       np.array([[2]]), np.zeros(4, dtype=np.int64))
    assert Y.shape == (1, 1) and Y[0, 0] == 5.0


def _brute(X, packed, scales, zeros, g_idx):
    M, d_in = X.shape
    d_out = packed.shape[0]
    Y = [[0.0] * d_out for _ in range(M)]
    for m in range(M):
        for n in range(d_out):
            acc = 0.0
            for c in range(d_in):
                byte = int(packed[n, c // 2])
                q = (byte >> 4) if c % 2 else (byte & 0xF)
                gi = int(g_idx[c])
                acc += float(X[m, c]) * float(scales[n, gi]) * (q - int(zeros[n, gi]))
            Y[m][n] = acc
    return np.array(Y)


def test_brute_force_with_act_order_groups():
    """Three tokens, five output rows, 16 input channels in groups of 4 whose
    membership follows a permutation (act-order g_idx): Y must be X times the
    transposed dequantized weights, not X times W or a row-major mix-up."""
    r = np.random.default_rng([77, 1])
    d_in, d_out, g = 16, 5, 4
    codes = r.integers(0, 16, (d_out, d_in))
    packed = O.pack_int4(codes)
    scales = r.uniform(0.01, 0.1, (d_out, d_in // g)).astype(np.float16).astype(np.float32)
    zeros = r.integers(0, 16, (d_out, d_in // g))
    perm = r.permutation(d_in)
    g_idx = np.empty(d_in, dtype=np.int64)
    g_idx[perm] = np.arange(d_in) // g
    X = r.standard_normal((3, d_in)).astype(np.float16).astype(np.float64)
    np.testing.assert_allclose(O.w4a16_matmul(X, packed, scales, zeros, g_idx),
                               _brute(X, packed, scales, zeros, g_idx), rtol=1e-13, atol=1e-15)


def test_codes_at_their_zero_give_zero_output():
    z = np.full((7, 2), 9)
    packed = O.pack_int4(np.full((7, 256), 9))
    X = np.random.default_rng([77, 2]).standard_normal((4, 256))
    Y = O.w4a16_matmul(X, packed, np.ones((7, 2), np.float32), z, np.arange(256) // 128)
    assert np.all(Y == 0.0)
