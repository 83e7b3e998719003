"""gptq_prepare_hinv alone, at sizes that are not multiples of the 64-wide
leaf: the factor U (U^T U = Hd^-1) and the act-order permutation against the
oracle on the same (S, D, N).  Every GPU call goes through the C ABI."""
import numpy as np
import pytest

import oracle as O
from tests.gpu_run import log

pytestmark = pytest.mark.gpu

# sizes around the leaf (64) and the fused two-leaf block (128), ragged tails
# at several recursion depths, one larger odd size, and sizes whose root
# (2048 columns and more) runs its off-chain product on the second stream:
# 2100 and 4160
SIZES = [1, 7, 40, 64, 65, 100, 127, 128, 129, 200, 333, 520, 1000, 2100, 4160]


def _inputs(d: int, seed: int, batch: int = 1):
    """fp32 S (as the accumulator holds it), fp64 diagonal D and N per entry."""
    rng = np.random.default_rng([seed, d, batch])
    n = 3 * d + 16
    S32, D = [], []
    for _ in range(batch):
        X = rng.standard_normal((n, d))
        X[:, rng.integers(0, d, size=max(1, d // 50))] *= 20.0   # a few outlier channels
        S = X.T @ X
        S32.append(S.astype(np.float32))
        D.append(np.diag(S).copy())
    return np.stack(S32), np.stack(D), n


def _oracle(S32: np.ndarray, D: np.ndarray, n: int, damp_rel: float, act_order: bool):
    """The oracle on exactly the values the library reads: the lower triangle
    of S in fp32 and the fp64 diagonal."""
    L = np.tril(S32.astype(np.float64), -1)
    S = L + L.T + np.diag(D)
    H0 = O.hessian(S, n)
    _, Hd = O.damping(H0, damp_rel)
    perm = O.act_order_perm(H0) if act_order else np.arange(S.shape[0])
    return O.inverse_factor(Hd[np.ix_(perm, perm)]), perm


def _gpu(S32, D, n, damp_rel, act_order):
    import torch
    import post_weight_quantization_08_amd as G
    from post_weight_quantization_08_amd import pipeline as P
    b, d = D.shape
    st = P.HessianState(d, b, "cuda")
    st.S.copy_(torch.from_numpy(S32))
    st.D.copy_(torch.from_numpy(D))
    st.n[:] = n
    prep = P.prepare(st, G.GptqParams.make(damp_rel=damp_rel, act_order=act_order), check=False)
    torch.cuda.synchronize()
    perm = prep.perm.cpu().numpy() if act_order else None
    return prep.U.cpu().numpy(), perm, prep.info.cpu().numpy()


@pytest.mark.parametrize("act_order", [False, True])
@pytest.mark.parametrize("d", SIZES)
def test_factor_matches_oracle(d, act_order):
    S32, D, n = _inputs(d, 1101)
    U, perm, info = _gpu(S32, D, n, 0.01, act_order)
    assert info.tolist() == [0]
    Uo, po = _oracle(S32[0], D[0], n, 0.01, act_order)
    if act_order:
        np.testing.assert_array_equal(perm[0], po)
    rel = np.linalg.norm(U[0] - Uo) / np.linalg.norm(Uo)
    log(f"[gpu] factor d={d} act_order={act_order}: U rel {rel:.2e}")
    # U is returned in fp32: its rounding alone is about 3e-8 relative
    assert rel < 2e-6
    assert np.all(np.tril(U[0], -1) == 0.0)


@pytest.mark.parametrize("d,b", [(200, 3), (2100, 2)])
def test_factor_batch_entries_are_independent(d, b):
    S32, D, n = _inputs(d, 1102, batch=b)
    U, perm, info = _gpu(S32, D, n, 0.01, True)
    assert info.tolist() == [0] * b
    for e in range(b):
        Uo, po = _oracle(S32[e], D[e], n, 0.01, True)
        np.testing.assert_array_equal(perm[e], po)
        assert np.linalg.norm(U[e] - Uo) / np.linalg.norm(Uo) < 2e-6


@pytest.mark.parametrize("d,dead", [(200, 150), (129, 0), (333, 332)])
def test_dead_channel_reports_its_column(d, dead):
    """With no damping a channel that never fires gives an exactly zero pivot;
    the reversed factorization meets it after the channels to its right, so
    info is its 1-based column when those are healthy; the oracle refuses the
    same matrix."""
    S32, D, n = _inputs(d, 1103)
    S32[0][dead, :] = 0.0
    S32[0][:, dead] = 0.0
    D[0][dead] = 0.0
    _, _, info = _gpu(S32, D, n, 0.0, False)
    assert info.tolist() == [dead + 1]
    with pytest.raises(np.linalg.LinAlgError):
        _oracle(S32[0], D[0], n, 0.0, False)
