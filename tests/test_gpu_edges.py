"""Edge cases of the HIP path, each against the oracle or an exact expectation."""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_run import gpu_layer, log, oracle_hessians
from tests.parity import assert_verified, verify_layer

pytestmark = pytest.mark.gpu


def _G():
    import post_weight_quantization_08_amd as G
    from post_weight_quantization_08_amd import pipeline as P
    return G, P


def _parity(cfg, g, S, N, W, bits, group_size, what, act_order=None, sym=False, static_groups=False):
    act_order = cfg.act_order if act_order is None else act_order
    o = O.gptq_layer(W, S, N, bits=bits, group_size=group_size, block_size=128, damp_rel=cfg.damp_rel,
                     act_order=act_order, sym=sym, static_groups=static_groups)
    gb = g[bits]
    np.testing.assert_array_equal(gb["g_idx"][0], o["g_idx"])
    if act_order:
        np.testing.assert_array_equal(gb["perm"][0], o["perm"])
    rep = verify_layer(dict(codes=gb["codes"][0], scales=gb["scales_f32"][0], zeros=gb["zeros"][0]), W, o,
                       bits, group_size, sym=sym)
    Qg = O.dequantize(gb["codes"][0], gb["scales_f32"][0], gb["zeros"][0], gb["g_idx"][0])
    e_g, e_o = O.recon_error(W, Qg, S), O.recon_error(W, o["Q"], S)
    log(f"[gpu] {what}: match {rep['match']:.6f} {rep['counts']} ties followed {rep['forced_ties']} "
        f"in {rep['replayed_rows']} rows, E ratio {e_g / e_o:.6f}")
    assert_verified(rep, e_gpu=e_g, e_ora=e_o, what=what)
    return o


def test_empty_chunk_leaves_state_unchanged():
    import torch
    G, P = _G()
    st = P.HessianState(256, 1, "cuda")
    X = torch.zeros(0, 256, dtype=torch.float16, device="cuda")
    st.add(X)
    torch.cuda.synchronize()
    assert st.n[0] == 0
    assert float(st.S.abs().sum()) == 0.0 and float(st.D.abs().sum()) == 0.0


def test_singular_hessian_reports_info():
    """A dead channel with no damping gives an exactly zero pivot: the last
    column, which the reversed factorization meets first (info = d); the
    oracle's Cholesky refuses the same matrix."""
    import torch
    G, P = _G()
    d = 256
    X = np.random.default_rng([901, 1]).standard_normal((512, d)).astype(np.float16)
    X[:, d - 1] = 0
    st = P.HessianState(d, 1, "cuda")
    st.add(torch.from_numpy(X).cuda())
    params = G.GptqParams.make(damp_rel=0.0)
    prep = P.prepare(st, params, check=False)
    torch.cuda.synchronize()
    assert int(prep.info.cpu()[0]) == d
    with pytest.raises(G.GptqError):
        P.prepare(st, params, check=True)
    S, N = O.hessian_sum([X.astype(np.float64)])
    with pytest.raises(np.linalg.LinAlgError):
        O.gptq_layer(np.zeros((4, d)), S, N, damp_rel=0.0)


def test_dead_channel_with_damping_and_zero_groups():
    """A dead input channel is fine once damped; all-zero weight groups give
    scale 1 (fp16 0x3C00), zero 0, codes 0 and an exactly zero Q."""
    cfg = synth.test_config("q_proj_7b").scaled("edge:zero", 301, d_out=70, d_in=384, n_tokens=1500)
    xs = [synth.x_chunk(cfg, c) for c in range(cfg.n_chunks)]
    for x in xs:
        x[:, 5] = 0
    W = synth.weights(cfg).copy()
    W[3, :128] = 0
    W[10, 128:256] = 0
    g = gpu_layer(cfg, (4,), want_q=True, x_chunks=xs, W=W[None])
    S, N = oracle_hessians(cfg, xs)
    Wf = synth.to_f64(W, cfg.w_dtype)
    _parity(cfg, g, S[0], N[0], Wf, 4, 128, "zero groups")
    gb = g[4]
    assert gb["scales"][0][3, 0] == np.int16(0x3C00) and gb["zeros"][0][3, 0] == 0
    assert np.all(gb["codes"][0][3, :128] == 0) and np.all(gb["Q"][0][3, :128] == 0.0)
    # zeroed weights of a later group are not zero when that group starts:
    # earlier columns' errors have been fed into them (checked by the parity above)


@pytest.mark.parametrize("group_size,bits", [(64, 4), (256, 4), (512, 3), (32, 2), (128, 8)])
def test_other_group_sizes_and_widths(group_size, bits):
    cfg = synth.test_config("up_proj_70b").scaled(f"edge:g{group_size}b{bits}", 310 + bits,
                                                  d_out=130, d_in=512, n_tokens=2100)
    g = gpu_layer(cfg, (bits,), want_q=True, params_over=dict(group_size=group_size))
    S, N = oracle_hessians(cfg)
    W = synth.to_f64(synth.weights(cfg), cfg.w_dtype)
    _parity(cfg, g, S[0], N[0], W, bits, group_size, f"g={group_size} bits={bits}")


# symmetric groups: natural and act-order, 2/3/4/8 bits, groups narrower and
# wider than the 128-column tile, per-channel (g = d_in), and a layer tall
# enough for the four-lanes-per-row variant of the column loop
SYM_CASES = [(128, 4, False, 130), (128, 4, True, 130), (64, 3, True, 130), (256, 4, False, 130),
             (32, 2, False, 130), (128, 8, True, 130), (512, 4, True, 130), (128, 4, True, 8300)]


@pytest.mark.parametrize("group_size,bits,act_order,d_out", SYM_CASES)
def test_symmetric_groups(group_size, bits, act_order, d_out):
    seed = 330 + SYM_CASES.index((group_size, bits, act_order, d_out))
    cfg = synth.test_config("up_proj_70b").scaled(f"edge:sym{group_size}b{bits}", seed,
                                                  d_out=d_out, d_in=512, n_tokens=2100)
    g = gpu_layer(cfg, (bits,), want_q=True,
                  params_over=dict(group_size=group_size, act_order=act_order, sym=True))
    S, N = oracle_hessians(cfg)
    W = synth.to_f64(synth.weights(cfg), cfg.w_dtype)
    what = f"sym g={group_size} bits={bits} act_order={act_order} d_out={d_out}"
    _parity(cfg, g, S[0], N[0], W, bits, group_size, what, act_order=act_order, sym=True)
    gb = g[bits]
    assert np.all(gb["zeros"][0] == 1 << (bits - 1))
    # Q = s (code - 2^(b-1)): the signed code times the group's scale
    Qg = O.dequantize(gb["codes"][0], gb["scales_f32"][0], gb["zeros"][0], gb["g_idx"][0])
    np.testing.assert_array_equal(Qg.astype(np.float32), gb["Q"][0])


# static groups (parameters fixed before the loop from W, groups of original
# columns): natural and act-order, both quantizers, group sizes below, at and
# above the tile, per-channel, a tall layer, 2/3/4/8 bits
STATIC_CASES = [(128, 4, False, False, 130), (128, 4, True, False, 130), (128, 4, True, True, 8300),
                (64, 3, True, False, 130), (256, 4, True, False, 130), (32, 2, True, True, 130),
                (512, 4, True, False, 130), (128, 8, True, False, 130)]


@pytest.mark.parametrize("group_size,bits,act_order,sym,d_out", STATIC_CASES)
def test_static_groups(group_size, bits, act_order, sym, d_out):
    seed = 350 + STATIC_CASES.index((group_size, bits, act_order, sym, d_out))
    cfg = synth.test_config("down_proj_7b").scaled(f"edge:static{group_size}b{bits}", seed,
                                                   d_out=d_out, d_in=512, n_tokens=2100)
    g = gpu_layer(cfg, (bits,), want_q=True,
                  params_over=dict(group_size=group_size, act_order=act_order, sym=sym, static_groups=True))
    S, N = oracle_hessians(cfg)
    W = synth.to_f64(synth.weights(cfg), cfg.w_dtype)
    what = f"static g={group_size} bits={bits} act_order={act_order} sym={sym} d_out={d_out}"
    _parity(cfg, g, S[0], N[0], W, bits, group_size, what, act_order=act_order, sym=sym, static_groups=True)
    gb = g[bits]
    np.testing.assert_array_equal(gb["g_idx"][0], np.arange(512) // group_size)
    # the parameters depend on W alone: bit-exact against group-wise rounding's
    t = O.rtn_quantize(W, bits, group_size, sym=sym)
    np.testing.assert_array_equal(gb["scales_f32"][0], t["scales"])
    np.testing.assert_array_equal(gb["zeros"][0], t["zeros"])
    Qg = O.dequantize(gb["codes"][0], gb["scales_f32"][0], gb["zeros"][0], gb["g_idx"][0])
    np.testing.assert_array_equal(Qg.astype(np.float32), gb["Q"][0])


def test_out_of_range_gather_rows_contribute_nothing():
    import torch
    G, P = _G()
    d = 128
    X = np.random.default_rng([902, 1]).standard_normal((300, d)).astype(np.float16)
    idx = np.array([0, 5, -1, 7, 300, 299, 1000], dtype=np.int32)
    st = P.HessianState(d, 1, "cuda")
    st.add(torch.from_numpy(X).cuda(), torch.from_numpy(idx).cuda(), [0, len(idx)])
    torch.cuda.synchronize()
    assert st.n[0] == len(idx)
    ok = idx[(idx >= 0) & (idx < 300)]
    S, _ = O.hessian_sum([X[ok].astype(np.float64)])
    L = np.tril(st.S[0].cpu().numpy().astype(np.float64))
    np.testing.assert_allclose(L, np.tril(S), rtol=1e-6, atol=1e-3)


def test_workspace_too_small_is_rejected():
    import torch
    G, P = _G()
    st = P.HessianState(4096, 1, "cuda")
    X = torch.zeros(70000, 4096, dtype=torch.float16, device="cuda")
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(G.GptqError) as e:
        G.gptq_hessian_accumulate(st.S, st.D, st.n, X, 4096, 70000, 4096, None, None, None, 1, ws, 1024)
    assert e.value.status == G.ENOMEM
