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
    assert int(st.n[0]) == 0
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


def test_entry_without_rows_reports_info_minus_one():
    """Two experts, every gathered row of the second one out of range: its
    count stays 0 and prepare reports info = -1 for it, while the first one
    factors normally (U against the oracle's)."""
    import torch
    G, P = _G()
    d = 128
    X = np.random.default_rng([901, 2]).standard_normal((400, d)).astype(np.float16)
    idx = np.concatenate([np.arange(0, 400, 2), [400, -3, 10 ** 6]]).astype(np.int32)
    st = P.HessianState(d, 2, "cuda")
    st.add(torch.from_numpy(X).cuda(), torch.from_numpy(idx).cuda(), [0, 200, 203])
    prep = P.prepare(st, G.GptqParams.make(), check=False)
    torch.cuda.synchronize()
    assert st.n.cpu().tolist() == [200, 0]
    assert prep.info.cpu().tolist() == [0, -1]
    S, N = O.hessian_sum([X[::2].astype(np.float64)])
    _, Hd = O.damping(O.hessian(S, N), 0.01)
    U = O.inverse_factor(Hd)
    Ug = prep.U[0].cpu().numpy().astype(np.float64)
    assert np.linalg.norm(Ug - U) / np.linalg.norm(U) < 1e-4
    with pytest.raises(G.GptqError):
        P.prepare(st, G.GptqParams.make(), check=True)


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


@pytest.mark.parametrize("group_size,bits", [(64, 4), (256, 4), (512, 3), (32, 2), (128, 8), (16, 4)])
def test_other_group_sizes_and_widths(group_size, bits):
    cfg = synth.test_config("up_proj_70b").scaled(f"edge:g{group_size}b{bits}", 310 + bits,
                                                  d_out=130, d_in=512, n_tokens=2100)
    g = gpu_layer(cfg, (bits,), want_q=True, params_over=dict(group_size=group_size))
    S, N = oracle_hessians(cfg)
    W = synth.to_f64(synth.weights(cfg), cfg.w_dtype)
    _parity(cfg, g, S[0], N[0], W, bits, group_size, f"g={group_size} bits={bits}")


# dynamic asymmetric groups (the workloads' quantizer) on a layer tall enough
# for the 64-row workgroups of the column loop: groups narrower than, equal
# to and wider than the 128-column tile, per-channel (g = d_in), 2/3/4 bits,
# natural and act-order
TALL_CASES = [(128, 4, False), (128, 3, True), (256, 4, False), (512, 4, True), (16, 4, False), (32, 2, True),
              (64, 4, False)]


@pytest.mark.parametrize("group_size,bits,act_order", TALL_CASES)
def test_tall_layer_dynamic_groups(group_size, bits, act_order):
    seed = 380 + TALL_CASES.index((group_size, bits, act_order))
    cfg = synth.test_config("up_proj_70b").scaled(f"edge:tall{group_size}b{bits}", seed,
                                                  d_out=8300, d_in=512, n_tokens=2100)
    g = gpu_layer(cfg, (bits,), want_q=True, params_over=dict(group_size=group_size, act_order=act_order))
    S, N = oracle_hessians(cfg)
    W = synth.to_f64(synth.weights(cfg), cfg.w_dtype)
    _parity(cfg, g, S[0], N[0], W, bits, group_size,
            f"tall g={group_size} bits={bits} act_order={act_order}", act_order=act_order)


# a layer of 16500 rows (258 workgroups of 64 rows, the last one with 52):
# groups equal to and wider than the tile, per-channel (g = d_in), 3/4 bits,
# natural and act-order, symmetric; the dequantized output against the codes
WIDE_CASES = [(128, 4, False, False), (128, 3, True, False), (256, 4, False, False), (512, 4, True, False),
              (128, 4, True, True)]


@pytest.mark.parametrize("group_size,bits,act_order,sym", WIDE_CASES)
def test_taller_layer_wide_groups(group_size, bits, act_order, sym):
    seed = 390 + WIDE_CASES.index((group_size, bits, act_order, sym))
    cfg = synth.test_config("up_proj_70b").scaled(f"edge:tall16500g{group_size}b{bits}", seed,
                                                  d_out=16500, d_in=512, n_tokens=2100)
    g = gpu_layer(cfg, (bits,), want_q=True,
                  params_over=dict(group_size=group_size, act_order=act_order, sym=sym))
    S, N = oracle_hessians(cfg)
    W = synth.to_f64(synth.weights(cfg), cfg.w_dtype)
    _parity(cfg, g, S[0], N[0], W, bits, group_size,
            f"16500 rows g={group_size} bits={bits} act_order={act_order} sym={sym}", act_order=act_order, sym=sym)
    gb = g[bits]
    Qg = O.dequantize(gb["codes"][0], gb["scales_f32"][0], gb["zeros"][0], gb["g_idx"][0])
    np.testing.assert_allclose(gb["Q"][0], Qg, rtol=1e-6, atol=0.0)


# a layer of 33000 rows: 516 workgroups of 64 rows, more than one round of
# two per CU, the last one with 40 rows; natural and act-order
TALLEST_CASES = [(128, 4, False), (256, 4, True), (128, 3, True)]


@pytest.mark.parametrize("group_size,bits,act_order", TALLEST_CASES)
def test_tallest_layer_two_rounds_of_workgroups(group_size, bits, act_order):
    seed = 420 + TALLEST_CASES.index((group_size, bits, act_order))
    cfg = synth.test_config("up_proj_70b").scaled(f"edge:tall33000g{group_size}b{bits}", seed,
                                                  d_out=33000, d_in=512, n_tokens=2100)
    g = gpu_layer(cfg, (bits,), want_q=True, params_over=dict(group_size=group_size, act_order=act_order))
    S, N = oracle_hessians(cfg)
    W = synth.to_f64(synth.weights(cfg), cfg.w_dtype)
    _parity(cfg, g, S[0], N[0], W, bits, group_size,
            f"33000 rows g={group_size} bits={bits} act_order={act_order}", act_order=act_order)
    gb = g[bits]
    Qg = O.dequantize(gb["codes"][0], gb["scales_f32"][0], gb["zeros"][0], gb["g_idx"][0])
    np.testing.assert_allclose(gb["Q"][0], Qg, rtol=1e-6, atol=0.0)


@pytest.mark.parametrize("x_rows", [262144, 300000, 540000])
def test_gather_over_x_of_2gib_and_more(x_rows):
    """X of exactly 2^31 bytes, of 2.46 GB and of 4.42 GB (rows of 4096 fp16):
    the first two are addressed as one buffer with 32-bit byte offsets, the
    last one (past 2^32 bytes) with 64-bit addresses.  The gathered rows sit
    on both sides of the 2^31- and 2^32-byte boundaries that X crosses, in
    random order, with indices outside X mixed in; S (every entry), D and N
    against the oracle over the valid rows."""
    import torch
    G, P = _G()
    d = 4096
    rng = np.random.default_rng([903, x_rows])
    parts = [rng.choice(x_rows - 131072, 1000, replace=False), x_rows - 131072 + rng.choice(131072, 1000, replace=False)]
    for edge in (1 << 31) // (2 * d), (1 << 32) // (2 * d):
        if edge + 500 <= x_rows - 131072:
            parts.append(edge - 500 + rng.choice(1000, 500, replace=False))
    valid = np.unique(np.concatenate(parts))
    data = rng.standard_normal((len(valid), d)).astype(np.float16)
    X = torch.zeros(x_rows, d, dtype=torch.float16, device="cuda")
    X[torch.from_numpy(valid).cuda()] = torch.from_numpy(data).cuda()
    order = rng.permutation(len(valid))
    bad = np.array([-1, x_rows, x_rows + 7, -(1 << 30)], dtype=np.int64)
    idx = np.concatenate([valid[order][:1000], bad[:2], valid[order][1000:], bad[2:]]).astype(np.int32)
    st = P.HessianState(d, 1, "cuda")
    st.add(X, torch.from_numpy(idx).cuda(), [0, len(idx)])
    torch.cuda.synchronize()
    del X
    assert int(st.n[0]) == len(valid)
    S, _ = O.hessian_sum([data.astype(np.float64)])
    L = np.tril(st.S[0].cpu().numpy().astype(np.float64))
    Sg = L + np.tril(L, -1).T
    rel = np.linalg.norm(Sg - S) / np.linalg.norm(S)
    log(f"[gpu] gather over {x_rows} rows ({x_rows * d * 2} bytes): S rel {rel:.2e}")
    assert rel <= 1e-5
    np.testing.assert_allclose(st.D[0].cpu().numpy(), np.diag(S), rtol=1e-12)


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


def test_out_of_range_gather_rows_are_skipped_and_not_counted():
    import torch
    G, P = _G()
    d = 128
    X = np.random.default_rng([902, 1]).standard_normal((300, d)).astype(np.float16)
    idx = np.array([0, 5, -1, 7, 300, 299, 1000], dtype=np.int32)
    st = P.HessianState(d, 1, "cuda")
    st.add(torch.from_numpy(X).cuda(), torch.from_numpy(idx).cuda(), [0, len(idx)])
    torch.cuda.synchronize()
    ok = idx[(idx >= 0) & (idx < 300)]
    assert int(st.n[0]) == len(ok)          # N counts only rows that contributed
    S, _ = O.hessian_sum([X[ok].astype(np.float64)])
    L = np.tril(st.S[0].cpu().numpy().astype(np.float64))
    np.testing.assert_allclose(L, np.tril(S), rtol=1e-6, atol=1e-3)


def _h_rel_lower(S32, S64):
    """Relative Frobenius error of the whole symmetric matrix from lower triangles."""
    a = np.tril(S32.astype(np.float64))
    b = np.tril(S64)
    w = np.tril(np.ones_like(b), -1) * 2.0 + np.eye(b.shape[0])
    return float(np.sqrt(np.sum(w * (a - b) ** 2) / np.sum(w * b * b)))


@pytest.mark.parametrize("d,n,gather", [(200, 1000, False), (328, 77, False), (1024, 5000, False),
                                        (64, 31, False), (136, 600, True), (4104, 300, True)])
def test_fp32_activations_accumulate_on_mfma(d, n, gather):
    """fp32 activations take their own product kernel (fp32 MFMA, 32-token
    stages, 64 x 64 tiles, or 128 x 128 once there are 256 of them as at
    d_in = 4104): ragged channel counts and token counts, a diagonal-only
    layer and gathers with rows outside X, against the float64 sum of outer
    products."""
    import torch
    G, P = _G()
    rng = np.random.default_rng([903, d, n])
    X = rng.standard_normal((n, d)).astype(np.float32)
    X[:, rng.choice(d, size=max(1, d // 50), replace=False)] *= 30.0   # a few outlier channels
    st = P.HessianState(d, 1, "cuda")
    if gather:
        idx = rng.integers(-5, n + 5, size=n // 2).astype(np.int32)
        st.add(torch.from_numpy(X).cuda(), torch.from_numpy(idx).cuda(), [0, len(idx)])
        ok = idx[(idx >= 0) & (idx < n)]
        rows = X[ok]
    else:
        st.add(torch.from_numpy(X).cuda())
        rows = X
    torch.cuda.synchronize()
    S, N = O.hessian_sum([rows.astype(np.float64)])
    assert int(st.n[0]) == N
    rel = _h_rel_lower(st.S[0].cpu().numpy(), S)
    log(f"[gpu] fp32 Hessian d={d} n={n} gather={gather}: H rel Frobenius {rel:.3e}")
    assert rel <= 1e-5
    np.testing.assert_allclose(st.D[0].cpu().numpy(), np.diag(S), rtol=1e-12)


# a wider layer of 20 tiles (ranges that halve into uneven parts, the first
# update over 8 or 10 tiles): groups equal to and wider than the tile,
# natural and act-order
WIDER_CASES = [(128, 4, False), (256, 4, True), (512, 3, False), (128, 4, True)]


@pytest.mark.parametrize("group_size,bits,act_order", WIDER_CASES)
def test_wider_layer_dynamic_groups(group_size, bits, act_order):
    seed = 410 + WIDER_CASES.index((group_size, bits, act_order))
    cfg = synth.test_config("up_proj_70b").scaled(f"edge:wider{group_size}b{bits}", seed,
                                                  d_out=700, d_in=2560, n_tokens=6000)
    g = gpu_layer(cfg, (bits,), want_q=True, params_over=dict(group_size=group_size, act_order=act_order))
    S, N = oracle_hessians(cfg)
    W = synth.to_f64(synth.weights(cfg), cfg.w_dtype)
    _parity(cfg, g, S[0], N[0], W, bits, group_size,
            f"700x2560 g={group_size} bits={bits} act_order={act_order}", act_order=act_order)


def test_bit_widths_on_two_streams_match_one_stream():
    """The benchmark quantizes its bit widths (same S and U) concurrently, each
    with its own workspace on a stream of its own: the outputs equal those of
    the same calls made one after the other on one stream, bit for bit."""
    import torch
    G, P = _G()
    cfg = synth.CONFIGS["up_proj_70b"].scaled("edge:streams", 905, d_out=700, d_in=2560, n_tokens=4096)
    W = P.to_device(synth.weights(cfg), cfg.w_dtype)
    st = P.HessianState(cfg.d_in, 1, "cuda")
    st.add(P.to_device(synth.x_all(cfg), cfg.x_dtype))
    plist = [G.GptqParams.make(bits=b, group_size=128, block_size=128, damp_rel=0.01) for b in (4, 3)]
    prep = P.prepare(st, plist[0])
    seq = [P.quantize(W, prep, p) for p in plist]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in plist]
    ready = torch.cuda.Event()
    ready.record()
    par = []
    for p, s in zip(plist, streams):
        s.wait_event(ready)
        with torch.cuda.stream(s):
            par.append(P.quantize(W, prep, p, stream=s))
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for a, b in zip(seq, par):
        for key in ("codes", "scales", "zeros", "g_idx"):
            assert torch.equal(a[key], b[key]), key


def test_workspace_too_small_is_rejected():
    import torch
    G, P = _G()
    st = P.HessianState(4096, 1, "cuda")
    X = torch.zeros(70000, 4096, dtype=torch.float16, device="cuda")
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(G.GptqError) as e:
        G.gptq_hessian_accumulate(st.S, st.D, st.n, X, 4096, 70000, 4096, None, None, None, 1, ws, 1024)
    assert e.value.status == G.ENOMEM
