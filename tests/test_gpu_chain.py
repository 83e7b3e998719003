"""Sequential block calibration on the GPU: the forward of a quantized layer
against the oracle (element by element, within one unit in the last place of
the output format plus the fp32 evaluation bound), and the two-layer chain
against the oracle's chain.  Every GPU call goes through the C ABI."""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_run import log, to_device
from tests.parity import assert_verified, follow_gpu_ties, verify_layer

pytestmark = pytest.mark.gpu


def _ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    """One unit in the last place of the 16-bit format at |v| (normal range)."""
    mant = {"f16": 10, "bf16": 7}[dtype]
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -14)))
    return 2.0 ** (e - mant)


@pytest.mark.parametrize("xdt,act,strided,d_in", [("f16", 0, False, 512), ("f16", 2, False, 512),
                                                  ("bf16", 1, False, 512), ("bf16", 2, False, 512),
                                                  ("f16", 2, True, 512), ("bf16", 0, True, 512),
                                                  ("f16", 1, False, 160), ("f16", 2, True, 96)])
def test_forward_matches_oracle(xdt, act, strided, d_in):
    """Dense 16-bit rows feed the MFMA as they are (fp16: Q as row-scaled fp16
    terms; bf16: Q as bf16 terms); rows that are not 16-byte aligned take
    the copied-operand path.  d_in 160 and 96 end on half a 64-wide k stage;
    300 tokens and 200 channels leave ragged tiles on both sides."""
    import torch
    from post_weight_quantization_08_amd import pipeline as P
    cfg = synth.CONFIGS["q_proj_7b"].scaled(f"fw:{xdt}{act}", 470 + act, d_out=200, d_in=d_in, x_dtype=xdt,
                                            group_size=128 if d_in % 128 == 0 else 32)
    codes, scales, zeros, _, g_idx = synth.w4_layer(cfg)
    Qh = O.dequantize(codes, scales.view(np.float16).astype(np.float32), zeros, g_idx).astype(np.float32)
    Xh = synth.w4_tokens(cfg, 300)
    Xd = to_device(Xh, xdt)
    if strided:   # row stride d_in + 3 elements, first element 2 bytes past an aligned address
        wide = torch.zeros(300, d_in + 3, dtype=Xd.dtype, device=Xd.device)
        wide[:, 1:d_in + 1] = Xd
        Xd = wide[:, 1:d_in + 1]
        assert Xd.stride(0) == d_in + 3 and Xd.data_ptr() % 16 != 0
    Y = P.layer_forward(Xd, torch.from_numpy(Qh).cuda(), act)
    torch.cuda.synchronize()
    Yg = synth.to_f64(Y.view(torch.int16).cpu().numpy().view(np.uint16 if xdt == "bf16" else np.float16), xdt)
    Xf = synth.to_f64(Xh, xdt)
    Yo = O.layer_forward(Xf, Qh.astype(np.float64), act, xdt)
    bound = 2.0 * (d_in * 2.0 ** -24 + 2.0 ** -17) * (np.abs(Xf) @ np.abs(Qh.astype(np.float64)).T)
    err = np.abs(Yg - Yo)
    tol = _ulp(Yo, xdt) + bound
    log(f"[gpu] forward {xdt} act={act} strided={strided} d_in={d_in}: exact {np.mean(err == 0):.4f}, "
        f"worst err/tol {np.max(err / tol):.3f}")
    assert np.all(err <= tol)
    # Q as two bf16 terms (2^-17): about 1.6% of fp16 roundings may flip
    assert np.mean(err == 0) > 0.95


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_forward_rows_of_extreme_magnitude(xdt):
    """Rows of Q that are zero, tiny (1e-6) or large (1e3) relative to the
    others: every row's power-of-two scaling (fp16 path) or bf16 terms keep
    the same bound."""
    import torch
    from post_weight_quantization_08_amd import pipeline as P
    cfg = synth.CONFIGS["q_proj_7b"].scaled(f"fwx:{xdt}", 476, d_out=96, d_in=256, x_dtype=xdt)
    codes, scales, zeros, _, g_idx = synth.w4_layer(cfg)
    Qh = O.dequantize(codes, scales.view(np.float16).astype(np.float32), zeros, g_idx).astype(np.float32)
    Qh[0] = 0.0
    Qh[1] *= np.float32(1e-6)
    Qh[2] *= np.float32(1e3)
    Qh[3, :128] *= np.float32(1e-4)        # two magnitudes inside one row
    Xh = synth.w4_tokens(cfg, 130)
    Y = P.layer_forward(to_device(Xh, xdt), torch.from_numpy(Qh).cuda(), O.ACT_NONE)
    torch.cuda.synchronize()
    Yg = synth.to_f64(Y.view(torch.int16).cpu().numpy().view(np.uint16 if xdt == "bf16" else np.float16), xdt)
    Xf = synth.to_f64(Xh, xdt)
    Yo = O.layer_forward(Xf, Qh.astype(np.float64), O.ACT_NONE, xdt)
    bound = 2.0 * (256 * 2.0 ** -24 + 2.0 ** -17) * (np.abs(Xf) @ np.abs(Qh.astype(np.float64)).T)
    err = np.abs(Yg - Yo)
    tol = _ulp(Yo, xdt) + bound
    log(f"[gpu] forward extreme rows {xdt}: worst err/tol {np.max(err / tol):.3f}")
    assert np.all(Yg[:, 0] == 0.0)
    assert np.all(err <= tol)


@pytest.mark.parametrize("act", [0, 2])
def test_forward_fp32_activations(act):
    """fp32 activations take the copied form: X and Q each as two bf16 terms
    (about 2^-17 relative each), three products; the dropped lo*lo product
    adds about 2^-18.  Bound: 2 (d_in 2^-24 + 2^-16) sum |x||q| plus one fp32
    ulp of the output."""
    import torch
    from post_weight_quantization_08_amd import pipeline as P
    cfg = synth.CONFIGS["q_proj_7b"].scaled(f"fw32:{act}", 478 + act, d_out=136, d_in=352, x_dtype="f32",
                                            group_size=32)
    codes, scales, zeros, _, g_idx = synth.w4_layer(cfg)
    Qh = O.dequantize(codes, scales.view(np.float16).astype(np.float32), zeros, g_idx).astype(np.float32)
    Xh = synth.w4_tokens(cfg, 270)
    assert Xh.dtype == np.float32
    Y = P.layer_forward(to_device(Xh, "f32"), torch.from_numpy(Qh).cuda(), act)
    torch.cuda.synchronize()
    assert Y.dtype == torch.float32
    Yg = Y.cpu().numpy().astype(np.float64)
    Xf = Xh.astype(np.float64)
    Yo = O.layer_forward(Xf, Qh.astype(np.float64), act, "f32")
    bound = 2.0 * (352 * 2.0 ** -24 + 2.0 ** -16) * (np.abs(Xf) @ np.abs(Qh.astype(np.float64)).T)
    err = np.abs(Yg - Yo)
    tol = np.spacing(np.abs(Yo).astype(np.float32)).astype(np.float64) + bound
    log(f"[gpu] forward f32 act={act}: worst err/tol {np.max(err / tol):.3f}")
    assert np.all(err <= tol)


def test_block_chain_against_oracle():
    """Layer 1 to the usual parity bar.  Layer 2's oracle input is the
    oracle's own forward of its layer 1 on the GPU's side of every tie the
    replay followed (both sides are correct results); that layer 1 must equal
    the GPU's bit for bit.  Layer 2 is then held to the same bar: H within
    1e-5, every mismatch a verified tie, output error within 1%."""
    import torch
    import post_weight_quantization_08_amd as G
    from post_weight_quantization_08_amd import pipeline as P
    cfg = synth.CONFIGS["q_proj_7b"].scaled("chain", 480, d_out=512, d_in=256, n_tokens=2048, chunk_tokens=1024)
    X = np.concatenate([synth.x_chunk(cfg, c) for c in range(cfg.n_chunks)])
    r = np.random.default_rng([480, 1])
    W1h = (r.standard_normal((512, 256)) * 0.05).astype(np.float16)
    W2h = (r.standard_normal((256, 512)) * 0.05).astype(np.float16)
    p = G.GptqParams.make()
    chunks = [to_device(X[i:i + 1024], "f16") for i in range(0, 2048, 1024)]
    res = P.calibrate_block(chunks, torch.from_numpy(W1h).cuda(), torch.from_numpy(W2h).cuda(), p, O.ACT_SILU)
    torch.cuda.synchronize()
    Xf = synth.to_f64(X, "f16")
    W1, W2 = W1h.astype(np.float64), W2h.astype(np.float64)
    S1, N1 = O.hessian_sum([Xf])
    ora1 = O.gptq_layer(W1, S1, N1)
    g1 = {k: res["layer1"][k][0].cpu().numpy() for k in ("codes", "scales", "zeros", "g_idx", "Q")}
    s1 = g1["scales"].astype(np.uint16).view(np.float16).astype(np.float32)
    rep = verify_layer(dict(codes=g1["codes"], scales=s1, zeros=g1["zeros"]), W1, ora1, 4, 128, follow_all=True)
    e_g = O.recon_error(W1, g1["Q"].astype(np.float64), S1)
    e_o = O.recon_error(W1, ora1["Q"], S1)
    assert_verified(rep, e_g, e_o, "block layer 1")
    Q1 = follow_gpu_ties(ora1, rep)
    np.testing.assert_array_equal(Q1.astype(np.float32), g1["Q"])
    # layer 2 from the oracle's forward of that layer 1
    X2 = O.layer_forward(Xf, Q1, O.ACT_SILU, "f16")
    S2, N2 = O.hessian_sum([X2])
    ora2 = O.gptq_layer(W2, S2, N2)
    st2 = res["state2"]
    L = np.tril(st2.S[0].cpu().numpy().astype(np.float64))
    S2g = L + np.tril(L, -1).T
    h_rel = np.linalg.norm(S2g - S2) / np.linalg.norm(S2)
    g2 = {k: res["layer2"][k][0].cpu().numpy() for k in ("codes", "scales", "zeros", "g_idx", "Q")}
    s2 = g2["scales"].astype(np.uint16).view(np.float16).astype(np.float32)
    rep2 = verify_layer(dict(codes=g2["codes"], scales=s2, zeros=g2["zeros"]), W2, ora2, 4, 128)
    e_g2 = O.recon_error(W2, g2["Q"].astype(np.float64), S2)
    e_o2 = O.recon_error(W2, ora2["Q"], S2)
    # the block's output with the GPU's quantized layers against the oracle chain's
    y_ref = O.activation(Xf @ W1.T, O.ACT_SILU) @ W2.T
    y_g = O.layer_forward(Xf, g1["Q"].astype(np.float64), O.ACT_SILU, "f16") @ g2["Q"].astype(np.float64).T
    y_o = X2 @ ora2["Q"].T
    eg, eo = np.linalg.norm(y_g - y_ref), np.linalg.norm(y_o - y_ref)
    log(f"[gpu] block chain: layer 1 match {rep['match']:.6f} ({rep['forced_ties']} ties followed), "
        f"layer-2 H rel {h_rel:.2e}, layer 2 match {rep2['match']:.6f} {rep2['counts']} "
        f"({rep2['forced_ties']} ties followed), block error GPU/oracle {eg / eo:.5f}")
    assert h_rel <= 1e-5
    assert_verified(rep2, e_g2, e_o2, "block layer 2")
    assert abs(eg / eo - 1.0) < 0.01
