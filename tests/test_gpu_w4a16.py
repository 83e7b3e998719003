"""W4A16 consumer of the packed format on the GPU against the float64 oracle
(Y = X Q^T), on seeded stand-ins for a quantized layer: codes, fp16 scales,
zeros and (act-order) a column permutation.  The tolerance is the forward
error bound of an fp32 evaluation (tests/parity.w4a16_error_bound), checked
element by element.  Every GPU call goes through the C ABI."""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_run import log
from tests.parity import w4a16_error_bound

pytestmark = pytest.mark.gpu


def _run(cfg, m, act_order, tag=0, reps=1):
    import torch
    from post_weight_quantization_08_amd import pipeline as P

    codes, scales, zeros, perm, g_idx = synth.w4_layer(cfg, act_order, tag)
    X = synth.w4_tokens(cfg, m, tag)
    dt = {"f16": torch.float16, "bf16": torch.bfloat16}[cfg.x_dtype]
    Xd = torch.from_numpy(X.view(np.int16)).cuda().view(dt)
    cd = torch.from_numpy(codes).cuda()
    pd = torch.from_numpy(perm).cuda() if perm is not None else None
    qw = P.pack_int4_permuted(cd, pd) if pd is not None else P.pack(cd, 4)
    sd = torch.from_numpy(scales.view(np.int16)).cuda()
    zd = torch.from_numpy(zeros).cuda()
    outs = [P.w4a16_matmul(Xd, qw, sd, zd, cfg.group_size, perm=pd) for _ in range(reps)]
    torch.cuda.synchronize()
    Y = [o.cpu().numpy() for o in outs]
    Xf = synth.to_f64(X, cfg.x_dtype)
    s32 = scales.view(np.float16).astype(np.float32)
    return Y, Xf, codes, s32, zeros, g_idx, (qw.cpu().numpy() if pd is not None else None)


def _check(cfg, m, act_order, what, tag=0):
    Y, Xf, codes, s32, zeros, g_idx, _ = _run(cfg, m, act_order, tag)
    Yo = O.w4a16_matmul(Xf, O.pack_int4(codes), s32, zeros, g_idx)
    bias = 128.0 if cfg.x_dtype == "bf16" else 0.0
    tol = w4a16_error_bound(Xf, codes, s32, zeros, g_idx, bias=bias)
    err = np.abs(Y[0].astype(np.float64) - Yo)
    rel = np.linalg.norm(Y[0] - Yo) / np.linalg.norm(Yo)
    log(f"[gpu] w4a16 {what}: rel {rel:.2e}, max err / bound {np.max(err / tol):.3e}")
    assert Y[0].shape == Yo.shape
    assert np.all(err <= tol), f"{what}: worst {np.max(err / tol):.3f} of the bound"
    return rel


# (d_out, d_in, M, g, x dtype, act_order): one k-split and several, token
# counts 1..64 across all three token-tile widths, ragged row blocks, groups
# of one chunk, of two, and per-channel
CASES = [
    (130, 512, 1, 128, "f16", False),
    (130, 512, 5, 128, "bf16", True),
    (1000, 2048, 3, 128, "bf16", True),
    (1000, 2048, 16, 128, "f16", True),
    (300, 1024, 17, 256, "f16", False),
    (70, 384, 33, 128, "bf16", False),
    (64, 1024, 64, 1024, "f16", True),
    (1, 128, 1, 128, "bf16", False),
    # bf16 with four token tiles over many chunks: the operands of every MFMA
    # come straight from the code unpacking, the case that needs its full
    # wait before the MFMA reads them
    (2000, 1024, 64, 128, "bf16", True),
    (2000, 8192, 33, 128, "bf16", True),
    (500, 4096, 48, 128, "bf16", False),
]


@pytest.mark.parametrize("d_out,d_in,m,g,xdt,act_order", CASES)
def test_w4a16_matches_oracle(d_out, d_in, m, g, xdt, act_order):
    cfg = synth.CONFIGS["up_proj_70b"].scaled(f"w4:{d_out}x{d_in}", 400 + CASES.index(
        (d_out, d_in, m, g, xdt, act_order)), d_out=d_out, d_in=d_in, group_size=g, x_dtype=xdt)
    _check(cfg, m, act_order, f"{d_out}x{d_in} M={m} g={g} {xdt} act_order={act_order}")


@pytest.mark.parametrize("name,m", [("up_proj_70b", 1), ("q_proj_7b", 1), ("moe_w1_8x7b", 16)])
def test_w4a16_full_size(name, m):
    """The shapes the benchmark times, every output checked."""
    cfg = synth.CONFIGS[name]
    rel = _check(cfg, m, name == "up_proj_70b", f"{name} M={m}")
    assert rel < 1e-5


@pytest.mark.parametrize("m,xdt", [(4, "f16"), (64, "bf16"), (24, "bf16")])
def test_w4a16_is_reproducible_and_packs_in_order(m, xdt):
    cfg = synth.CONFIGS["up_proj_70b"].scaled("w4:rep", 420, d_out=500, d_in=1024, x_dtype=xdt)
    Y, _, codes, _, _, _, qw = _run(cfg, m, True, reps=3)
    for y in Y[1:]:
        np.testing.assert_array_equal(y, Y[0])
    perm = synth.w4_layer(cfg, True)[3]
    np.testing.assert_array_equal(qw, O.pack_int4(codes[:, perm]))
