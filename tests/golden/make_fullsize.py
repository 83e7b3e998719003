"""Writes the full-size oracle fixtures ``fullsize_<workload>.npz``.

For every workload at its real size this runs the float64 oracle on the whole
Hessian (streamed over the same 16384-token chunks the GPU sees), factors the
damped inverse, and quantizes a fixed sample of weight rows (rows are
independent given U, so the sample's results equal those of the whole layer).
It stores, for the sampled rows only: codes, fp16 scale bits, zeros, a
three-level flag per rounding decision (0: clear, 1: within 0.05 steps of a
midpoint, 2: within 1e-3 steps; scales: 2 = within 1e-5 relative of an fp16
midpoint), the output error ||(W - Q) X^T||^2 of each sampled row for the
oracle and for plain rounding, the act-order permutation, and a few entries of
U and H.  Only ``oracle`` and the seeded input generators are used.

    python tests/golden/make_fullsize.py [workload ...]
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synth  # noqa: E402

ROWS_DENSE = 16
ROWS_PER_EXPERT = 4
TAU, CASCADE, SCALE_TIE = 1e-3, 0.05, 1e-5


def sample_rows(cfg: synth.LayerConfig, expert: int) -> np.ndarray:
    k = ROWS_PER_EXPERT if cfg.n_experts else ROWS_DENSE
    rng = np.random.default_rng([777, cfg.cfg_id, expert])
    return np.sort(rng.choice(cfg.d_out, size=k, replace=False))


def flags(m: np.ndarray, tie: float, casc: float) -> np.ndarray:
    return np.where(m < tie, 2, np.where(m < casc, 1, 0)).astype(np.uint8)


def hessians(cfg: synth.LayerConfig):
    routes = synth.routing(cfg) if cfg.n_experts else None
    f = synth.channel_factor(cfg)
    S = [np.zeros((cfg.d_in, cfg.d_in)) for _ in range(cfg.batch)]
    N = [0] * cfg.batch
    for c in range(cfg.n_chunks):
        t0, t1 = cfg.chunk_range(c)
        X = synth.to_f64(synth.x_chunk(cfg, c, f), cfg.x_dtype)
        for e in range(cfg.batch):
            Xe = X if routes is None else X[routes[e][(routes[e] >= t0) & (routes[e] < t1)] - t0]
            S[e] += Xe.T @ Xe
            N[e] += Xe.shape[0]
        print(f"  chunk {c + 1}/{cfg.n_chunks}", flush=True)
    return S, N


def main(names) -> None:
    for name in names:
        cfg = synth.CONFIGS[name]
        t = time.time()
        print(f"{name}: Hessian over {cfg.n_tokens} tokens", flush=True)
        S, N = hessians(cfg)
        out = {"n_tokens": np.array(N, dtype=np.int64)}
        rng = np.random.default_rng([778, cfg.cfg_id])
        hi = rng.integers(0, cfg.d_in, 512)
        hj = rng.integers(0, cfg.d_in, 512)
        out["h_i"], out["h_j"] = hi, hj
        for e in range(cfg.batch):
            rows = sample_rows(cfg, e)
            W = synth.to_f64(synth.weights(cfg, e), cfg.w_dtype)[rows]
            out[f"e{e}_rows"] = rows
            out[f"e{e}_h"] = 2.0 * S[e][hi, hj] / N[e]
            for bits in cfg.bits:
                r = O.gptq_layer(W, S[e], N[e], bits=bits, group_size=cfg.group_size,
                                 block_size=cfg.block_size, damp_rel=cfg.damp_rel, act_order=cfg.act_order)
                m = O.decision_margins(r, bits, cfg.group_size)
                p = f"e{e}_b{bits}_"
                out[p + "codes"] = r["codes"].astype(np.uint8)
                out[p + "scales"] = r["scales"].astype(np.float16).view(np.uint16)
                out[p + "zeros"] = r["zeros"].astype(np.uint8)
                out[p + "code_flag"] = flags(m["code"], TAU, CASCADE)
                out[p + "zero_flag"] = flags(m["zero"], TAU, CASCADE)
                out[p + "scale_flag"] = np.where(m["scale"] < SCALE_TIE, 2, 1).astype(np.uint8)
                D = W - r["Q"]
                out[p + "err_rows"] = np.einsum("ij,jk,ik->i", D, S[e], D)
                Dr = W - O.rtn_quantize(W, bits, cfg.group_size)["Q"]
                out[p + "err_rows_rtn"] = np.einsum("ij,jk,ik->i", Dr, S[e], Dr)
                if bits == cfg.bits[0]:
                    out[f"e{e}_perm"] = r["perm"].astype(np.int32)
                    ui = rng.integers(0, cfg.d_in, 256)
                    uj = rng.integers(0, cfg.d_in, 256)
                    lo, hi2 = np.minimum(ui, uj), np.maximum(ui, uj)
                    out[f"e{e}_u_i"], out[f"e{e}_u_j"] = lo, hi2
                    out[f"e{e}_u"] = r["U"][lo, hi2]
                print(f"  expert {e} bits {bits}: rows {rows[:4]}..., "
                      f"E/E_rtn {out[p + 'err_rows'].sum() / out[p + 'err_rows_rtn'].sum():.4f}", flush=True)
        path = os.path.join(HERE, f"fullsize_{name}.npz")
        np.savez_compressed(path, **out)
        print(f"{name}: wrote {path} ({os.path.getsize(path)} bytes) in {time.time() - t:.0f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or [n for n in synth.CONFIG_ORDER if n != "tiny"])
