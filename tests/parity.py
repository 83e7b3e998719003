"""GPU-vs-oracle comparison of one quantized layer (test infrastructure).

Codes must be identical in at least 99.9% of entries; every mismatch must be
off by exactly one and explained by one of
  (i)   the oracle's value sat within TAU steps of a rounding midpoint;
  (ii)  the (row, group)'s zero or fp16 scale sat at a near-tie, shifting the
        whole group, or the group's parameters themselves differ at such a tie;
  (iii) a cascade: an admissible mismatch earlier in the same row changed the
        feedback, and the value sat within CASCADE steps of a midpoint.
Scales must agree within 1e-3 relative (one fp16 ulp), zeros exactly except in
class (ii), and the output error ||(W - Q) X^T||_F^2 within 1% of the oracle's.

verify_layer() goes further where the oracle's inputs are at hand: a row whose
mismatches are not all plain ties is replayed through the oracle, which is
made to take the GPU's side of each tie it meets (both sides of a tie are
correct results); everything after the tie must then agree again.  A row is
accepted only if every divergence it shows is such a tie.  The replays are
returned, so a later step (the next layer of a block) can be computed by the
oracle from its own result on the GPU's side of the ties.
"""
from __future__ import annotations

from collections import Counter
from typing import Dict

import numpy as np

TAU = 1e-3
CASCADE = 0.05
SCALE_TIE = 1e-5


def classify(gpu: Dict[str, np.ndarray], ora: Dict[str, np.ndarray], margins: Dict[str, np.ndarray],
             group_size: int) -> Dict[str, object]:
    codes_g, codes_o = gpu["codes"].astype(np.int64), ora["codes"].astype(np.int64)
    rows, d = codes_o.shape
    perm = np.asarray(ora["perm"], dtype=np.int64)
    pos = np.empty(d, dtype=np.int64)
    pos[perm] = np.arange(d)
    sc_g, sc_o = gpu["scales"].astype(np.float64), ora["scales"].astype(np.float64)
    z_g, z_o = gpu["zeros"].astype(np.int64), ora["zeros"].astype(np.int64)

    # static groups: parameters are fixed before the loop and a group holds
    # original columns
    static = ora.get("static") is not None
    events = []   # (row, k, kind, index)
    pr, pg = np.nonzero((sc_g != sc_o) | (z_g != z_o))
    for r, gi in zip(pr.tolist(), pg.tolist()):
        events.append((r, -1 if static else gi * group_size, 0, gi))
    cr, cc = np.nonzero(codes_g != codes_o)
    for r, c in zip(cr.tolist(), cc.tolist()):
        events.append((r, int(pos[c]), 1, c))
    events.sort()

    counts = Counter()
    unexplained = []
    shifted_groups = set()
    admissible_rows = set()
    for r, k, kind, idx in events:
        if kind == 0:
            gi = idx
            scale_rel = abs(sc_g[r, gi] - sc_o[r, gi]) / max(sc_o[r, gi], 1e-30)
            zero_d = abs(z_g[r, gi] - z_o[r, gi])
            tie = margins["scale"][r, gi] < SCALE_TIE or margins["zero"][r, gi] < TAU
            if scale_rel <= 1.0e-3 and zero_d <= 1 and tie:
                counts["ii_param"] += 1
            elif scale_rel <= 1.0e-3 and zero_d <= 1 and r in admissible_rows:
                counts["iii_param"] += 1
            else:
                unexplained.append(("param", r, gi, scale_rel, zero_d))
                continue
            shifted_groups.add((r, gi))
            admissible_rows.add(r)
        else:
            c = idx
            gi = c // group_size if static else k // group_size
            delta = abs(codes_g[r, c] - codes_o[r, c])
            m = margins["code"][r, c]
            if delta != 1:
                unexplained.append(("code", r, c, int(delta), float(m)))
                continue
            if (r, gi) in shifted_groups:
                counts["ii_code"] += 1
            elif m < TAU:
                counts["i"] += 1
            elif r in admissible_rows and m < CASCADE:
                counts["iii"] += 1
            else:
                unexplained.append(("code", r, c, int(delta), float(m)))
                continue
            admissible_rows.add(r)
    n_code_mis = int((codes_g != codes_o).sum())
    return dict(match=1.0 - n_code_mis / codes_o.size, mismatches=n_code_mis, counts=dict(counts),
                unexplained=unexplained, scale_max_rel=float(np.max(np.abs(sc_g - sc_o) / np.maximum(sc_o, 1e-30))))


def dequant(codes, scales, zeros, g_idx) -> np.ndarray:
    s = np.asarray(scales, dtype=np.float64)[:, g_idx]
    z = np.asarray(zeros, dtype=np.int64)[:, g_idx]
    return s * (np.asarray(codes, dtype=np.int64) - z)


def assert_layer_parity(rep: Dict[str, object], e_gpu: float, e_ora: float, what: str = "") -> None:
    assert not rep["unexplained"], f"{what}: unexplained mismatches {rep['unexplained'][:10]} counts={rep['counts']}"
    assert rep["match"] >= 0.999, f"{what}: code match {rep['match']:.6f} {rep['counts']}"
    assert rep["scale_max_rel"] <= 1.0e-3, f"{what}: scale rel diff {rep['scale_max_rel']}"
    assert abs(e_gpu - e_ora) <= 0.01 * e_ora, f"{what}: recon error {e_gpu} vs {e_ora}"


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits).astype(np.uint16).view(np.float16).astype(np.float32)


def _first_divergence(gq, gs, gz, oq, os_, oz, group_size, static=False):
    """First (k, kind) where a GPU row and an oracle row differ, in
    quantization order; kind 'param' at a group start, 'code' otherwise.
    Static groups are fixed before the loop: a parameter difference comes
    first, reported at k = group * group_size."""
    d = len(oq)
    pd = np.nonzero((gs != os_) | (gz != oz))[0]
    cd = np.nonzero(gq != oq)[0]
    if static and len(pd):
        return int(pd[0]) * group_size, "param"
    kp = pd[0] * group_size if len(pd) else d
    kc = cd[0] if len(cd) else d
    if kp >= d and kc >= d:
        return None
    if kp <= kc:
        return int(kp), "param"
    return int(kc), "code"


def verify_layer(gpu: Dict[str, np.ndarray], W: np.ndarray, ora: Dict[str, np.ndarray], bits: int,
                 group_size: int, max_ties_per_row: int = 16, sym: bool = False,
                 follow_all: bool = False) -> Dict[str, object]:
    """Classify every mismatch; rows whose mismatches are not all plain near-ties
    (every row with a mismatch, with ``follow_all``) are replayed through the
    oracle, following the GPU's side of each tie (rows are independent given
    U), until the row agrees or a decision that was not a tie differs."""
    import oracle as O

    rep = classify(gpu, ora, O.decision_margins(ora, bits, group_size, sym), group_size)
    perm = np.asarray(ora["perm"], dtype=np.int64)
    d = len(perm)
    static = ora.get("static")
    # group of each column in quantization order (static groups: the original
    # column's group)
    qgroup = static["col_group"] if static is not None else np.arange(d) // group_size
    plain = {"i", "ii_code", "ii_param"}
    bad_rows = sorted({u[1] for u in rep["unexplained"]})
    if follow_all or set(rep["counts"]) - plain:
        # rows with cascade classes: find them by re-classifying per row
        codes_g, codes_o = gpu["codes"], ora["codes"]
        rows = np.nonzero((codes_g != codes_o).any(1) | (gpu["scales"] != ora["scales"]).any(1)
                          | (gpu["zeros"] != ora["zeros"]).any(1))[0]
        bad_rows = sorted(set(bad_rows) | set(rows.tolist()))
    unexplained = []
    ties = 0
    replayed = 0
    followed = {}
    for r in bad_rows:
        force = {}
        gq = gpu["codes"][r][perm].astype(np.int64)
        gs = gpu["scales"][r].astype(np.float32)
        gz = gpu["zeros"][r].astype(np.int64)
        replayed += 1
        st_r = None
        if static is not None:
            st_r = {k: (v[r:r + 1].copy() if k != "col_group" else v) for k, v in static.items()}
        while True:
            o = O.gptq_quantize(W[r:r + 1, perm], ora["U"], bits=bits, group_size=group_size,
                                block_size=128, force=force, sym=sym, static=st_r)
            oq, os_, oz = o["codes"][0], o["scales"][0], o["zeros"][0]
            div = _first_divergence(gq, gs, gz, oq, os_, oz, group_size, static is not None)
            if div is None:
                followed[int(r)] = o
                break
            k, kind = div
            m = O.decision_margins(dict(scales=o["scales"], g_idx=qgroup, pre=o["pre"],
                                        gmin=o["gmin"], gmax=o["gmax"]), bits, group_size, sym)
            gi = k // group_size
            if kind == "param":
                srel = abs(float(gs[gi]) - float(os_[gi])) / max(float(os_[gi]), 1e-30)
                tie = m["scale"][0, gi] < SCALE_TIE or m["zero"][0, gi] < TAU
                ok = tie and srel <= 1.0e-3 and abs(int(gz[gi]) - int(oz[gi])) <= 1
                fix = {"s": gs[gi], "z": int(gz[gi])}
            else:
                ok = m["code"][0, k] < TAU and abs(int(gq[k]) - int(oq[k])) == 1
                fix = {"q": int(gq[k])}
            if not ok or len(force) >= max_ties_per_row:
                unexplained.append((kind, int(r), int(k)))
                break
            if st_r is not None and kind == "param":
                # static parameters are set before the loop: change the group's
                st_r["s"][0, gi] = gs[gi]
                st_r["z"][0, gi] = gz[gi]
                force[-1 - gi] = fix      # a key no column has: counts toward the row limit only
            else:
                force[k] = {**force.get(k, {}), **fix}
            ties += 1
    out = dict(rep)
    out.update(unexplained=unexplained, forced_ties=ties, replayed_rows=replayed, followed=followed)
    return out


def follow_gpu_ties(ora: Dict[str, np.ndarray], rep: Dict[str, object]) -> np.ndarray:
    """The oracle's dequantized weights (original column order) with every
    replayed row taken from its replay, i.e. the oracle's own result on the
    GPU's side of each tie."""
    Q = np.array(ora["Q"], dtype=np.float64, copy=True)
    perm = np.asarray(ora["perm"], dtype=np.int64)
    for r, o in rep["followed"].items():
        Q[r, perm] = o["Q"][0]
    return Q


def assert_verified(rep: Dict[str, object], e_gpu: float, e_ora: float, what: str = "") -> None:
    assert not rep["unexplained"], f"{what}: mismatches not at a tie {rep['unexplained'][:10]}"
    assert rep["match"] >= 0.999, f"{what}: code match {rep['match']:.6f}"
    assert abs(e_gpu - e_ora) <= 0.01 * e_ora, f"{what}: recon error {e_gpu} vs {e_ora}"


def w4a16_error_bound(X: np.ndarray, codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                      g_idx: np.ndarray, bias: float = 0.0, unit: float = 2.0 ** -24) -> np.ndarray:
    """Tolerance of an fp32 evaluation of Y = X Q^T, per output element.

    Any evaluation that forms the terms x * s * (q + bias) and x * s * (z +
    bias) exactly or with one rounding each, and sums them in any order with
    one rounding per addition, is within d_in * unit * sum_c |x_c| s (q_c + z
    + 2 bias) of the exact value (first-order forward error of summation); the
    factor 2 covers the scaling of each group's partial sum.  ``bias`` is a
    constant added to every code and taken off again through the zero (the
    integers re-encoded in a narrower float format)."""
    s = np.asarray(scales, dtype=np.float64)[:, g_idx]
    z = np.asarray(zeros, dtype=np.float64)[:, g_idx]
    mag = s * (np.asarray(codes, dtype=np.float64) + z + 2.0 * bias)
    k = mag.shape[1]
    return 2.0 * k * unit * (np.abs(np.asarray(X, dtype=np.float64)) @ mag.T)
