#!/usr/bin/env python3
"""GPTQ layer quantization benchmark on one MI355X.

One step = the whole path for one layer (or all experts of an MoE layer):
zero the Hessian state, accumulate every calibration chunk, damp + order +
factor, quantize every column with error feedback, pack codes and zeros.
Inputs (W and all of X) are resident in HBM before the timed region.

    python bench.py [--steps K] [--warmup W] [--config up_proj_70b]

Prints one JSON line.  The default workload is the Llama-70B-shaped FFN
up_proj layer (W 28672x8192 bf16, X 262144x8192 bf16 streamed in 16 chunks of
16384 tokens, INT4 and INT3 g128 on the same Hessian and factor).

The K timed steps run with no per-kernel event records (ms_per_step); the
same K steps then run again with the library's per-launch HIP events on, which
gives the phase times and the roofline kernel's mean launch duration.  Two
reference kernels (an MFMA loop on registers, a 1 GiB device copy) give the
rates this GPU sustains, reported next to the published peaks.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms per layer & weights/s for GPTQ INT4 g128; % MFMA peak per phase"
PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3, "f64": 78.6}
HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_syrk.json")
SYRK_SRC = os.path.join(ROOT, "post_weight_quantization_08_amd", "csrc", "hessian.hip")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def describe(cfg, sym: bool = False, static_groups: bool = False, awq: bool = False) -> str:
    e = f"{cfg.n_experts} experts x " if cfg.n_experts else ""
    chunks = f", {cfg.n_chunks} chunks of {cfg.chunk_tokens}" if cfg.name == "up_proj_70b" else ""
    bits = "/".join(f"INT{b}" for b in cfg.bits)
    ao = ", act-order" if cfg.act_order else ""
    sy = (", symmetric" if sym else "") + (", static groups" if static_groups else "")
    sy += ", activation-aware scaling first (20 candidates, 512 sample tokens)" if awq else ""
    return (f"{cfg.name}: W {e}{cfg.d_out}x{cfg.d_in} {cfg.w_dtype}, X {cfg.n_tokens}x{cfg.d_in} {cfg.x_dtype}"
            f"{chunks}, {bits} g{cfg.group_size}{ao}{sy}")


def source_sha(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def _oracle_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(cfg, W_host, x_host, routes, budget_chunks: int = 8, rows: int = 1024, sym: bool = False,
                 static_groups: bool = False):
    """The float64 oracle on a bounded sample of the same workload, scaled to
    the whole layer: the Hessian over `budget_chunks` chunks (scaled by the
    token count), the full factorization, and the column loop over `rows`
    weight rows (scaled by d_out and by the number of bit widths)."""
    import oracle as O
    import synth
    cores = _oracle_threads()
    e0 = 0
    chunk = cfg.chunk_tokens
    n_used = min(cfg.n_tokens, budget_chunks * chunk)
    t = time.perf_counter()
    S = np.zeros((cfg.d_in, cfg.d_in))
    n = 0
    for c in range(0, n_used, chunk):
        X = synth.to_f64(x_host[c:c + chunk], cfg.x_dtype)
        if routes is not None:
            r = routes[e0]
            X = X[r[(r >= c) & (r < c + chunk)] - c]
        S += X.T @ X
        n += X.shape[0]
    t_h = time.perf_counter() - t
    tokens_total = len(routes[e0]) if routes is not None else cfg.n_tokens
    tokens_sample = n
    t = time.perf_counter()
    H0 = O.hessian(S, n)
    _, Hd = O.damping(H0, cfg.damp_rel)
    perm = O.act_order_perm(H0) if cfg.act_order else np.arange(cfg.d_in)
    U = O.inverse_factor(Hd[np.ix_(perm, perm)])
    t_f = time.perf_counter() - t
    rows = min(rows, cfg.d_out)
    W0 = synth.to_f64(W_host[e0][:rows], cfg.w_dtype)
    Wr = W0[:, perm]
    t = time.perf_counter()
    st = None
    if static_groups:
        st = O.static_group_params(W0, cfg.bits[0], cfg.group_size, sym)
        st["col_group"] = perm // cfg.group_size
    O.gptq_quantize(Wr, U, bits=cfg.bits[0], group_size=cfg.group_size, block_size=cfg.block_size, sym=sym,
                    static=st)
    t_q = time.perf_counter() - t
    nb = len(cfg.bits)
    per_entry = t_h * tokens_total / max(tokens_sample, 1) + t_f + t_q * nb * cfg.d_out / rows
    if routes is not None:
        # other experts: Hessian work scales with their token counts
        per_entry_total = sum(t_h * len(r) / max(tokens_sample, 1) + t_f + t_q * nb * cfg.d_out / rows for r in routes)
    else:
        per_entry_total = per_entry
    weights = cfg.batch * cfg.d_out * cfg.d_in
    return {
        "value": weights / per_entry_total,
        "unit": "weights/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle: Hessian over {tokens_sample} of {tokens_total} tokens "
                   f"({t_h:.2f} s), full {cfg.d_in}x{cfg.d_in} factor ({t_f:.2f} s), column loop over "
                   f"{rows} of {cfg.d_out} rows ({t_q:.2f} s, x{nb} bit widths); scaled to the whole layer = "
                   f"{per_entry_total:.1f} s"),
    }


def bench_w4a16(args) -> int:
    """The W4A16 consumer of the packed format on one layer shape: M tokens
    (decode: 1) times the layer's 4-bit weights, inputs resident in HBM.  One
    step is one gptq_w4a16_matmul call (staging + main kernel)."""
    import torch

    import synth
    import post_weight_quantization_08_amd as G
    from post_weight_quantization_08_amd import pipeline as P

    cfg = synth.CONFIGS[args.config]
    if cfg.x_dtype not in ("f16", "bf16"):
        raise SystemExit("W4A16 needs fp16 or bf16 activations")
    m = args.tokens
    act_order = cfg.act_order or args.config == "up_proj_70b"
    log(f"[bench] W4A16 {cfg.name}: {cfg.d_out}x{cfg.d_in}, {m} token(s) {cfg.x_dtype}, g{cfg.group_size}"
        f"{', act-order' if act_order else ''}")
    codes, scales, zeros, perm, g_idx = synth.w4_layer(cfg, act_order)
    X = synth.w4_tokens(cfg, m)
    dt = {"f16": torch.float16, "bf16": torch.bfloat16}[cfg.x_dtype]
    Xd = torch.from_numpy(X.view(np.int16)).cuda().view(dt)
    cd = torch.from_numpy(codes).cuda()
    pd = torch.from_numpy(perm).cuda() if perm is not None else None
    qw = P.pack_int4_permuted(cd, pd) if pd is not None else P.pack(cd, 4)
    del cd
    sd = torch.from_numpy(scales.view(np.int16)).cuda()
    zd = torch.from_numpy(zeros).cuda()
    Y = torch.empty(m, cfg.d_out, dtype=torch.float32, device="cuda")
    ws = torch.empty(G.gptq_workspace_size(G.OP_W4A16, None, cfg.d_out, cfg.d_in, m, 1), dtype=torch.uint8,
                     device="cuda")
    for _ in range(args.warmup):
        P.w4a16_matmul(Xd, qw, sd, zd, cfg.group_size, perm=pd, Y=Y, ws=ws)
    # wall clock with no event records between the launches, then the same
    # number of calls again with per-kernel events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        P.w4a16_matmul(Xd, qw, sd, zd, cfg.group_size, perm=pd, Y=Y, ws=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    G.gptq_timing_reset()
    G.gptq_timing_enable(True)
    for _ in range(args.steps):
        P.w4a16_matmul(Xd, qw, sd, zd, cfg.group_size, perm=pd, Y=Y, ws=ws)
    torch.cuda.synchronize()
    G.gptq_timing_enable(False)
    main_ms, main_n = G.gptq_timing_read(G.TIME_W4_MAIN)
    stage_ms, _ = G.gptq_timing_read(G.TIME_W4_STAGE)
    G.gptq_timing_reset()
    ms = (t1 - t0) * 1e3 / args.steps
    avg_main = main_ms / max(main_n, 1)
    ng = cfg.d_in // cfg.group_size
    xb = 2
    algo = cfg.d_out * cfg.d_in // 2 + cfg.d_out * ng * 3 + m * cfg.d_in * xb + m * cfg.d_out * 4
    achieved = algo / (avg_main * 1e-3) / 1e9
    traffic = None
    tf = os.path.join(ROOT, "profiles", "traffic_w4a16.json")
    if os.path.exists(tf):
        tr = json.load(open(tf))
        src = os.path.join(ROOT, "post_weight_quantization_08_amd", "csrc", "w4a16.hip")
        if tr.get("source_sha256") == source_sha(src) and tr.get("workload") == f"{cfg.name}:{m}":
            traffic = tr.get("bytes_per_launch")
    weights = cfg.d_out * cfg.d_in
    line = {
        "metric": "W4A16 matmul of a packed 4-bit layer: weights consumed per second",
        "value": weights / (ms * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.x_dtype,
        "data": "synthetic",
        "config": {"workload": f"W4A16 {cfg.name}: {cfg.d_out}x{cfg.d_in} INT4 g{cfg.group_size}"
                               f"{' act-order' if act_order else ''}, {m} token(s) {cfg.x_dtype}",
                   "d_out": cfg.d_out, "d_in": cfg.d_in, "tokens": m, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "w4_main_kernel", "achieved": achieved, "peak": 8000.0,
                     "unit": "GB/s", "frac": achieved / 8000.0, "traffic": traffic,
                     "avg_launch_ms": avg_main, "bytes_per_launch": algo},
        "phases_ms": {"stage": stage_ms / args.steps, "main": main_ms / args.steps},
    }
    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        t = time.perf_counter()
        b.copy_(a)
        torch.cuda.synchronize()
        line["copy_probe"] = {"bytes": 1 << 30, "ms": (time.perf_counter() - t) * 1e3}
        del a, b
    if not args.no_cpu_baseline:
        import oracle as O
        rows = min(cfg.d_out, 4096)
        Xf = synth.to_f64(X, cfg.x_dtype)
        s32 = scales.view(np.float16).astype(np.float32)
        t = time.perf_counter()
        O.w4a16_matmul(Xf, O.pack_int4(codes[:rows]), s32[:rows], zeros[:rows], g_idx)
        tc = (time.perf_counter() - t) * cfg.d_out / rows
        line["cpu_baseline"] = {"value": weights / tc, "unit": "weights/s", "cores": _oracle_threads(),
                                "kind": "oracle",
                                "sample": f"float64 oracle (unpack, dequantize, matmul) over {rows} of "
                                          f"{cfg.d_out} rows, scaled to the layer: {tc:.2f} s"}
    log(f"[bench] W4A16 {ms * 1e3:.1f} us/call, main kernel {avg_main * 1e3:.1f} us = {achieved:.0f} GB/s")
    print(json.dumps(line), flush=True)
    return 0


def bench_block(args) -> int:
    """Sequential calibration of a Llama-7B-shaped MLP block (up 4096 -> 11008,
    SiLU, down 11008 -> 4096, fp16): layer 1 on the calibration tokens, layer
    2 on the rounded activations of the quantized layer 1.  One step is the
    whole chain, inputs resident in HBM."""
    import torch

    import synth
    import post_weight_quantization_08_amd as G
    from post_weight_quantization_08_amd import pipeline as P

    d, h, n = 4096, 11008, args.block_tokens
    cfg = synth.CONFIGS["q_proj_7b"].scaled("block", 490, d_out=h, d_in=d, n_tokens=n)
    log(f"[bench] block: up {d}->{h}, SiLU, down {h}->{d}, {n} calibration tokens f16, INT4 g128")
    X = synth.x_all(cfg, threads=16)
    r = np.random.default_rng([490, 7])
    W1 = torch.from_numpy((r.standard_normal((h, d), dtype=np.float32) * 0.02).astype(np.float16)).cuda()
    W2 = torch.from_numpy((r.standard_normal((d, h), dtype=np.float32) * 0.02).astype(np.float16)).cuda()
    Xd = torch.from_numpy(X).cuda()
    chunks = [Xd[i:i + cfg.chunk_tokens] for i in range(0, n, cfg.chunk_tokens)]
    p = G.GptqParams.make()
    for _ in range(args.warmup):
        P.calibrate_block(chunks, W1, W2, p, G.ACT_SILU)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        P.calibrate_block(chunks, W1, W2, p, G.ACT_SILU)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    G.gptq_timing_reset()
    G.gptq_timing_enable(True)
    P.calibrate_block(chunks, W1, W2, p, G.ACT_SILU)
    torch.cuda.synchronize()
    G.gptq_timing_enable(False)
    kinds = {"hessian_mfma": G.TIME_SYRK, "hessian_split_reduce": G.TIME_SYRK_REDUCE, "diag_fp64": G.TIME_DIAG,
             "factor_fp64": G.TIME_FACTOR, "prep": G.TIME_PREP, "block_quant": G.TIME_BLOCK_QUANT,
             "deferred_update_mfma": G.TIME_TRAILING, "forward": G.TIME_FORWARD}
    phases = {k: G.gptq_timing_read(v)[0] for k, v in kinds.items()}
    G.gptq_timing_reset()
    fw_flops = 2.0 * n * d * h * 2        # two fp16 products per multiply-add (X times Q's hi and lo terms)
    weights = 2 * d * h
    line = {
        "metric": "sequential calibration of an MLP block: weights quantized per second",
        "value": weights / (ms * 1e-3), "unit": "weights/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"MLP block up {d}->{h}, SiLU, down {h}->{d}, {n} tokens f16, INT4 g128",
                   "tokens": n, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "split_gemm_kernel (layer 1 output for layer 2)",
                     "achieved": fw_flops / (phases["forward"] * 1e-3) / 1e12, "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": fw_flops / (phases["forward"] * 1e-3) / 1e12 / 2500.0, "traffic": None},
        "phases_ms": phases,
    }
    log(f"[bench] block {ms:.1f} ms, phases {json.dumps(phases)}")
    print(json.dumps(line), flush=True)
    return 0


PHASE_KINDS = ["hessian_mfma", "hessian_split_reduce", "diag_fp64", "factor_fp64", "prep", "block_quant",
               "deferred_update_mfma", "pack"]


def _kind_ids(G):
    return {"hessian_mfma": G.TIME_SYRK, "hessian_split_reduce": G.TIME_SYRK_REDUCE, "diag_fp64": G.TIME_DIAG,
            "factor_fp64": G.TIME_FACTOR, "prep": G.TIME_PREP, "block_quant": G.TIME_BLOCK_QUANT,
            "deferred_update_mfma": G.TIME_TRAILING, "pack": G.TIME_PACK, "abs_sum": G.TIME_ABS,
            "awq_search": G.TIME_AWQ_SEARCH, "awq_apply": G.TIME_AWQ_APPLY}


def reference_rates(G, torch, dev) -> dict:
    """Measured ceilings on this GPU: MFMA loops (fp16, bf16, fp64) and a 1 GiB copy."""
    sink = torch.empty(G.gptq_probe_sink_bytes() // 4, dtype=torch.float32, device=dev)
    # kinds 0-2 keep one operand set in registers; 3 and 4 feed every MFMA new
    # random operands, as the Hessian product's streamed tokens do
    out = {"mfma_f16_tflops": G.gptq_probe_mfma(0, 20000, sink),
           "mfma_bf16_tflops": G.gptq_probe_mfma(1, 20000, sink),
           "mfma_f64_tflops": G.gptq_probe_mfma(2, 20000, sink),
           "mfma_f16_streaming_tflops": G.gptq_probe_mfma(3, 20000, sink),
           "mfma_bf16_streaming_tflops": G.gptq_probe_mfma(4, 20000, sink)}
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    gbs, ms = G.gptq_probe_copy(a, b, 1 << 30)
    out.update({"copy_gbs": gbs, "copy_bytes": 1 << 30, "copy_ms": ms})
    del a, b, sink
    torch.cuda.synchronize()
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="up_proj_70b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sym", action="store_true", help="symmetric groups (fixed zero 2^(bits-1))")
    ap.add_argument("--group-size", type=int, default=None, help="override the workload's group size")
    ap.add_argument("--static-groups", action="store_true",
                    help="fix every group's scale and zero from W before the column loop")
    ap.add_argument("--w4a16", action="store_true",
                    help="time the W4A16 consumer of the packed format instead of quantization")
    ap.add_argument("--tokens", type=int, default=1, help="tokens per W4A16 call")
    ap.add_argument("--block", action="store_true",
                    help="sequential calibration of a Llama-7B-shaped MLP block instead of one layer")
    ap.add_argument("--block-tokens", type=int, default=65536, help="calibration tokens for --block")
    ap.add_argument("--awq", action="store_true",
                    help="activation-aware channel scaling before GPTQ (20 candidates, 512 sample tokens)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="W4A16 mode: also run a plain device copy of 1 GiB (scales HBM counters)")
    ap.add_argument("--hessian-only", action="store_true",
                    help="time only the Hessian accumulation of the workload (S, D, N from zero)")
    ap.add_argument("--x-fill", choices=["random", "zeros"], default="random",
                    help="calibration tokens: the workload's random recipe, or all zeros (with --hessian-only: "
                         "the same launches on operands that draw less power)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2
    if args.x_fill == "zeros" and not args.hessian_only:
        print("--x-fill zeros needs --hessian-only (an all-zero Hessian has no factor)", file=sys.stderr)
        return 2

    if args.w4a16:
        return bench_w4a16(args)
    if args.block:
        return bench_block(args)

    import torch

    import synth
    import post_weight_quantization_08_amd as G
    from post_weight_quantization_08_amd import pipeline as P

    cfg = synth.CONFIGS[args.config]
    if args.group_size:
        cfg = dataclasses.replace(cfg, group_size=args.group_size)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    log(f"[bench] {describe(cfg, args.sym, args.static_groups, args.awq)}"
        f"{' (Hessian only, X ' + args.x_fill + ')' if args.hessian_only else ''}")

    t = time.perf_counter()
    W_host = np.stack([synth.weights(cfg, e) for e in range(cfg.batch)])
    routes = synth.routing(cfg) if cfg.n_experts else None
    from post_weight_quantization_08_amd.pipeline import to_device
    W = to_device(W_host, cfg.w_dtype, dev)
    if args.x_fill == "zeros":
        x_host = None
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[cfg.x_dtype]
        X = torch.zeros(cfg.n_tokens, cfg.d_in, dtype=tdt, device=dev)
    else:
        x_host = synth.x_all(cfg, threads=16)
        X = to_device(x_host, cfg.x_dtype, dev)
    log(f"[bench] inputs generated and uploaded in {time.perf_counter() - t:.1f} s")
    calls = []
    if routes is not None:
        idx = torch.from_numpy(np.concatenate(routes).astype(np.int32)).to(dev)
        ptr = np.zeros(cfg.batch + 1, dtype=np.int64)
        ptr[1:] = np.cumsum([len(r) for r in routes])
        calls.append((X, idx, ptr.tolist()))
    elif cfg.name == "up_proj_70b":
        for c in range(cfg.n_chunks):       # streamed in 16384-token chunks
            t0, t1 = cfg.chunk_range(c)
            calls.append((X[t0:t1], None, None))
    else:
        calls.append((X, None, None))
    torch.cuda.synchronize()

    if args.awq and cfg.batch != 1:
        print("bench.py --awq times one layer (not the expert batch)", file=sys.stderr)
        return 2
    state = P.HessianState(cfg.d_in, cfg.batch, dev, track_abs=args.awq)
    alphas = [i / 20 for i in range(20)]
    Xs = calls[0][0][:512]
    plist = [G.GptqParams.make(bits=b, group_size=cfg.group_size, block_size=cfg.block_size,
                               damp_rel=cfg.damp_rel, act_order=cfg.act_order, sym=args.sym,
                               static_groups=args.static_groups) for b in cfg.bits]
    prep_ws = torch.empty(G.gptq_workspace_size(G.OP_PREPARE, None, 1, cfg.d_in, 0, cfg.batch),
                          dtype=torch.uint8, device=dev)
    # one quantize workspace per bit width: with several widths (70B: INT4 and
    # INT3 from the same S and U) each runs on a stream of its own, so one
    # width's latency-bound column loop overlaps the other's update GEMMs
    q_ws = [torch.empty(G.gptq_workspace_size(G.OP_QUANTIZE, p, cfg.d_out, cfg.d_in, 0, cfg.batch),
                        dtype=torch.uint8, device=dev) for p in plist]
    q_streams = [torch.cuda.Stream() for _ in plist] if len(plist) > 1 else None
    for Xc, idx, ptr in calls:
        state.workspace(Xc.shape[0] if idx is None else int(np.max(np.diff(ptr))))

    out = {}

    def step():
        state.zero()
        for Xc, idx, ptr in calls:
            state.add(Xc, idx, ptr)
        if args.hessian_only:
            return
        Wq = W
        if args.awq:
            r = P.awq_search(W[0], state, Xs, plist[0], alphas)
            Wq = P.awq_apply(W[0], state, r["s"])
        prep = P.prepare(state, plist[0], ws=prep_ws, check=False)
        if q_streams is None:
            res = P.quantize(Wq, prep, plist[0], ws=q_ws[0])
            out[plist[0].bits] = (P.pack(res["codes"], plist[0].bits), P.pack(res["zeros"], plist[0].bits), res, prep)
            return
        ready = torch.cuda.Event()
        ready.record()
        cur = torch.cuda.current_stream()
        for p, ws, st in zip(plist, q_ws, q_streams):
            st.wait_event(ready)
            with torch.cuda.stream(st):
                res = P.quantize(Wq, prep, p, ws=ws, stream=st)
                out[p.bits] = (P.pack(res["codes"], p.bits, stream=st), P.pack(res["zeros"], p.bits, stream=st),
                               res, prep)
        for st in q_streams:
            cur.wait_stream(st)

    def run(k: int) -> float:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(k):
            step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3

    G.gptq_timing_enable(False)
    run(args.warmup)
    # the timed steps: no event records between the launches
    ms = run(args.steps) / args.steps
    # the same steps again with the library's per-launch events on
    G.gptq_timing_reset()
    G.gptq_timing_enable(True)
    ms_events = run(args.steps) / args.steps
    G.gptq_timing_enable(False)
    if not args.hessian_only:
        info = out[plist[0].bits][3].info.cpu().numpy()
        if np.any(info != 0):
            raise G.GptqError(G.ENOTPD, f"prepare info {info.tolist()}")

    ids = _kind_ids(G)
    kinds = list(PHASE_KINDS) + (["abs_sum", "awq_search", "awq_apply"] if args.awq else [])
    phases, launches = {}, {}
    for name in kinds:
        tot, n = G.gptq_timing_read(ids[name])
        phases[name] = tot / args.steps
        launches[name] = n // args.steps
    G.gptq_timing_reset()
    rates = reference_rates(G, torch, dev)

    d, dout, nb = cfg.d_in, cfg.d_out, cfg.batch
    nbits = len(cfg.bits)
    rows_total = sum(len(r) for r in routes) if routes is not None else cfg.n_tokens
    hess_flops = rows_total * d * (d + 1)                          # lower triangle, 2 flops per MAC
    trail_flops = nb * dout * d * (d - 128) * nbits               # one product per multiply-add
    factor_flops = nb * 2.0 * d ** 3 / 3.0
    xdt = cfg.x_dtype
    syrk_launches = max(launches["hessian_mfma"], 1)
    syrk_avg_ms = phases["hessian_mfma"] / syrk_launches
    achieved = hess_flops / syrk_launches / (syrk_avg_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[xdt]
    onbox_mm = rates["mfma_bf16_tflops"] if xdt == "bf16" else rates["mfma_f16_tflops"]
    onbox_stream = rates["mfma_bf16_streaming_tflops"] if xdt == "bf16" else rates["mfma_f16_streaming_tflops"]

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        ent = tr.get("workloads", {}).get(cfg.name)
        if ent and tr.get("source_sha256") == source_sha(SYRK_SRC):
            traffic = ent.get("bytes_per_launch")
    # algorithmic bytes of one accumulation launch: its token rows of X read
    # once, and the lower triangle of S read and written once
    xbytes = {"f32": 4, "f16": 2, "bf16": 2}[xdt]
    syrk_algo_bytes = (rows_total / syrk_launches) * d * xbytes + 8.0 * d * (d + 1) / 2

    def pct(flops, ms_, pk):
        return 100.0 * flops / max(ms_ * 1e-3, 1e-12) / 1e12 / pk

    weights = nb * dout * d
    line = {
        "metric": METRIC,
        "value": (rows_total * d if args.hessian_only else weights) / (ms * 1e-3),
        "unit": "tokens x channels/s" if args.hessian_only else "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": xdt,
        "data": "synthetic" + (" (all-zero X)" if args.x_fill == "zeros" else ""),
        "config": {"workload": describe(cfg, args.sym, args.static_groups, args.awq)
                   + (" -- Hessian accumulation only" if args.hessian_only else ""),
                   "d_out": dout, "d_in": d, "experts": cfg.n_experts,
                   "n_tokens": cfg.n_tokens, "bits": list(cfg.bits), "group_size": cfg.group_size,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "syrk_dma_kernel (Hessian X^T X)",
                     "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": traffic, "algorithmic_bytes_per_launch": syrk_algo_bytes,
                     "traffic_ratio": (traffic / syrk_algo_bytes) if traffic else None,
                     "launches_per_step": syrk_launches, "avg_launch_ms": syrk_avg_ms,
                     "flops_per_launch": hess_flops / syrk_launches,
                     "onbox_peak": onbox_mm, "frac_of_onbox_peak": achieved / onbox_mm,
                     "onbox_streaming_peak": onbox_stream, "frac_of_onbox_streaming_peak": achieved / onbox_stream},
        "ms_per_step_with_events": ms_events,
        "phases_ms": phases,
        "launches_per_step": launches,
        "reference_rates": rates,
    }
    if not args.hessian_only:
        # algorithmic bytes: block quantizer reads the fp32 working tile and
        # writes codes (1 B), the tile's errors as two bf16 terms (4 B) and each
        # group's scale and zero (3 B); packing reads a code byte and writes
        # bits/8 bytes, plus the zeros (one byte read, bits/8 written per group)
        ng = d // cfg.group_size
        bq_bytes = nbits * nb * dout * (d * (4 + 1 + 4) + ng * 3)
        pack_bytes = sum(nb * dout * (d * (1 + b / 8) + ng * (1 + b / 8)) for b in cfg.bits)
        gbs = {"block_quant": bq_bytes / max(phases["block_quant"] * 1e-3, 1e-12) / 1e9,
               "pack": pack_bytes / max(phases["pack"] * 1e-3, 1e-12) / 1e9}
        line["phase_gbs"] = gbs
        line["phase_bytes"] = {"block_quant": bq_bytes, "pack": pack_bytes}
        spec_f64, onbox_f64 = PEAK_TFLOPS["f64"], rates["mfma_f64_tflops"]
        line["phase_pct_peak"] = {
            "hessian_mfma_pct_peak": 100.0 * achieved / peak,
            "hessian_mfma_pct_onbox": 100.0 * achieved / onbox_mm,
            "hessian_with_reduce_pct_peak": pct(hess_flops, phases["hessian_mfma"] + phases["hessian_split_reduce"], peak),
            "deferred_update_pct_bf16_peak": pct(trail_flops, phases["deferred_update_mfma"], 2500.0),
            # the split-bf16 update issues three bf16 products per multiply-add
            "deferred_update_3products_pct_bf16_peak": pct(3 * trail_flops, phases["deferred_update_mfma"], 2500.0),
            "deferred_update_pct_onbox": pct(trail_flops, phases["deferred_update_mfma"], rates["mfma_bf16_tflops"]),
            "factor_pct_fp64_peak": pct(factor_flops, phases["factor_fp64"], spec_f64),
            "factor_pct_onbox": pct(factor_flops, phases["factor_fp64"], onbox_f64),
            "block_quant_pct_hbm": 100.0 * gbs["block_quant"] / HBM_GBS,
            "block_quant_pct_copy": 100.0 * gbs["block_quant"] / rates["copy_gbs"],
            "pack_pct_hbm": 100.0 * gbs["pack"] / HBM_GBS,
            "pack_pct_copy": 100.0 * gbs["pack"] / rates["copy_gbs"],
        }
    if not args.no_cpu_baseline and not args.hessian_only:
        log("[bench] timing the float64 oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline(cfg, W_host, x_host, routes, sym=args.sym,
                                            static_groups=args.static_groups)
    log(f"[bench] {ms:.2f} ms/step ({ms_events:.2f} with events), phases {json.dumps(phases)}")
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
