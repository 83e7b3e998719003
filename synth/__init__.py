"""Seeded synthetic inputs for the GPTQ layer workloads.

This module only *makes inputs*: weights W, calibration activations X (in
16384-token chunks that can be regenerated independently and in any order),
and the top-2 expert routing of the mixture-of-experts layer.  It holds none
of the quantization method's arithmetic; both the float64 CPU oracle and the
GPU path take their inputs from here and from nowhere else.

Shapes and value structure follow the workloads the pages describe:

* calibration sets of 128-512 sequences (the "校准集 128~512 条" advice in
  "大模型量化实战（上）", selection-table notes);
* a small, fixed set of activation channels that are one to two orders of
  magnitude larger than the rest, 0.1%-1% of the channels, stable across
  inputs ("INT4/INT8 量化推理：从 GPTQ 到 AWQ 的取舍", §二 离群通道);
* for the MoE layer, cold experts that receive few tokens, topped up so every
  expert sees at least 128 samples (same page, §五 实测对比, the note under
  the table).

Seeds: every array is drawn from ``numpy.random.default_rng([cfg_id, stream,
index...])`` so that it depends only on (config, stream, index):
stream 0 = W (index = expert), 1 = outlier subset, 2 = per-channel std,
3 = X chunk (index = chunk), 4 = routing, 5 = stored form of a 4-bit layer
for the W4A16 consumer, 6 = its activation rows.  Values are drawn in float32 and cast
to the workload dtype with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterator, List, Optional, Sequence, Tuple

import numpy as np

CHUNK_TOKENS = 16384

DTYPES = ("f32", "f16", "bf16")


# ----------------------------------------------------------------------------
# dtype casts (round-to-nearest-even), storage as numpy arrays:
#   f32  -> float32, f16 -> float16, bf16 -> uint16 bit patterns
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, IEEE round-to-nearest-even.

    NaN inputs map to a quiet NaN; finite values that round past the bf16
    range become +-inf, as RNE requires.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def cast(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Cast a float32 array to the storage form of ``dtype`` (RNE)."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x32.astype(np.float16))
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of a stored array to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(stored).astype(np.float64)
    return np.asarray(stored).astype(np.float64)


def to_f32(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of a stored array to float32."""
    if dtype == "bf16":
        return bf16_bits_to_f32(stored)
    return np.asarray(stored).astype(np.float32)


# ----------------------------------------------------------------------------
# workload descriptions
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    cfg_id: int
    d_out: int
    d_in: int
    n_tokens: int
    w_dtype: str
    x_dtype: str
    w_std: float
    outlier_frac: float = 0.0          # fraction of channels (fixed random subset)
    outlier_mult: float = 1.0
    outlier_channels: Tuple[int, ...] = ()   # explicit list (overrides frac)
    chan_std_loguniform: Optional[Tuple[float, float]] = None
    bits: Tuple[int, ...] = (4,)
    group_size: int = 128
    block_size: int = 128
    damp_rel: float = 0.01
    act_order: bool = False
    chunk_tokens: int = CHUNK_TOKENS
    n_experts: int = 0                # 0 = dense layer
    zipf_s: float = 1.2
    top_k: int = 2
    min_expert_tokens: int = 128
    correlated: bool = False          # X = Z @ (I + 0.5 G / sqrt(d))

    @property
    def n_chunks(self) -> int:
        return max(1, math.ceil(self.n_tokens / self.chunk_tokens))

    @property
    def batch(self) -> int:
        return max(1, self.n_experts)

    def chunk_range(self, c: int) -> Tuple[int, int]:
        t0 = c * self.chunk_tokens
        return t0, min(self.n_tokens, t0 + self.chunk_tokens)

    @property
    def n_outliers(self) -> int:
        if self.outlier_channels:
            return len(self.outlier_channels)
        return int(round(self.outlier_frac * self.d_in))

    def scaled(self, name: str, cfg_id: int, **kw) -> "LayerConfig":
        """A smaller workload with the same recipe (used for parity tests)."""
        return dataclasses.replace(self, name=name, cfg_id=cfg_id, **kw)


# The five workloads: a tiny layer; Llama-7B q_proj and down_proj; a
# Llama-70B up_proj; a Mixtral-8x7B expert w1 with 8 experts.
CONFIGS = {
    "tiny": LayerConfig(
        name="tiny", cfg_id=1, d_out=64, d_in=256, n_tokens=512,
        w_dtype="f32", x_dtype="f32", w_std=0.02,
        outlier_channels=(3, 77), outlier_mult=20.0),
    "q_proj_7b": LayerConfig(
        name="q_proj_7b", cfg_id=2, d_out=4096, d_in=4096, n_tokens=128 * 2048,
        w_dtype="f16", x_dtype="f16", w_std=0.02,
        outlier_frac=0.005, outlier_mult=50.0),
    "down_proj_7b": LayerConfig(
        name="down_proj_7b", cfg_id=3, d_out=4096, d_in=11008, n_tokens=262144,
        w_dtype="f16", x_dtype="f16", w_std=0.02,
        chan_std_loguniform=(0.1, 10.0), outlier_frac=0.01, outlier_mult=30.0,
        act_order=True),
    "up_proj_70b": LayerConfig(
        name="up_proj_70b", cfg_id=4, d_out=28672, d_in=8192, n_tokens=262144,
        w_dtype="bf16", x_dtype="bf16", w_std=0.015,
        outlier_frac=0.003, outlier_mult=60.0, bits=(4, 3)),
    "moe_w1_8x7b": LayerConfig(
        name="moe_w1_8x7b", cfg_id=5, d_out=14336, d_in=4096, n_tokens=262144,
        w_dtype="bf16", x_dtype="bf16", w_std=0.02,
        outlier_frac=0.005, outlier_mult=40.0, n_experts=8),
}
CONFIG_ORDER = ["tiny", "q_proj_7b", "down_proj_7b", "up_proj_70b", "moe_w1_8x7b"]


def _rng(cfg: LayerConfig, *idx: int) -> np.random.Generator:
    return np.random.default_rng([cfg.cfg_id, *idx])


def outlier_channels(cfg: LayerConfig) -> np.ndarray:
    if cfg.outlier_channels:
        return np.asarray(cfg.outlier_channels, dtype=np.int64)
    k = cfg.n_outliers
    if k == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(cfg, 1).choice(cfg.d_in, size=k, replace=False))


def channel_factor(cfg: LayerConfig) -> np.ndarray:
    """Per-input-channel multiplier of the N(0,1) activations (float32)."""
    f = np.ones(cfg.d_in, dtype=np.float64)
    if cfg.chan_std_loguniform is not None:
        lo, hi = cfg.chan_std_loguniform
        f = np.exp(_rng(cfg, 2).uniform(math.log(lo), math.log(hi), cfg.d_in))
    oc = outlier_channels(cfg)
    f[oc] *= cfg.outlier_mult
    return f.astype(np.float32)


def weights(cfg: LayerConfig, expert: int = 0) -> np.ndarray:
    """W (d_out x d_in, row-major) in storage form of cfg.w_dtype."""
    z = _rng(cfg, 0, expert).standard_normal((cfg.d_out, cfg.d_in), dtype=np.float32)
    z *= np.float32(cfg.w_std)
    return cast(z, cfg.w_dtype)


def x_chunk(cfg: LayerConfig, c: int, factor: Optional[np.ndarray] = None) -> np.ndarray:
    """Calibration chunk c (n_c x d_in, token-major) in storage form."""
    t0, t1 = cfg.chunk_range(c)
    if factor is None:
        factor = channel_factor(cfg)
    z = _rng(cfg, 3, c).standard_normal((t1 - t0, cfg.d_in), dtype=np.float32)
    if cfg.correlated:
        z = z @ correlated_mixer(cfg)
    z *= factor[None, :]
    return cast(z, cfg.x_dtype)


def x_chunks(cfg: LayerConfig) -> Iterator[np.ndarray]:
    f = channel_factor(cfg)
    for c in range(cfg.n_chunks):
        yield x_chunk(cfg, c, f)


def x_all(cfg: LayerConfig, threads: int = 8) -> np.ndarray:
    """All of X (n_tokens x d_in) in storage form; chunks drawn in parallel."""
    from concurrent.futures import ThreadPoolExecutor

    f = channel_factor(cfg)
    st = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[cfg.x_dtype]
    out = np.empty((cfg.n_tokens, cfg.d_in), dtype=st)

    def work(c: int) -> None:
        t0, t1 = cfg.chunk_range(c)
        out[t0:t1] = x_chunk(cfg, c, f)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(work, range(cfg.n_chunks)))
    return out


# ----------------------------------------------------------------------------
# MoE routing (top-k over Zipf popularity, then a >= min_expert_tokens top-up)
# ----------------------------------------------------------------------------
def expert_popularity(cfg: LayerConfig) -> np.ndarray:
    p = (np.arange(cfg.n_experts, dtype=np.float64) + 1.0) ** (-cfg.zipf_s)
    return p / p.sum()


def routing(cfg: LayerConfig) -> List[np.ndarray]:
    """Sorted int64 token indices per expert.

    Each token picks ``top_k`` distinct experts with probability proportional
    to the Zipf popularity (Gumbel-top-k, i.e. sampling without replacement).
    An expert left with fewer than ``min_expert_tokens`` tokens is topped up
    with tokens drawn without replacement from those not routed to it.
    """
    E, N = cfg.n_experts, cfg.n_tokens
    if E == 0:
        return [np.arange(N, dtype=np.int64)]
    rng = _rng(cfg, 4)
    logp = np.log(expert_popularity(cfg))
    keys = logp[None, :] + rng.gumbel(size=(N, E))
    top = np.argsort(-keys, axis=1, kind="stable")[:, : cfg.top_k]
    out = []
    for e in range(E):
        mine = np.nonzero((top == e).any(axis=1))[0]
        if mine.size < cfg.min_expert_tokens:
            need = min(cfg.min_expert_tokens, N) - mine.size
            pool = np.setdiff1d(np.arange(N), mine, assume_unique=True)
            extra = _rng(cfg, 4, 1, e).choice(pool, size=need, replace=False)
            mine = np.sort(np.concatenate([mine, extra]))
        out.append(mine.astype(np.int64))
    return out


# ----------------------------------------------------------------------------
# Reduced workloads with the same recipes, sized so the oracle finishes in
# seconds while the GPU kernels still see several tiles and ragged tails.
# ----------------------------------------------------------------------------
def test_config(base: str, variant: str = "small") -> LayerConfig:
    c = CONFIGS[base]
    if variant == "small":
        sizes = {
            "tiny": dict(),
            "q_proj_7b": dict(d_out=200, d_in=640, n_tokens=3000, chunk_tokens=1024),
            "down_proj_7b": dict(d_out=136, d_in=1152, n_tokens=5000, chunk_tokens=2048),
            "up_proj_70b": dict(d_out=333, d_in=768, n_tokens=4099, chunk_tokens=1024),
            "moe_w1_8x7b": dict(d_out=96, d_in=512, n_tokens=1024, chunk_tokens=1024),
        }[base]
        return c.scaled(f"{base}:small", 100 + c.cfg_id, **sizes)
    raise ValueError(variant)


def correlated_config() -> LayerConfig:
    """Supplementary input with strongly correlated channels (not a workload
    of its own): X = Z @ A with A = I + 0.5 G / sqrt(d).  Its error feedback
    moves pre-rounding values by whole quantization steps, which iid
    activations do not."""
    return LayerConfig(name="correlated", cfg_id=50, d_out=256, d_in=1024,
                       n_tokens=4096, w_dtype="f16", x_dtype="f16", w_std=0.02,
                       chunk_tokens=1024, correlated=True)


def correlated_mixer(cfg: LayerConfig) -> np.ndarray:
    g = _rng(cfg, 2, 7).standard_normal((cfg.d_in, cfg.d_in))
    return (np.eye(cfg.d_in) + 0.5 * g / math.sqrt(cfg.d_in)).astype(np.float32)


# ----------------------------------------------------------------------------
# Stored form of a 4-bit layer for the W4A16 consumer (stream 5)
# ----------------------------------------------------------------------------
def w4_layer(cfg: LayerConfig, act_order: bool = False, tag: int = 0):
    """Stand-in for a quantized layer of cfg's shape: 4-bit codes (d_out x d_in,
    original column order), fp16 scale bits and integer zeros per (row, group),
    and with ``act_order`` a column permutation whose consecutive runs of g
    entries form the groups.  Zeros are drawn in 5..10 and codes around their
    group's zero with std 3, clipped to 0..15 (the spread an asymmetric
    min-max grid gives roughly Gaussian weights); scales are cfg.w_std/4
    times U(0.5, 2).  Returns (codes uint8, scales uint16, zeros uint8,
    perm int32 or None, g_idx int32)."""
    r = np.random.default_rng([cfg.cfg_id, 5, tag])
    d_out, d_in, g = cfg.d_out, cfg.d_in, cfg.group_size
    ng = d_in // g
    perm = r.permutation(d_in).astype(np.int32) if act_order else None
    g_idx = np.empty(d_in, dtype=np.int32)
    if perm is not None:
        g_idx[perm] = np.arange(d_in) // g
    else:
        g_idx[:] = np.arange(d_in) // g
    zeros = r.integers(5, 11, (d_out, ng)).astype(np.uint8)
    codes = np.empty((d_out, d_in), dtype=np.uint8)
    for r0 in range(0, d_out, 1024):
        r1 = min(d_out, r0 + 1024)
        v = r.standard_normal((r1 - r0, d_in), dtype=np.float32) * np.float32(3.0)
        v += zeros[r0:r1][:, g_idx].astype(np.float32)
        codes[r0:r1] = np.clip(np.rint(v), 0, 15).astype(np.uint8)
    s = r.uniform(0.5, 2.0, (d_out, ng)).astype(np.float32) * np.float32(cfg.w_std / 4)
    scales = s.astype(np.float16).view(np.uint16)
    return codes, scales, zeros, perm, g_idx


def w4_tokens(cfg: LayerConfig, m: int, tag: int = 0) -> np.ndarray:
    """M activation rows with the workload's channel recipe (outliers,
    per-channel spread), in storage form of cfg.x_dtype (stream 6)."""
    z = np.random.default_rng([cfg.cfg_id, 6, tag]).standard_normal((m, cfg.d_in), dtype=np.float32)
    z *= channel_factor(cfg)[None, :]
    return cast(z, cfg.x_dtype)
