"""Seeded synthetic inputs for the compressed attention path.

This module holds the workload shapes and the random draws only; it contains
none of the method's arithmetic.  Draws use NumPy's PCG64 ``default_rng(seed)``
``standard_normal`` in float32 and a fixed order per workload; bf16 tensors are
the float32 draws rounded to nearest-even and kept as raw uint16 bit patterns.

Workloads follow the shapes of DeepSeek-V4-Pro's attention ("DeepSeek-V4-Pro
架构：一个 token 的旅程": 128 query heads of 512 dims, RoPE on the last 64 dims,
indexer 64 heads x 128 dims, weights scaled by 1/sqrt(128)/sqrt(64); "图解DeepSeek
V4": C4A ratio 4 with an overlapping 2*ratio state, C128A ratio 128, window KV
ring, top-k compressed entries).  I.i.d. N(0,1) data has no locality, so the
selected entries are scattered uniformly: the worst case for the gathers.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

CHUNK = 1 << 24


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


class Draw:
    """Sequential N(0,1) draws in a fixed order from one PCG64 stream."""

    def __init__(self, seed: int):
        self.rng = np.random.default_rng(seed)

    def f32(self, shape, scale: float = 1.0, shift: float = 0.0) -> np.ndarray:
        n = int(np.prod(shape))
        out = np.empty(n, dtype=np.float32)
        for i in range(0, n, CHUNK):
            m = min(CHUNK, n - i)
            out[i:i + m] = self.rng.standard_normal(m, dtype=np.float32)
        if scale != 1.0:
            out *= np.float32(scale)
        if shift != 0.0:
            out += np.float32(shift)
        return out.reshape(shape)

    def bf16(self, shape, scale: float = 1.0) -> np.ndarray:
        """N(0, scale^2) draws in float32, rounded to bf16 bit patterns."""
        n = int(np.prod(shape))
        out = np.empty(n, dtype=np.uint16)
        for i in range(0, n, CHUNK):
            m = min(CHUNK, n - i)
            v = self.rng.standard_normal(m, dtype=np.float32)
            if scale != 1.0:
                v *= np.float32(scale)
            out[i:i + m] = bf16_bits(v)
        return out.reshape(shape)

    def data(self, shape, dtype: str) -> np.ndarray:
        return self.bf16(shape) if dtype == "bf16" else self.f32(shape)


@dataclasses.dataclass
class Shape:
    """Everything that sizes one pass of the path."""
    name: str
    B: int = 1
    S: int = 1
    q_pos: int = 0            # position of query 0 (every batch row alike)
    H: int = 128
    D: int = 512
    rope: int = 64
    ratio: int = 4
    overlap: bool = True      # C4A overlapping state; False for C128A
    N_cap: int = 8192         # compressed entries per sequence
    n_pre: int = 0            # entries already in the cache (rows [0, n_pre) are drawn)
    window: int = 128
    W_cap: int = 128          # window buffer rows (ring unless win_linear)
    win_linear: bool = False  # linear window rows starting at win_pos0
    win_pos0: int = 0
    state_pos0: int = 0       # absolute position of compressor state row 0
    state_len: int = 8
    indexer: bool = True
    swa: bool = False         # sliding-window layer: no compressed channel at all
    Hi: int = 64
    di: int = 128
    idx_rope: int = 64
    k: int = 1024
    dtype: str = "bf16"
    seed: int = 0

    @property
    def w_scale(self) -> float:
        return 1.0 / math.sqrt(self.di) / math.sqrt(self.Hi)

    @property
    def queries(self) -> int:
        return self.B * self.S

    @property
    def kind(self) -> str:
        return "swa" if self.swa else ("csa" if self.indexer else "hca")


def generate(sh: Shape, seed: Optional[int] = None) -> dict:
    """Draw every input of one pass, in a fixed order.  Returns numpy arrays:
    bf16 tensors as uint16 bit patterns, fp32 tensors as float32; small
    per-head vectors (sink, w, gamma) are always float32."""
    dr = Draw(sh.seed if seed is None else seed)
    dt = sh.dtype
    m = 2 if sh.overlap else 1
    out = {"shape": sh}
    out["q"] = dr.data((sh.B, sh.S, sh.H, sh.D), dt)
    out["sink"] = dr.f32((sh.H,))
    if sh.indexer:
        out["q_idx"] = dr.data((sh.B, sh.S, sh.Hi, sh.di), dt)
        out["w"] = dr.f32((sh.B, sh.S, sh.Hi), scale=sh.w_scale)
    out["cmp_cache"] = dr.data((sh.B, sh.N_cap, sh.D), dt)
    if sh.indexer:
        out["idx_cache"] = dr.data((sh.B, sh.N_cap, sh.di), dt)
    out["win_kv"] = dr.data((sh.B, sh.W_cap, sh.D), dt)
    out["kv_state"] = dr.data((sh.B, sh.state_len, m * sh.D), dt)
    out["score_state"] = dr.data((sh.B, sh.state_len, m * sh.D), dt)
    if sh.indexer:
        out["idx_kv_state"] = dr.data((sh.B, sh.state_len, 2 * sh.di), dt)
        out["idx_score_state"] = dr.data((sh.B, sh.state_len, 2 * sh.di), dt)
    out["gamma"] = dr.f32((sh.D,), scale=0.1, shift=1.0)
    if sh.indexer:
        out["idx_gamma"] = dr.f32((sh.di,), scale=0.1, shift=1.0)
    out["q_pos"] = np.full((sh.B,), sh.q_pos, dtype=np.int32)
    out["state_pos0"] = np.full((sh.B,), sh.state_pos0, dtype=np.int32)
    out["win_pos0"] = np.full((sh.B,), sh.win_pos0, dtype=np.int32) if sh.win_linear else None
    return out


def tiny_fp32() -> dict:
    """Tiny fp32 CSA: one sequence of 64 tokens, every token queried causally.
    4 heads x 64 dims, RoPE on the last 16, ratio 4, window 8, top-4, indexer
    2 heads x 32 dims.  Own draw order (kv/score states first)."""
    sh = Shape(name="tiny_fp32", B=1, S=64, q_pos=0, H=4, D=64, rope=16, ratio=4, overlap=True, N_cap=16,
               n_pre=0, window=8, W_cap=64, win_linear=True, win_pos0=0, state_pos0=0, state_len=64,
               indexer=True, Hi=2, di=32, idx_rope=16, k=4, dtype="fp32", seed=0)
    dr = Draw(0)
    T = 64
    out = {"shape": sh}
    out["kv_state"] = dr.f32((1, T, 128))
    out["score_state"] = dr.f32((1, T, 128))
    out["idx_kv_state"] = dr.f32((1, T, 64))
    out["idx_score_state"] = dr.f32((1, T, 64))
    out["q"] = dr.f32((1, T, 4, 64))
    out["sink"] = dr.f32((4,))
    out["q_idx"] = dr.f32((1, T, 2, 32))
    out["w"] = dr.f32((1, T, 2), scale=sh.w_scale)
    out["gamma"] = dr.f32((64,), scale=0.1, shift=1.0)
    out["idx_gamma"] = dr.f32((32,), scale=0.1, shift=1.0)
    out["win_kv"] = dr.f32((1, T, 64))
    out["cmp_cache"] = np.zeros((1, 16, 64), dtype=np.float32)
    out["idx_cache"] = np.zeros((1, 16, 32), dtype=np.float32)
    out["q_pos"] = np.zeros((1,), dtype=np.int32)
    out["state_pos0"] = np.zeros((1,), dtype=np.int32)
    out["win_pos0"] = np.zeros((1,), dtype=np.int32)
    return out


def csa_decode_32k(B: int = 32) -> Shape:
    """CSA decode at 32K context: B queries at position 32767; 8192 entries,
    the last written by this step's compressor from tokens 32760..32767."""
    t = 32767
    return Shape(name="csa_decode_32k", B=B, S=1, q_pos=t, N_cap=8192, n_pre=8191, window=128, W_cap=128,
                 state_pos0=t - 7, state_len=8, k=1024, seed=1)


def csa_prefill_32k() -> Shape:
    """CSA prefill chunk: 8192 new tokens after 24576 cached (32K total);
    the compressor writes entries 6144..8191; window rows linear from 24449."""
    return Shape(name="csa_prefill_8k_at_24k", B=1, S=8192, q_pos=24576, N_cap=8192, n_pre=6144, window=128,
                 W_cap=8192 + 127, win_linear=True, win_pos0=24576 - 127, state_pos0=24572, state_len=8196, k=1024,
                 seed=2)


def hca_decode_128k(B: int = 64) -> Shape:
    """HCA decode at 128K: C128A non-overlapping groups, 1024 entries, the last
    written by this step from tokens 130944..131071; no indexer."""
    t = 131071
    return Shape(name="hca_decode_128k", B=B, S=1, q_pos=t, ratio=128, overlap=False, N_cap=1024, n_pre=1023,
                 window=128, W_cap=128, state_pos0=t - 127, state_len=128, indexer=False, seed=3)


def hca_decode_32k(B: int = 32) -> Shape:
    """HCA decode at 32K: 256 entries, the last written by this step."""
    t = 32767
    return Shape(name="hca_decode_32k", B=B, S=1, q_pos=t, ratio=128, overlap=False, N_cap=256, n_pre=255,
                 window=128, W_cap=128, state_pos0=t - 127, state_len=128, indexer=False, seed=5)


def swa_decode_32k(B: int = 32) -> Shape:
    """Sliding-window layer at 32K: the 128 window rows only (no compressed
    cache, no compressor)."""
    t = 32767
    return Shape(name="swa_decode_32k", B=B, S=1, q_pos=t, ratio=1, overlap=False, N_cap=0, n_pre=0, window=128,
                 W_cap=128, state_pos0=t, state_len=0, indexer=False, swa=True, seed=6)


def layer_shape(kind: str, B: int, t: int, seed: int) -> Shape:
    """Shape of one decode layer of the given attention type at position t
    (sizes of the Pro model; small contexts give small caches)."""
    if kind == "csa":
        n = (t + 1) // 4
        return Shape(name=f"csa_t{t}", B=B, S=1, q_pos=t, N_cap=n, n_pre=n - 1, state_pos0=t - 7, state_len=8,
                     k=min(1024, max(n, 1)), seed=seed)
    if kind == "hca":
        n = max((t + 1) // 128, 1)
        return Shape(name=f"hca_t{t}", B=B, S=1, q_pos=t, ratio=128, overlap=False, N_cap=n, n_pre=n - 1,
                     state_pos0=t - 127, state_len=128, indexer=False, seed=seed)
    if kind == "swa":
        return Shape(name=f"swa_t{t}", B=B, S=1, q_pos=t, ratio=1, overlap=False, N_cap=0, state_pos0=t,
                     state_len=0, indexer=False, swa=True, seed=seed)
    raise ValueError(f"unknown attention type {kind}")


def csa_decode_1m(B: int = 8) -> Shape:
    """CSA decode at 1M context: 262144 entries; the indexer scan dominates."""
    t = 1048575
    return Shape(name="csa_decode_1m", B=B, S=1, q_pos=t, N_cap=262144, n_pre=262143, window=128, W_cap=128,
                 state_pos0=t - 7, state_len=8, k=1024, seed=4)


def slice_batch(inp: dict, n: int) -> dict:
    """The first n batch rows of a generated workload (pure slicing)."""
    sh = dataclasses.replace(inp["shape"], B=n)
    out = {"shape": sh}
    per_head = {"sink", "gamma", "idx_gamma"}
    for key, val in inp.items():
        if key == "shape":
            continue
        out[key] = val if (val is None or key in per_head) else val[:n]
    return out


@dataclasses.dataclass
class ProjShape:
    """Sizes of the projections around one attention layer ("DeepSeek-V4-Pro
    架构": d_model 7168, low-rank Q of rank 1536 into 128 heads x 512, output
    in 16 groups of 8 heads, each projected to 1024, then 16384 -> 7168)."""
    name: str
    B: int = 32
    S: int = 1
    q_pos: int = 32767
    d_model: int = 7168
    q_rank: int = 1536
    H: int = 128
    D: int = 512
    rope: int = 64
    groups: int = 16
    o_rank: int = 1024
    seed: int = 7

    @property
    def M(self) -> int:
        return self.B * self.S


def proj_decode_32k(B: int = 32) -> ProjShape:
    """Decode projections: B tokens at position 32767."""
    return ProjShape(name="proj_decode_32k", B=B)


def generate_proj(ps: ProjShape, seed: Optional[int] = None) -> dict:
    """Inputs and random-init weights of the projections, in a fixed order.
    Activations are N(0,1); every weight matrix is N(0, 1/K) for its input
    width K, so products stay O(1); gamma_q is 1 + 0.1 N(0,1)."""
    dr = Draw(ps.seed if seed is None else seed)
    gdim = ps.H // ps.groups * ps.D
    out = {"shape": ps}
    out["x"] = dr.bf16((ps.M, ps.d_model))
    out["wq_a"] = dr.bf16((ps.q_rank, ps.d_model), scale=1.0 / math.sqrt(ps.d_model))
    out["gamma_q"] = dr.f32((ps.q_rank,), scale=0.1, shift=1.0)
    out["wq_b"] = dr.bf16((ps.H * ps.D, ps.q_rank), scale=1.0 / math.sqrt(ps.q_rank))
    out["o"] = dr.bf16((ps.M, ps.H, ps.D))
    out["wo_a"] = dr.bf16((ps.groups, ps.o_rank, gdim), scale=1.0 / math.sqrt(gdim))
    out["wo_b"] = dr.bf16((ps.d_model, ps.groups * ps.o_rank), scale=1.0 / math.sqrt(ps.groups * ps.o_rank))
    out["pos"] = np.full((ps.B,), ps.q_pos, dtype=np.int32)
    return out
