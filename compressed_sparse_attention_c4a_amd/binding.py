"""ctypes binding of libcsa.so: the same entry points as include/csa.h, taking
torch tensors.  It only checks devices, dtypes and contiguity, derives sizes
from tensor shapes and passes raw device pointers; every computation runs in
the HIP kernels.  There is no fallback: if libcsa.so is missing or a call
fails, a RuntimeError is raised.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "csa.h")

CSA_F32, CSA_BF16 = 0, 1
CSA_INDEX_NO_RELU = 1

_lib = None


def load() -> ctypes.CDLL:
    """Load libcsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m compressed_sparse_attention_c4a_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, u32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_uint, ctypes.c_size_t
    sigs = {
        "csa_version": ([], i32),
        "csa_error_string": ([i32], ctypes.c_char_p),
        "csa_last_error": ([], ctypes.c_char_p),
        "csa_compress": ([vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, f32, i32, vp], i32),
        "csa_compress_kv_index": ([vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, i32, i32, i32, vp, i32, i32,
                                   i32, f32, f32, i32, vp], i32),
        "csa_index_scores": ([vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, u32, i32, vp], i32),
        "csa_topk_workspace_size": ([i32, i32, i32, i32], sz),
        "csa_topk": ([vp, vp, vp, vp, vp, sz, i32, i32, i32, i32, i32, vp], i32),
        "csa_index_topk_workspace_size": ([i32, i32, i32, i32], sz),
        "csa_index_topk": ([vp, vp, vp, vp, vp, vp, vp, sz, i32, i32, i32, i32, i32, i32, i32, u32, i32, vp], i32),
        "csa_compress_index_topk": ([vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, i32, vp, i32, vp, vp, vp, vp, vp,
                                     vp, sz, i32, i32, i32, i32, i32, i32, i32, u32, f32, f32, i32, vp], i32),
        "csa_compress_index_topk_noalloc": ([vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, i32, vp, i32, vp, vp, vp,
                                             vp, vp, i32, i32, i32, i32, i32, i32, i32, u32, f32, f32, i32, vp], i32),
        "csa_attn_workspace_size": ([i32, i32, i32, i32, i32], sz),
        "csa_sparse_attn": ([vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                             f32, f32, i32, vp], i32),
        "hca_attn": ([vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i32, i32, i32, i32, i32, i32, i32, i32, i32, f32, f32,
                      i32, vp], i32),
        "swa_attn": ([vp, vp, vp, vp, vp, vp, vp, vp, sz, i32, i32, i32, i32, i32, i32, i32, f32, f32, i32, vp], i32),
        "csa_pack_weights": ([vp, vp, i32, i32, i32, vp], i32),
        "csa_quantize_rows": ([vp, vp, ctypes.c_long, i32, i32, vp], i32),
        "csa_dequantize_rows": ([vp, vp, ctypes.c_long, i32, i32, vp], i32),
        "csa_q_proj_workspace_size": ([i32, i32, i32, i32, i32], sz),
        "csa_q_proj": ([vp, vp, vp, vp, vp, vp, vp, vp, sz, i32, i32, i32, i32, i32, i32, i32, f32, f32, vp], i32),
        "csa_o_proj_workspace_size": ([i32, i32, i32, i32, i32, i32], sz),
        "csa_o_proj": ([vp, vp, vp, vp, vp, vp, sz, i32, i32, i32, i32, i32, i32, vp], i32),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def declared_functions() -> list:
    """Names of the functions include/csa.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*((?:csa|hca)_\w+)\s*\(", text, flags=re.M)))


# ----------------------------------------------------------------------------- marshalling helpers
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


CSA_BF16_KV_FP8 = 2


def _cache(cache, states):
    """(d, dtype code, torch dtype of the cache) of a compressor's output
    cache: uint8 [.., 640] rows are FP8 rows of d = 512 written from bf16
    states (CSA_BF16_KV_FP8); otherwise the cache has the states' dtype."""
    if cache.dtype == torch.uint8:
        if cache.shape[-1] != 640 or states.dtype != torch.bfloat16:
            raise TypeError("an FP8 cache has 640-byte rows and bf16 states")
        return 512, CSA_BF16_KV_FP8, torch.uint8
    return cache.shape[-1], _dtype_code(states), states.dtype


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(rc: int, name: str):
    if rc != 0:
        L = load()
        raise RuntimeError(f"{name} failed ({L.csa_error_string(rc).decode()}): {L.csa_last_error().decode()}")


class Prepared:
    """One library call with its arguments marshalled once.  Calling it issues
    the same launch again (same tensors, sizes and stream), without the
    per-call Python work of the wrappers below."""

    __slots__ = ("name", "fn", "args", "keep")

    def __init__(self, name, fn, args, keep=()):
        self.name, self.fn, self.args = name, fn, args
        self.keep = keep  # tensors the call owns (a workspace allocated here)

    def __call__(self):
        rc = self.fn(*self.args)
        if rc != 0:
            _check(rc, self.name)


def _run(name: str, args: tuple, prepare: bool, keep=()):
    fn = getattr(load(), name)
    if prepare:
        return Prepared(name, fn, args, keep)
    _check(fn(*args), name)
    return None


# ----------------------------------------------------------------------------- entry points
# Every entry point takes `prepare=True` to return a Prepared call instead of
# running it.


def csa_version() -> int:
    return load().csa_version()


def csa_compress(kv_state, score_state, gamma, cache, pos0, *, ratio: int, overlap: bool, rope_dim: int,
                 eps: float = 1e-6, rope_base: float = 10000.0, stream=None, prepare: bool = False):
    B, L, md = kv_state.shape
    d, code, ct = _cache(cache, kv_state)
    if md != (2 if overlap else 1) * d or score_state.shape != kv_state.shape:
        raise ValueError("state width must be (2 if overlap else 1) * d and kv/score shapes must match")
    dt = kv_state.dtype
    args = (_ptr(kv_state, dt, "kv_state"), _ptr(score_state, dt, "score_state"), _ptr(gamma, torch.float32, "gamma"),
            _ptr(cache, ct, "cache"), _ptr(pos0, torch.int32, "pos0"), B, L, d, rope_dim, ratio, int(overlap),
            cache.shape[1], eps, rope_base, code, _stream(stream))
    return _run("csa_compress", args, prepare)


def csa_compress_kv_index(kv_state, score_state, gamma, cache, idx_kv_state, idx_score_state, idx_gamma, idx_cache,
                          pos0, *, ratio: int, overlap: bool, rope_dim: int, idx_rope_dim: int, eps: float = 1e-6,
                          rope_base: float = 10000.0, stream=None, prepare: bool = False):
    B, L, md = kv_state.shape
    (d, code, ct), di = _cache(cache, kv_state), idx_cache.shape[-1]
    if md != (2 if overlap else 1) * d or score_state.shape != kv_state.shape:
        raise ValueError("state width must be (2 if overlap else 1) * d and kv/score shapes must match")
    if idx_kv_state.shape != (B, L, 2 * di) or idx_score_state.shape != idx_kv_state.shape:
        raise ValueError("index states must be [B, L, 2 * di] over the same tokens")
    dt = kv_state.dtype
    args = (_ptr(kv_state, dt, "kv_state"), _ptr(score_state, dt, "score_state"), _ptr(gamma, torch.float32, "gamma"),
            _ptr(cache, ct, "cache"), d, rope_dim, int(overlap), cache.shape[1],
            _ptr(idx_kv_state, dt, "idx_kv_state"), _ptr(idx_score_state, dt, "idx_score_state"),
            _ptr(idx_gamma, torch.float32, "idx_gamma"), _ptr(idx_cache, dt, "idx_cache"), di, idx_rope_dim,
            idx_cache.shape[1], _ptr(pos0, torch.int32, "pos0"), B, L, ratio, eps, rope_base, code, _stream(stream))
    return _run("csa_compress_kv_index", args, prepare)


def csa_index_scores(q_idx, w, idx_cache, q_pos, scores, *, ratio: int, relu: bool = True, stream=None,
                     prepare: bool = False):
    B, S, Hi, di = q_idx.shape
    N_cap = idx_cache.shape[1]
    args = (_ptr(q_idx, q_idx.dtype, "q_idx"), _ptr(w, torch.float32, "w"), _ptr(idx_cache, q_idx.dtype, "idx_cache"),
            _ptr(q_pos, torch.int32, "q_pos"), _ptr(scores, torch.float32, "scores"), B, S, Hi, di, N_cap, ratio,
            0 if relu else CSA_INDEX_NO_RELU, _dtype_code(q_idx), _stream(stream))
    return _run("csa_index_scores", args, prepare)


def csa_topk_workspace_size(B: int, S: int, N_cap: int, k: int) -> int:
    return load().csa_topk_workspace_size(B, S, N_cap, k)


def csa_topk(scores, q_pos, topk_idx, topk_score=None, *, ratio: int, workspace=None, stream=None,
             prepare: bool = False):
    B, S, N_cap = scores.shape
    k = topk_idx.shape[-1]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(scores, torch.float32, "scores"), _ptr(q_pos, torch.int32, "q_pos"),
            _ptr(topk_idx, torch.int32, "topk_idx"), _ptr(topk_score, torch.float32, "topk_score"),
            _ptr(workspace, None, "workspace"), ws_bytes, B, S, N_cap, k, ratio, _stream(stream))
    return _run("csa_topk", args, prepare)


def csa_index_topk_workspace_size(B: int, S: int, N_cap: int, k: int) -> int:
    return load().csa_index_topk_workspace_size(B, S, N_cap, k)


def csa_index_topk(q_idx, w, idx_cache, q_pos, topk_idx, topk_score=None, *, ratio: int, workspace,
                   relu: bool = True, stream=None, prepare: bool = False):
    B, S, Hi, di = q_idx.shape
    N_cap = idx_cache.shape[1]
    k = topk_idx.shape[-1]
    ws_bytes = workspace.numel() * workspace.element_size()
    args = (_ptr(q_idx, q_idx.dtype, "q_idx"), _ptr(w, torch.float32, "w"), _ptr(idx_cache, q_idx.dtype, "idx_cache"),
            _ptr(q_pos, torch.int32, "q_pos"), _ptr(topk_idx, torch.int32, "topk_idx"),
            _ptr(topk_score, torch.float32, "topk_score"), _ptr(workspace, None, "workspace"), ws_bytes, B, S, Hi, di,
            N_cap, k, ratio, 0 if relu else CSA_INDEX_NO_RELU, _dtype_code(q_idx), _stream(stream))
    return _run("csa_index_topk", args, prepare)


def csa_compress_index_topk(kv_state, score_state, gamma, cache, idx_kv_state, idx_score_state, idx_gamma, idx_cache,
                            state_pos0, q_idx, w, q_pos, topk_idx, topk_score=None, *, ratio: int, overlap: bool,
                            rope_dim: int, idx_rope_dim: int, workspace, relu: bool = True, eps: float = 1e-6,
                            rope_base: float = 10000.0, stream=None, prepare: bool = False):
    """csa_compress_kv_index followed by csa_index_topk over idx_cache, one
    call (one fused launch plus top-k for decode).  workspace=None calls
    csa_compress_index_topk_noalloc (the library's static scratch)."""
    B, L, md = kv_state.shape
    (d, code, ct), di = _cache(cache, kv_state), idx_cache.shape[-1]
    _, S, Hi, qdi = q_idx.shape
    N_cap = idx_cache.shape[1]
    k = topk_idx.shape[-1]
    if md != (2 if overlap else 1) * d or score_state.shape != kv_state.shape:
        raise ValueError("state width must be (2 if overlap else 1) * d and kv/score shapes must match")
    if idx_kv_state.shape != (B, L, 2 * di) or idx_score_state.shape != idx_kv_state.shape:
        raise ValueError("index states must be [B, L, 2 * di] over the same tokens")
    if qdi != di or cache.shape[1] != N_cap:
        raise ValueError("q_idx dims must equal the index cache's, and both caches must hold N_cap entries")
    dt = kv_state.dtype
    head = (_ptr(kv_state, dt, "kv_state"), _ptr(score_state, dt, "score_state"), _ptr(gamma, torch.float32, "gamma"),
            _ptr(cache, ct, "cache"), d, rope_dim, int(overlap), _ptr(idx_kv_state, dt, "idx_kv_state"),
            _ptr(idx_score_state, dt, "idx_score_state"), _ptr(idx_gamma, torch.float32, "idx_gamma"),
            _ptr(idx_cache, dt, "idx_cache"), idx_rope_dim, _ptr(state_pos0, torch.int32, "state_pos0"), L,
            _ptr(q_idx, dt, "q_idx"), _ptr(w, torch.float32, "w"), _ptr(q_pos, torch.int32, "q_pos"),
            _ptr(topk_idx, torch.int32, "topk_idx"), _ptr(topk_score, torch.float32, "topk_score"))
    tail = (B, S, Hi, di, N_cap, k, ratio, 0 if relu else CSA_INDEX_NO_RELU, eps, rope_base, code, _stream(stream))
    if workspace is None:
        return _run("csa_compress_index_topk_noalloc", head + tail, prepare)
    ws_bytes = workspace.numel() * workspace.element_size()
    return _run("csa_compress_index_topk", head + (_ptr(workspace, None, "workspace"), ws_bytes) + tail, prepare)


def _kv(q, *rows):
    """(dtype code, torch dtype of the KV rows): uint8 rows are FP8 rows read
    with bf16 q (CSA_BF16_KV_FP8); otherwise the rows have q's dtype."""
    fp8 = [r is not None and r.dtype == torch.uint8 for r in rows]
    if any(fp8):
        if not all(f for f, r in zip(fp8, rows) if r is not None):
            raise TypeError("either all KV rows are FP8 rows (uint8) or none")
        if q.dtype != torch.bfloat16:
            raise TypeError("FP8 KV rows are read with a bf16 q")
        return CSA_BF16_KV_FP8, torch.uint8
    return _dtype_code(q), q.dtype


def csa_attn_workspace_size(B: int, S: int, H: int, D: int, n_cand: int) -> int:
    return load().csa_attn_workspace_size(B, S, H, D, n_cand)


def attn_workspace(B: int, S: int, H: int, D: int, n_cand: int, device) -> Optional[torch.Tensor]:
    """An attention workspace of the size the library asks for (None when it
    needs none); its contents need no initialisation."""
    n = csa_attn_workspace_size(B, S, H, D, n_cand)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def csa_sparse_attn(q, cmp_cache, topk_idx, win_kv, win_pos0, sink, q_pos, out, lse=None, *, rope_dim: int,
                    window: int, softmax_scale: Optional[float] = None, rope_base: float = 10000.0, workspace=None,
                    stream=None, prepare: bool = False):
    B, S, H, D = q.shape
    N_cap = cmp_cache.shape[1]
    k = topk_idx.shape[-1]
    W_cap = win_kv.shape[1]
    scale = softmax_scale if softmax_scale is not None else D ** -0.5
    if workspace is None:
        workspace = attn_workspace(B, S, H, D, window + k, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code, kvt = _kv(q, cmp_cache, win_kv)
    args = (_ptr(q, q.dtype, "q"), _ptr(cmp_cache, kvt, "cmp_cache"), _ptr(topk_idx, torch.int32, "topk_idx"),
            _ptr(win_kv, kvt, "win_kv"), _ptr(win_pos0, torch.int32, "win_pos0"), _ptr(sink, torch.float32, "sink"),
            _ptr(q_pos, torch.int32, "q_pos"), _ptr(out, q.dtype, "out"), _ptr(lse, torch.float32, "lse"),
            _ptr(workspace, None, "workspace"), ws_bytes, B, S, H, D, rope_dim, N_cap, k, W_cap, window, scale,
            rope_base, code, _stream(stream))
    return _run("csa_sparse_attn", args, prepare, keep=(workspace,))


def hca_attn(q, cmp_cache, win_kv, win_pos0, sink, q_pos, out, lse=None, *, ratio: int, rope_dim: int, window: int,
             softmax_scale: Optional[float] = None, rope_base: float = 10000.0, workspace=None, stream=None,
             prepare: bool = False):
    B, S, H, D = q.shape
    N_cap = cmp_cache.shape[1]
    W_cap = win_kv.shape[1]
    scale = softmax_scale if softmax_scale is not None else D ** -0.5
    if workspace is None:
        workspace = attn_workspace(B, S, H, D, window + N_cap, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code, kvt = _kv(q, cmp_cache, win_kv)
    args = (_ptr(q, q.dtype, "q"), _ptr(cmp_cache, kvt, "cmp_cache"), _ptr(win_kv, kvt, "win_kv"),
            _ptr(win_pos0, torch.int32, "win_pos0"), _ptr(sink, torch.float32, "sink"), _ptr(q_pos, torch.int32, "q_pos"),
            _ptr(out, q.dtype, "out"), _ptr(lse, torch.float32, "lse"), _ptr(workspace, None, "workspace"), ws_bytes,
            B, S, H, D, rope_dim, N_cap, ratio, W_cap, window, scale, rope_base, code, _stream(stream))
    return _run("hca_attn", args, prepare, keep=(workspace,))


def swa_attn(q, win_kv, win_pos0, sink, q_pos, out, lse=None, *, rope_dim: int, window: int,
             softmax_scale: Optional[float] = None, rope_base: float = 10000.0, workspace=None, stream=None,
             prepare: bool = False):
    """Sliding-window attention layer: the window rows, the sink and the
    inverse RoPE, no compressed channel."""
    B, S, H, D = q.shape
    W_cap = win_kv.shape[1]
    scale = softmax_scale if softmax_scale is not None else D ** -0.5
    if workspace is None:
        workspace = attn_workspace(B, S, H, D, window, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code, kvt = _kv(q, win_kv)
    args = (_ptr(q, q.dtype, "q"), _ptr(win_kv, kvt, "win_kv"), _ptr(win_pos0, torch.int32, "win_pos0"),
            _ptr(sink, torch.float32, "sink"), _ptr(q_pos, torch.int32, "q_pos"), _ptr(out, q.dtype, "out"),
            _ptr(lse, torch.float32, "lse"), _ptr(workspace, None, "workspace"), ws_bytes, B, S, H, D, rope_dim, W_cap,
            window, scale, rope_base, code, _stream(stream))
    return _run("swa_attn", args, prepare, keep=(workspace,))


FP8_ROW_BYTES = 640


def csa_quantize_rows(src, dst=None, *, stream=None, prepare: bool = False):
    """bf16 KV rows [..., 512] -> FP8 rows uint8 [..., 640] (see include/csa.h)."""
    if src.shape[-1] != 512:
        raise ValueError("FP8 rows hold 512 values")
    rows = src.numel() // 512
    if dst is None:
        dst = torch.empty(src.shape[:-1] + (FP8_ROW_BYTES,), dtype=torch.uint8, device=src.device)
    if rows == 0:
        return dst
    args = (_ptr(src, torch.bfloat16, "src"), _ptr(dst, torch.uint8, "dst"), rows, 512, 64, _stream(stream))
    _run("csa_quantize_rows", args, prepare)
    return dst


def csa_dequantize_rows(src, dst=None, *, stream=None, prepare: bool = False):
    """FP8 rows uint8 [..., 640] -> bf16 [..., 512] (exact)."""
    if src.shape[-1] != FP8_ROW_BYTES:
        raise ValueError("FP8 rows are 640 bytes")
    rows = src.numel() // FP8_ROW_BYTES
    if dst is None:
        dst = torch.empty(src.shape[:-1] + (512,), dtype=torch.bfloat16, device=src.device)
    if rows == 0:
        return dst
    args = (_ptr(src, torch.uint8, "src"), _ptr(dst, torch.bfloat16, "dst"), rows, 512, 64, _stream(stream))
    _run("csa_dequantize_rows", args, prepare)
    return dst


def csa_pack_weights(w, packed=None, *, stream=None, prepare: bool = False):
    """Pack a bf16 weight [N, K] (or a group stack [G, N, K]) into the layout
    csa_q_proj / csa_o_proj read.  Returns the packed tensor (same shape and
    size; the contents are a permutation)."""
    groups = 1 if w.dim() == 2 else w.shape[0]
    N, Kd = w.shape[-2], w.shape[-1]
    if packed is None:
        packed = torch.empty_like(w)
    args = (_ptr(w, torch.bfloat16, "w"), _ptr(packed, torch.bfloat16, "packed"), groups, N, Kd, _stream(stream))
    _run("csa_pack_weights", args, prepare)
    return packed


def csa_q_proj_workspace_size(M: int, d_model: int, q_rank: int, H: int, D: int) -> int:
    return load().csa_q_proj_workspace_size(M, d_model, q_rank, H, D)


def csa_q_proj(x, wq_a, gamma_q, wq_b, pos, qr, q, *, B: int, S: int, rope_dim: int, eps: float = 1e-6,
               rope_base: float = 10000.0, workspace=None, stream=None, prepare: bool = False):
    """Low-rank query: x [B*S, d_model] -> qr [B*S, q_rank], q [B*S, H, D]
    (bf16 throughout); wq_a and wq_b packed by csa_pack_weights."""
    M, d_model = x.shape
    q_rank = wq_a.shape[0]
    H, D = q.shape[-2], q.shape[-1]
    if M != B * S:
        raise ValueError(f"x has {M} rows, expected B*S = {B * S}")
    if workspace is None:
        workspace = torch.empty(csa_q_proj_workspace_size(M, d_model, q_rank, H, D), dtype=torch.uint8,
                                device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    bf = torch.bfloat16
    args = (_ptr(x, bf, "x"), _ptr(wq_a, bf, "wq_a"), _ptr(gamma_q, torch.float32, "gamma_q"), _ptr(wq_b, bf, "wq_b"),
            _ptr(pos, torch.int32, "pos"), _ptr(qr, bf, "qr"), _ptr(q, bf, "q"), _ptr(workspace, None, "workspace"),
            ws_bytes, B, S, d_model, q_rank, H, D, rope_dim, eps, rope_base, _stream(stream))
    return _run("csa_q_proj", args, prepare, keep=(workspace,))


def csa_o_proj_workspace_size(M: int, H: int, D: int, groups: int, o_rank: int, d_model: int) -> int:
    return load().csa_o_proj_workspace_size(M, H, D, groups, o_rank, d_model)


def csa_o_proj(o, wo_a, wo_b, r, y, *, groups: int, workspace=None, stream=None, prepare: bool = False):
    """Grouped output projection: o [M, H, D] -> r [M, groups*o_rank] ->
    y [M, d_model] (bf16 throughout); wo_a and wo_b packed by
    csa_pack_weights."""
    M, H, D = o.shape
    o_rank = wo_a.shape[1]
    d_model = wo_b.shape[0]
    if workspace is None:
        workspace = torch.empty(csa_o_proj_workspace_size(M, H, D, groups, o_rank, d_model), dtype=torch.uint8,
                                device=o.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    bf = torch.bfloat16
    args = (_ptr(o, bf, "o"), _ptr(wo_a, bf, "wo_a"), _ptr(wo_b, bf, "wo_b"), _ptr(r, bf, "r"), _ptr(y, bf, "y"),
            _ptr(workspace, None, "workspace"), ws_bytes, M, H, D, groups, o_rank, d_model, _stream(stream))
    return _run("csa_o_proj", args, prepare, keep=(workspace,))
