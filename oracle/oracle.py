"""Python front end of the fp64 CPU oracle (``oracle.c``) and a second,
independent NumPy dense-mask formulation of the same path.

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It never imports the HIP package and
the HIP package never imports it.

Sources: "DeepSeek-V4-Pro 架构：一个 token 的旅程" (hs-black.github.io) and
"图解DeepSeek V4：详细计算流程解析" (jsqmd.com); the C file names the sections each
function follows.

Input arrays may be float32, float64, or uint16 holding bf16 bit patterns;
they are widened exactly inside the C code.  Outputs are float64.  Fresh
cache entries are stored in the cache's own type: bf16 caches receive the
fp64 value rounded once to nearest-even bf16 (round_bf16).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A different build of this same file may be substituted (mutation checks of the pins).
_LIB_OVERRIDE = os.environ.get("CSA_ORACLE_LIB")

F32, BF16, F64 = 0, 1, 2
NO_RELU = 1


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (plain gcc, OpenMP over queries)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            L = ctypes.CDLL(_LIB_PATH)
        vp, i32, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        L.orc_rope.argtypes = [vp, i32, dbl, dbl, i32]
        L.orc_pool.argtypes = [vp, vp, i32, i32, i32, i32, i32, ctypes.c_long, ctypes.c_long, vp]
        L.orc_pool.restype = i32
        L.orc_compress.argtypes = [vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, dbl, dbl]
        L.orc_compress.restype = ctypes.c_long
        L.orc_compress_rolling.argtypes = [vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, dbl, dbl]
        L.orc_compress_rolling.restype = ctypes.c_long
        L.orc_index_scores.argtypes = [vp, i32, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, ctypes.c_uint, vp, vp]
        L.orc_topk.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp]
        L.orc_attn.argtypes = [vp, i32, vp, i32, vp, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp,
                               i32, i32, i32, i32, i32, i32, i32, i32, dbl, dbl]
        L.orc_attn.restype = i32
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = i32
        _lib = L
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().orc_num_threads())


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"unsupported oracle input dtype {a.dtype}")


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
def rope(x: np.ndarray, pos: float, base: float = 10000.0, inverse: bool = False) -> np.ndarray:
    """RoPE of a 1-D vector x (the whole vector is the rotated part)."""
    y = np.array(x, dtype=np.float64, copy=True)
    lib().orc_rope(_p(y), y.shape[0], float(pos), float(base), -1 if inverse else 1)
    return y


def pool(kv, sc, d, ratio, overlap, pos0, g):
    """Pooled entry g (before RMSNorm) of one sequence; kv, sc: [L, m*d]."""
    kv, sc = _c(kv), _c(sc)
    assert kv.dtype == sc.dtype
    out = np.zeros(d, dtype=np.float64)
    rc = lib().orc_pool(_p(kv), _p(sc), _dt(kv), kv.shape[0], d, ratio, int(overlap), int(pos0), int(g), _p(out))
    if rc != 0:
        raise ValueError("group not fully inside the state buffer")
    return out


def compress(kv_state, score_state, gamma, pos0, ratio, overlap, N_cap, rope_dim, cache=None,
             eps=1e-6, rope_base=10000.0):
    """Parallel-form compressor.  Returns (cache f64 [B,N_cap,d], written bool [B,N_cap])."""
    kv_state, score_state = _c(kv_state), _c(score_state)
    B, L, md = kv_state.shape
    d = md // (2 if overlap else 1)
    if cache is None:
        cache = np.zeros((B, N_cap, d), dtype=np.float64)
    else:
        cache = np.array(cache, dtype=np.float64, copy=True)
    written = np.zeros((B, N_cap), dtype=np.uint8)
    g64 = _c(np.asarray(gamma, dtype=np.float64))
    p0 = _c(np.asarray(pos0, dtype=np.int32))
    lib().orc_compress(_p(kv_state), _p(score_state), _dt(kv_state), _p(g64), _p(cache), _p(written), _p(p0),
                       B, L, d, rope_dim, ratio, int(overlap), N_cap, float(eps), float(rope_base))
    return cache, written.astype(bool)


def compress_rolling(kv_state, score_state, gamma, ratio, N_cap, rope_dim, eps=1e-6, rope_base=10000.0):
    """Literal rolling-state (concat + roll) form; sequences start at position 0."""
    kv_state, score_state = _c(kv_state), _c(score_state)
    B, L, md = kv_state.shape
    d = md // 2
    cache = np.zeros((B, N_cap, d), dtype=np.float64)
    g64 = _c(np.asarray(gamma, dtype=np.float64))
    lib().orc_compress_rolling(_p(kv_state), _p(score_state), _dt(kv_state), _p(g64), _p(cache), B, L, d,
                               rope_dim, ratio, N_cap, float(eps), float(rope_base))
    return cache


def index_scores(q_idx, w, idx_cache, q_pos, ratio, relu=True):
    """Scores [B,S,N_cap] (-inf past the visible count) and nvis [B,S]."""
    q_idx, idx_cache = _c(q_idx), _c(idx_cache)
    B, S, Hi, di = q_idx.shape
    N_cap = idx_cache.shape[1]
    w64 = _c(np.asarray(w, dtype=np.float64).reshape(B, S, Hi))
    qp = _c(np.asarray(q_pos, dtype=np.int32))
    scores = np.empty((B, S, N_cap), dtype=np.float64)
    nvis = np.empty((B, S), dtype=np.int32)
    lib().orc_index_scores(_p(q_idx), _dt(q_idx), _p(w64), _p(idx_cache), _dt(idx_cache), _p(qp), B, S, Hi, di,
                           N_cap, ratio, 0 if relu else NO_RELU, _p(scores), _p(nvis))
    return scores, nvis


def topk(scores, nvis, k):
    """Indices [B,S,k] (descending score, ties to lower index, -1 padded) and k-th score [B,S]."""
    scores = _c(np.asarray(scores, dtype=np.float64))
    nvis = _c(np.asarray(nvis, dtype=np.int32))
    B, S, N_cap = scores.shape
    idx = np.empty((B, S, k), dtype=np.int32)
    kth = np.empty((B, S), dtype=np.float64)
    lib().orc_topk(_p(scores), _p(nvis), B, S, N_cap, k, _p(idx), _p(kth))
    return idx, kth


def attn(q, cmp_cache, win_kv, sink, q_pos, *, topk_idx=None, ratio=4, win_pos0=None, window=128,
         rope_dim=64, scale=None, rope_base=10000.0):
    """Sparse (topk_idx given) or dense (topk_idx None: all visible entries) MQA with sink.

    FP8 rows (uint8 [..., 640], see quantize_rows_fp8) are read as their
    dequantised values.

    Returns (out f64 [B,S,H,D], lse [B,S,H], ncand [B,S])."""
    q, cmp_cache, win_kv = _c(q), _c(widen_kv(cmp_cache)), _c(widen_kv(win_kv))
    B, S, H, D = q.shape
    N_cap = cmp_cache.shape[1]
    W_cap = win_kv.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    s64 = _c(np.asarray(sink, dtype=np.float64))
    qp = _c(np.asarray(q_pos, dtype=np.int32))
    k = 0
    ti = None
    if topk_idx is not None:
        ti = _c(np.asarray(topk_idx, dtype=np.int32))
        k = ti.shape[-1]
    wp = None if win_pos0 is None else _c(np.asarray(win_pos0, dtype=np.int32))
    out = np.empty((B, S, H, D), dtype=np.float64)
    lse = np.empty((B, S, H), dtype=np.float64)
    ncand = np.empty((B, S), dtype=np.int32)
    rc = lib().orc_attn(_p(q), _dt(q), _p(cmp_cache), _dt(cmp_cache), _p(ti), k, ratio, _p(win_kv), _dt(win_kv),
                        _p(wp), _p(s64), _p(qp), _p(out), _p(lse), _p(ncand), B, S, H, D, rope_dim, N_cap, W_cap,
                        window, float(scale), float(rope_base))
    if rc != 0:
        raise ValueError("a window row lies outside the window buffer")
    return out, lse, ncand


# --------------------------------------------------------------------------
# Second formulation: dense masks over whole sequences, no gathers.  Used to
# cross-check the C oracle on small inputs.
# --------------------------------------------------------------------------
def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _rope_mat(x, pos, rope_dim, base, sign):
    """Rotate the last rope_dim entries of x[..., D] at per-row positions pos[...]."""
    x = np.array(x, dtype=np.float64, copy=True)
    if rope_dim == 0:
        return x
    i = np.arange(rope_dim // 2, dtype=np.float64)
    theta = sign * np.asarray(pos, dtype=np.float64)[..., None] * base ** (-2.0 * i / rope_dim)
    tail = x[..., x.shape[-1] - rope_dim:]
    a, b = tail[..., 0::2].copy(), tail[..., 1::2].copy()
    tail[..., 0::2] = a * np.cos(theta) - b * np.sin(theta)
    tail[..., 1::2] = a * np.sin(theta) + b * np.cos(theta)
    return x


def _bf16_exact(x: float) -> float:
    """x rounded to the nearest bf16 value (8 significant bits, exponent down
    to -126, then subnormals of spacing 2^-133), ties to the even significand,
    in exact rational arithmetic.  Finite inputs below 2^128 only."""
    from fractions import Fraction
    a = abs(Fraction(x))
    if a == 0:
        return float(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()   # 2^e <= a < 2^(e+2)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (max(e, -126) - 7)
    q = a / ulp
    n = q.numerator // q.denominator
    rest = q - n
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and n % 2 == 1):
        n += 1
    y = float(n * ulp)
    return -y if x < 0 else y


def dense_pipeline(inp: dict) -> dict:
    """Whole CSA (or HCA when inp['hca']) path for sequences that start at
    position 0 and are queried causally at every token, via dense masks.
    With inp['store'] == 'bf16' the compressed entries are rounded to bf16
    (nearest, ties to even) before the indexer and the attention read them,
    as a bf16 cache stores them."""
    kv = _f64(inp["kv_state"])          # [B, T, m*d]
    sc = _f64(inp["score_state"])
    B, T, md = kv.shape
    ratio, overlap = inp["ratio"], inp["overlap"]
    d = md // (2 if overlap else 1)
    rope_dim, base, eps = inp["rope_dim"], inp.get("rope_base", 10000.0), inp.get("eps", 1e-6)
    G = T // ratio
    tok = np.arange(T)

    def entries(kv, sc, d, gamma, rope_dim):
        out = np.zeros((B, G, d))
        for g in range(G):
            own = (tok // ratio) == g
            prev = (tok // ratio) == g - 1
            if overlap:
                s_all = np.concatenate([np.where(prev[None, :, None], sc[:, :, :d], -np.inf),
                                        np.where(own[None, :, None], sc[:, :, d:], -np.inf)], axis=1)
                v_all = np.concatenate([kv[:, :, :d], kv[:, :, d:]], axis=1)
            else:
                s_all = np.where(own[None, :, None], sc, -np.inf)
                v_all = kv
            wgt = np.exp(s_all - s_all.max(axis=1, keepdims=True))
            wgt = wgt / wgt.sum(axis=1, keepdims=True)
            pooled = (wgt * np.where(np.isfinite(s_all), v_all, 0.0)).sum(axis=1)
            y = pooled / np.sqrt((pooled ** 2).mean(axis=-1, keepdims=True) + eps) * np.asarray(gamma)
            out[:, g] = _rope_mat(y, np.full((B,), g * ratio), rope_dim, base, +1)
        return out

    def store(vals):
        if inp.get("store") != "bf16":
            return vals
        return np.vectorize(_bf16_exact, otypes=[np.float64])(vals)

    cache = store(entries(kv, sc, d, inp["gamma"], rope_dim))
    q = _f64(inp["q"])                 # [B, T, H, D]
    win = _f64(inp["win_kv"])          # [B, T, D] linear rows for positions 0..T-1
    H = q.shape[2]
    t = tok
    nvis = (t + 1) // ratio            # [T]
    vis = np.arange(G)[None, :] < nvis[:, None]          # [T, G]
    res = {"cache": cache}
    if not inp.get("hca", False):
        ikv, isc = _f64(inp["idx_kv_state"]), _f64(inp["idx_score_state"])
        di = ikv.shape[-1] // 2
        icache = store(entries(ikv, isc, di, inp["idx_gamma"], inp["idx_rope_dim"]))
        qi = _f64(inp["q_idx"])        # [B, T, Hi, di]
        w = np.asarray(inp["w"], dtype=np.float64)       # [B, T, Hi]
        dots = np.einsum("bthc,bgc->bthg", qi, icache)
        score = np.einsum("bth,bthg->btg", w, np.maximum(dots, 0.0))
        score = np.where(vis[None], score, -np.inf)
        k = inp["k"]
        sel = np.zeros((B, T, G), dtype=bool)
        for b in range(B):
            for tt in range(T):
                order = np.argsort(-score[b, tt], kind="stable")[: min(k, nvis[tt])]
                sel[b, tt, order] = True
        res["icache"], res["scores"], res["sel"] = icache, score, sel
        cmp_mask = sel
    else:
        cmp_mask = np.broadcast_to(vis[None], (B, T, G))
    window = inp["window"]
    win_mask = (tok[None, :] <= t[:, None]) & (tok[None, :] > t[:, None] - window)   # [T, T]
    keys = np.concatenate([win, cache], axis=1)                                        # [B, T+G, D]
    mask = np.concatenate([np.broadcast_to(win_mask[None], (B, T, T)), cmp_mask], axis=2)  # [B, T, T+G]
    D = q.shape[-1]
    scale = inp.get("scale", 1.0 / np.sqrt(D))
    logits = scale * np.einsum("bthc,bjc->bthj", q, keys)
    logits = np.where(mask[:, :, None, :], logits, -np.inf)
    sink = np.asarray(inp["sink"], dtype=np.float64)
    mx = np.maximum(logits.max(axis=-1), sink[None, None, :])
    e = np.exp(logits - mx[..., None])
    Z = e.sum(axis=-1) + np.exp(sink[None, None, :] - mx)
    o = np.einsum("bthj,bjc->bthc", e / Z[..., None], keys)
    res["out"] = _rope_mat(o, np.broadcast_to(t[None, :, None], o.shape[:3]), rope_dim, base, -1)
    res["lse"] = mx + np.log(Z)
    return res


# --------------------------------------------------------------------------
# Stage composition (C oracle)
# --------------------------------------------------------------------------
def round_bf16(values64) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp64 values, rounded once to the nearest
    bf16 value, ties to the even significand (IEEE round-to-nearest-even).

    bf16 keeps 8 significant bits.  A value with frexp exponent E (|x| in
    [2^(E-1), 2^E)) has bf16 spacing 2^(E-8); below the smallest normal 2^-126
    the spacing stays 2^-133 (subnormals).  Scaling by a power of two is
    exact, numpy's round() takes ties to even, and the rounded value has at
    most 8 significant bits, so its float32 form is exact and its upper 16
    bits are the bf16 pattern (a carry past 2^128 gives infinity)."""
    x = np.asarray(values64, dtype=np.float64)
    _, E = np.frexp(x)
    E = np.maximum(E, -125)
    y = np.ldexp(np.round(np.ldexp(x, 8 - E)), E - 8)
    with np.errstate(over="ignore"):
        y32 = y.astype(np.float32)
    return (y32.view(np.uint32) >> 16).astype(np.uint16)


def is_fp8_rows(a) -> bool:
    return a is not None and a.dtype == np.uint8 and a.shape[-1] == FP8_ROW_BYTES


def widen_kv(a):
    """Cache or window rows as stored -> values the attention reads (FP8 rows
    dequantised, other types unchanged)."""
    return dequantize_rows_fp8(a) if is_fp8_rows(a) else a


def _store_like(raw: np.ndarray, values64: np.ndarray) -> np.ndarray:
    """Round fp64 values once to the storage type of ``raw``: bf16 bits by
    round_bf16, fp32 by numpy's nearest-even cast, fp64 unchanged, FP8 rows by
    quantize_rows_fp8.  The caches are bf16 in the bf16 configurations, so the
    attention and index stages read entries rounded this way."""
    if is_fp8_rows(raw):
        return quantize_rows_fp8(values64)
    if raw.dtype == np.uint16:
        return round_bf16(values64)
    if raw.dtype == np.float32:
        return np.asarray(values64, dtype=np.float64).astype(np.float32)
    return np.asarray(values64, dtype=np.float64)


def widen(raw: np.ndarray) -> np.ndarray:
    return dequantize_rows_fp8(raw) if is_fp8_rows(raw) else _f64(raw)


def compress_into(raw_cache, kv_state, score_state, gamma, pos0, ratio, overlap, rope_dim, eps=1e-6,
                  rope_base=10000.0):
    """Compress into a copy of ``raw_cache`` (storage dtype kept).  Returns
    (new raw cache, written mask, fp64 values of the written rows)."""
    N_cap = raw_cache.shape[1]
    vals, written = compress(kv_state, score_state, gamma, pos0, ratio, overlap, N_cap, rope_dim, eps=eps,
                             rope_base=rope_base)
    new = np.array(raw_cache, copy=True)
    new[written] = _store_like(raw_cache, vals[written])
    return new, written, vals


def pipeline(inp: dict, eps: float = 1e-6, rope_base: float = 10000.0, topk_override=None) -> dict:
    """One pass of the whole path for a workload dict (see the workloads
    module): compress -> [index scores -> top-k] -> attention."""
    sh = inp["shape"]
    res = {}
    if getattr(sh, "swa", False):
        # sliding-window layer ("图解DeepSeek V4" 1: SWA): the window rows only,
        # with the sink and the inverse RoPE; no compressed channel
        q = inp["q"]
        none = np.zeros((sh.B, 0, q.shape[-1]), dtype=q.dtype)
        out, lse, ncand = attn(q, none, inp["win_kv"], inp["sink"], inp["q_pos"],
                               topk_idx=np.zeros((sh.B, sh.S, 0), dtype=np.int32), ratio=1,
                               win_pos0=inp.get("win_pos0"), window=sh.window, rope_dim=sh.rope, rope_base=rope_base)
        res["out"], res["lse"], res["ncand"] = out, lse, ncand
        return res
    cmp_new, written, vals = compress_into(inp["cmp_cache"], inp["kv_state"], inp["score_state"], inp["gamma"],
                                           inp["state_pos0"], sh.ratio, sh.overlap, sh.rope, eps, rope_base)
    res["cmp_cache"], res["written"], res["cmp_vals"] = cmp_new, written, vals
    topk_idx = None
    if sh.indexer:
        idx_new, iw, ivals = compress_into(inp["idx_cache"], inp["idx_kv_state"], inp["idx_score_state"],
                                           inp["idx_gamma"], inp["state_pos0"], sh.ratio, True, sh.idx_rope, eps,
                                           rope_base)
        res["idx_cache"], res["idx_written"], res["idx_vals"] = idx_new, iw, ivals
        scores, nvis = index_scores(inp["q_idx"], inp["w"], idx_new, inp["q_pos"], sh.ratio)
        topk_idx, kth = topk(scores, nvis, sh.k)
        res["scores"], res["nvis"], res["topk_idx"], res["kth"] = scores, nvis, topk_idx, kth
        if topk_override is not None:
            topk_idx = topk_override
    out, lse, ncand = attn(inp["q"], cmp_new, inp["win_kv"], inp["sink"], inp["q_pos"], topk_idx=topk_idx,
                           ratio=sh.ratio, win_pos0=inp.get("win_pos0"), window=sh.window, rope_dim=sh.rope,
                           rope_base=rope_base)
    res["out"], res["lse"], res["ncand"] = out, lse, ncand
    return res


# --------------------------------------------------------------------------
# Projections around the attention ("DeepSeek-V4-Pro 架构：一个 token 的旅程")
# --------------------------------------------------------------------------
def _rows_pos(pos, M: int, S: int) -> np.ndarray:
    """Position of each of the M = B*S rows: row m is token m % S of sequence
    m // S, whose first token sits at pos[m // S]."""
    pos = np.asarray(pos, dtype=np.int64).reshape(-1)
    m = np.arange(M)
    return pos[m // S] + m % S


def q_proj(x, wq_a, gamma_q, wq_b, pos, *, H: int, D: int, rope_dim: int, S: int = 1, eps: float = 1e-6,
           rope_base: float = 10000.0, store=None):
    """Low-rank query, section "低秩 Q：两次矩阵乘法接起来".

    x [M, d_model] (M = B*S rows), wq_a [q_rank, d_model], gamma_q [q_rank],
    wq_b [H*D, q_rank], pos [B].  In order:
      qr = RMSNorm(x wq_a^T) with gain gamma_q (the page writes rms_norm);
      q  = qr wq_b^T viewed as [M, H, D];
      every head divided by sqrt(mean over its D dims of q^2 + eps);
      RoPE on the last rope_dim dims at the row's position (the same pair
      rotation as the compressed entries).
    store == 'bf16' rounds qr once to bf16 before the second product, the
    precision in which it is held between the two matrix products.
    Returns (q [M, H, D], qr [M, q_rank]) in fp64."""
    X = _f64(x)
    M = X.shape[0]
    qr = X @ _f64(wq_a).T
    qr = qr / np.sqrt(np.mean(qr * qr, axis=-1, keepdims=True) + eps) * _f64(gamma_q)[None, :]
    if store == "bf16":
        qr = _f64(round_bf16(qr))
    q = (qr @ _f64(wq_b).T).reshape(M, H, D)
    q = q / np.sqrt(np.mean(q * q, axis=-1, keepdims=True) + eps)
    t = _rows_pos(pos, M, S)
    for m in range(M):
        for h in range(H):
            q[m, h, D - rope_dim:] = rope(q[m, h, D - rope_dim:], float(t[m]), rope_base)
    return q, qr


def o_proj(o, wo_a, wo_b, *, groups: int, store=None):
    """Grouped output projection, section "输出投影也分组，并且降低中间维度".

    o [M, H, D] is the attention output with the inverse RoPE already applied
    (the attention stage does it).  Heads h = 8g .. 8g+7 (H/groups of them,
    in order) form group g, whose H*D/groups inputs are projected by its own
    wo_a[g] [o_rank, H*D/groups]; the groups*o_rank results, group-major, are
    projected by wo_b [d_model, groups*o_rank].
    store == 'bf16' rounds r once to bf16 before the second product.
    Returns (y [M, d_model], r [M, groups, o_rank]) in fp64."""
    O = _f64(o)
    M = O.shape[0]
    Wa = _f64(wo_a)
    og = O.reshape(M, groups, -1)
    r = np.empty((M, groups, Wa.shape[1]), dtype=np.float64)
    for g in range(groups):
        r[:, g, :] = og[:, g, :] @ Wa[g].T
    if store == "bf16":
        r = _f64(round_bf16(r))
    y = r.reshape(M, -1) @ _f64(wo_b).T
    return y, r


# --------------------------------------------------------------------------
# FP8 cache rows ("图解DeepSeek V4：详细计算流程解析" 2, CSA模块: the rope_head_dim
# part of a KV row is rotated, the rest is quantised; the page gives no format)
# --------------------------------------------------------------------------
# Reading: OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
# largest finite 448, codes 0x7F/0xFF NaN, no infinity) for the first D - rope
# dims, one power-of-two scale 2^k per 64-dim block (k the smallest integer with
# max|x| <= 448 * 2^k, k = 0 for an all-zero block, clamped to [-120, 120]),
# values rounded to the nearest E4M3 value of x / 2^k, ties to the even code;
# the rope dims kept as bf16.  Row of D = 512, rope = 64: bytes [0, 448) codes,
# [448, 576) the 64 bf16 rope dims, [576, 583) the 7 exponents k as int8,
# [583, 640) zero.  Dequantised value: E4M3 value x 2^k, exact in bf16.
FP8_ROW_BYTES = 640
FP8_BLOCK = 64


def e4m3_value(code) -> np.ndarray:
    """The value of each E4M3 code (fp64; NaN for 0x7F and 0xFF)."""
    c = np.asarray(code).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (8.0 + m) * np.exp2(e.astype(np.float64) - 10.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def e4m3_rne(v) -> np.ndarray:
    """E4M3 codes of values |v| <= 448: nearest representable value, ties to
    the even code.  Below 2^-6 the spacing is 2^-9 (subnormals); above, a
    value in [2^e, 2^(e+1)) has spacing 2^(e-3)."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.abs(v) > 448.0) or np.any(np.isnan(v)):
        raise ValueError("e4m3_rne takes finite values of magnitude <= 448")
    a = np.abs(v)
    sign = (np.signbit(v)).astype(np.int64) << 7
    sub = a < 2.0 ** -6
    # subnormal codes 0..8 (8 is the smallest normal, 2^-6)
    code_sub = np.rint(a * 512.0).astype(np.int64)
    _, E = np.frexp(np.where(sub, 1.0, a))          # a = f 2^E, f in [0.5, 1)
    e = E - 1                                         # a in [2^e, 2^(e+1))
    mant = np.rint((np.ldexp(np.where(sub, 1.0, a), -e) - 1.0) * 8.0).astype(np.int64)
    carry = mant == 8
    e = np.where(carry, e + 1, e)
    mant = np.where(carry, 0, mant)
    code_norm = ((e + 7) << 3) | mant
    code = np.where(sub, code_sub, code_norm)
    return (sign | code).astype(np.uint8)


def fp8_block_exp(amax) -> np.ndarray:
    """Smallest integer k with amax <= 448 * 2^k (0 for amax == 0), clamped to
    [-120, 120].  With amax in [2^(E-1), 2^E): 448 * 2^(E-10) = 0.4375 * 2^E
    is too small and 448 * 2^(E-8) = 1.75 * 2^E always enough, so k is E - 9
    when amax <= 448 * 2^(E-9) (= 0.875 * 2^E) and E - 8 otherwise."""
    amax = np.asarray(amax, dtype=np.float64)
    _, E = np.frexp(np.where(amax > 0, amax, 1.0))
    k = np.where(amax <= np.ldexp(448.0, E - 9), E - 9, E - 8)
    k = np.where(amax > 0, k, 0)
    return np.clip(k, -120, 120).astype(np.int64)


def quantize_rows_fp8(values, rope_dim: int = 64, decide_in_float32: bool = True) -> np.ndarray:
    """FP8 rows (uint8 [..., 640]) of D = 512 values per row (see the reading
    above).  With decide_in_float32 the values are first rounded to float32,
    the precision in which the kernels hold them when they quantise."""
    x = np.asarray(values, dtype=np.float64)
    if decide_in_float32:
        x = x.astype(np.float32).astype(np.float64)
    D = x.shape[-1]
    if D != 512 or rope_dim != 64:
        raise ValueError("FP8 rows are defined for D = 512, rope_dim = 64")
    lead = x.shape[:-1]
    x = x.reshape(-1, D)
    nq = D - rope_dim
    blocks = x[:, :nq].reshape(-1, nq // FP8_BLOCK, FP8_BLOCK)
    k = fp8_block_exp(np.max(np.abs(blocks), axis=-1))             # [R, 7]
    codes = e4m3_rne(np.ldexp(blocks, -k[..., None])).reshape(-1, nq)
    out = np.zeros((x.shape[0], FP8_ROW_BYTES), dtype=np.uint8)
    out[:, :nq] = codes
    out[:, nq:nq + 2 * rope_dim] = round_bf16(x[:, nq:]).view(np.uint8).reshape(-1, 2 * rope_dim)
    out[:, nq + 2 * rope_dim:nq + 2 * rope_dim + nq // FP8_BLOCK] = k.astype(np.int8).view(np.uint8)
    return out.reshape(lead + (FP8_ROW_BYTES,))


def dequantize_rows_fp8(rows, rope_dim: int = 64) -> np.ndarray:
    """fp64 values [..., 512] of FP8 rows."""
    r = np.asarray(rows, dtype=np.uint8)
    lead = r.shape[:-1]
    r = r.reshape(-1, FP8_ROW_BYTES)
    nq = 512 - rope_dim
    k = r[:, nq + 2 * rope_dim:nq + 2 * rope_dim + nq // FP8_BLOCK].view(np.int8).astype(np.int64)
    vals = e4m3_value(r[:, :nq]).reshape(-1, nq // FP8_BLOCK, FP8_BLOCK)
    out = np.empty((r.shape[0], 512), dtype=np.float64)
    out[:, :nq] = np.ldexp(vals, k[..., None]).reshape(-1, nq)
    out[:, nq:] = _f64(np.ascontiguousarray(r[:, nq:nq + 2 * rope_dim]).view(np.uint16))
    return out.reshape(lead + (512,))
