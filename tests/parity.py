"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (stated once, used everywhere):
  * floating-point outputs: normwise relative error max|gpu - ref| / max|ref|
    <= 1e-2 for bf16 outputs and <= 1e-4 for fp32 outputs; every comparison
    also records the rms-scaled error max|gpu - ref| / rms(ref) and the
    elementwise relative error max |gpu - ref| / max(|ref|, 1e-3 rms(ref)),
    printed per case and summarised at the end of the session;
  * index-score buffers (fp32 outputs of bf16 or fp32 inputs): <= 1e-3 for
    bf16 inputs (bf16 products are exact in fp32; the bound covers fp32
    accumulation order) and <= 1e-4 for fp32 inputs;
  * top-k index sets: exact, except that an entry may be swapped for another
    whose oracle score lies within 1e-3 of the oracle's k-th score;
  * visibility (which entries are -inf, which cache rows are written) and
    top-k on identical fp32 scores: exact.
"""
import numpy as np
import torch

TOL = {"bf16": 1e-2, "fp32": 1e-4}
SCORE_TOL = {"bf16": 1e-3, "fp32": 1e-4}
TIE_BAND = 1e-3


def to_np(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 (bf16 widened exactly) or int numpy array."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return (t.view(torch.int16).numpy().astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if t.dtype in (torch.float32, torch.float64):
        return t.numpy().astype(np.float64)
    return t.numpy()


def raw_np(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> its storage (bf16 as uint16 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().astype(np.uint16)
    return t.numpy()


def elementwise(gpu, ref, floor=1e-3) -> float:
    """max_i |gpu_i - ref_i| / max(|ref_i|, floor * rms(ref)): the relative
    error of every element, with a floor for elements near zero."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    den = np.maximum(np.abs(ref), floor * rms)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(gpu - ref) / den))


def rmswise(gpu, ref) -> float:
    """max_i |gpu_i - ref_i| / rms(ref): the largest error on the scale of a
    typical element (stricter than the normwise form by max|ref| / rms)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    d = float(np.max(np.abs(gpu - ref)))
    return d / rms if rms > 0 else d


# (what, normwise, rms-scaled, elementwise) of every comparison made in this session
REPORT = []


def normwise(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    return float(np.max(np.abs(gpu - ref)) / den) if den > 0 else float(np.max(np.abs(gpu - ref), initial=0.0))


def assert_close(gpu, ref, tol, what):
    """Asserts the normwise bar; also records and prints the rms-scaled and
    the elementwise error of the same comparison."""
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    err = normwise(gpu, ref)
    rw, el = rmswise(gpu, ref), elementwise(gpu, ref)
    REPORT.append((what, err, rw, el))
    print(f"[parity] {what}: normwise {err:.3e} rms-scaled {rw:.3e} elementwise {el:.3e}", flush=True)
    assert err <= tol, f"{what}: normwise relative error {err:.3e} > {tol:.1e}"
    return err


def check_topk_sets(gpu_idx, orc_idx, orc_scores, nvis, k, band=TIE_BAND, exact=False):
    """gpu_idx, orc_idx: [Q, k]; orc_scores: [Q, N] (fp64); nvis: [Q]."""
    gpu_idx = np.asarray(gpu_idx).reshape(-1, k)
    orc_idx = np.asarray(orc_idx).reshape(-1, k)
    orc_scores = np.asarray(orc_scores).reshape(gpu_idx.shape[0], -1)
    nvis = np.asarray(nvis).reshape(-1)
    swaps = 0
    for qi in range(gpu_idx.shape[0]):
        keep = min(k, int(nvis[qi]))
        g = gpu_idx[qi]
        sel = g[g >= 0]
        assert len(sel) == keep, f"query {qi}: {len(sel)} entries kept, expected {keep}"
        assert np.all(g[keep:] == -1) or np.sum(g == -1) == k - keep, f"query {qi}: bad padding"
        assert len(np.unique(sel)) == keep, f"query {qi}: duplicate entries"
        assert np.all(sel < nvis[qi]), f"query {qi}: entry beyond the visible range"
        G, O = set(sel.tolist()), set(orc_idx[qi][orc_idx[qi] >= 0].tolist())
        diff = G ^ O
        if exact:
            assert not diff, f"query {qi}: sets differ in {sorted(diff)[:8]}"
            continue
        if diff:
            kth = orc_scores[qi, orc_idx[qi][keep - 1]]
            bad = [e for e in diff if abs(orc_scores[qi, e] - kth) > band]
            assert not bad, f"query {qi}: entries {bad[:8]} differ by more than {band} from the k-th score"
            swaps += len(diff) // 2
    return swaps
