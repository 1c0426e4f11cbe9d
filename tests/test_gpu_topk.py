"""GPU parity of csa_topk on its own, on fp32 score arrays both sides read
identically, so the selection must match the oracle exactly: the min(k,
visible) largest scores, ties to the lower entry index, -1 padding.  Covers
one-chunk rows (8, 16 or 32 keys per thread), rows cut into chunks whose kept
lists are selected from again (two and three rounds, chunk edges inside the
visible range), heavy ties across the k-th score -- also across chunk edges
--, all-equal scores, negative and mixed-magnitude values, k larger than the
visible range, k = 1 and the largest k.  The kept entries come out in
ascending entry order."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_c4a_amd import binding as K
from parity import check_topk_sets

pytestmark = pytest.mark.gpu


def _scores(kind, Q, N, rng):
    if kind == "normal":
        return rng.normal(0.0, 0.05, (Q, N)).astype(np.float32)
    if kind == "ties":          # a handful of levels: many keys equal the k-th score
        return rng.integers(0, 7, (Q, N)).astype(np.float32) * 0.25 - 0.5
    if kind == "equal":
        return np.full((Q, N), 0.125, dtype=np.float32)
    if kind == "wide":          # signs and exponents spread over many binades
        m = rng.normal(0.0, 1.0, (Q, N))
        return (m * np.exp2(rng.integers(-30, 30, (Q, N)))).astype(np.float32)
    raise ValueError(kind)


CASES = [
    # (N_cap, k, q_pos list, kind)
    (100, 16, [399, 63, 3], "normal"),          # 100 visible, 15 visible, 1 visible (< k)
    (8192, 1024, [32767, 20000, 4099], "normal"),
    (8192, 1024, [32767, 32767], "ties"),
    (8192, 1, [32767, 100], "wide"),
    (8192, 4096, [32767, 8000], "wide"),
    (12000, 700, [47999, 40000], "normal"),     # 16 keys per thread
    (20000, 1024, [79999, 50000], "normal"),    # 32 keys per thread
    (20000, 512, [79999], "ties"),
    (40000, 1024, [159999, 70000], "normal"),   # two rounds, 8192-entry chunks
    (40000, 2048, [159999, 65539], "ties"),     # two rounds, 16384-entry chunks
    (262144, 1024, [1048575, 600003], "normal"),
    (262144, 1024, [1048575], "equal"),         # every chunk ties at the k-th score
    (300000, 4096, [1199999, 140000], "ties"),  # three rounds
    (5000, 300, [19999, 19999], "equal"),
]


@pytest.mark.parametrize("N_cap,k,q_pos,kind", CASES)
def test_topk_matches_oracle(orc, N_cap, k, q_pos, kind):
    rng = np.random.default_rng(N_cap + k + len(kind))
    B, S = len(q_pos), 1
    s32 = _scores(kind, B, N_cap, rng).reshape(B, S, N_cap)
    qp = np.asarray(q_pos, dtype=np.int32)
    nvis = np.minimum((qp[:, None] + np.arange(S)[None] + 1) // 4, N_cap)
    s64 = s32.astype(np.float64)
    o_idx, _ = orc.topk(s64, nvis, k)
    idx = torch.empty((B, S, k), dtype=torch.int32, device="cuda")
    val = torch.empty((B, S, k), dtype=torch.float32, device="cuda")
    nws = K.csa_topk_workspace_size(B, S, N_cap, k)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
    K.csa_topk(torch.from_numpy(s32).cuda(), torch.from_numpy(qp).cuda(), idx, val, ratio=4, workspace=ws)
    gi = idx.cpu().numpy()
    check_topk_sets(gi, o_idx, s64, nvis, k, exact=True)
    for row in gi.reshape(-1, k):
        n = int((row >= 0).sum())
        assert np.all(row[n:] == -1), "padding follows the kept entries"
        assert np.all(np.diff(row[:n]) > 0), "kept entries in ascending entry order"
    gv = val.cpu().numpy().reshape(-1, k)
    for qi, row in enumerate(gi.reshape(-1, k)):
        m = row >= 0
        np.testing.assert_array_equal(gv[qi, m], s32.reshape(-1, N_cap)[qi, row[m]])
        assert np.all(np.isneginf(gv[qi, ~m]))


def test_topk_is_deterministic():
    rng = np.random.default_rng(5)
    s32 = _scores("ties", 4, 8192, rng).reshape(4, 1, 8192)
    qp = torch.full((4,), 32767, dtype=torch.int32, device="cuda")
    outs = []
    for _ in range(3):
        idx = torch.empty((4, 1, 1024), dtype=torch.int32, device="cuda")
        K.csa_topk(torch.from_numpy(s32).cuda(), qp, idx, ratio=4)
        outs.append(idx.cpu().numpy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
