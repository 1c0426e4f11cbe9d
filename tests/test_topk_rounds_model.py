"""Host check of the rule the chunked top-k rounds rely on: selecting the k
best (score descending, ties to the lower entry index) of each chunk, then
the k best of the concatenated kept lists, gives the k best of the whole row.
A plain NumPy model of the rounds (chunk sizes as the library picks them for
long rows, and deliberately awkward ones) against the oracle's top-k, on
rows with heavy ties, all-equal rows, short visible ranges and k larger than
a chunk's visible part."""
import numpy as np
import pytest


def _best(vals, idx, k):
    """The k best of (vals, idx) by (value descending, index ascending), in index order."""
    order = np.lexsort((idx, -vals))[:k]
    keep = np.sort(idx[order])
    return keep


def _rounds(scores, nv, k, ch):
    """Chunked selection: every round keeps the k best of each chunk of ch
    list elements (lists stay in entry order), until one chunk remains."""
    vals = scores[:nv].astype(np.float64)
    idx = np.arange(nv)
    while True:
        out_v, out_i = [], []
        for c0 in range(0, max(len(idx), 1), ch):
            kv = _best(vals[c0:c0 + ch], idx[c0:c0 + ch], k)
            sel = np.searchsorted(idx, kv)
            out_v.append(vals[sel])
            out_i.append(kv)
        vals, idx = np.concatenate(out_v), np.concatenate(out_i)
        if len(out_i) == 1:
            return idx


@pytest.mark.parametrize("N,k,ch,kind", [
    (40000, 1024, 8192, "normal"),
    (40000, 2048, 16384, "ties"),
    (262144, 1024, 16384, "normal"),
    (262144, 1024, 16384, "equal"),
    (300000, 4096, 32768, "ties"),
    (5000, 700, 1000, "ties"),        # awkward: k close to the chunk size
    (3000, 1, 1024, "ties"),
])
def test_chunked_rounds_equal_direct_topk(orc, N, k, ch, kind):
    rng = np.random.default_rng(N + k + ch)
    if kind == "normal":
        s = rng.normal(0.0, 1.0, N)
    elif kind == "ties":
        s = rng.integers(0, 5, N).astype(np.float64)
    else:
        s = np.zeros(N)
    for nv in (N, N // 3, min(N, k + 7), min(N, k // 2 + 1)):
        exp, _ = orc.topk(s.reshape(1, 1, N), np.asarray([[nv]], dtype=np.int32), k)
        exp = exp[0, 0]
        exp = np.sort(exp[exp >= 0])
        got = _rounds(s, nv, k, ch)
        np.testing.assert_array_equal(got, exp)
