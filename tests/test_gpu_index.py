"""GPU parity of csa_index_scores on its own against the oracle, for the
query layouts the scoring kernels distinguish: one position per sequence
(each workgroup scores one query over a chunk of candidates) and chunks of
positions (S >= 4: a workgroup scores four consecutive queries against shared
key tiles).  Covers S not a multiple of four (idle waves in the last group),
candidate ranges split over several chunks with a ragged last tile, queries
whose visible range ends inside a tile or covers nothing, and the signed
(no-ReLU) form.  Visibility must match exactly; scores to the bf16 score
tolerance."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_c4a_amd import binding as K
from compressed_sparse_attention_c4a_amd.workloads import bf16_bits
from parity import SCORE_TOL, assert_close

pytestmark = pytest.mark.gpu

CASES = [
    # (B, S, N_cap, q_pos list, relu)
    (2, 1, 700, [2799, 1001], True),
    (1, 4, 700, [2795], True),
    (2, 6, 1000, [3990, 100], True),        # second sequence: few visible entries
    (1, 9, 300, [1100], False),             # signed form, ragged last group
    (1, 37, 64, [130], True),               # early positions: visible range inside one tile
    (3, 5, 2000, [7999, 2, 5000], True),    # positions 2..6: nothing visible for the first ones
    (1, 64, 4096, [16320], True),           # many chunks per group
]


@pytest.mark.parametrize("B,S,N_cap,q_pos,relu", CASES)
def test_index_scores_match_oracle(orc, B, S, N_cap, q_pos, relu):
    rng = np.random.default_rng(B * 1000 + S * 10 + N_cap)
    Hi, di = 64, 128
    q_idx = bf16_bits(rng.standard_normal((B, S, Hi, di)).astype(np.float32))
    kc = bf16_bits(rng.standard_normal((B, N_cap, di)).astype(np.float32))
    w = (rng.standard_normal((B, S, Hi)) / np.sqrt(di) / np.sqrt(Hi)).astype(np.float32)
    qp = np.asarray(q_pos, dtype=np.int32)
    exp, _ = orc.index_scores(q_idx, w, kc, qp, 4, relu=relu)
    dev = lambda a: torch.from_numpy(a).cuda().view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a).cuda()
    scores = torch.empty((B, S, N_cap), dtype=torch.float32, device="cuda")
    K.csa_index_scores(dev(q_idx), dev(w), dev(kc), dev(qp), scores, ratio=4, relu=relu)
    got = scores.cpu().numpy().astype(np.float64)
    vis = np.isfinite(exp)
    np.testing.assert_array_equal(np.isfinite(got), vis)     # visibility is exact
    if vis.any():
        assert_close(got[vis], exp[vis], SCORE_TOL["bf16"], "index scores")
