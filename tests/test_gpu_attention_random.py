"""GPU parity of the attention entry points on seeded random configurations:
batch, heads (16 to 128, so both head groupings and the generic kernel's
H = 8), sparse or dense candidates, ring or linear windows of 8 to 1024 rows,
lists of 0 to 2048 entries with scattered -1 padding, positions from 0 to
deep contexts (several splits, empty splits, ragged tails), bf16 or FP8 rows,
each compared with the oracle on the same inputs.  The configurations are
drawn once from a fixed seed, so a failure names a reproducible case."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_c4a_amd import binding as K
from parity import TOL, assert_close, to_np
from test_gpu_attention import _dev, _inputs

pytestmark = pytest.mark.gpu


def _configs(n=24, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H = int(rng.choice([8, 16, 32, 48, 64, 128]))
        B = int(rng.integers(1, 9)) if H >= 64 else int(rng.integers(1, 17))
        window = int(rng.choice([8, 64, 128, 256, 1024]))
        linear = bool(rng.integers(0, 2))
        S = int(rng.choice([1, 1, 1, 3, 17])) if linear else 1
        B = min(B, 2) if S > 1 else B
        W_cap = window + S - 1 if linear else window
        N_cap = int(rng.choice([16, 300, 1500, 4000]))
        k = int(rng.choice([0, 16, 256, 1024, 2048]))
        dense = bool(rng.integers(0, 2))
        fp8 = bool(rng.integers(0, 4) == 0) and H % 16 == 0 and window <= 1024 and k <= 2048
        top = 4 * N_cap + 400
        q_pos = [int(rng.integers(0, top)) for _ in range(B)]
        out.append(dict(name=f"r{i:02d}", B=B, S=S, H=H, N_cap=N_cap, W_cap=W_cap, k=k, q_pos=q_pos,
                        linear=linear, window=window, dense=dense, fp8=fp8, seed=1000 + i))
    return out


CONFIGS = _configs()


@pytest.mark.parametrize("c", CONFIGS, ids=[c["name"] for c in CONFIGS])
def test_attention_random_configuration(orc, c):
    print(f"[attn-random] {c}", flush=True)
    B, S, H = c["B"], c["S"], c["H"]
    k = max(c["k"], 1)
    x = _inputs(c["seed"], B, S, H, c["N_cap"], c["W_cap"], k, c["q_pos"], c["linear"])
    topk = x["topk"][..., :c["k"]]
    cmp, win = _dev(x["cmp"]), _dev(x["win"])
    cmp_ref, win_ref = x["cmp"], x["win"]
    if c["fp8"]:
        cmp, win = K.csa_quantize_rows(cmp), K.csa_quantize_rows(win)
        cmp_ref, win_ref = cmp.cpu().numpy(), win.cpu().numpy()
    out = torch.empty((B, S, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, S, H), dtype=torch.float32, device="cuda")
    if c["dense"]:
        K.hca_attn(_dev(x["q"]), cmp, win, _dev(x["win_pos0"]), _dev(x["sink"]), _dev(x["q_pos"]), out, lse,
                   ratio=4, rope_dim=64, window=c["window"])
    else:
        K.csa_sparse_attn(_dev(x["q"]), cmp, _dev(np.ascontiguousarray(topk)), win, _dev(x["win_pos0"]),
                          _dev(x["sink"]), _dev(x["q_pos"]), out, lse, rope_dim=64, window=c["window"])
    torch.cuda.synchronize()
    ref, rlse, _ = orc.attn(x["q"], cmp_ref, win_ref, x["sink"], x["q_pos"],
                            topk_idx=None if c["dense"] else topk, ratio=4, win_pos0=x["win_pos0"],
                            window=c["window"], rope_dim=64)
    assert_close(to_np(out), ref, TOL["bf16"], f"{c['name']}: output")
    assert_close(lse.cpu().numpy(), rlse, 1e-3, f"{c['name']}: lse")
