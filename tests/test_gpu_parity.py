"""GPU parity: every libcsa entry point against the fp64 oracle, stage by stage
on identical inputs and end to end, at sizes the oracle finishes in seconds
(several tiles, ragged tails, edge cases).  Calls go through the C ABI."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_c4a_amd import binding as K
from compressed_sparse_attention_c4a_amd import path as P
from compressed_sparse_attention_c4a_amd import workloads as W
from parity import (SCORE_TOL, TOL, assert_close, check_topk_sets, raw_np, to_np)

pytestmark = pytest.mark.gpu


def _with_positions(inp, q_pos, state_back=7):
    """Give every batch row its own query position (ragged contexts)."""
    inp = dict(inp)
    q_pos = np.asarray(q_pos, dtype=np.int32)
    inp["q_pos"] = q_pos
    sh = inp["shape"]
    inp["state_pos0"] = (q_pos - state_back).astype(np.int32) if sh.S == 1 else inp["state_pos0"]
    return inp


def _cases():
    c = {}
    c["tiny_fp32"] = W.tiny_fp32()
    sh = W.Shape(name="csa_decode_small", B=3, S=1, N_cap=700, window=128, W_cap=128, state_len=8, k=64, seed=11)
    c["csa_decode_ragged_bf16"] = _with_positions(W.generate(sh), [2799, 2000, 1235])
    sh = W.Shape(name="csa_decode_short", B=3, S=1, N_cap=64, window=128, W_cap=128, state_len=8, k=64, seed=12)
    c["csa_decode_short_ctx_bf16"] = _with_positions(W.generate(sh), [200, 2, 71])   # nvis < k, nvis == 0, t < window
    sh = W.Shape(name="csa_prefill_small", B=1, S=37, q_pos=130, N_cap=64, window=128, W_cap=37 + 127,
                 win_linear=True, win_pos0=130 - 127, state_pos0=128, state_len=39, k=16, seed=13)
    c["csa_prefill_small_bf16"] = W.generate(sh)
    sh = W.Shape(name="hca_small", B=2, S=1, ratio=128, overlap=False, N_cap=8, window=128, W_cap=128,
                 state_len=128, indexer=False, seed=14)
    c["hca_decode_small_bf16"] = _with_positions(W.generate(sh), [639, 1023], state_back=127)
    sh = W.Shape(name="csa_decode_fp32", B=2, S=1, H=16, D=128, rope=32, N_cap=300, window=16, W_cap=16,
                 state_len=8, Hi=4, di=64, idx_rope=16, k=40, dtype="fp32", seed=15)
    c["csa_decode_fp32"] = _with_positions(W.generate(sh), [1199, 503])
    return c


CASES = _cases()


def _dt(sh):
    return "fp32" if sh.dtype == "fp32" else "bf16"


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request, orc):
    inp = CASES[request.param]
    ref = orc.pipeline(inp)
    return request.param, inp, ref


def test_compress_stage(case, orc):
    name, inp, ref = case
    sh = inp["shape"]
    dev = P.to_device(inp)
    K.csa_compress(dev["kv_state"], dev["score_state"], dev["gamma"], dev["cmp_cache"], dev["state_pos0"],
                   ratio=sh.ratio, overlap=sh.overlap, rope_dim=sh.rope)
    got = to_np(dev["cmp_cache"])
    wr = ref["written"]
    if wr.any():
        assert_close(got[wr], ref["cmp_vals"][wr], TOL[_dt(sh)], f"{name}: compressed rows")
    # rows that are not complete stay untouched
    np.testing.assert_array_equal(raw_np(dev["cmp_cache"])[~wr], inp["cmp_cache"][~wr])
    if sh.indexer:
        K.csa_compress(dev["idx_kv_state"], dev["idx_score_state"], dev["idx_gamma"], dev["idx_cache"],
                       dev["state_pos0"], ratio=sh.ratio, overlap=True, rope_dim=sh.idx_rope)
        iw = ref["idx_written"]
        if iw.any():
            assert_close(to_np(dev["idx_cache"])[iw], ref["idx_vals"][iw], TOL[_dt(sh)], f"{name}: index rows")
        np.testing.assert_array_equal(raw_np(dev["idx_cache"])[~iw], inp["idx_cache"][~iw])


def test_paired_compress_equals_two_calls(case):
    """csa_compress_kv_index (one launch) writes exactly what two csa_compress
    calls write, and nothing else."""
    name, inp, _ = case
    sh = inp["shape"]
    if not sh.indexer:
        pytest.skip("HCA has no index-key compressor")
    a, b = P.to_device(inp), P.to_device(inp)
    K.csa_compress(a["kv_state"], a["score_state"], a["gamma"], a["cmp_cache"], a["state_pos0"], ratio=sh.ratio,
                   overlap=sh.overlap, rope_dim=sh.rope)
    K.csa_compress(a["idx_kv_state"], a["idx_score_state"], a["idx_gamma"], a["idx_cache"], a["state_pos0"],
                   ratio=sh.ratio, overlap=True, rope_dim=sh.idx_rope)
    K.csa_compress_kv_index(b["kv_state"], b["score_state"], b["gamma"], b["cmp_cache"], b["idx_kv_state"],
                            b["idx_score_state"], b["idx_gamma"], b["idx_cache"], b["state_pos0"], ratio=sh.ratio,
                            overlap=sh.overlap, rope_dim=sh.rope, idx_rope_dim=sh.idx_rope)
    np.testing.assert_array_equal(raw_np(a["cmp_cache"]), raw_np(b["cmp_cache"]))
    np.testing.assert_array_equal(raw_np(a["idx_cache"]), raw_np(b["idx_cache"]))


def _separate_and_fused(inp):
    """csa_compress_kv_index + csa_index_topk on one device copy of the
    inputs, csa_compress_index_topk on another; returns both copies with
    their top-k lists and workspaces."""
    sh = inp["shape"]
    out = []
    for fused in (False, True):
        d = P.to_device(inp)
        idx = torch.empty((sh.B, sh.S, sh.k), dtype=torch.int32, device="cuda")
        ws = torch.empty(K.csa_index_topk_workspace_size(sh.B, sh.S, sh.N_cap, sh.k), dtype=torch.uint8,
                         device="cuda")
        if fused:
            K.csa_compress_index_topk(d["kv_state"], d["score_state"], d["gamma"], d["cmp_cache"], d["idx_kv_state"],
                                      d["idx_score_state"], d["idx_gamma"], d["idx_cache"], d["state_pos0"],
                                      d["q_idx"], d["w"], d["q_pos"], idx, ratio=sh.ratio, overlap=sh.overlap,
                                      rope_dim=sh.rope, idx_rope_dim=sh.idx_rope, workspace=ws)
        else:
            K.csa_compress_kv_index(d["kv_state"], d["score_state"], d["gamma"], d["cmp_cache"], d["idx_kv_state"],
                                    d["idx_score_state"], d["idx_gamma"], d["idx_cache"], d["state_pos0"],
                                    ratio=sh.ratio, overlap=sh.overlap, rope_dim=sh.rope, idx_rope_dim=sh.idx_rope)
            K.csa_index_topk(d["q_idx"], d["w"], d["idx_cache"], d["q_pos"], idx, ratio=sh.ratio, workspace=ws)
        out.append((d, idx, ws))
    return out


def _assert_fused_equal(inp):
    sh = inp["shape"]
    (a, ia, wa), (b, ib, wb) = _separate_and_fused(inp)
    np.testing.assert_array_equal(raw_np(a["cmp_cache"]), raw_np(b["cmp_cache"]))
    np.testing.assert_array_equal(raw_np(a["idx_cache"]), raw_np(b["idx_cache"]))
    n = sh.B * sh.S * sh.N_cap
    np.testing.assert_array_equal(wa[:4 * n].view(torch.float32).cpu().numpy(),
                                  wb[:4 * n].view(torch.float32).cpu().numpy())   # the scores, bit for bit
    np.testing.assert_array_equal(ia.cpu().numpy(), ib.cpu().numpy())


def test_fused_compress_index_topk_equals_separate_calls(case):
    """csa_compress_index_topk (fused launch for decode, two launches
    otherwise) writes the same caches, scores and top-k as the separate calls."""
    name, inp, _ = case
    if not inp["shape"].indexer:
        pytest.skip("HCA has no indexer")
    _assert_fused_equal(inp)


def test_fused_decode_new_entry_at_tile_and_chunk_edges():
    """Decode at full N_cap with the freshly written index entry at the
    first/last row of a wave tile, of a workgroup chunk and of the cache: the
    wave that scores it computes it in the fused launch.  Entry 1 (position 7,
    state starting at position 0) completes entries 0 and 1 in the same step:
    both must be scored from their new values."""
    entries = [0, 1, 31, 32, 255, 256, 4095, 5000, 8191]
    q_pos = [4 * e + 3 for e in entries]
    sh = W.Shape(name="csa_decode_edges", B=len(entries), S=1, N_cap=8192, window=128, W_cap=128, state_len=8,
                 k=1024, seed=21)
    inp = dict(W.generate(sh))
    inp["q_pos"] = np.asarray(q_pos, dtype=np.int32)
    inp["state_pos0"] = (inp["q_pos"] - 7).astype(np.int32)
    assert inp["state_pos0"][1] == 0
    print(f"[fused] entries {entries}", flush=True)
    _assert_fused_equal(inp)


def test_index_score_stage(case, orc):
    name, inp, ref = case
    sh = inp["shape"]
    if not sh.indexer:
        pytest.skip("HCA has no indexer")
    dev = P.to_device(inp)
    idx_cache = P._dev(ref["idx_cache"], "cuda")          # the oracle's compressed index rows
    scores = torch.empty((sh.B, sh.S, sh.N_cap), dtype=torch.float32, device="cuda")
    K.csa_index_scores(dev["q_idx"], dev["w"], idx_cache, dev["q_pos"], scores, ratio=sh.ratio)
    got = scores.cpu().numpy().astype(np.float64)
    exp = ref["scores"]
    vis = np.isfinite(exp)
    np.testing.assert_array_equal(np.isfinite(got), vis)     # visibility is exact
    if vis.any():
        assert_close(got[vis], exp[vis], SCORE_TOL[_dt(sh)], f"{name}: index scores")


def test_topk_stage_exact_on_identical_scores(case, orc):
    name, inp, ref = case
    sh = inp["shape"]
    if not sh.indexer:
        pytest.skip("HCA has no indexer")
    s32 = ref["scores"].astype(np.float32)
    s64 = s32.astype(np.float64)                    # both sides decide on the same fp32 scores
    o_idx, _ = orc.topk(s64, ref["nvis"], sh.k)
    scores = torch.from_numpy(s32).cuda()
    idx = torch.empty((sh.B, sh.S, sh.k), dtype=torch.int32, device="cuda")
    val = torch.empty((sh.B, sh.S, sh.k), dtype=torch.float32, device="cuda")
    K.csa_topk(scores, torch.from_numpy(inp["q_pos"]).cuda(), idx, val, ratio=sh.ratio)
    gi = idx.cpu().numpy()
    check_topk_sets(gi, o_idx, s64, ref["nvis"], sh.k, exact=True)
    gv = val.cpu().numpy()
    for qi, (row_i, row_v) in enumerate(zip(gi.reshape(-1, sh.k), gv.reshape(-1, sh.k))):
        m = row_i >= 0
        np.testing.assert_array_equal(row_v[m], s32.reshape(-1, sh.N_cap)[qi, row_i[m]])


def test_attention_stage(case, orc):
    name, inp, ref = case
    sh = inp["shape"]
    dev = P.to_device(inp)
    cmp = P._dev(ref["cmp_cache"], "cuda")
    out = torch.empty_like(dev["q"])
    lse = torch.empty((sh.B, sh.S, sh.H), dtype=torch.float32, device="cuda")
    if sh.indexer:
        topk = torch.from_numpy(ref["topk_idx"]).cuda()
        K.csa_sparse_attn(dev["q"], cmp, topk, dev["win_kv"], dev.get("win_pos0"), dev["sink"], dev["q_pos"], out,
                          lse, rope_dim=sh.rope, window=sh.window)
    else:
        K.hca_attn(dev["q"], cmp, dev["win_kv"], dev.get("win_pos0"), dev["sink"], dev["q_pos"], out, lse,
                   ratio=sh.ratio, rope_dim=sh.rope, window=sh.window)
    assert_close(to_np(out), ref["out"], TOL[_dt(sh)], f"{name}: attention output")
    assert_close(lse.cpu().numpy(), ref["lse"], TOL["fp32"] if sh.dtype == "fp32" else 1e-3, f"{name}: lse")


def test_end_to_end(case, orc):
    name, inp, ref = case
    sh = inp["shape"]
    dev = P.to_device(inp)
    step = P.Step(dev)
    out = step.run(dev)
    torch.cuda.synchronize()
    tol = TOL[_dt(sh)]
    wr = ref["written"]
    if wr.any():
        assert_close(to_np(dev["cmp_cache"])[wr], ref["cmp_vals"][wr], tol, f"{name}: compressed rows")
    if sh.indexer:
        gi = step.topk_idx.cpu().numpy()
        check_topk_sets(gi, ref["topk_idx"], ref["scores"], ref["nvis"], sh.k)
        # attention of the oracle on the GPU's own selection (a legitimate tie swap is not an error)
        o2, _, _ = orc.attn(inp["q"], ref["cmp_cache"], inp["win_kv"], inp["sink"], inp["q_pos"], topk_idx=gi,
                            ratio=sh.ratio, win_pos0=inp.get("win_pos0"), window=sh.window, rope_dim=sh.rope)
        assert_close(to_np(out), o2, tol, f"{name}: output")
    else:
        assert_close(to_np(out), ref["out"], tol, f"{name}: output")


def test_repeat_runs_are_bitwise_identical(case):
    name, inp, _ = case
    dev = P.to_device(inp)
    step = P.Step(dev)
    a = raw_np(step.run(dev)).copy()
    b = raw_np(step.run(dev))
    np.testing.assert_array_equal(a, b)


def _random_decode_cases(n=8, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 13))
        N_cap = int(rng.choice([64, 700, 3000, 8192, 9000]))
        k = int(rng.choice([16, 256, 1024, 2048]))
        state_len = 8 if rng.integers(0, 4) else int(rng.integers(4, 8))   # 2 * ratio tokens, sometimes fewer
        q_pos = rng.integers(0, 4 * N_cap + 64, B)
        q_pos[rng.integers(0, B)] = 4 * int(rng.integers(0, N_cap)) + 3   # one sequence completes an entry
        q_pos = np.maximum(q_pos, state_len - 1)    # the state starts at position 0 or later
        out.append((f"d{i}", B, N_cap, k, state_len, q_pos.astype(np.int32), 900 + i))
    return out


@pytest.mark.parametrize("case", _random_decode_cases(), ids=lambda c: c[0])
def test_fused_decode_random_positions(orc, case):
    """Seeded random decode batches (ragged positions, states of 8 tokens (at
    times 4 to 7) ending at each query's position, caches of 64 to 9000 entries, k of 16
    to 2048): the fused call equals the separate calls bit for bit, and the
    cache rows it writes and its top-k sets match the oracle."""
    name, B, N_cap, k, L, q_pos, seed = case
    print(f"[fused-random] {name}: B={B} N_cap={N_cap} k={k} L={L} q_pos={q_pos.tolist()}", flush=True)
    sh = W.Shape(name=f"fused_random_{name}", B=B, S=1, N_cap=N_cap, window=128, W_cap=128, state_len=L, k=k,
                 seed=seed)
    inp = dict(W.generate(sh))
    inp["q_pos"] = q_pos
    inp["state_pos0"] = (q_pos - (L - 1)).astype(np.int32)
    _assert_fused_equal(inp)
    ref = orc.pipeline(inp)
    (d, idx, _), _ = _separate_and_fused(inp)
    wr = ref["written"]
    if wr.any():
        assert_close(to_np(d["cmp_cache"])[wr], ref["cmp_vals"][wr], TOL["bf16"], f"{name}: compressed rows")
    iw = ref["idx_written"]
    if iw.any():
        assert_close(to_np(d["idx_cache"])[iw], ref["idx_vals"][iw], TOL["bf16"], f"{name}: index rows")
    nvis = np.minimum((q_pos + 1) // 4, N_cap)
    check_topk_sets(idx.cpu().numpy().reshape(B, k), ref["topk_idx"].reshape(B, k), ref["scores"].reshape(B, -1),
                    nvis, k)
