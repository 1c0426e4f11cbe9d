"""The allocation-free entry point (csa_compress_index_topk_noalloc, its
scratch in the library's static device array) against the workspace form of
the same call: identical caches, top-k lists and scores of the kept entries,
on two calls in a row (the second smaller), through the C ABI."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_c4a_amd import binding as K
from compressed_sparse_attention_c4a_amd import path as P
from compressed_sparse_attention_c4a_amd import workloads as W
from parity import raw_np

pytestmark = pytest.mark.gpu


def _call(inp, workspace):
    sh = inp["shape"]
    d = P.to_device(inp)
    idx = torch.full((sh.B, sh.S, sh.k), -7, dtype=torch.int32, device="cuda")
    val = torch.full((sh.B, sh.S, sh.k), 7.0, dtype=torch.float32, device="cuda")
    ws = None
    if workspace:
        ws = torch.empty(K.csa_index_topk_workspace_size(sh.B, sh.S, sh.N_cap, sh.k), dtype=torch.uint8,
                         device="cuda")
    K.csa_compress_index_topk(d["kv_state"], d["score_state"], d["gamma"], d["cmp_cache"], d["idx_kv_state"],
                              d["idx_score_state"], d["idx_gamma"], d["idx_cache"], d["state_pos0"], d["q_idx"],
                              d["w"], d["q_pos"], idx, val, ratio=sh.ratio, overlap=sh.overlap, rope_dim=sh.rope,
                              idx_rope_dim=sh.idx_rope, workspace=ws)
    torch.cuda.synchronize()
    return raw_np(d["cmp_cache"]), raw_np(d["idx_cache"]), idx.cpu().numpy(), val.cpu().numpy()


def _shapes():
    a = W.Shape(name="noalloc_32k", B=32, S=1, q_pos=32767, N_cap=8192, state_pos0=32760, state_len=8, k=1024,
                seed=41)
    b = W.Shape(name="noalloc_small", B=3, S=1, q_pos=4095, N_cap=1024, state_pos0=4088, state_len=8, k=128,
                seed=42)
    return a, b


def test_noalloc_equals_workspace_form_twice():
    for sh in _shapes():        # the second call is smaller than the first
        inp = W.generate(sh)
        print(f"[noalloc] {sh.name}: B={sh.B} N_cap={sh.N_cap} k={sh.k}", flush=True)
        ref = _call(inp, workspace=True)
        got = _call(inp, workspace=False)
        for r, g, what in zip(ref, got, ("compressed cache", "index cache", "top-k indices", "top-k scores")):
            np.testing.assert_array_equal(g, r, err_msg=f"{sh.name}: {what}")
        assert (got[2] >= 0).all()


def test_noalloc_rejects_more_than_the_static_array():
    sh = W.Shape(name="noalloc_too_big", B=1, S=4096, q_pos=0, N_cap=8192, state_pos0=0, state_len=8, k=16,
                 seed=43, H=16, Hi=16)
    need = K.csa_index_topk_workspace_size(sh.B, sh.S, sh.N_cap, sh.k)
    assert need > 64 << 20
    inp = W.generate(sh)
    d = P.to_device(inp)
    idx = torch.empty((sh.B, sh.S, sh.k), dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError, match="scratch"):
        K.csa_compress_index_topk(d["kv_state"], d["score_state"], d["gamma"], d["cmp_cache"], d["idx_kv_state"],
                                  d["idx_score_state"], d["idx_gamma"], d["idx_cache"], d["state_pos0"], d["q_idx"],
                                  d["w"], d["q_pos"], idx, ratio=sh.ratio, overlap=sh.overlap, rope_dim=sh.rope,
                                  idx_rope_dim=sh.idx_rope, workspace=None)
