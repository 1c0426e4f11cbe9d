"""GPU parity of the attention entry points on shapes that select each
kernel variant (16 or 32 heads per workgroup, candidate lists split over 1 to
16 workgroups, including splits left with no tile), in sparse (CSA) and dense
(HCA) mode, with ring and linear windows, -1 padding anywhere in the
selection, short contexts, the largest window and list, and ragged tile
tails."""
import zlib

import numpy as np
import pytest
import torch

from compressed_sparse_attention_c4a_amd import binding as K
from compressed_sparse_attention_c4a_amd import workloads as W
from parity import TOL, assert_close, to_np

pytestmark = pytest.mark.gpu


def _inputs(seed, B, S, H, N_cap, W_cap, k, q_pos, linear=False, D=512, dtype="bf16"):
    dr = W.Draw(seed)
    q = dr.data((B, S, H, D), dtype)
    cmp = dr.data((B, N_cap, D), dtype)
    win = dr.data((B, W_cap, D), dtype)
    sink = dr.f32((H,))
    rng = np.random.default_rng(seed + 1000)
    q_pos = np.asarray(q_pos, dtype=np.int32)
    topk = np.full((B, S, k), -1, dtype=np.int32)
    for b in range(B):
        for s in range(S):
            nv = min((int(q_pos[b]) + s + 1) // 4, N_cap)
            m = min(k, nv)
            if m:
                sel = rng.choice(nv, size=m, replace=False).astype(np.int32)
                slots = rng.choice(k, size=m, replace=False)     # padding scattered through the list
                topk[b, s, slots] = sel
    win_pos0 = (q_pos - (W_cap - S)).astype(np.int32) if linear else None
    return dict(q=q, cmp=cmp, win=win, sink=sink, q_pos=q_pos, topk=topk, win_pos0=win_pos0)


def _dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


VARIANTS = {
    # name: (B, S, H, N_cap, W_cap, k, q_pos, linear window, window)
    # (the plan, 16 or 32 heads per workgroup and the splits, is the cost model's choice)
    # 16 heads per workgroup, 2 splits (sparse) / 6 splits, most of them empty (dense)
    "split_decode_short_ctx": (5, 1, 128, 600, 128, 96, [2399, 1000, 130, 7, 0], False, 128),
    # 32 heads per workgroup, 64 items, 4 splits
    "h128_four_splits": (16, 1, 128, 2000, 128, 1024, list(range(7999, 7999 - 16 * 37, -37)), False, 128),
    # 256 (query, head group) items: no split
    "nosplit_decode": (64, 1, 128, 300, 128, 40, list(range(400, 1040, 10)), False, 128),
    "prefill_linear_window": (1, 160, 128, 200, 160 + 127, 48, [600], True, 128),
    # 16 heads per workgroup (H % 32 != 0)
    "h48_groups_of_16": (3, 1, 48, 100, 64, 33, [399, 250, 60], False, 64),
    "h96_window_gt_ctx": (100, 1, 96, 64, 128, 20, list(range(0, 200, 2)), False, 128),
    # largest list and window: 48 tiles in 16 splits of 3 (16 heads per workgroup)
    "max_list_16_splits": (2, 1, 32, 4096, 1024, 2048, [16383, 9000], False, 1024),
    # 16 heads, one item, 6 splits
    "h16_one_item_splits": (1, 1, 16, 2000, 256, 512, [7999], False, 256),
    # 256 items, no split, dense lists of 3100-3200 entries: candidates past the 3072-slot table
    "dense_past_table_nosplit": (64, 1, 128, 3200, 128, 16, [12399 + 7 * i for i in range(64)], False, 128),
}


def _seed(name):
    return zlib.crc32(name.encode()) % 1000


@pytest.mark.parametrize("name", sorted(VARIANTS))
@pytest.mark.parametrize("dense", [False, True])
def test_attention_variants(orc, name, dense):
    B, S, H, N_cap, W_cap, k, q_pos, linear, window = VARIANTS[name]
    x = _inputs(_seed(name), B, S, H, N_cap, W_cap, k, q_pos, linear)
    out = torch.empty((B, S, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, S, H), dtype=torch.float32, device="cuda")
    if dense:
        K.hca_attn(_dev(x["q"]), _dev(x["cmp"]), _dev(x["win"]), _dev(x["win_pos0"]), _dev(x["sink"]),
                   _dev(x["q_pos"]), out, lse, ratio=4, rope_dim=64, window=window)
        ref, rlse, _ = orc.attn(x["q"], x["cmp"], x["win"], x["sink"], x["q_pos"], topk_idx=None, ratio=4,
                                win_pos0=x["win_pos0"], window=window, rope_dim=64)
    else:
        K.csa_sparse_attn(_dev(x["q"]), _dev(x["cmp"]), _dev(x["topk"]), _dev(x["win"]), _dev(x["win_pos0"]),
                          _dev(x["sink"]), _dev(x["q_pos"]), out, lse, rope_dim=64, window=window)
        ref, rlse, _ = orc.attn(x["q"], x["cmp"], x["win"], x["sink"], x["q_pos"], topk_idx=x["topk"],
                                win_pos0=x["win_pos0"], window=window, rope_dim=64)
    torch.cuda.synchronize()
    assert_close(to_np(out), ref, TOL["bf16"], f"{name} dense={dense}: output")
    assert_close(lse.cpu().numpy(), rlse, 1e-3, f"{name} dense={dense}: lse")


def test_sparse_with_every_visible_entry_equals_dense(orc):
    B, S, H, N_cap = 4, 1, 128, 256

    def both(q_pos):
        x = _inputs(7, B, S, H, N_cap, 128, 256, q_pos)
        topk = np.full((B, S, 256), -1, dtype=np.int32)
        for b in range(B):
            nv = min((int(x["q_pos"][b]) + 1) // 4, N_cap)
            topk[b, 0, :nv] = np.arange(nv)
        o1 = torch.empty((B, S, H, 512), dtype=torch.bfloat16, device="cuda")
        o2 = torch.empty_like(o1)
        K.csa_sparse_attn(_dev(x["q"]), _dev(x["cmp"]), _dev(topk), _dev(x["win"]), None, _dev(x["sink"]),
                          _dev(x["q_pos"]), o1, rope_dim=64, window=128)
        K.hca_attn(_dev(x["q"]), _dev(x["cmp"]), _dev(x["win"]), None, _dev(x["sink"]), _dev(x["q_pos"]), o2,
                   ratio=4, rope_dim=64, window=128)
        return x, topk, o1, o2

    # every entry visible (k == N_cap == visible): the two calls see the same
    # candidates in the same slots and the same split of them, so they agree
    # bit for bit
    _, _, o1, o2 = both([1023, 2000, 1500, 4000])
    assert torch.equal(o1, o2)
    # fewer visible entries than k: the sparse list is padded with -1, the
    # slots differ, the values agree within the bar
    x, topk, o1, o2 = both([1023, 700, 300, 40])
    ref, _, _ = orc.attn(x["q"], x["cmp"], x["win"], x["sink"], x["q_pos"], topk_idx=None, ratio=4, window=128,
                         rope_dim=64)
    assert_close(to_np(o1), ref, TOL["bf16"], "sparse over every visible entry")
    assert_close(to_np(o2), ref, TOL["bf16"], "dense")


@pytest.mark.parametrize("B,H,N_cap,k,q_pos", [(2, 64, 50, 16, [199, 150]), (1, 32, 2000, 1024, [7000])])
def test_sink_minus_infinity_and_no_rope(orc, B, H, N_cap, k, q_pos):
    S = 1
    x = _inputs(9, B, S, H, N_cap, 128, k, q_pos)
    sink = np.full((H,), -np.inf, dtype=np.float32)
    out = torch.empty((B, S, H, 512), dtype=torch.bfloat16, device="cuda")
    K.csa_sparse_attn(_dev(x["q"]), _dev(x["cmp"]), _dev(x["topk"]), _dev(x["win"]), None, _dev(sink),
                      _dev(x["q_pos"]), out, rope_dim=0, window=128, softmax_scale=0.03)
    ref, _, _ = orc.attn(x["q"], x["cmp"], x["win"], sink, x["q_pos"], topk_idx=x["topk"], window=128, rope_dim=0,
                         scale=0.03)
    assert_close(to_np(out), ref, TOL["bf16"], "no sink, no rope")


@pytest.mark.parametrize("H,q_pos", [(128, [5000, 90, 0]), (48, [300, 127, 1])])
def test_window_only_layer(orc, H, q_pos):
    """A sliding-window-only layer (window plus sink, no compressed channel):
    csa_sparse_attn with an empty selection (k = 0)."""
    B, S = len(q_pos), 1
    x = _inputs(11, B, S, H, 64, 128, 1, q_pos)
    topk = torch.empty((B, S, 0), dtype=torch.int32, device="cuda")
    out = torch.empty((B, S, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, S, H), dtype=torch.float32, device="cuda")
    K.csa_sparse_attn(_dev(x["q"]), _dev(x["cmp"]), topk, _dev(x["win"]), None, _dev(x["sink"]), _dev(x["q_pos"]),
                      out, lse, rope_dim=64, window=128)
    ref, rlse, _ = orc.attn(x["q"], x["cmp"], x["win"], x["sink"], x["q_pos"],
                            topk_idx=np.zeros((B, S, 0), dtype=np.int32), window=128, rope_dim=64)
    assert_close(to_np(out), ref, TOL["bf16"], "window only: output")
    assert_close(lse.cpu().numpy(), rlse, 1e-3, "window only: lse")


@pytest.mark.parametrize("sink_inf", [False, True])
@pytest.mark.parametrize("dense", [False, True])
def test_moving_maximum_and_short_contexts_32_heads(orc, dense, sink_inf):
    """32 heads per workgroup in 4 candidate splits with logits of a wide
    spread (softmax scale 1, standard deviation about 22): the running maximum
    leaves its headroom in many tiles, so the rescale of P and of the
    accumulated output is taken again and again; with a -inf sink it is taken
    on the first valid logit.  Contexts from 1 to 4800 positions leave dense
    splits with no tile and tiles with a ragged tail."""
    B, S, H, N_cap, W_cap, k = 16, 1, 128, 1200, 128, 1024
    q_pos = [0, 1, 2, 30, 31, 32, 63, 64, 95, 127, 128, 200, 700, 2047, 4000, 4799]
    x = _inputs(23 + dense, B, S, H, N_cap, W_cap, k, q_pos)
    sink = np.full((H,), -np.inf, dtype=np.float32) if sink_inf else x["sink"] * np.float32(8.0)
    out = torch.empty((B, S, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, S, H), dtype=torch.float32, device="cuda")
    print(f"[attn] moving max dense={dense} sink_inf={sink_inf}", flush=True)
    if dense:
        K.hca_attn(_dev(x["q"]), _dev(x["cmp"]), _dev(x["win"]), None, _dev(sink), _dev(x["q_pos"]), out, lse,
                   ratio=4, rope_dim=64, window=128, softmax_scale=1.0)
    else:
        K.csa_sparse_attn(_dev(x["q"]), _dev(x["cmp"]), _dev(x["topk"]), _dev(x["win"]), None, _dev(sink),
                          _dev(x["q_pos"]), out, lse, rope_dim=64, window=128, softmax_scale=1.0)
    ref, rlse, _ = orc.attn(x["q"], x["cmp"], x["win"], sink, x["q_pos"], topk_idx=None if dense else x["topk"],
                            ratio=4, window=128, rope_dim=64, scale=1.0)
    torch.cuda.synchronize()
    assert_close(to_np(out), ref, TOL["bf16"], f"moving max dense={dense} sink_inf={sink_inf}: output")
    assert_close(lse.cpu().numpy(), rlse, 1e-3, f"moving max dense={dense} sink_inf={sink_inf}: lse")


@pytest.mark.parametrize("H,B", [(128, 16), (48, 3), (8, 2)])
def test_list_entries_past_the_cache_are_skipped(orc, H, B):
    """Top-k entries at or past N_cap (and negative ones other than -1) select
    nothing, on the GPU as in the oracle (both head groupings and the generic
    kernel)."""
    N_cap, k = 500, 256
    x = _inputs(41 + H, B, 1, H, N_cap, 128, k, [1999 - 37 * i for i in range(B)])
    topk = x["topk"].copy()
    rng = np.random.default_rng(H)
    bad = rng.random(topk.shape) < 0.2
    topk[bad] = rng.choice(np.array([N_cap, N_cap + 3, 2 ** 30, -7, -2 ** 31], dtype=np.int64),
                           size=int(bad.sum())).astype(np.int32)
    out = torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 1, H), dtype=torch.float32, device="cuda")
    print(f"[attn] out-of-range list entries H={H} B={B}", flush=True)
    K.csa_sparse_attn(_dev(x["q"]), _dev(x["cmp"]), _dev(topk), _dev(x["win"]), None, _dev(x["sink"]),
                      _dev(x["q_pos"]), out, lse, rope_dim=64, window=128)
    torch.cuda.synchronize()
    ref, rlse, _ = orc.attn(x["q"], x["cmp"], x["win"], x["sink"], x["q_pos"], topk_idx=topk, window=128, rope_dim=64)
    assert_close(to_np(out), ref, TOL["bf16"], f"out-of-range entries H={H}: output")
    assert_close(lse.cpu().numpy(), rlse, 1e-3, f"out-of-range entries H={H}: lse")
