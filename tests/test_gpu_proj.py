"""GPU parity of the projections around the attention (low-rank Q with the
per-head norm and RoPE, grouped O-proj) against the oracle, element by
element: small shapes spanning several column tiles, K splits and a ragged
row tail, both row-tile widths (<= 32 rows and 64-row tiles), and the full
DeepSeek-V4-Pro decode sizes (B=32: 7168 -> 1536 -> 128 x 512, and
128 x 512 -> 16 x 1024 -> 7168), where every output element is compared."""
import dataclasses

import numpy as np
import pytest
import torch

from compressed_sparse_attention_c4a_amd import binding as K
from compressed_sparse_attention_c4a_amd import path as P
from compressed_sparse_attention_c4a_amd import workloads as W
from parity import TOL, assert_close, to_np

pytestmark = pytest.mark.gpu


def _packed(dev):
    """The weights in the layout the projections read (packed on the GPU)."""
    return {k: K.csa_pack_weights(dev[k]) for k in ("wq_a", "wq_b", "wo_a", "wo_b")}


def _run_q(dev, ps):
    qr = torch.empty(ps.M, ps.q_rank, dtype=torch.bfloat16, device="cuda")
    q = torch.empty(ps.M, ps.H, ps.D, dtype=torch.bfloat16, device="cuda")
    pw = _packed(dev)
    K.csa_q_proj(dev["x"], pw["wq_a"], dev["gamma_q"], pw["wq_b"], dev["pos"], qr, q, B=ps.B, S=ps.S,
                 rope_dim=ps.rope)
    torch.cuda.synchronize()
    return to_np(qr), to_np(q)


def _run_o(dev, ps):
    r = torch.empty(ps.M, ps.groups * ps.o_rank, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(ps.M, ps.d_model, dtype=torch.bfloat16, device="cuda")
    pw = _packed(dev)
    K.csa_o_proj(dev["o"], pw["wo_a"], pw["wo_b"], r, y, groups=ps.groups)
    torch.cuda.synchronize()
    return to_np(r), to_np(y)


def _check_q(orc, inp, ps, tag):
    print(f"[proj] {tag}: q_proj M={ps.M} d_model={ps.d_model} q_rank={ps.q_rank} H={ps.H} D={ps.D}", flush=True)
    qr, q = _run_q(P.to_device(inp), ps)
    q_ref, qr_ref = orc.q_proj(inp["x"], inp["wq_a"], inp["gamma_q"], inp["wq_b"], inp["pos"], H=ps.H, D=ps.D,
                               rope_dim=ps.rope, S=ps.S, store="bf16")
    assert_close(qr, qr_ref, TOL["bf16"], f"{tag}: qr")
    assert_close(q, q_ref, TOL["bf16"], f"{tag}: q")
    # each head has unit RMS before RoPE, which keeps pair lengths: so after it
    assert np.max(np.abs(np.sqrt(np.mean(q * q, axis=-1)) - 1.0)) < 1e-2


def _check_o(orc, inp, ps, tag):
    print(f"[proj] {tag}: o_proj M={ps.M} H={ps.H} D={ps.D} groups={ps.groups} o_rank={ps.o_rank} "
          f"d_model={ps.d_model}", flush=True)
    r, y = _run_o(P.to_device(inp), ps)
    y_ref, r_ref = orc.o_proj(inp["o"], inp["wo_a"], inp["wo_b"], groups=ps.groups, store="bf16")
    assert_close(r, r_ref.reshape(ps.M, -1), TOL["bf16"], f"{tag}: r")
    assert_close(y, y_ref, TOL["bf16"], f"{tag}: y")


SMALL = [
    # name, B, S, pos, d_model, q_rank, H, D, rope, groups, o_rank
    ("rows6", 2, 3, 5, 1024, 512, 4, 512, 64, 2, 256),
    ("rows32_split", 32, 1, 4095, 3072, 1024, 6, 256, 32, 3, 512),
    ("rows70_tm64", 7, 10, 100000, 1536, 1024, 6, 256, 64, 3, 512),
    ("rows1", 1, 1, 0, 512, 2048, 2, 2048, 64, 1, 512),
    # 1024 column tiles and a 1024 + 512 split: two tiles per workgroup
    ("wide_multi_tile", 2, 1, 77, 512, 1536, 128, 512, 64, 16, 512),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_projections_small(orc, case):
    name, B, S, pos, dm, qrk, H, D, rope, G, orank = case
    ps = W.ProjShape(name=name, B=B, S=S, q_pos=pos, d_model=dm, q_rank=qrk, H=H, D=D, rope=rope, groups=G,
                     o_rank=orank, seed=11)
    inp = W.generate_proj(ps)
    # distinct positions per sequence, so a wrong row->position map shows
    inp["pos"] = (pos + 37 * np.arange(B)).astype(np.int32)
    _check_q(orc, inp, ps, name)
    _check_o(orc, inp, ps, name)


def test_projections_full_size_decode(orc):
    ps = W.proj_decode_32k()
    inp = W.generate_proj(ps)
    _check_q(orc, inp, ps, "proj_decode_32k")
    _check_o(orc, inp, ps, "proj_decode_32k")


def test_projection_prefill_rows(orc):
    """A 512-row chunk (eight 64-row tiles) at the full widths of Q."""
    ps = dataclasses.replace(W.proj_decode_32k(), name="proj_rows512", B=1, S=512, q_pos=24576, H=16, groups=2)
    inp = W.generate_proj(ps)
    _check_q(orc, inp, ps, "proj_rows512")
    _check_o(orc, inp, ps, "proj_rows512")


def test_projections_repeatable():
    """Split-K partials are summed in a fixed order: two calls agree bit for bit."""
    ps = W.ProjShape(name="rep", B=4, S=1, d_model=2048, q_rank=1024, H=8, D=512, groups=2, o_rank=512)
    dev = P.to_device(W.generate_proj(ps))
    a = _run_q(dev, ps)[1], _run_o(dev, ps)[1]
    b = _run_q(dev, ps)[1], _run_o(dev, ps)[1]
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_pack_weights_is_the_documented_permutation():
    """Packed element (g, c, h, j, l, e) is W[g][16c + l%16][512h + 32j + 8(l/16) + e],
    bit for bit; checked with NumPy reshapes on the host."""
    rng = np.random.default_rng(12)
    G, N, Kd = 3, 128, 1024
    w = rng.integers(0, 1 << 16, size=(G, N, Kd), dtype=np.uint16)
    dev = torch.from_numpy(w.view(np.int16)).cuda().view(torch.bfloat16)
    got = K.csa_pack_weights(dev).cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1)
    # W[g, 16c + n, 512h + 32j + 8q + e] -> order (g, c, h, j, q, n, e)
    ref = w.reshape(G, N // 16, 16, Kd // 512, 16, 4, 8).transpose(0, 1, 3, 4, 5, 2, 6).reshape(-1)
    assert np.array_equal(got, ref)
