"""GPU parity of a stack of attention layers following the model's schedule:
HCA, HCA, CSA, HCA, CSA and the final SWA layer, every layer with its own
caches and inputs, one decode position through all of them, each layer
against the oracle.  Also: the SWA entry point equals csa_sparse_attn with an
empty selection, bit for bit."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_c4a_amd import binding as K
from compressed_sparse_attention_c4a_amd import path as P
from compressed_sparse_attention_c4a_amd import schedule as SCH
from compressed_sparse_attention_c4a_amd import workloads as W
from parity import TOL, assert_close, check_topk_sets, to_np

pytestmark = pytest.mark.gpu


def test_layer_stack_against_the_oracle(orc):
    kinds = SCH.attention_kinds(6)
    t = 8191
    inps = [W.generate(W.layer_shape(kind, B=2, t=t, seed=60 + i)) for i, kind in enumerate(kinds)]
    print(f"[layers] {kinds} at position {t}", flush=True)
    stack = P.LayerStack([P.to_device(x) for x in inps])
    outs = stack.run()
    torch.cuda.synchronize()
    for i, (kind, inp, st, out) in enumerate(zip(kinds, inps, stack.steps, outs)):
        sh = inp["shape"]
        ref = orc.pipeline(inp)
        if kind == "csa":
            gi = st.topk_idx.cpu().numpy()
            check_topk_sets(gi, ref["topk_idx"], ref["scores"], ref["nvis"], sh.k)
            o2, l2, _ = orc.attn(inp["q"], ref["cmp_cache"], inp["win_kv"], inp["sink"], inp["q_pos"], topk_idx=gi,
                                 ratio=sh.ratio, window=sh.window, rope_dim=sh.rope)
        else:
            o2, l2 = ref["out"], ref["lse"]
        assert_close(to_np(out), o2, TOL["bf16"], f"layer {i} ({kind}): output")
        assert_close(st.lse.cpu().numpy(), l2, 1e-3, f"layer {i} ({kind}): lse")


@pytest.mark.parametrize("q_pos", [[32767, 5000, 40], [127, 64, 0]])
def test_swa_equals_empty_selection(q_pos):
    sh = W.swa_decode_32k(B=3)
    inp = W.generate(sh)
    inp["q_pos"] = np.asarray(q_pos, dtype=np.int32)
    d = P.to_device(inp)
    o1 = torch.empty_like(d["q"])
    o2 = torch.empty_like(d["q"])
    K.swa_attn(d["q"], d["win_kv"], None, d["sink"], d["q_pos"], o1, rope_dim=64, window=128)
    empty = torch.empty((sh.B, sh.S, 0), dtype=torch.int32, device="cuda")
    K.csa_sparse_attn(d["q"], d["cmp_cache"], empty, d["win_kv"], None, d["sink"], d["q_pos"], o2, rope_dim=64,
                      window=128)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
