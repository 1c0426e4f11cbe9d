"""A decode pass captured into a HIP graph (path.GraphStep) gives, on every
replay, exactly the outputs of the eager calls: replayed several times, with
eager work and synchronisations of the program between the replays."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_c4a_amd import path as P
from compressed_sparse_attention_c4a_amd import workloads as W

pytestmark = pytest.mark.gpu


def _state(step, dev, sh):
    out = [step.out.clone(), step.lse.clone(), dev["cmp_cache"].clone()]
    if sh.indexer:
        out += [step.topk_idx.clone(), dev["idx_cache"].clone()]
    return out


@pytest.mark.parametrize("name", ["csa_decode_32k", "hca_decode_32k", "swa_decode_32k"])
def test_graph_replays_equal_eager(name):
    sh = getattr(W, name)()
    inp = W.generate(sh)
    print(f"[graph] {name}", flush=True)
    dev_e = P.to_device(inp)
    eager = P.Step(dev_e)
    eager.run(dev_e)
    torch.cuda.synchronize()
    ref = _state(eager, dev_e, sh)
    dev_g = P.to_device(inp)
    gs = P.GraphStep(dev_g)
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        gs.run()
        junk.mul_(1.0001).add_(0.5)         # the program's own eager work between replays
        torch.cuda.synchronize()
        got = _state(gs.step, dev_g, sh)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager pass"
        eager.run(dev_e)                      # and an eager pass of the other copy
        torch.cuda.synchronize()
