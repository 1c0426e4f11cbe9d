"""One pass of the compressed attention hot path on device tensors:

    csa_compress_index_topk (both compressors, index scores, top-k)
      -> csa_sparse_attn                                  (CSA layers)
    csa_compress (C128A) -> hca_attn                      (HCA layers)

Every step is a libcsa call; this module only moves the generated inputs to
the device and allocates outputs and workspaces.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as K
from .workloads import Shape


def _dev(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_device(inp: dict, device="cuda") -> dict:
    """Copy a generated workload (numpy) to the device."""
    out = {"shape": inp["shape"]}
    for key, val in inp.items():
        if key != "shape":
            out[key] = None if val is None else _dev(val, device)
    return out


class Step:
    """Outputs and workspaces of one pass, allocated once and reused."""

    def __init__(self, dev: dict):
        sh: Shape = dev["shape"]
        self.sh = sh
        q = dev["q"]
        device = q.device
        self.out = torch.empty_like(q)
        self.lse = torch.empty((sh.B, sh.S, sh.H), dtype=torch.float32, device=device)
        if sh.swa:
            n_cand = sh.window
        elif sh.indexer:
            self.topk_idx = torch.empty((sh.B, sh.S, sh.k), dtype=torch.int32, device=device)
            ws = K.csa_index_topk_workspace_size(sh.B, sh.S, sh.N_cap, sh.k)
            self.idx_ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
            n_cand = sh.window + sh.k
        else:
            n_cand = sh.window + sh.N_cap
        self.attn_ws = K.attn_workspace(sh.B, sh.S, sh.H, sh.D, n_cand, device)

    def calls(self, dev: dict, stream=None, prepare: bool = False):
        """The pass as a list of (name, thunk), in launch order.  With
        prepare=True the thunks are binding.Prepared calls: their arguments
        are marshalled once and every call re-issues the same launches."""
        sh = self.sh
        P = dict(stream=stream, prepare=True)

        def thunk(fn, *a, **kw):
            if prepare:
                return fn(*a, **kw, **P)
            return lambda: fn(*a, **kw, stream=stream)

        if sh.swa:
            # sliding-window layer: the window rows, the sink and the inverse RoPE only
            return [("attn", thunk(K.swa_attn, dev["q"], dev["win_kv"], dev.get("win_pos0"), dev["sink"], dev["q_pos"],
                                   self.out, self.lse, rope_dim=sh.rope, window=sh.window, workspace=self.attn_ws))]
        if sh.indexer:
            # both compressors (main KV and index keys), index scores and top-k
            c = [("compress_index_topk",
                  thunk(K.csa_compress_index_topk, dev["kv_state"], dev["score_state"], dev["gamma"], dev["cmp_cache"],
                        dev["idx_kv_state"], dev["idx_score_state"], dev["idx_gamma"], dev["idx_cache"],
                        dev["state_pos0"], dev["q_idx"], dev["w"], dev["q_pos"], self.topk_idx, ratio=sh.ratio,
                        overlap=sh.overlap, rope_dim=sh.rope, idx_rope_dim=sh.idx_rope, workspace=self.idx_ws))]
            c.append(("attn", thunk(K.csa_sparse_attn, dev["q"], dev["cmp_cache"], self.topk_idx, dev["win_kv"],
                                    dev.get("win_pos0"), dev["sink"], dev["q_pos"], self.out, self.lse,
                                    rope_dim=sh.rope, window=sh.window, workspace=self.attn_ws)))
        else:
            c = [("compress", thunk(K.csa_compress, dev["kv_state"], dev["score_state"], dev["gamma"],
                                    dev["cmp_cache"], dev["state_pos0"], ratio=sh.ratio, overlap=sh.overlap,
                                    rope_dim=sh.rope))]
            c.append(("attn", thunk(K.hca_attn, dev["q"], dev["cmp_cache"], dev["win_kv"], dev.get("win_pos0"),
                                    dev["sink"], dev["q_pos"], self.out, self.lse, ratio=sh.ratio, rope_dim=sh.rope,
                                    window=sh.window, workspace=self.attn_ws)))
        return c

    def run(self, dev: dict, stream=None):
        for _, fn in self.calls(dev, stream):
            fn()
        return self.out

    def run_timed(self, dev: dict, stream, events: dict, calls=None):
        """As run(); calls named in `events` are bracketed by timing events
        recorded on `stream` (the stream the kernels are launched on).  `calls`
        may pass a prepared call list for this dev and stream."""
        for name, fn in (calls if calls is not None else self.calls(dev, stream)):
            if name in events:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                events[name].append((a, b))
            else:
                fn()
        return self.out


class LayerStack:
    """One decode pass through a stack of attention layers, each of its own
    type (CSA, HCA or SWA; see schedule.attention_kinds) with its own caches
    and inputs.  The Q/O projections between layers are outside this path, so
    every layer's q is its own generated input."""

    def __init__(self, devs: list):
        self.devs = devs
        self.steps = [Step(d) for d in devs]

    def calls(self, stream=None, prepare: bool = False):
        out = []
        for i, (st, d) in enumerate(zip(self.steps, self.devs)):
            for name, fn in st.calls(d, stream, prepare=prepare):
                out.append((f"layer{i}.{d['shape'].kind}.{name}", fn))
        return out

    def run(self, stream=None):
        for _, fn in self.calls(stream):
            fn()
        return [st.out for st in self.steps]


class GraphStep:
    """One pass of the path captured once into a HIP graph and replayed: the
    same library launches (the Prepared calls of Step, on the capture stream),
    issued by one graph launch instead of one host call each.  Nothing is
    allocated during capture (outputs and workspaces belong to the Step) and
    no launch path of the library records a memset.  Replays overwrite the
    Step's outputs in place."""

    def __init__(self, dev: dict, step: "Step" = None):
        self.dev = dev
        self.step = step if step is not None else Step(dev)
        self.step.run(dev)  # first calls outside the capture (library load, one-time host work)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            cs = torch.cuda.current_stream()
            for _, fn in self.step.calls(dev, cs, prepare=True):
                fn()
        torch.cuda.synchronize()

    @property
    def out(self):
        return self.step.out

    def run(self):
        self.graph.replay()
        return self.step.out
