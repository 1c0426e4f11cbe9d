"""Throughput of one pass of the compressed attention hot path on one MI355X.

A step = csa_compress_index_topk (both compressors, index scores, top-k) +
csa_sparse_attn over one batch of seeded synthetic inputs (CSA), or
csa_compress (C128A) + hca_attn (HCA).  Inputs are resident in HBM before the
timed region; R copies of every input rotate from step to step so the 256 MB
Infinity Cache cannot keep the working set between steps.

Prints one JSON line (rank 0).  Default workload: CSA decode at 32K context,
B=32 queries, 128 heads x 512 dims, top-1024 of 8192 entries, window 128.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA decode queries/s at 32K ctx (B=32, 128 heads); % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0

WORKLOADS = {
    "csa_decode_32k": "csa_decode_32k",
    "csa_prefill_8k_at_24k": "csa_prefill_32k",
    "hca_decode_128k": "hca_decode_128k",
    "csa_decode_1m": "csa_decode_1m",
}


def _kernel_sources_hash(files):
    """Hash of the kernel sources with // comments and blank lines removed, so
    that counter records stay valid across comment-only edits."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "compressed_sparse_attention_c4a_amd", "csrc", f), encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode("utf-8") + b"\n")
    return h.hexdigest()[:16]


def algorithmic(sh):
    """Algorithmic bytes and flops per QUERY of each call (what the method must
    move or compute; re-reads and temporary score buffers are excluded)."""
    e = 2 if sh.dtype == "bf16" else 4
    t_last = sh.q_pos + sh.S - 1
    nvis = min((t_last + 1) // sh.ratio, sh.N_cap)
    nwin = min(sh.window, t_last + 1)
    m = 2 if sh.overlap else 1
    groups = max(1, sh.S // sh.ratio) if sh.S > 1 else 1
    per = {}
    cmp = {"bytes": (2 * sh.state_len * m * sh.D * e + groups * sh.D * e) / sh.S, "flops": 0.0}
    if sh.indexer:  # both compressors, the index scores and the top-k in one call
        cmp["bytes"] += (2 * sh.state_len * 2 * sh.di * e + groups * sh.di * e) / sh.S
        per["compress_index_topk"] = {
            "bytes": cmp["bytes"] + nvis * sh.di * e + sh.Hi * sh.di * e + sh.Hi * 4 + sh.k * 4,
            "flops": 2.0 * sh.Hi * sh.di * nvis}
        reads = nwin + min(sh.k, nvis)
        per["attn"] = {"bytes": reads * sh.D * e + 2 * sh.H * sh.D * e + sh.k * 4,
                       "flops": 4.0 * sh.H * reads * sh.D}
    else:
        per["compress"] = cmp
        reads = nwin + nvis
        per["attn"] = {"bytes": reads * sh.D * e + 2 * sh.H * sh.D * e, "flops": 4.0 * sh.H * reads * sh.D}
    return per, reads


def load_traffic(workload: str, kernel_call: str, src_hash: str):
    """HBM traffic per launch of `kernel_call` in `workload` from committed
    rocprofv3 counter runs, if they were taken on the current kernel sources
    (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f).get("workloads", {}).get(workload, {}).get(kernel_call)
    except (OSError, ValueError, AttributeError):
        return None
    if not rec or rec.get("src_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(inp, seconds: float):
    """The oracle (as it stands) on the host cores: full passes over the whole
    batch, repeated until about `seconds` of wall time have been spent."""
    from oracle import oracle as O
    from compressed_sparse_attention_c4a_amd import workloads as W
    sh = inp["shape"]
    O.pipeline(W.slice_batch(inp, 1))           # warm-up (library load, page-in)
    reps, t0 = 0, time.perf_counter()
    while True:
        O.pipeline(inp)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds or reps >= 1000:
            break
    q = reps * sh.B * sh.S
    return {"value": q / dt, "unit": "queries/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"{reps} full passes (compress, index scores, top-k, attention; fp64) over the whole batch of "
                      f"{sh.name} ({sh.B * sh.S} queries each), {dt:.1f} s wall"}


def copy_calibration(nbytes: int, reps: int = 5):
    """A plain device-to-device copy of known size (nbytes read, nbytes
    written per launch): what FETCH_SIZE / WRITE_SIZE report for it scales
    the counters of the hot-path kernels to bytes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="csa_decode_32k", choices=sorted(WORKLOADS))
    ap.add_argument("--rotate", type=int, default=0, help="input copies to rotate (0: enough to defeat the MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="wall time of the CPU oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (HBM counter calibration) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1"}))
        sys.exit(2)

    import torch
    from compressed_sparse_attention_c4a_amd import binding as K
    from compressed_sparse_attention_c4a_amd import path as P
    from compressed_sparse_attention_c4a_amd import workloads as W

    K.load()
    sh = getattr(W, WORKLOADS[args.workload])()
    inp = W.generate(sh)
    dev0 = P.to_device(inp, "cuda")
    # bytes one copy of the inputs occupies; rotate enough copies to exceed 2x the 256 MB MALL
    copy_bytes = sum(v.numel() * v.element_size() for k, v in dev0.items() if k != "shape" and v is not None)
    R = args.rotate or max(2, int(np.ceil(2 * 256e6 / copy_bytes)) + 1)
    R = min(R, 64)
    devs = [dev0] + [{k: (v.clone() if (k != "shape" and v is not None) else v) for k, v in dev0.items()}
                     for _ in range(R - 1)]
    steps = [P.Step(d) for d in devs]
    stream = torch.cuda.current_stream()
    # every library call of a step marshalled once per input copy
    prepared = [st.calls(d, stream, prepare=True) for st, d in zip(steps, devs)]

    per, reads = algorithmic(sh)
    calls = list(per)
    Q = sh.B * sh.S

    def run_one(i, events=None):
        d, st, pc = devs[i % R], steps[i % R], prepared[i % R]
        if events is None:
            for _, fn in pc:
                fn()
        else:
            st.run_timed(d, stream, events, pc)

    # warm-up, then a probe pass with events around every call to find the
    # dominant one (the timed region below brackets only that call)
    for i in range(args.warmup):
        run_one(i)
    torch.cuda.synchronize()
    ev_probe = {c: [] for c in calls}
    n_probe = max(10, min(args.steps, 50))
    for i in range(n_probe):
        run_one(args.warmup + i, ev_probe)
    torch.cuda.synchronize()
    avg_probe = {c: float(np.mean([a.elapsed_time(b) for a, b in ev_probe[c]])) for c in calls}
    dominant = max(avg_probe, key=avg_probe.get)

    # timed region: exactly K steps.  The dominant call is bracketed by HIP
    # events on every EVERY-th step only: an event record costs the stream a
    # few microseconds, so bracketing every step would inflate the step time.
    EVERY = 8
    dom_events = {dominant: []}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_one(args.warmup + n_probe + i, dom_events if i % EVERY == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_ms = float(np.mean([a.elapsed_time(b) for a, b in dom_events[dominant]]))

    ms_per_step = wall * 1e3 / args.steps
    value = Q * args.steps / wall
    src = {"attn": ["attn.hip", "common.hpp"],
           "compress_index_topk": ["index.hip", "topk.hip", "compress_dev.hpp", "common.hpp"],
           "compress": ["compress.hip", "compress_dev.hpp", "common.hpp"]}[dominant]
    src_hash = _kernel_sources_hash(src)
    alg_bytes = per[dominant]["bytes"] * Q
    alg_flops = per[dominant]["flops"] * Q
    gbs = alg_bytes / (dom_ms * 1e-3) / 1e9
    tfl = alg_flops / (dom_ms * 1e-3) / 1e12
    hbm_t = alg_bytes / (HBM_PEAK_GBS * 1e9)
    mfma_t = alg_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if mfma_t > hbm_t:
        roof = {"bound": "mfma", "achieved": round(tfl, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    roof["traffic"] = load_traffic(sh.name, dominant, src_hash)
    roof["kernel"] = dominant
    roof["avg_launch_us"] = round(dom_ms * 1e3, 2)
    roof["algorithmic_bytes_per_launch"] = int(alg_bytes)
    roof["algorithmic_flops_per_launch"] = int(alg_flops)

    step_bytes = sum(p["bytes"] for p in per.values()) * Q
    whole = {"bytes_per_step": int(step_bytes), "hbm_roofline_step_us": round(step_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
             "frac_of_hbm_roofline": round(step_bytes / (HBM_PEAK_GBS * 1e9) / (ms_per_step * 1e-3), 4)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_seconds)

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": sh.dtype, "data": "synthetic (seeded N(0,1), PCG64)",
        "config": {"workload": sh.name, "B": sh.B, "S": sh.S, "context": sh.q_pos + sh.S, "heads": sh.H,
                   "head_dim": sh.D, "rope_dim": sh.rope, "ratio": sh.ratio, "entries": sh.N_cap,
                   "topk": sh.k if sh.indexer else None, "window": sh.window,
                   "indexer": f"{sh.Hi}x{sh.di}" if sh.indexer else None, "reads_per_query": reads,
                   "input_copies_rotated": R},
        "roofline": roof,
        "whole_step": whole,
        "call_us": {c: round(v * 1e3, 2) for c, v in avg_probe.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
