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

# name: (workload generator, KV rows in FP8)
WORKLOADS = {
    "csa_decode_32k": ("csa_decode_32k", False),
    "csa_prefill_8k_at_24k": ("csa_prefill_32k", False),
    "hca_decode_128k": ("hca_decode_128k", False),
    "csa_decode_1m": ("csa_decode_1m", False),
    "hca_decode_32k": ("hca_decode_32k", False),
    "swa_decode_32k": ("swa_decode_32k", False),
    "csa_decode_32k_fp8": ("csa_decode_32k", True),
    "hca_decode_128k_fp8": ("hca_decode_128k", True),
}
FP8_ROW_BYTES = 640


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


def algorithmic(sh, kv_fp8: bool = False):
    """Algorithmic bytes and flops per QUERY of each call: what the method
    must move or compute.  Re-reads and the temporary score buffer are
    excluded: with one position per sequence (decode) every gathered row is a
    distinct read; with a chunk of positions (prefill) each sequence's
    compressed and window rows count once for the whole chunk (consecutive
    queries share them), q, out, q_idx, w and the index lists once per query.
    With FP8 KV rows a compressed or window row is 640 bytes."""
    e = 2 if sh.dtype == "bf16" else 4
    rb = FP8_ROW_BYTES if kv_fp8 else sh.D * e  # bytes of one compressed / window row
    t_last = sh.q_pos + sh.S - 1
    nvis = min((t_last + 1) // sh.ratio, sh.N_cap)
    nwin = min(sh.window, t_last + 1)
    m = 2 if sh.overlap else 1
    groups = max(1, sh.S // sh.ratio) if sh.S > 1 else 1
    per = {}
    if sh.swa:  # window rows, q and out only
        win_rows = min(sh.S + sh.window - 1, t_last + 1) if sh.S > 1 else nwin
        per["attn"] = {"bytes": win_rows / sh.S * rb + 2 * sh.H * sh.D * e, "flops": 4.0 * sh.H * nwin * sh.D}
        return per, nwin
    cmp = {"bytes": (2 * sh.state_len * m * sh.D * e + groups * rb) / sh.S, "flops": 0.0}
    # rows of the window span of the chunk (decode: the window itself)
    win_rows = min(sh.S + sh.window - 1, t_last + 1) if sh.S > 1 else nwin
    if sh.indexer:  # both compressors, the index scores and the top-k in one call
        cmp["bytes"] += (2 * sh.state_len * 2 * sh.di * e + groups * sh.di * e) / sh.S
        nvis_avg = np.mean([min((sh.q_pos + s + 1) // sh.ratio, sh.N_cap) for s in range(sh.S)])
        per["compress_index_topk"] = {
            "bytes": cmp["bytes"] + nvis * sh.di * e / sh.S + sh.Hi * sh.di * e + sh.Hi * 4 + sh.k * 4,
            "flops": 2.0 * sh.Hi * sh.di * nvis_avg}
        reads = nwin + min(sh.k, nvis)
        rows = (win_rows + min(sh.N_cap, nvis if sh.S > 1 else min(sh.k, nvis))) / sh.S if sh.S > 1 else reads
        per["attn"] = {"bytes": rows * rb + 2 * sh.H * sh.D * e + sh.k * 4,
                       "flops": 4.0 * sh.H * reads * sh.D}
    else:
        per["compress"] = cmp
        reads = nwin + nvis
        rows = (win_rows + nvis) / sh.S if sh.S > 1 else reads
        per["attn"] = {"bytes": rows * rb + 2 * sh.H * sh.D * e, "flops": 4.0 * sh.H * reads * sh.D}
    return per, reads


def roofline_of(alg_bytes, alg_flops, seconds):
    """The bound (whichever of HBM and MFMA time is larger), what was
    achieved against it, and the fraction of its peak."""
    gbs = alg_bytes / seconds / 1e9
    tfl = alg_flops / seconds / 1e12
    if alg_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > alg_bytes / (HBM_PEAK_GBS * 1e9):
        return {"bound": "mfma", "achieved": round(tfl, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4)}
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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


def cpu_baseline(inp, seconds: float, kv_fp8: bool = False):
    """The oracle (as it stands) on the host cores: full passes over the whole
    batch, repeated until about `seconds` of wall time have been spent."""
    from oracle import oracle as O
    from compressed_sparse_attention_c4a_amd import workloads as W
    sh = inp["shape"]
    if kv_fp8:
        inp = dict(inp)
        inp["cmp_cache"] = O.quantize_rows_fp8(O.widen(inp["cmp_cache"]))
        inp["win_kv"] = O.quantize_rows_fp8(O.widen(inp["win_kv"]))
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
            "cpu_model": cpu_model(),
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


def measure_projections(B: int, iters: int = 30):
    """Time the projections around one attention layer at decode (B tokens):
    csa_q_proj (x -> qr -> q, with the norms and RoPE) and csa_o_proj
    (o -> r -> y), weights packed once beforehand.  The 592 MB of bf16
    weights exceed the 256 MB Infinity Cache, so every call streams them from
    HBM; algorithmic bytes = weights + activations read and written once."""
    import torch
    from compressed_sparse_attention_c4a_amd import binding as K
    from compressed_sparse_attention_c4a_amd import path as P
    from compressed_sparse_attention_c4a_amd import workloads as W

    ps = W.proj_decode_32k(B)
    dev = P.to_device(W.generate_proj(ps), "cuda")
    for k in ("wq_a", "wq_b", "wo_a", "wo_b"):
        dev[k] = K.csa_pack_weights(dev[k])
    M, bf = ps.M, torch.bfloat16
    qr = torch.empty(M, ps.q_rank, dtype=bf, device="cuda")
    q = torch.empty(M, ps.H, ps.D, dtype=bf, device="cuda")
    r = torch.empty(M, ps.groups * ps.o_rank, dtype=bf, device="cuda")
    y = torch.empty(M, ps.d_model, dtype=bf, device="cuda")
    stream = torch.cuda.current_stream()
    cq = K.csa_q_proj(dev["x"], dev["wq_a"], dev["gamma_q"], dev["wq_b"], dev["pos"], qr, q, B=ps.B, S=ps.S,
                      rope_dim=ps.rope, stream=stream, prepare=True)
    co = K.csa_o_proj(dev["o"], dev["wo_a"], dev["wo_b"], r, y, groups=ps.groups, stream=stream, prepare=True)
    HD = ps.H * ps.D
    w_q = 2 * (ps.q_rank * ps.d_model + HD * ps.q_rank)
    w_o = 2 * (ps.o_rank * HD + ps.d_model * ps.groups * ps.o_rank)
    alg_q = w_q + 2 * M * (ps.d_model + 2 * ps.q_rank + HD) + 4 * ps.q_rank
    alg_o = w_o + 2 * M * (HD + 2 * ps.groups * ps.o_rank + ps.d_model)
    fl_q = 2 * M * (ps.d_model * ps.q_rank + ps.q_rank * HD)
    fl_o = 2 * M * (HD * ps.o_rank + ps.groups * ps.o_rank * ps.d_model)
    out = {"workload": ps.name, "tokens": M, "d_model": ps.d_model, "q_rank": ps.q_rank,
           "groups": ps.groups, "o_rank": ps.o_rank, "weight_bytes": w_q + w_o}
    for name, c, alg, fl in [("q_proj", cq, alg_q, fl_q), ("o_proj", co, alg_o, fl_o)]:
        for _ in range(5):
            c()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            c()
        e1.record(stream)
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3 / iters
        out[name] = {"us": round(sec * 1e6, 2), **roofline_of(alg, fl, sec)}
    out["us_per_layer"] = round(out["q_proj"]["us"] + out["o_proj"]["us"], 2)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="csa_decode_32k", choices=sorted(WORKLOADS))
    ap.add_argument("--rotate", type=int, default=0, help="input copies to rotate (0: enough to defeat the MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="wall time of the CPU oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-projections", action="store_true", help="skip the Q/O projection measurement")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as replays of one captured HIP graph per input copy (path.GraphStep)")
    ap.add_argument("--projections-only", action="store_true",
                    help="only measure the Q/O projections at decode (B=32) and print their JSON")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (HBM counter calibration) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1"}))
        sys.exit(2)
    if args.projections_only:
        print(json.dumps({"projections": measure_projections(32, iters=max(1, args.steps))}))
        return

    import torch
    from compressed_sparse_attention_c4a_amd import binding as K
    from compressed_sparse_attention_c4a_amd import path as P
    from compressed_sparse_attention_c4a_amd import workloads as W

    K.load()
    gen, kv_fp8 = WORKLOADS[args.workload]
    sh = getattr(W, gen)()
    inp = W.generate(sh)
    dev0 = P.to_device(inp, "cuda")
    if kv_fp8:  # compressed cache and window rows in FP8 (the library's own quantisation)
        dev0["cmp_cache"] = K.csa_quantize_rows(dev0["cmp_cache"])
        dev0["win_kv"] = K.csa_quantize_rows(dev0["win_kv"])
        torch.cuda.synchronize()
    # rotate enough input copies that the bytes one step touches, summed over
    # the copies, exceed 4x the 256 MB Infinity Cache (bounded by memory)
    per, reads = algorithmic(sh, kv_fp8)
    touched = sum(p["bytes"] for p in per.values()) * sh.B * sh.S
    if sh.indexer:
        touched += 4.0 * sh.B * sh.S * sh.N_cap            # the score buffer
    copy_bytes = sum(v.numel() * v.element_size() for k, v in dev0.items() if k != "shape" and v is not None)
    R = args.rotate or max(2, int(np.ceil(4 * 256e6 / touched)) + 1)
    R = max(1, min(R, 64, int(100e9 // copy_bytes)))
    devs = [dev0] + [{k: (v.clone() if (k != "shape" and v is not None) else v) for k, v in dev0.items()}
                     for _ in range(R - 1)]
    steps = [P.Step(d) for d in devs]
    stream = torch.cuda.current_stream()
    # every library call of a step marshalled once per input copy
    prepared = [st.calls(d, stream, prepare=True) for st, d in zip(steps, devs)]

    calls = list(per)
    Q = sh.B * sh.S
    graphs = [P.GraphStep(d, st) for d, st in zip(devs, steps)] if args.graph else None

    def run_one(i, events=None):
        d, st, pc = devs[i % R], steps[i % R], prepared[i % R]
        if events is None:
            if graphs is not None:
                graphs[i % R].run()
            else:
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
    dom_events = {dominant: []} if graphs is None else {dominant: list(ev_probe[dominant])}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        # (graph replays are not bracketed: the dominant call's time is the probe's)
        run_one(args.warmup + n_probe + i, dom_events if (i % EVERY == 0 and graphs is None) else None)
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
    roof = roofline_of(alg_bytes, alg_flops, dom_ms * 1e-3)
    roof["traffic"] = load_traffic(args.workload, dominant, src_hash)
    roof["kernel"] = dominant
    roof["avg_launch_us"] = round(dom_ms * 1e3, 2)
    roof["algorithmic_bytes_per_launch"] = int(alg_bytes)
    roof["algorithmic_flops_per_launch"] = int(alg_flops)

    step_bytes = sum(p["bytes"] for p in per.values()) * Q
    step_flops = sum(p["flops"] for p in per.values()) * Q
    step_roof_s = max(step_bytes / (HBM_PEAK_GBS * 1e9), step_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12))
    whole = {"bytes_per_step": int(step_bytes), "flops_per_step": int(step_flops),
             "bound": "mfma" if step_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > step_bytes / (HBM_PEAK_GBS * 1e9)
             else "hbm",
             "roofline_step_us": round(step_roof_s * 1e6, 2),
             "frac_of_roofline": round(step_roof_s / (ms_per_step * 1e-3), 4),
             "per_call": {c: roofline_of(per[c]["bytes"] * Q, per[c]["flops"] * Q, avg_probe[c] * 1e-3)
                          for c in calls}}

    proj = measure_projections(sh.B) if (sh.S == 1 and not args.no_projections) else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_seconds, kv_fp8)

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": sh.dtype, "data": "synthetic (seeded N(0,1), PCG64)",
        "config": {"workload": args.workload, "kv_rows": "fp8 (e4m3, 640 B)" if kv_fp8 else sh.dtype, "B": sh.B,
                   "S": sh.S, "context": sh.q_pos + sh.S, "heads": sh.H,
                   "head_dim": sh.D, "rope_dim": sh.rope, "ratio": sh.ratio, "entries": sh.N_cap,
                   "topk": sh.k if sh.indexer else None, "window": sh.window,
                   "indexer": f"{sh.Hi}x{sh.di}" if sh.indexer else None, "reads_per_query": reads,
                   "input_copies_rotated": R},
        "roofline": roof,
        "whole_step": whole,
        "call_us": {c: round(v * 1e3, 2) for c, v in avg_probe.items()},
        "launch": "hip graph replay per step" if graphs is not None else "eager library calls",
        # the projections around the same layer (not part of `value`): the
        # decode step of a whole attention block adds their time
        "projections": proj,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
