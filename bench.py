#!/usr/bin/env python3
"""Benchmark of the GPTQ layer-quantization path on one MI355X.

One step = the whole path for one layer: zero H, H += 2·XᵀX over all
calibration tokens, prepare (dead fix, damping, factor U of H_d⁻¹), and the
blocked sweep with lazy updates, packing and Ŵ.  Inputs (W, X) are synthetic,
seeded, and resident in HBM before timing starts.

    python bench.py [--steps K] [--warmup W] [--workload llama7b-attn]

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "ms per layer quantize (4096×4096, 4-bit g128) & weights/s; % MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 MFMA
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def work_figures(m, d, n_tok, B=128):
    """Algorithmic work of each stage (flops / bytes), as defined for the roofline."""
    upd = 0
    for b0 in range(0, d, B):
        b1 = min(b0 + B, d)
        upd += 2 * m * (b1 - b0) * (d - b1)
    return {
        "hessian_flop": d * (d + 1) * n_tok,               # SYRK: upper triangle only
        "hessian_bytes": 2 * n_tok * d + 4 * d * d,        # read X (bf16) once, write H
        "prepare_flop": 2 * d ** 3 // 3,                   # Cholesky + triangular inverse
        "update_flop": upd,                                # lazy block updates
        "sweep_flop": m * d * (B - 1),                     # in-block rank-1 updates
    }


# HBM bytes per gptq_hessian_accumulate call on the 4096x4096, 131072-token
# workload, from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs of
# `bench.py --steps 2 --warmup 1 --no-cpu-baseline` (KiB per dispatch, summed
# over the call's two kernels), each scaled by the counter's reading for a
# plain copy of known size (`bench.py --copy-calibration 512`).  Valid only
# for the Hessian source they were taken on: any change to it reports null.
HESSIAN_TRAFFIC = {
    "source_sha256": "f02b59cf2282f2d04e0f8cfb33a2b948c71b5a9e45235e99ec2d766f33e9a542",
    # zero_chunk_kernel + syrk256_kernel + reduce_mirror_kernel, KiB per call
    "fetch_kib": 1.5 + 2255284.3 + 134888.2, "fetch_scale": 524288 / 262159.7,
    "write_kib": 0.3 + 236544.0 + 65652.9, "write_scale": 524288 / 524288.0,
}


def hessian_traffic():
    import hashlib
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                       "post_weight_quantization_16_amd", "csrc", "hessian.hip")
    t = HESSIAN_TRAFFIC
    if t["source_sha256"] is None:
        return None
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != t["source_sha256"]:
            return None
    return (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024.0


def copy_calibration(mib):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 copies of {mib} MiB (read {mib} MiB, write {mib} MiB each)")


def cpu_baseline(wl, W, X, tok_sample, row_sample):
    """Time the fp64 oracle as it stands on a bounded sample and scale to one layer."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    p = oracle.Params(bits=wl.bits, group_size=wl.group_size, block_size=wl.block_size,
                      percdamp=wl.percdamp, act_order=wl.act_order, sym=wl.sym)
    t0 = time.perf_counter()
    H = oracle.hessian(X[:tok_sample], wl.x_dtype)
    t_h = time.perf_counter() - t0
    H *= wl.n_tok / tok_sample
    t0 = time.perf_counter()
    prep = oracle.prepare(H, p.percdamp, p.act_order)
    t_p = time.perf_counter() - t0
    import synth
    Wr = synth.to_f64(W[:row_sample], wl.w_dtype)
    if prep["perm"] is not None:
        Wr = Wr[:, prep["perm"]]
    t0 = time.perf_counter()
    oracle.gptq_sweep(Wr, prep["U"], p)
    t_s = time.perf_counter() - t0
    total = t_h * wl.n_tok / tok_sample + t_p + t_s * wl.d_out / row_sample
    return {
        "value": wl.d_out * wl.d_in / total,
        "unit": "weights/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"fp64 oracle: H over {tok_sample} of {wl.n_tok} tokens ({t_h:.2f}s, scaled x"
                   f"{wl.n_tok / tok_sample:g}), full prepare ({t_p:.2f}s), sweep of {row_sample} of "
                   f"{wl.d_out} rows ({t_s:.2f}s, scaled x{wl.d_out / row_sample:g}); "
                   f"extrapolated {total:.1f}s per layer"),
        "ms_per_layer": total * 1e3,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama7b-attn")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=16384)
    ap.add_argument("--cpu-rows", type=int, default=512)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the single-GPU path only (the layer runs on one MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import numpy as np
    import torch

    import post_weight_quantization_16_amd as gq
    import synth

    wl = synth.WORKLOADS[args.workload]
    m, d, N = wl.d_out, wl.d_in, wl.n_tok
    log(f"bench: {wl.name}; library {gq.version()}")
    t0 = time.time()
    W_host = synth.make_weights(wl)
    X_host = synth.make_activations(wl)
    log(f"bench: inputs generated in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")

    def up(a, dt):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16) \
            if dt == "bf16" else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        return t.to(dev)

    W = up(W_host, wl.w_dtype)
    X = up(X_host, wl.x_dtype)
    params = gq.GPTQParams(bits=wl.bits, group_size=wl.group_size, block_size=wl.block_size,
                           percdamp=wl.percdamp, act_order=wl.act_order, sym=wl.sym)
    H = torch.empty(d, d, dtype=torch.float32, device=dev)
    ws_h = torch.empty(gq.workspace_bytes(0, 0, d, N), dtype=torch.uint8, device=dev)
    ws_p = torch.empty(gq.workspace_bytes(1, 0, d, 0, params), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(gq.workspace_bytes(2, m, d, 0, params), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        H.zero_()
        if ev: ev[0].record(stream)
        gq.hessian_accumulate(H, X, ws=ws_h)
        if ev: ev[1].record(stream)
        prep = gq.prepare_hinv(H, params, ws=ws_p)
        if ev: ev[2].record(stream)
        out = gq.quantize_layer(W, prep, params, ws=ws_q)
        if ev: ev[3].record(stream)
        return out

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    st = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])]
                   for e in evs])
    h_ms, p_ms, q_ms = (float(x) for x in st.mean(axis=0))
    wf = work_figures(m, d, N)
    log(f"bench: {ms_step:.3f} ms/step; hessian {h_ms:.3f} ms, prepare {p_ms:.3f} ms, "
        f"quantize {q_ms:.3f} ms")
    h_tflops = wf["hessian_flop"] / (h_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": m * d / (ms_step * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16/f32",
        "data": "synthetic",
        "config": {"workload": wl.name, **{k: v for k, v in wl.describe().items() if k != "workload"}},
        "stages_ms": {"hessian": h_ms, "prepare": p_ms, "quantize": q_ms},
        "stage_rates": {
            "hessian_tflops": h_tflops,
            "hessian_frac_bf16_peak": h_tflops / PEAK_BF16_TFLOPS,
            "prepare_tflops": wf["prepare_flop"] / (p_ms * 1e-3) / 1e12,
            "quantize_update_tflops": wf["update_flop"] / (q_ms * 1e-3) / 1e12,
        },
        "roofline": {
            "kernel": "gptq_hessian_accumulate (syrk256_kernel + reduce_mirror_kernel)",
            "bound": "mfma",
            "achieved": h_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": h_tflops / PEAK_BF16_TFLOPS,
            "traffic": hessian_traffic(),
        },
    }
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on the host ...")
        result["cpu_baseline"] = cpu_baseline(wl, W_host, X_host, min(args.cpu_tokens, N),
                                              min(args.cpu_rows, m))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
