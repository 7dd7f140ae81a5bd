#!/usr/bin/env python3
"""Benchmark of the GPTQ layer-quantization path on one MI355X.

One step = the whole path for one layer: H = 2·XᵀX over all calibration
tokens, prepare (dead fix, damping, factor U of H_d⁻¹), and the blocked
sweep with lazy updates, packing and Ŵ.  Inputs (W, X) are synthetic,
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
PEAK_FP64_TFLOPS = 78.6     # MI355X fp64 (vector and matrix)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def work_figures(m, d, n_tok, B=128, g=128, w_bytes=2, x_bytes=2):
    """Algorithmic work of each stage (flops / bytes), as defined for the roofline."""
    upd = 0
    for b0 in range(0, d, B):
        b1 = min(b0 + B, d)
        upd += 2 * m * (b1 - b0) * (d - b1)
    # the part the GEMM launches do: each 512-column super-block's update of
    # everything right of it (the updates inside a super-block run in the
    # sweep kernel, timed with the sweep)
    sup = 0
    for s0 in range(0, d, 4 * B):
        s1 = min(s0 + 4 * B, d)
        sup += 2 * m * (s1 - s0) * (d - s1)
    ng = (d + g - 1) // g
    return {
        "hessian_flop": d * (d + 1) * n_tok,               # SYRK: upper triangle only
        "hessian_bytes": x_bytes * n_tok * d + 4 * d * d,  # read X once, write H
        "prepare_flop": 2 * d ** 3 // 3,                   # Cholesky + triangular inverse
        "update_flop": upd,                                # lazy block updates, all
        "superblock_update_flop": sup,                     # those done by the GEMM launches
        "sweep_flop": m * d * (B - 1),                     # in-block rank-1 updates
        # the whole layer's compulsory traffic: X and W read once; H written
        # and read, U written and read; codes (4-bit), Ŵ (fp32), scales and
        # zeros written
        "layer_bytes": (x_bytes * n_tok * d + w_bytes * m * d + 4 * 4 * d * d
                        + m * d // 2 + 4 * m * d + 5 * m * ng),
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# HBM bytes per gptq_hessian call on the 4096x4096, 131072-token
# workload, from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs of
# `bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-extras` (KiB per
# dispatch, summed over the call's four kernels), each scaled by the counter's reading for a
# plain copy of known size (`bench.py --copy-calibration 512`).  Valid only
# for the Hessian source they were taken on: any change to it reports null.
HESSIAN_TRAFFIC = {
    "source_sha256": "6fb1320b11bb3bddd82f3a7a19ad510aa0149d858edcefd4a191d080e04ecc53",
    # zero_chunk + shift_mean + syrk256 + reduce_mirror kernels, KiB per call
    "fetch_kib": 1.1 + 16417.5 + 2647161.9 + 127117.1, "fetch_scale": 524288 / 262159.4,
    "write_kib": 0.2 + 8.0 + 253952.0 + 65652.4, "write_scale": 524288 / 524288.0,
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
    """Time the fp64 oracle as it stands on the host cores: the whole layer
    (every token, every row) unless a smaller sample is asked for, in which
    case the measured stages are scaled to one layer and the line says so."""
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
    whole = tok_sample == wl.n_tok and row_sample == wl.d_out
    if whole:
        sample = (f"fp64 oracle over the whole layer: H over all {wl.n_tok} tokens ({t_h:.2f}s), "
                  f"prepare ({t_p:.2f}s), sweep of all {wl.d_out} rows ({t_s:.2f}s); "
                  f"{total:.1f}s per layer")
    else:
        sample = (f"fp64 oracle: H over {tok_sample} of {wl.n_tok} tokens ({t_h:.2f}s, scaled x"
                  f"{wl.n_tok / tok_sample:g}), full prepare ({t_p:.2f}s), sweep of {row_sample} of "
                  f"{wl.d_out} rows ({t_s:.2f}s, scaled x{wl.d_out / row_sample:g}); "
                  f"extrapolated {total:.1f}s per layer")
    return {
        "value": wl.d_out * wl.d_in / total,
        "unit": "weights/s",
        "cores": int(cores),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": sample,
        "ms_per_layer": total * 1e3,
        "stage_s": {"hessian": t_h, "prepare": t_p, "sweep": t_s},
    }


def time_events(fn, reps, stream):
    """Average milliseconds of fn() over reps calls, HIP events on `stream`.
    A spin kernel first holds the GPU while the host queues all the calls, so
    short calls are timed back to back on the GPU, not at the host's pace."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    torch.cuda._sleep(10_000_000)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def extras(gq, torch, wl, W, X, params, H, ws_h, ws_p, stream):
    """Throughput of the rows beyond the single layer, on the same inputs:
    several layers against one factor, independent small layers run
    concurrently, the exported layer's W4A16 product, and the OBQ comparator
    on a tiny layer."""
    import numpy as np
    import synth
    out = {}
    m, d = W.shape
    # three layers fed the same X (query/key/value): one H, one factor, one call
    Ws = [W] + [torch.from_numpy(synth.make_weights(wl.scaled(seed=wl.seed + 100 + i)).view(np.int16))
                .view(torch.bfloat16).to(W.device) for i in range(2)]
    ws_q3 = torch.empty(gq.workspace_bytes(2, 3 * m, d, 0, params), dtype=torch.uint8, device=W.device)

    def batched():
        H.zero_()
        gq.hessian_accumulate(H, X, ws=ws_h)
        prep = gq.prepare_hinv(H, params, ws=ws_p)
        gq.quantize_layers(Ws, prep, params, ws=ws_q3)

    def separate():
        H.zero_()
        gq.hessian_accumulate(H, X, ws=ws_h)
        prep = gq.prepare_hinv(H, params, ws=ws_p)
        for Wi in Ws:
            gq.quantize_layer(Wi, prep, params, ws=ws_q3)

    tb, ts = time_events(batched, 5, stream), time_events(separate, 5, stream)
    out["three_layers_one_factor"] = {
        "shape": f"3 x {m}x{d}, one H over {X.shape[0]} tokens", "ms": tb,
        "weights_per_s": 3 * m * d / (tb * 1e-3), "ms_separate_calls": ts,
        "weights_per_s_separate_calls": 3 * m * d / (ts * 1e-3)}
    # independent small layers (each its own X, H and factor): eight
    # 1024x1024 layers over 16384 tokens each, one concurrent call against the
    # three calls per layer made one layer after the other
    nl, ds, ns = 8, 1024, 16384
    gen = torch.Generator(device=W.device).manual_seed(11)
    small = [((torch.randn(ds, ds, device=W.device, generator=gen) * 0.02).to(torch.bfloat16),
              torch.randn(ns, ds, device=W.device, generator=gen).to(torch.bfloat16))
             for _ in range(nl)]
    ws_l = [torch.empty(gq.workspace_bytes(5, ds, ds, ns, params), dtype=torch.uint8, device=W.device)
            for _ in range(nl)]
    Hs = torch.empty(ds, ds, device=W.device)
    ws_hs = torch.empty(gq.workspace_bytes(0, 0, ds, ns), dtype=torch.uint8, device=W.device)
    ws_ps = torch.empty(gq.workspace_bytes(1, 0, ds, 0, params), dtype=torch.uint8, device=W.device)
    ws_qs = torch.empty(gq.workspace_bytes(2, ds, ds, 0, params), dtype=torch.uint8, device=W.device)

    def one_by_one():
        for Wi, Xi in small:
            Hs.zero_()
            gq.hessian_accumulate(Hs, Xi, ws=ws_hs)
            gq.quantize_layer(Wi, gq.prepare_hinv(Hs, params, ws=ws_ps), params, ws=ws_qs)

    ti = time_events(lambda: gq.quantize_independent(small, params, ws=ws_l), 5, stream)
    to = time_events(one_by_one, 5, stream)
    out["independent_layers"] = {
        "shape": f"{nl} x {ds}x{ds}, each its own X of {ns} bf16 tokens", "ms": ti,
        "weights_per_s": nl * ds * ds / (ti * 1e-3), "ms_one_after_another": to,
        "weights_per_s_one_after_another": nl * ds * ds / (to * 1e-3)}
    del small, ws_l
    # W4A16 product with the exported headline layer (4-bit, g128)
    H.zero_()
    gq.hessian_accumulate(H, X, ws=ws_h)
    prep = gq.prepare_hinv(H, params, ws=ws_p)
    q = gq.quantize_layer(W, prep, params)
    ex = gq.export(q, params, d)
    ng = ex.scales_f16.shape[1]
    for M in (1, 4, 64, 512):
        A = torch.randn(M, d, device=W.device).to(torch.float16)
        C = torch.empty(M, m, device=W.device)
        ws_w = torch.empty(gq.workspace_bytes(4, m, d, M), dtype=torch.uint8, device=W.device)
        t = time_events(lambda: gq.w4a16_gemm(A, ex, params.bits, params.group_size, out=C, ws=ws_w),
                        50, stream)
        wbytes = m * ((d * params.bits + 31) // 32) * 4 + 2 * 2 * m * ng
        byts = wbytes + M * d * 2 + M * m * 4
        flop = 2 * M * m * d
        out[f"w4a16_M{M}"] = {
            "ms": t, "GB_per_s": byts / (t * 1e-3) / 1e9, "frac_hbm": byts / (t * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "TFLOP_per_s": flop / (t * 1e-3) / 1e12,
            "frac_f16_mfma": flop / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "bytes": byts}
    # the same product on a large layer's shape (28672 x 8192, 4-bit g128): any
    # word stream is a valid dense code stream, so the export is random words
    # with random half scales and zero codes
    Nl, Kl = 28672, 8192
    gen = torch.Generator(device=W.device).manual_seed(7)
    exl = gq.Exported(
        torch.randint(-2**31, 2**31 - 1, (Nl, Kl * 4 // 32), dtype=torch.int32, device=W.device,
                      generator=gen),
        (torch.rand(Nl, Kl // 128, device=W.device, generator=gen) * 0.01 + 1e-3).to(torch.float16),
        torch.randint(0, 16, (Nl, Kl // 128), device=W.device, generator=gen).to(torch.float16))
    for M in (1, 4, 64):
        A = torch.randn(M, Kl, device=W.device).to(torch.float16)
        C = torch.empty(M, Nl, device=W.device)
        ws_w = torch.empty(gq.workspace_bytes(4, Nl, Kl, M), dtype=torch.uint8, device=W.device)
        t = time_events(lambda: gq.w4a16_gemm(A, exl, 4, 128, out=C, ws=ws_w), 20, stream)
        byts = Nl * Kl // 2 + 2 * 2 * Nl * (Kl // 128) + M * Kl * 2 + M * Nl * 4
        flop = 2 * M * Nl * Kl
        out[f"w4a16_28672x8192_M{M}"] = {
            "ms": t, "GB_per_s": byts / (t * 1e-3) / 1e9, "frac_hbm": byts / (t * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "TFLOP_per_s": flop / (t * 1e-3) / 1e12,
            "frac_f16_mfma": flop / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "bytes": byts}
    del exl
    # OBQ comparator on a tiny layer: 2048 rows x 128 columns
    Wt = torch.randn(2048, 128, device=W.device) * 0.02
    Xt = torch.randn(4096, 128, device=W.device).to(torch.bfloat16)
    Ht = torch.zeros(128, 128, device=W.device)
    gq.hessian_accumulate(Ht, Xt)
    po = gq.GPTQParams(bits=4, group_size=-1)
    t = time_events(lambda: gq.obq_layer(Wt, Ht, po), 3, stream)
    dd = 128
    flop = 2048 * sum(2 * (dd - k) ** 2 for k in range(dd))   # per-step downdate, fp64
    out["obq_2048x128"] = {"ms": t, "weights_per_s": 2048 * 128 / (t * 1e-3),
                           "fp64_TFLOP_per_s": flop / (t * 1e-3) / 1e12,
                           "frac_fp64_peak": flop / (t * 1e-3) / 1e12 / PEAK_FP64_TFLOPS}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama7b-attn")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the multi-layer, W4A16 and OBQ throughput figures")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle token sample (0: all)")
    ap.add_argument("--cpu-rows", type=int, default=0, help="oracle row sample (0: all)")
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
        # the preparation is queued without its wait (its status is checked
        # once the quantization is queued behind it), so the GPU never idles
        # between the stages
        if ev: ev[0].record(stream)
        gq.hessian(H, X, ws=ws_h)   # H = 2·XᵀX, H not read
        if ev: ev[1].record(stream)
        prep = gq.prepare_hinv(H, params, ws=ws_p, sync=False)
        if ev: ev[2].record(stream)
        out = gq.quantize_layer(W, prep, params, ws=ws_q)
        if ev: ev[3].record(stream)
        prep.check()
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
    wf = work_figures(m, d, N, g=wl.group_size if wl.group_size > 0 else d,
                      w_bytes=2 if wl.w_dtype == "bf16" else 4, x_bytes=2 if wl.x_dtype == "bf16" else 4)
    # one more step with the library's per-stage event timing (outside the
    # timed steps): the block-update products, sweeps, Cholesky and inverse
    gq.timing(True)
    step()
    torch.cuda.synchronize()
    stage = gq.timing_read()
    gq.timing(False)
    log("bench: timed stages (ms): " + ", ".join(f"{k} {v:.3f}" for k, v in stage.items()))
    log(f"bench: {ms_step:.3f} ms/step; hessian {h_ms:.3f} ms, prepare {p_ms:.3f} ms, "
        f"quantize {q_ms:.3f} ms")
    h_tflops = wf["hessian_flop"] / (h_ms * 1e-3) / 1e12
    upd_tflops = (wf["superblock_update_flop"] / (stage["block_update"] * 1e-3) / 1e12
                  if stage["block_update"] else None)
    hbm_gbs = wf["layer_bytes"] / (ms_step * 1e-3) / 1e9
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
        "timed_stages_ms": stage,
        "stage_rates": {
            "hessian_tflops": h_tflops,
            "hessian_frac_bf16_peak": h_tflops / PEAK_BF16_TFLOPS,
            "prepare_tflops": wf["prepare_flop"] / (p_ms * 1e-3) / 1e12,
            "block_update_tflops": upd_tflops,
            "block_update_frac_fp32_peak": upd_tflops / PEAK_FP32_TFLOPS if upd_tflops else None,
        },
        "roofline_block_update": {
            "kernel": "super-block update products inside gptq_quantize_layer (fp32 MFMA GEMM)",
            "bound": "mfma",
            "achieved": upd_tflops,
            "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s",
            "frac": upd_tflops / PEAK_FP32_TFLOPS if upd_tflops else None,
            "flop_per_layer": wf["superblock_update_flop"],
            "ms_per_layer": stage["block_update"],
        },
        "hbm_end_to_end": {
            "algorithmic_bytes": wf["layer_bytes"],
            "achieved": hbm_gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": hbm_gbs / PEAK_HBM_GBS,
        },
        "roofline": {
            "kernel": "gptq_hessian (syrk256_kernel + reduce_mirror_kernel)",
            "bound": "mfma",
            "achieved": h_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": h_tflops / PEAK_BF16_TFLOPS,
            "traffic": hessian_traffic(),
        },
    }
    if not args.no_extras:
        log("bench: multi-layer, W4A16 and OBQ figures ...")
        result["extras"] = extras(gq, torch, wl, W, X, params, H, ws_h, ws_p, stream)
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on the host ...")
        result["cpu_baseline"] = cpu_baseline(wl, W_host, X_host,
                                              min(args.cpu_tokens, N) if args.cpu_tokens else N,
                                              min(args.cpu_rows, m) if args.cpu_rows else m)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
