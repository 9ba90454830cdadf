"""Benchmark of the speculative-decoding verification step on one MI355X.

One step = the whole hot path over one batch: the scoring GEMM over the
gamma+1 positions of every sequence (one pass over the LM-head weights) and
the rejection-sampling kernels.  Inputs are synthetic, seeded, and resident in
HBM before timing starts.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --projection-sweep     (the decoder-projection GEMM sweep over N; one JSON line)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published peak
METRIC = "verified positions/sec and achieved HBM GB/s (% of peak) per verify step"
HERE = os.path.dirname(os.path.abspath(__file__))
# The sources of the dominant kernel (the sweep scoring GEMM) that the traffic record below was measured on.
GEMM_SOURCES = [os.path.join(HERE, "speculative_decoding_verification_09_amd", "csrc", f)
                for f in ("gemm_common.h", "gemm_sweep.hip")]

# HBM bytes per scoring launch, from hardware counters (FETCH_SIZE and WRITE_SIZE, each in its own rocprofv3
# --pmc run of this script, scaled by what the same counter reads for a plain device copy of known size: 2.0 for
# FETCH_SIZE, 1.0 for WRITE_SIZE).  Keyed by workload, weight layout and the SHA-256 of the GEMM source the
# counters were taken on: once that source changes, the record no longer describes the kernel and traffic is null.
MEASURED_TRAFFIC = {
    ("lmhead_b1_g4", "packed"): {"fetch_bytes": 1051182331, "write_bytes": 2565120,
                                 "source_sha256": "0081623de30eb1123662d03e456909cadd21e9ce09a1c73bf16c4b87c1645281"},
}


def measured_traffic(workload: str, layout: str):
    rec = MEASURED_TRAFFIC.get((workload, layout))
    if rec is None:
        return None
    h = hashlib.sha256()
    for path in GEMM_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def algorithmic_bytes(w):
    """Bytes the step must move at minimum: W and X read once, fp32 logits written once and read once by the
    statistics pass, draft logits read once, and the one (target, draft) row pair where each sequence ends
    read again by the draw."""
    N = w.B * (w.gamma + 1)
    gemm = w.V * w.d * 2 + N * w.d * 2 + N * w.V * 4
    if w.temperature == 0.0:
        reject = N * w.V * 4
    else:
        reject = N * w.V * 4 + w.B * w.gamma * w.V * 4 + w.B * w.V * 8
    return gemm, gemm + reject


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="lmhead_b1_g4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="the CPU baseline times whole oracle sequences until this much time has passed")
    ap.add_argument("--projection-sweep", action="store_true",
                    help="time the scoring GEMM on the decoder projection shapes over N instead of the step")
    ap.add_argument("--layout", choices=["packed", "rowmajor"], default="packed", help="weight layout")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (a known byte count for hardware counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import speculative_decoding_verification_09_amd as sd
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.projection_sweep:
        projection_sweep(args)
        return
    w = synth.WORKLOADS[args.workload]
    if w.d == 0:
        print(f"workload {w.name} has no scoring GEMM; pick an LM-head workload", file=sys.stderr)
        sys.exit(2)
    B, g, V, d, T = w.B, w.gamma, w.V, w.d, w.temperature
    N = B * (g + 1)
    dev = torch.device("cuda")

    # ---- inputs (untimed): hidden states and weights from the seeded generator
    Xb, Wb = synth.lm_head_inputs(w)
    X = torch.from_numpy(Xb.view(np.int16)).to(dev).view(torch.bfloat16)
    W_rows = torch.from_numpy(Wb.view(np.int16)).to(dev).view(torch.bfloat16)
    del Xb, Wb
    # One-time weight preparation, as at model load: the packed tile layout.  Every step still reads all of it.
    W = sd.specdec_pack_weights(W_rows) if args.layout == "packed" else W_rows
    torch.cuda.synchronize()
    if args.layout == "packed":
        del W_rows
    logits = torch.empty((N, V), dtype=torch.float32, device=dev)
    out_tok = torch.empty((B, g + 1), dtype=torch.int32, device=dev)
    out_num = torch.empty((B,), dtype=torch.int32, device=dev)
    layout = sd.SPECDEC_WEIGHTS_PACKED if args.layout == "packed" else sd.SPECDEC_WEIGHTS_ROW_MAJOR
    ws = sd.new_step_workspace(B, g, d, V, layout)
    gemm_ws = torch.empty(max(1, sd.logits_workspace_bytes(N, d, V, layout)), dtype=torch.uint8, device=dev)
    uni = torch.from_numpy(synth.step_uniforms(w)).to(dev)
    # Draft logits = target logits + N(0, noise) and drafted tokens ~ q: built with the library itself
    # (one scoring pass, then one draw per drafted row as gamma = 0 steps), outside the timed region.
    sd.specdec_verify_logits(X, W, logits, workspace=gemm_ws)
    if T > 0:
        tl = logits.view(B, g + 1, V)[:, :g]
        noise = torch.from_numpy(synth.normal_f32((B, g, V), w.noise_std, w.seed, synth.STREAM_DRAFT_NOISE)).to(dev)
        draft = (tl + noise).contiguous()
        du = torch.zeros((B * g, 1, 2), dtype=torch.float32, device=dev)
        du[:, 0, 1] = torch.from_numpy(synth.draft_sample_uniforms(w).reshape(-1)).to(dev)
        dt = torch.empty((B * g, 1), dtype=torch.int32, device=dev)
        dn = torch.empty((B * g,), dtype=torch.int32, device=dev)
        dws = sd.new_workspace(B * g, 0, V)
        sd.specdec_reject_sample(draft.view(B * g, 1, V), None, torch.empty((B * g, 0), dtype=torch.int32, device=dev),
                                 T, du, dt, dn, dws)
        tokens = dt.view(B, g).contiguous()
        del noise, dws
    else:
        draft = None
        am = logits.view(B, g + 1, V)[:, :g].argmax(dim=2).to(torch.int32)
        rep = torch.from_numpy(synth.bernoulli((B, g), w.replace_prob, w.seed, synth.STREAM_REPLACE)).to(dev)
        rnd = torch.from_numpy(synth.integers((B, g), 0, V, w.seed, synth.STREAM_REPLACE + 10)).to(dev)
        tokens = torch.where(rep, rnd, am).contiguous()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    probs = None
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        sd.specdec_verify_step(X, W, draft, tokens, T, uni if T > 0 else None, logits, out_tok, out_num, ws,
                               out_probs=probs, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region 1 (the headline): K whole steps back to back, events on the launch stream
    K = args.steps
    evs = torch.cuda.Event(enable_timing=True)
    eve = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    evs.record(stream)
    for _ in range(K):
        step()
    eve.record(stream)
    torch.cuda.synchronize()
    ms_step = evs.elapsed_time(eve) / K
    emitted = int(out_num.sum().item())

    # ---- timed region 2 (the roofline of the dominant kernel): K scoring launches back to back on the same
    # stream between two events.  (An event between every launch would add its own release to each interval.)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(K):
        sd.specdec_verify_logits(X, W, logits, workspace=gemm_ws, stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    gemm_ms = ev0.elapsed_time(ev1) / K

    gemm_bytes, step_bytes = algorithmic_bytes(w)
    gemm_gbps = gemm_bytes / (gemm_ms * 1e-3) / 1e9
    step_gbps = step_bytes / (ms_step * 1e-3) / 1e9
    positions_per_s = N / (ms_step * 1e-3)

    # ---- CPU baseline: the oracle as it stands, single-threaded, on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        orc = oracle.load()
        Xh, Wh = synth.lm_head_inputs(w)
        rows_per_seq = g + 1
        uh = synth.step_uniforms(w)
        toks = tokens.cpu().numpy()
        dr = draft.cpu().numpy() if draft is not None else None
        reps = 0
        t0 = time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < args.cpu_seconds:
            b = reps % B
            zb = orc.linear(Xh[b * rows_per_seq:(b + 1) * rows_per_seq], Wh).astype(np.float32)
            orc.verify(zb[None], dr[b:b + 1] if dr is not None else None, toks[b:b + 1], uh[b:b + 1], T)
            reps += 1
        cpu_s = time.perf_counter() - t0
        cpu = {"value": reps * rows_per_seq / cpu_s, "unit": "positions/s", "cores": 1, "kind": "oracle",
               "sample": f"{reps} sequence(s) of {rows_per_seq} positions (B={B}: "
                         f"{'whole steps' if B == 1 else 'sequences of one step'}): fp64 scoring over the full "
                         f"{V}x{d} weights plus the rule, single-threaded C, {cpu_s:.1f} s"}

    out = {
        "metric": METRIC,
        "value": positions_per_s,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "gamma": g, "d": d, "V": V, "N": N, "temperature": T,
                   "draft_noise_std": w.noise_std, "weight_layout": args.layout},
        "step_hbm_gbps": step_gbps,
        "step_frac_of_peak": step_gbps / HBM_PEAK_GBPS,
        "step_bytes": step_bytes,
        "emitted_tokens_per_s": emitted / (ms_step * 1e-3),
        "roofline": {"kernel": "scoring GEMM (specdec_verify_logits)", "bound": "hbm", "achieved": gemm_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": gemm_gbps / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(w.name, args.layout), "bytes_per_launch": gemm_bytes,
                     "avg_launch_ms": gemm_ms},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published


def projection_sweep(args):
    """The scoring GEMM on the decoder projection shapes [N x d_in] . [d_in x d_out] (W stored [d_out, d_in],
    packed, bf16 out), for each N: K back-to-back launches between two events.  Reports achieved HBM GB/s
    (algorithmic bytes: W once, X once, Y once) and MFMA utilisation (2 N d_in d_out flops against the dense bf16
    peak)."""
    import numpy as np
    import torch

    import speculative_decoding_verification_09_amd as sd
    import synth

    cfg = synth.PROJECTION_SWEEP
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    points = []
    Nmax = max(cfg["N"])
    for d_in, d_out in cfg["shapes"]:
        seed = cfg["seed"] + d_in
        W_rows = torch.from_numpy(synth.normal_bf16((d_out, d_in), cfg["w_std"], seed, synth.STREAM_W).view(np.int16))
        W = sd.specdec_pack_weights(W_rows.to(dev).view(torch.bfloat16))
        torch.cuda.synchronize()
        del W_rows
        Xall = torch.from_numpy(synth.normal_bf16((Nmax, d_in), cfg["x_std"], seed, synth.STREAM_X).view(np.int16))
        Xall = Xall.to(dev).view(torch.bfloat16)
        for N in cfg["N"]:
            X = Xall[:N].contiguous()
            Y = torch.empty((N, d_out), dtype=torch.bfloat16, device=dev)
            need = sd.logits_workspace_bytes(N, d_in, d_out, sd.SPECDEC_WEIGHTS_PACKED)
            ws = torch.empty(max(1, need), dtype=torch.uint8, device=dev)
            for _ in range(args.warmup):
                sd.specdec_verify_logits(X, W, Y, sd.SPECDEC_OUT_BF16, workspace=ws, stream=stream)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(args.steps):
                sd.specdec_verify_logits(X, W, Y, sd.SPECDEC_OUT_BF16, workspace=ws, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            nbytes = 2 * d_in * d_out + 2 * N * d_in + 2 * N * d_out
            flops = 2.0 * N * d_in * d_out
            gbps = nbytes / (ms * 1e-3) / 1e9
            tflops = flops / (ms * 1e-3) / 1e12
            points.append({"d_in": d_in, "d_out": d_out, "N": N, "us": ms * 1e3, "gbps": gbps,
                           "hbm_frac": gbps / HBM_PEAK_GBPS, "tflops": tflops,
                           "mfma_util": tflops / MFMA_BF16_PEAK_TFLOPS, "k_groups": need // max(1, N * d_out * 4)})
        del W, Xall
    low = min(p["hbm_frac"] for p in points if p["N"] <= 64)
    out = {
        "metric": "projection GEMM sweep: lowest fraction of HBM peak over N <= 64 (per-N GB/s and MFMA use listed)",
        "value": low, "unit": "fraction of 8 TB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "projection_sweep", "shapes": cfg["shapes"], "N": cfg["N"], "weight_layout": "packed",
                   "out_dtype": "bf16"},
        "points": points,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
