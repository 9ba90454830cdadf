"""Benchmark of the speculative-decoding verification step on one MI355X.

One step = the whole hot path over one batch: the scoring GEMM over the
gamma+1 positions of every sequence (one pass over the LM-head weights) and
the rejection-sampling kernels.  Inputs are synthetic, seeded, and resident in
HBM before timing starts.  Prints one JSON line.

The headline is the larger Llama-8B-shaped step (B=8, gamma=7, d=8192,
V=128256, 64 positions); the one-sequence step (B=1, gamma=4, d=4096) is timed
in the same run and reported beside it.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-b1]
    python bench.py --projection-sweep     (the decoder-projection GEMM sweep over N; one JSON line)
    python bench.py --extensions           (warping, one-hot drafts, tree verification, paged KV; one JSON line)
    python bench.py --pmc-summary FETCH_CSV WRITE_CSV   (per-kernel HBM bytes from two rocprofv3 --pmc runs)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
METRIC = "verified positions/sec and achieved HBM GB/s (% of peak) per verify step"
HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "speculative_decoding_verification_09_amd", "csrc")

# HBM bytes per launch of the dominant kernel, from hardware counters: FETCH_SIZE and WRITE_SIZE, each in its own
# rocprofv3 --pmc run of this script with --copy-calibration, scaled by what the same counter reads for a plain
# device copy of known size (2.0 for FETCH_SIZE, 1.0 for WRITE_SIZE); `python bench.py --pmc-summary` prints them.
# Keyed by workload and weight layout, with the SHA-256 of the kernel's sources at the time of measurement: once a
# source changes, the record no longer describes the kernel and traffic is reported as null.
MEASURED_TRAFFIC = {
    ("lmhead_b8_g7", "packed"): {"kernel": "panel_kernel", "sources": ["gemm_common.h", "gemm_tiled.hip"],
                                 "fetch_bytes": 2109581097, "write_bytes": 32833426,
                                 "source_sha256": "57ed4f6bbeaa5359ecf8f139e23aac4400163d42446a32ae4d716ae085eec8ff"},
    ("lmhead_b1_g4", "packed"): {"kernel": "sweep_kernel", "sources": ["gemm_common.h", "gemm_sweep.hip"],
                                 "fetch_bytes": 1051032073, "write_bytes": 2616919,
                                 "source_sha256": "71a5ef05d4525c34539ab421a9d4ec98c8a843dc7aadc5c111ec70439d1dfb6b"},
}


def sources_sha256(names) -> str:
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, layout: str):
    rec = MEASURED_TRAFFIC.get((workload, layout))
    if rec is None or sources_sha256(rec["sources"]) != rec["source_sha256"]:
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def algorithmic_bytes(w, fused: bool, with_logits: bool):
    """Bytes the step must move at minimum, and those of its scoring GEMM.  The GEMM reads W and X once and writes
    the fp32 logits once (not at all when a greedy step keeps no logits).  The sampling stage reads the target
    logits once more unless the GEMM forms their statistics itself (fused), reads the draft logits once, and reads
    the one (target, draft) row pair where each sequence ends a second time (T > 0)."""
    N = w.B * (w.gamma + 1)
    y = N * w.V * 4
    gemm = w.V * w.d * 2 + N * w.d * 2 + y
    step = w.V * w.d * 2 + N * w.d * 2 + (y if with_logits else 0)
    if not fused:
        step += y
    if w.temperature > 0.0:
        step += w.B * w.gamma * w.V * 4 + w.B * w.V * 8
    return gemm, step


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps before each timed region (300: about 0.1 s of the eight-sequence step, "
                    "enough for the clocks to settle after the setup; after 10 the step measured ~2%% slower)")
    ap.add_argument("--workload", default="lmhead_b8_g7")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-b1", action="store_true", help="do not also time the one-sequence step (lmhead_b1_g4)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="the CPU baseline times whole oracle sequences until this much time has passed")
    ap.add_argument("--projection-sweep", action="store_true",
                    help="time the scoring GEMM on the decoder projection shapes over N instead of the step")
    ap.add_argument("--projection-n", type=int, nargs="+", default=None, metavar="N",
                    help="with --projection-sweep: only these N")
    ap.add_argument("--layout", choices=["packed", "rowmajor"], default="packed", help="weight layout")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (a known byte count for hardware counters)")
    ap.add_argument("--extensions", action="store_true",
                    help="time the extensions (warping, one-hot drafts, tree verification, paged KV) instead")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, WRITE_SIZE)")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import speculative_decoding_verification_09_amd as sd  # noqa: F401  (fails loudly without the HIP library)
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.projection_sweep:
        projection_sweep(args)
        return
    if args.extensions:
        extensions(args)
        return
    w = synth.WORKLOADS[args.workload]
    if w.d == 0:
        toy_reject(args, w)
        return

    m = measure_step(w, args)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, m, args.cpu_seconds)
    state = m.pop("_state")
    del state
    b1 = None
    if not args.no_b1 and w.name != "lmhead_b1_g4":
        torch.cuda.empty_cache()
        m1 = measure_step(synth.WORKLOADS["lmhead_b1_g4"], args)
        m1.pop("_state")
        b1 = {k: m1[k] for k in ("ms_per_step", "positions_per_s", "step_hbm_gbps", "step_frac_of_peak",
                                 "step_bytes", "step_times_us", "roofline", "reject_stage")}
        b1["config"] = m1["config"]

    out = {
        "metric": METRIC,
        "value": m["positions_per_s"],
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": m["config"],
        "step_hbm_gbps": m["step_hbm_gbps"],
        "step_frac_of_peak": m["step_frac_of_peak"],
        "step_bytes": m["step_bytes"],
        "step_times_us": m["step_times_us"],
        "emitted_tokens_per_s": m["emitted_tokens_per_s"],
        "reject_stage": m["reject_stage"],
        "roofline": m["roofline"],
        "cpu_baseline": cpu,
        "b1_step": b1,
    }
    print(json.dumps(out), flush=True)


def _percentiles(times_ms):
    import numpy as np

    t = np.asarray(times_ms, dtype=np.float64) * 1e3
    return {"median": float(np.median(t)), "p10": float(np.percentile(t, 10)), "p90": float(np.percentile(t, 90)),
            "mean": float(t.mean()), "n": int(t.size)}


def measure_step(w, args):
    """Times one workload's verify step (inputs resident in HBM) and its dominant kernel.

    Timed region 1 (the headline): K whole steps back to back between two events on the launch stream; the mean.
    Timed region 2: K steps with an event between consecutive steps, for the median and p10/p90 of single steps
    (each interval also holds one event's own cost).  Timed region 3 (the roofline of the dominant kernel): K
    scoring launches back to back between two events."""
    import torch

    import speculative_decoding_verification_09_amd as sd

    B, g, V, d, T = w.B, w.gamma, w.V, w.d, w.temperature
    N = B * (g + 1)
    X, W, logits, out_tok, out_num, ws, gemm_ws, uni, draft, tokens = step_inputs(w, args.layout)
    layout = sd.SPECDEC_WEIGHTS_PACKED if args.layout == "packed" else sd.SPECDEC_WEIGHTS_ROW_MAJOR
    stream = torch.cuda.current_stream()
    fused = sd.step_fuses_statistics(B, g, d, V, layout)
    # A greedy step whose scoring kernel takes the argmax itself needs no logits buffer.
    step_logits = None if (T == 0.0 and sd.step_accepts_null_logits(B, g, d, V, layout)) else logits

    def step():
        sd.specdec_verify_step(X, W, draft, tokens, T, uni if T > 0 else None, step_logits, out_tok, out_num, ws,
                               stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    evs = torch.cuda.Event(enable_timing=True)
    eve = torch.cuda.Event(enable_timing=True)
    evs.record(stream)
    for _ in range(K):
        step()
    eve.record(stream)
    torch.cuda.synchronize()
    ms_step = evs.elapsed_time(eve) / K
    emitted = int(out_num.sum().item())

    evl = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    evl[0].record(stream)
    for i in range(K):
        step()
        evl[i + 1].record(stream)
    torch.cuda.synchronize()
    singles = [evl[i].elapsed_time(evl[i + 1]) for i in range(K)]

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(K):
        sd.specdec_verify_logits(X, W, logits, workspace=gemm_ws, stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    gemm_ms = ev0.elapsed_time(ev1) / K

    # The reject stage alone on the step's logits (specdec_reject_sample: its own statistics pass, then the rule),
    # warm (K back-to-back calls right after the logits were written) and flushed (a 512 MiB write before each
    # call, each call between its own two events; median of 10).
    rule = None
    if T > 0:
        rws = sd.new_workspace(B, g, V)
        tl = logits.view(B, g + 1, V)
        rule = {"warm_ms": _time_launches(lambda: sd.specdec_reject_sample(tl, draft, tokens, T, uni, out_tok, out_num,
                                                                           rws, stream=stream), K, args.warmup,
                                          stream)}
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        times = []
        for _ in range(10):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            sd.specdec_reject_sample(tl, draft, tokens, T, uni, out_tok, out_num, rws, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        rule["flushed_ms"] = _percentiles(times)["median"] * 1e-3
        del flush, rws
    # The step's outputs once more, with the logits kept, for the parity check of the CPU baseline (the outputs
    # are the same with or without a logits buffer).
    sd.specdec_verify_step(X, W, draft, tokens, T, uni if T > 0 else None, logits, out_tok, out_num, ws,
                           stream=stream)
    torch.cuda.synchronize()

    gemm_bytes, step_bytes = algorithmic_bytes(w, fused, step_logits is not None)
    gemm_gbps = gemm_bytes / (gemm_ms * 1e-3) / 1e9
    step_gbps = step_bytes / (ms_step * 1e-3) / 1e9
    flops = 2.0 * N * d * V
    roof = {"kernel": sd.scoring_kernel_name(N, d, V, layout), "bound": "hbm", "achieved": gemm_gbps,
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": gemm_gbps / HBM_PEAK_GBPS,
            "traffic": measured_traffic(w.name, args.layout), "bytes_per_launch": gemm_bytes,
            "avg_launch_ms": gemm_ms,
            "mfma_tflops": flops / (gemm_ms * 1e-3) / 1e12,
            "mfma_frac": flops / (gemm_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    return {
        "config": {"workload": w.name, "B": B, "gamma": g, "d": d, "V": V, "N": N, "temperature": T,
                   "draft_noise_std": w.noise_std, "weight_layout": args.layout,
                   "statistics_fused": bool(fused), "logits_written": step_logits is not None},
        "ms_per_step": ms_step,
        "positions_per_s": N / (ms_step * 1e-3),
        "step_hbm_gbps": step_gbps,
        "step_frac_of_peak": step_gbps / HBM_PEAK_GBPS,
        "step_bytes": step_bytes,
        "step_times_us": _percentiles(singles),
        "emitted_tokens_per_s": emitted / (ms_step * 1e-3),
        "reject_stage": rule,
        "roofline": roof,
        "_state": {"logits": logits, "out_tok": out_tok, "out_num": out_num, "draft": draft, "tokens": tokens},
    }


def cpu_baseline(w, m, seconds: float):
    """The oracle as it stands (single-threaded C, fp64), pinned to one host core, on whole sequences of the same
    workload until `seconds` have passed: scoring over the full weights, then the rule.  Each sequence it finishes
    is also compared with the GPU step's outputs on the same inputs: the logits (max |dz| against the oracle's fp64
    scores) and the emitted tokens and counts, element by element, near ties counted."""
    import numpy as np

    import oracle
    from oracle.parity import compare_steps, end_to_end_bands
    import synth

    orc = oracle.load()
    B, g, V, d, T = w.B, w.gamma, w.V, w.d, w.temperature
    st = m["_state"]
    Xh, Wh = synth.lm_head_inputs(w)
    g1 = g + 1
    uh = synth.step_uniforms(w) if T > 0 else None
    toks = st["tokens"].cpu().numpy()
    dr = st["draft"].cpu().numpy() if st["draft"] is not None else None
    gpu_logits = st["logits"].cpu().numpy()
    gpu_tok = st["out_tok"].cpu().numpy()
    gpu_num = st["out_num"].cpu().numpy()
    pinned = None
    if hasattr(os, "sched_setaffinity"):
        old_mask = os.sched_getaffinity(0)
        pinned = min(old_mask)
        os.sched_setaffinity(0, {pinned})
    reps, t_lin, t_rule = 0, 0.0, 0.0
    seqs, outs, dzs = [], [], []
    t0 = time.perf_counter()
    while reps == 0 or time.perf_counter() - t0 < seconds:
        b = reps % B
        ta = time.perf_counter()
        z64 = orc.linear(Xh[b * g1:(b + 1) * g1], Wh)
        tb = time.perf_counter()
        ora = orc.verify(z64.astype(np.float32)[None], dr[b:b + 1] if dr is not None else None, toks[b:b + 1],
                         uh[b:b + 1] if uh is not None else None, T)
        t_lin += tb - ta
        t_rule += time.perf_counter() - tb
        reps += 1
        if b not in seqs:
            seqs.append(b)
            outs.append(ora)
            dzs.append(float(np.abs(gpu_logits[b * g1:(b + 1) * g1].astype(np.float64) - z64).max()))
    cpu_s = time.perf_counter() - t0
    if pinned is not None:
        os.sched_setaffinity(0, old_mask)
    # Parity of the sequences the oracle finished.
    max_dz = max(dzs)
    exact = excused = 0
    failures = []
    for b, ora in zip(seqs, outs):
        acc_band, draw_band = end_to_end_bands(max_dz, T, ora["draw_mass"])
        r = compare_steps(gpu_tok[b:b + 1], gpu_num[b:b + 1], ora, acc_band, draw_band)
        exact += r["exact"]
        excused += r["excused"]
        failures += [b] if r["failures"] else []
    return {"value": reps * g1 / cpu_s, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} sequence(s) of {g1} positions ({'whole steps' if B == 1 else f'of the {B} in a step'}):"
                      f" fp64 scoring over the full {V}x{d} weights plus the rule, single-threaded C, {cpu_s:.1f} s",
            "scoring_s_per_sequence": t_lin / reps, "rule_s_per_sequence": t_rule / reps,
            "pinned_core": pinned, "host_cpus": os.cpu_count(), "cpu_model": _cpu_model(),
            "parity": {"sequences": seqs, "exact": exact, "excused": excused, "failures": failures,
                       "max_dz": max_dz}}


def pmc_summary(fetch_csv: str, write_csv: str):
    """Per-kernel HBM bytes per dispatch from the counter_collection.csv files of two rocprofv3 runs (one with
    --pmc FETCH_SIZE, one with --pmc WRITE_SIZE, both of `bench.py ... --copy-calibration`), one line per kernel and
    grid size.  Each counter is scaled by what it reads for the plain device copy (__amd_rocclr_copyBuffer, 256 MiB
    read and written)."""
    import csv
    from collections import defaultdict

    def load(path, counter):
        d = defaultdict(list)
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter:
                    d[(row["Kernel_Name"], int(row["Grid_Size"]))].append(float(row["Counter_Value"]))
        return d

    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    copy_kib = 256 * 1024.0

    def copy_total(d):
        return sum(sum(v) for (k, _), v in d.items() if k == "__amd_rocclr_copyBuffer") or copy_kib

    cf, cw = copy_kib / copy_total(fetch), copy_kib / copy_total(write)
    print(f"copy calibration: FETCH_SIZE x{cf:.4f}, WRITE_SIZE x{cw:.4f}")
    print("| kernel | grid (threads) | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM bytes per dispatch |")
    print("|---|---|---|---|---|---|")
    for key in sorted(fetch, key=lambda k: -sum(fetch[k])):
        k, grid = key
        if k == "__amd_rocclr_copyBuffer" or key not in write:
            continue
        f = sum(fetch[key]) / len(fetch[key])
        wr = sum(write[key]) / len(write[key])
        name = k.replace("(anonymous namespace)::", "").replace("specdec::", "").replace("void ", "").split("(")[0]
        print(f"| {name} | {grid} | {len(fetch[key])} | {f:.1f} | {wr:.1f} | {(f * cf + wr * cw) * 1024:.4e} |")
        print(f"    fetch_bytes={int(f * cf * 1024)} write_bytes={int(wr * cw * 1024)}")


def step_inputs(w, layout_name: str):
    """Device inputs of one verify step of workload w (untimed): X, W (packed or row-major), logits, outputs, the step
    and scoring workspaces, uniforms, draft logits (T > 0) and drafted tokens."""
    import numpy as np
    import torch

    import speculative_decoding_verification_09_amd as sd
    import synth

    B, g, V, d, T = w.B, w.gamma, w.V, w.d, w.temperature
    N = B * (g + 1)
    dev = torch.device("cuda")

    # ---- inputs (untimed): hidden states and weights from the seeded generator
    Xb, Wb = synth.lm_head_inputs(w)
    X = torch.from_numpy(Xb.view(np.int16)).to(dev).view(torch.bfloat16)
    W_rows = torch.from_numpy(Wb.view(np.int16)).to(dev).view(torch.bfloat16)
    del Xb, Wb
    # One-time weight preparation, as at model load: the packed tile layout.  Every step still reads all of it.
    W = sd.specdec_pack_weights(W_rows) if layout_name == "packed" else W_rows
    torch.cuda.synchronize()
    if layout_name == "packed":
        del W_rows
    logits = torch.empty((N, V), dtype=torch.float32, device=dev)
    out_tok = torch.empty((B, g + 1), dtype=torch.int32, device=dev)
    out_num = torch.empty((B,), dtype=torch.int32, device=dev)
    layout = sd.SPECDEC_WEIGHTS_PACKED if layout_name == "packed" else sd.SPECDEC_WEIGHTS_ROW_MAJOR
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

    return X, W, logits, out_tok, out_num, ws, gemm_ws, uni, draft, tokens


def toy_reject(args, w):
    """The reject-only toy workload (no scoring GEMM): one target row z ~ N(0, target_std) over V tokens and its
    draft z + N(0, noise_std), replicated over B trials of gamma drafts; drafted tokens x ~ q drawn with the
    library itself (gamma = 0 calls), per-position uniforms from the seeded generator.  Times
    specdec_reject_sample (K back-to-back calls between two events, inputs resident) and reports, from the
    outputs, the first emitted token's total-variation distance to p and the mean emitted count against the
    closed form (1 - alpha^(gamma+1)) / (1 - alpha), alpha = sum min(p, q)."""
    import numpy as np
    import torch

    import speculative_decoding_verification_09_amd as sd
    import synth

    B, g, V, T = w.B, w.gamma, w.V, w.temperature
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    z = synth.normal_f32((1, V), w.target_std, w.seed, synth.STREAM_TARGET)
    dz = z + synth.normal_f32((1, V), w.noise_std, w.seed, synth.STREAM_DRAFT_NOISE)
    zt = torch.from_numpy(z).to(dev).expand(B, g + 1, V).contiguous()
    zd = torch.from_numpy(dz).to(dev).expand(B, g, V).contiguous()
    du = torch.zeros((B * g, 1, 2), dtype=torch.float32, device=dev)
    du[:, 0, 1] = torch.from_numpy(synth.draft_sample_uniforms(w).reshape(-1)).to(dev)
    dt = torch.empty((B * g, 1), dtype=torch.int32, device=dev)
    dn = torch.empty((B * g,), dtype=torch.int32, device=dev)
    sd.specdec_reject_sample(zd.view(B * g, 1, V), None, torch.empty((B * g, 0), dtype=torch.int32, device=dev), T,
                             du, dt, dn, sd.new_workspace(B * g, 0, V))
    tokens = dt.view(B, g).contiguous()
    uni = torch.from_numpy(synth.step_uniforms(w)).to(dev)
    out_tok = torch.empty((B, g + 1), dtype=torch.int32, device=dev)
    out_num = torch.empty((B,), dtype=torch.int32, device=dev)
    ws = sd.new_workspace(B, g, V)
    torch.cuda.synchronize()
    ms = _time_launches(lambda: sd.specdec_reject_sample(zt, zd, tokens, T, uni, out_tok, out_num, ws, stream=stream),
                        args.steps, args.warmup, stream)
    first = out_tok[:, 0].cpu().numpy()
    num = out_num.cpu().numpy().astype(np.float64)

    def softmax(a):
        e = np.exp((a.astype(np.float64) / T) - (a.astype(np.float64) / T).max())
        return e / e.sum()

    p, q = softmax(z[0]), softmax(dz[0])
    tv = 0.5 * np.abs(np.bincount(first, minlength=V) / B - p).sum()
    alpha = float(np.minimum(p, q).sum())
    expected = (1 - alpha ** (g + 1)) / (1 - alpha)
    print(json.dumps({
        "metric": "verified positions/sec (reject stage alone)", "value": B * (g + 1) / (ms * 1e-3),
        "unit": "positions/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "gamma": g, "V": V, "temperature": T},
        "input_bytes": (B * (g + 1) * V + B * g * V) * 4,
        "tv_first_token": tv, "mean_emitted": float(num.mean()), "closed_form_emitted": expected,
        "emitted_se": float(num.std() / np.sqrt(B)),
    }))


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _time_launches(fn, K: int, warmup: int, stream) -> float:
    """Average ms of fn() over K back-to-back calls on one stream, between two events, after warmup calls."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(K):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / K


def extensions(args):
    """Times each extension on its synthetic workload (inputs resident in HBM, K back-to-back calls between two
    events on the launch stream): top-k / top-p warping and one-hot drafts on the larger LM-head step (each beside
    the plain step on the same inputs), greedy tree verification with its scoring GEMM, and the paged KV cache
    operations around a verify step."""
    import numpy as np
    import torch

    import speculative_decoding_verification_09_amd as sd
    import synth

    K, Wm = args.steps, args.warmup
    stream = torch.cuda.current_stream()
    dev = torch.device("cuda")
    res = {}

    # ---- warping and one-hot drafts on the larger LM-head step
    cfg = synth.EXTENSIONS["warp"]
    w = synth.WORKLOADS[cfg["workload"]]
    B, g, V, d, T = w.B, w.gamma, w.V, w.d, w.temperature
    N = B * (g + 1)
    X, W, logits, out_tok, out_num, ws, gemm_ws, uni, draft, tokens = step_inputs(w, "packed")
    k, p = cfg["top_k"], cfg["top_p"]
    plain = _time_launches(lambda: sd.specdec_verify_step(X, W, draft, tokens, T, uni, logits, out_tok, out_num, ws,
                                                          stream=stream), K, Wm, stream)
    warped = _time_launches(lambda: sd.specdec_verify_step_warped(X, W, draft, tokens, T, k, p, uni, logits, out_tok,
                                                                  out_num, ws, stream=stream), K, Wm, stream)
    emitted_w = int(out_num.sum().item())
    # top-p alone (its own path: a window of keys around a sampled estimate of the cut)
    p_only = cfg["top_p_alone"]
    warped_p = _time_launches(lambda: sd.specdec_verify_step_warped(X, W, draft, tokens, T, 0, p_only, uni, logits,
                                                                    out_tok, out_num, ws, stream=stream), K, Wm, stream)
    rws = sd.new_workspace(B, g, V)
    tl = logits.view(B, g + 1, V)
    rej = _time_launches(lambda: sd.specdec_reject_sample(tl, draft, tokens, T, uni, out_tok, out_num, rws,
                                                          stream=stream), K, Wm, stream)
    rej_w = _time_launches(lambda: sd.specdec_reject_sample_warped(tl, draft, tokens, T, k, p, uni, out_tok, out_num,
                                                                   rws, stream=stream), K, Wm, stream)
    rows = B * (g + 1) + B * g
    res["warp"] = {"workload": w.name, "top_k": k, "top_p": p, "plain_step_ms": plain, "warped_step_ms": warped,
                   "warped_positions_per_s": N / (warped * 1e-3), "warped_emitted_per_step": emitted_w,
                   "plain_rule_ms": rej, "warped_rule_ms": rej_w, "warp_overhead_ms": rej_w - rej,
                   "rows_warped": rows, "row_bytes_read_once": rows * V * 4,
                   "top_p_alone": p_only, "top_p_alone_step_ms": warped_p,
                   "top_p_alone_positions_per_s": N / (warped_p * 1e-3)}
    onehot = _time_launches(lambda: sd.specdec_verify_step(X, W, None, tokens, T, uni, logits, out_tok, out_num, ws,
                                                           draft_kind=sd.SPECDEC_DRAFT_ONEHOT, stream=stream),
                            K, Wm, stream)
    res["onehot"] = {"workload": w.name, "plain_step_ms": plain, "onehot_step_ms": onehot,
                     "onehot_positions_per_s": N / (onehot * 1e-3),
                     "draft_bytes_not_read": B * g * V * 4}
    del X, W, logits, ws, gemm_ws, draft, rws
    torch.cuda.empty_cache()

    # ---- greedy tree verification
    c = synth.EXTENSIONS["tree"]
    B, M, V, d = c["B"], c["M"], c["V"], c["d"]
    N = B * M
    X = torch.from_numpy(synth.normal_bf16((N, d), c["x_std"], c["seed"], synth.STREAM_X).view(np.int16))
    X = X.to(dev).view(torch.bfloat16)
    W_rows = torch.from_numpy(synth.normal_bf16((V, d), c["w_std"], c["seed"], synth.STREAM_W).view(np.int16))
    W = sd.specdec_pack_weights(W_rows.to(dev).view(torch.bfloat16))
    del W_rows
    parents = torch.from_numpy(np.tile((np.arange(M, dtype=np.int32) - 1) // 2, (B, 1))).to(dev)
    logits = torch.empty((N, V), dtype=torch.float32, device=dev)
    gws = torch.empty(max(1, sd.logits_workspace_bytes(N, d, V, sd.SPECDEC_WEIGHTS_PACKED)), dtype=torch.uint8,
                      device=dev)
    sd.specdec_verify_logits(X, W, logits, workspace=gws)
    am = logits.view(B, M, V).argmax(dim=2).to(torch.int32)
    par_l = parents.long().clamp(min=0)
    right = torch.from_numpy(synth.bernoulli((B, M), c["right"], c["seed"], synth.STREAM_REPLACE)).to(dev)
    rnd = torch.from_numpy(synth.integers((B, M), 0, V, c["seed"], synth.STREAM_REPLACE + 10)).to(dev)
    node_tok = torch.where(right, torch.gather(am, 1, par_l), rnd).to(torch.int32).contiguous()
    ot = torch.empty((B, M), dtype=torch.int32, device=dev)
    on = torch.empty((B,), dtype=torch.int32, device=dev)
    nd = torch.empty((B, M), dtype=torch.int32, device=dev)
    tws = torch.empty(sd.tree_step_workspace_bytes(B, M, d, V, sd.SPECDEC_WEIGHTS_PACKED), dtype=torch.uint8,
                      device=dev)
    tree_ms = _time_launches(lambda: sd.specdec_tree_verify_step(X, W, parents, node_tok, logits, ot, on, nd, tws,
                                                                 stream=stream), K, Wm, stream)
    gemm_ms = _time_launches(lambda: sd.specdec_verify_logits(X, W, logits, workspace=gws, stream=stream), K, Wm,
                             stream)
    gemm_bytes = V * d * 2 + N * d * 2 + N * V * 4
    res["tree"] = {"B": B, "M": M, "V": V, "d": d, "tree_step_ms": tree_ms, "positions_per_s": N / (tree_ms * 1e-3),
                   "mean_emitted": float(on.float().mean().item()), "gemm_ms": gemm_ms,
                   "gemm_hbm_gbps": gemm_bytes / (gemm_ms * 1e-3) / 1e9,
                   "gemm_hbm_frac": gemm_bytes / (gemm_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    del X, W, logits, gws, tws
    torch.cuda.empty_cache()

    # ---- paged KV cache around a verify step
    c = synth.EXTENSIONS["paged_kv"]
    R, H, D, bs, ctx, g = c["R"], c["heads"], c["head_dim"], c["block_size"], c["ctx"], c["gamma"]
    # Each call appends gamma + 1 positions and keeps the accepted ones, so the contexts grow with every call: a
    # short warm-up keeps them near the stated length (the clocks have settled over the parts timed before).
    Wkv = min(Wm, 10)
    max_len = ctx + (K + Wkv + 2) * (g + 1)
    mb = (max_len + bs - 1) // bs
    kv = sd.PagedKVCache(R, R * mb, H, bs, D, max_blocks=mb, dtype=torch.bfloat16)
    k0 = torch.from_numpy(synth.normal_bf16((R, H, ctx, D), 1.0, c["seed"], 0).view(np.int16)).to(dev)
    kv.append(k0.view(torch.bfloat16), k0.view(torch.bfloat16))
    del k0
    kn = torch.from_numpy(synth.normal_bf16((R, H, g + 1, D), 1.0, c["seed"], 1).view(np.int16)).to(dev)
    kn = kn.view(torch.bfloat16)
    num = torch.from_numpy(synth.integers((R,), 1, g + 2, c["seed"], 2)).to(dev)

    def kv_step():
        kv.append(kn, kn, stream=stream)
        kv.rollback_after_verify(num, g, stream=stream)

    kv_ms = _time_launches(kv_step, K, Wkv, stream)
    torch.cuda.synchronize()
    assert int(kv.status.item()) == 0
    cur = int(kv.lens.max().item())
    kout = torch.empty((R, H, cur, D), dtype=torch.bfloat16, device=dev)
    vout = torch.empty_like(kout)
    gather_ms = _time_launches(lambda: kv.gather(cur, kout, vout, stream=stream), K, Wkv, stream)
    gather_bytes = 2 * 2 * int(kv.lens.sum().item()) * H * D * 2
    res["paged_kv"] = {"R": R, "heads": H, "head_dim": D, "block_size": bs, "gamma": g,
                       "append_and_rollback_us": kv_ms * 1e3,
                       "append_bytes": 2 * 2 * R * H * (g + 1) * D * 2,
                       "gather_ms": gather_ms, "gather_hbm_gbps": gather_bytes / (gather_ms * 1e-3) / 1e9,
                       "gather_hbm_frac": gather_bytes / (gather_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}

    out = {
        "metric": "extensions: warped / one-hot / tree verify steps and paged-KV operations (times per call)",
        "value": res["warp"]["warped_positions_per_s"], "unit": "positions/s (warped step)", "n_gpus": 1,
        "steps": K, "warmup": Wm, "higher_is_better": True, "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": {"workload": "extensions"}, "results": res,
    }
    print(json.dumps(out), flush=True)




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
    Ns = args.projection_n or cfg["N"]
    Nmax = max(cfg["N"])
    for d_in, d_out in cfg["shapes"]:
        seed = cfg["seed"] + d_in
        W_rows = torch.from_numpy(synth.normal_bf16((d_out, d_in), cfg["w_std"], seed, synth.STREAM_W).view(np.int16))
        W = sd.specdec_pack_weights(W_rows.to(dev).view(torch.bfloat16))
        torch.cuda.synchronize()
        del W_rows
        Xall = torch.from_numpy(synth.normal_bf16((Nmax, d_in), cfg["x_std"], seed, synth.STREAM_X).view(np.int16))
        Xall = Xall.to(dev).view(torch.bfloat16)
        # Sustained load first (about 0.1 s): after the host-side setup the GPU needs tens of milliseconds of work
        # before its clocks settle, and each point below is only a few milliseconds long.
        Xw = Xall[:64].contiguous()
        Yw = torch.empty((64, d_out), dtype=torch.bfloat16, device=dev)
        wsw = torch.empty(max(1, sd.logits_workspace_bytes(64, d_in, d_out, sd.SPECDEC_WEIGHTS_PACKED)),
                          dtype=torch.uint8, device=dev)
        for _ in range(1200):
            sd.specdec_verify_logits(Xw, W, Yw, sd.SPECDEC_OUT_BF16, workspace=wsw, stream=stream)
        torch.cuda.synchronize()
        del Xw, Yw, wsw
        for N in Ns:
            X = Xall[:N].contiguous()
            Y = torch.empty((N, d_out), dtype=torch.bfloat16, device=dev)
            need = sd.logits_workspace_bytes(N, d_in, d_out, sd.SPECDEC_WEIGHTS_PACKED)
            kernel = sd.scoring_kernel_name(N, d_in, d_out, sd.SPECDEC_WEIGHTS_PACKED)
            # The deep kernel's workspace starts with the packed copy of X (16-row tiles, 256-byte aligned); the
            # rest, if any, holds the fp32 partials of the k-groups.
            xpack = ((N + 15) // 16 * 16 * d_in * 2 + 255) // 256 * 256 if kernel == "deep_kernel" else 0
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
                           "mfma_util": tflops / MFMA_BF16_PEAK_TFLOPS, "kernel": kernel,
                           "k_groups": (need - xpack) // max(1, N * d_out * 4)})
        del W, Xall
    # The value: the lowest fraction of HBM peak over N <= 64 (over the points run, if --projection-n left none).
    low = min((p["hbm_frac"] for p in points if p["N"] <= 64), default=min(p["hbm_frac"] for p in points))
    out = {
        "metric": "projection GEMM sweep: lowest fraction of HBM peak over N <= 64 (per-N GB/s and MFMA use listed)",
        "value": low, "unit": "fraction of 8 TB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "projection_sweep", "shapes": cfg["shapes"], "N": list(Ns), "weight_layout": "packed",
                   "out_dtype": "bf16"},
        "points": points,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
