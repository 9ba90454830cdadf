"""Benchmark of the speculative-decoding verification step on one MI355X.

One step = the whole hot path over one batch: the scoring GEMM over the
gamma+1 positions of every sequence (one pass over the LM-head weights) and
the rejection-sampling kernels.  Inputs are synthetic, seeded, and resident in
HBM before timing starts.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --projection-sweep     (the decoder-projection GEMM sweep over N; one JSON line)
    python bench.py --extensions           (warping, one-hot drafts, tree verification, paged KV; one JSON line)
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
    ("lmhead_b1_g4", "packed"): {"fetch_bytes": 1051154653, "write_bytes": 2616848,
                                 "source_sha256": "35f675362734d11c2eddaf9aedd8e3b18b35e6273c3fed0475eb69aedfa4d403"},
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
    ap.add_argument("--extensions", action="store_true",
                    help="time the extensions (warping, one-hot drafts, tree verification, paged KV) instead")
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
    if args.extensions:
        extensions(args)
        return
    w = synth.WORKLOADS[args.workload]
    if w.d == 0:
        toy_reject(args, w)
        return
    B, g, V, d, T = w.B, w.gamma, w.V, w.d, w.temperature
    N = B * (g + 1)
    dev = torch.device("cuda")
    X, W, logits, out_tok, out_num, ws, gemm_ws, uni, draft, tokens = step_inputs(w, args.layout)
    layout = sd.SPECDEC_WEIGHTS_PACKED if args.layout == "packed" else sd.SPECDEC_WEIGHTS_ROW_MAJOR
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

    # ---- the reject stage alone on the step's logits (specdec_reject_sample: statistics pass, then the rule),
    # warm (the logits just written, K back-to-back calls) and flushed (a 512 MiB write between calls, each call
    # between its own two events)
    rule = {}
    if T > 0:
        rws = sd.new_workspace(B, g, V)
        tl = logits.view(B, g + 1, V)
        rule["warm_ms"] = _time_launches(lambda: sd.specdec_reject_sample(tl, draft, tokens, T, uni, out_tok, out_num,
                                                                          rws, stream=stream), K, args.warmup, stream)
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        times = []
        for _ in range(10):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            sd.specdec_reject_sample(tl, draft, tokens, T, uni, out_tok, out_num, rws, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        rule["flushed_ms"] = float(np.median(times))
        del flush, rws
        # the step's own tokens again (the rule above wrote the same outputs from the same inputs)
        step()
        torch.cuda.synchronize()

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
        # One host core: the oracle is single-threaded C; the process is pinned to the core it runs on for the
        # duration, so that the scheduler does not move it.
        pinned = None
        if hasattr(os, "sched_setaffinity"):
            old_mask = os.sched_getaffinity(0)
            core = min(old_mask)
            os.sched_setaffinity(0, {core})
            pinned = core
        reps, t_lin, t_rule = 0, 0.0, 0.0
        t0 = time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < args.cpu_seconds:
            b = reps % B
            ta = time.perf_counter()
            zb = orc.linear(Xh[b * rows_per_seq:(b + 1) * rows_per_seq], Wh).astype(np.float32)
            tb = time.perf_counter()
            orc.verify(zb[None], dr[b:b + 1] if dr is not None else None, toks[b:b + 1], uh[b:b + 1], T)
            t_lin += tb - ta
            t_rule += time.perf_counter() - tb
            reps += 1
        cpu_s = time.perf_counter() - t0
        if pinned is not None:
            os.sched_setaffinity(0, old_mask)
        cpu = {"value": reps * rows_per_seq / cpu_s, "unit": "positions/s", "cores": 1, "kind": "oracle",
               "sample": f"{reps} sequence(s) of {rows_per_seq} positions (B={B}: "
                         f"{'whole steps' if B == 1 else 'sequences of one step'}): fp64 scoring over the full "
                         f"{V}x{d} weights plus the rule, single-threaded C, {cpu_s:.1f} s",
               "scoring_s_per_sequence": t_lin / reps, "rule_s_per_sequence": t_rule / reps,
               "pinned_core": pinned, "host_cpus": os.cpu_count(), "cpu_model": _cpu_model()}

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
        "reject_stage": rule or None,
        "roofline": {"kernel": "scoring GEMM (specdec_verify_logits)", "bound": "hbm", "achieved": gemm_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": gemm_gbps / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(w.name, args.layout), "bytes_per_launch": gemm_bytes,
                     "avg_launch_ms": gemm_ms},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


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
                   "rows_warped": rows, "row_bytes_read_once": rows * V * 4}
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
    max_len = ctx + (K + Wm + 2) * (g + 1)
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

    kv_ms = _time_launches(kv_step, K, Wm, stream)
    torch.cuda.synchronize()
    assert int(kv.status.item()) == 0
    cur = int(kv.lens.max().item())
    kout = torch.empty((R, H, cur, D), dtype=torch.bfloat16, device=dev)
    vout = torch.empty_like(kout)
    gather_ms = _time_launches(lambda: kv.gather(cur, kout, vout, stream=stream), K, Wm, stream)
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
