"""Throughput of exact tiled attention (forward + backward) on one MI355X.

One step = the whole path over one batch of the causal forward + backward
workload (B=2, Hq=Hkv=16, N=8192, d=128, bf16 iid N(0,1) Q, K, V, dO):
fa_fwd (O, LSE), then fa_bwd in both dQ modes the workload names: the
deterministic separate dQ pass and the atomic dQ.  FLOPs are counted
nominally: forward 4*B*Hq*N^2*d, halved when causal; each backward 2.5x the
forward, the same count for every dQ mode.  The step's value is
(forward + 2 backward) nominal FLOPs over the step time.

Prints ONE JSON line.  Inputs are resident in HBM before the timed region; the
region is bracketed by device synchronisation.  HIP events recorded on the
launch stream around each call give per-call durations for the roofline.  The
ordered-dQ and paired-atomic backward modes are timed after the step loop and
reported under "parts".
The fp64 CPU oracle is timed on bounded samples of every workload (whole
heads of the forward; whole key/value groups of the backward) as a reported
baseline.

"per_config" then times each of the five synthetic workloads on its own
(forward; the four dQ modes of the backward for the backward workload and for
the long-context GQA shape; the linear-position-bias forward and deterministic
backward on the backward workload's inputs): launches back to back after
0.3 s of untimed ones, an event pair around each launch, median and minimum
reported.  --no-per-config skips it (profiling runs use that, so the
kernel averages cover the step's launches only).
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA peak (published)
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def source_sha256():
    """Hash of the kernel sources and build flags (not of the binary, whose
    bytes depend on the checkout path), with comments, runs of white space and
    the debug build's `#if FA_DEBUG_COUNTERS` blocks removed: the stored
    counters stay valid exactly as long as the code of libfa.so they measured
    does."""
    import hashlib
    import importlib.util
    import re
    spec = importlib.util.spec_from_file_location(
        "_fa_build", os.path.join(ROOT, "exact_tiled_attention_27_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    h = hashlib.sha256(" ".join(b.FLAGS[:-2]).encode())
    csrc = os.path.join(ROOT, "exact_tiled_attention_27_amd", "csrc")
    paths = [os.path.join(csrc, n) for n in sorted(os.listdir(csrc))]
    for path in paths + [os.path.join(ROOT, "include", "fa.h")]:
        with open(path) as fh:
            code = re.sub(r"//[^\n]*|/\*.*?\*/", " ", fh.read(), flags=re.S)
            code = re.sub(r"#if FA_DEBUG_COUNTERS\b.*?#endif", " ", code, flags=re.S)
        code = " ".join(code.split())
        h.update(os.path.basename(path).encode() + b"\0" + code.encode())
    return h.hexdigest()


def measured_traffic(kernels, workload):
    """HBM bytes per launch (read + write) of `kernels` from the rocprofv3
    FETCH_SIZE / WRITE_SIZE passes stored in profiles/, or None when they were
    taken on another workload or with other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("source_sha256") != source_sha256():
        return None
    # A backward preprocess is stored under the kernel dispatched after it
    # (the dQ zeroing of the atomic modes makes its bytes mode-dependent).
    keys = [f"{k} (before {kernels[i + 1]})" if "bwd_pre_kernel" in k and i + 1 < len(kernels) else k
            for i, k in enumerate(kernels)]
    try:
        return sum(t["kernels"][k]["read_bytes"] + t["kernels"][k]["write_bytes"] for k in keys)
    except KeyError:
        return None


def time_launches(fn, reps, stream, warm_s=0.3):
    """Per-launch durations (ms) of `reps` back-to-back calls of fn, from an
    event pair recorded on `stream` around each call, after `warm_s` seconds of
    untimed calls (the clock drops while the host draws the next workload's
    inputs and needs tens of milliseconds of load to come back up)."""
    import torch
    t0 = time.perf_counter()
    while True:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= warm_s:
            break
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return sorted(e0.elapsed_time(e1) for e0, e1 in ev)


def per_config(fa, reps, dev, stream):
    """Forward (and, for the backward workload and the long-context GQA shape,
    every backward mode) of each synthetic workload, timed on its own; the
    backward workload also times the linear-position-bias forward and
    deterministic backward."""
    import numpy as np
    import torch
    from synth import WORKLOADS, make_inputs
    from dataclasses import replace

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    def one(w):
        x = make_inputs(w)
        q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
        B, Hq, Hkv, N, d = w.B, w.Hq, w.Hkv, w.N, w.d
        o = torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)

        def fwd():
            st = fa.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, w.scale, w.causal,
                           stream.cuda_stream)
            if st:
                raise fa.FAError(st, "fa_fwd")

        def entry(call, flops, ms):
            med = float(np.median(ms))
            tf = flops / (med * 1e-3) / 1e12
            return {"call": call, "ms_median": med, "ms_min": float(ms[0]),
                    "tflops": tf, "frac_peak": tf / PEAK_BF16_TFLOPS}

        row = {"workload": w.name, "B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "d": d,
               "causal": w.causal, "calls": [entry("fa_fwd", w.fwd_flops(),
                                                   time_launches(fwd, reps, stream))]}
        if w.backward:
            do = to_dev(x["dout"])
            dq = torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev)
            dk = torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev)
            dv = torch.empty_like(dk)
            for det in (fa.BWD_SEPARATE, fa.BWD_ATOMIC, fa.BWD_ORDERED, fa.BWD_ATOMIC_PAIRED):
                wsb = fa.fa_bwd_workspace_bytes(B, Hq, Hkv, N, d, det)
                ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

                def bwd():
                    st = fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, N, d, w.scale,
                                   w.causal, det, ws, wsb, stream.cuda_stream)
                    if st:
                        raise fa.FAError(st, "fa_bwd")

                name = {fa.BWD_SEPARATE: "fa_bwd deterministic", fa.BWD_ATOMIC: "fa_bwd atomic",
                        fa.BWD_ORDERED: "fa_bwd ordered",
                        fa.BWD_ATOMIC_PAIRED: "fa_bwd atomic paired"}[det]
                row["calls"].append(entry(name, w.bwd_flops(), time_launches(bwd, reps, stream)))
            if w.name == "fwdbwd_causal_n8192":
                # The linear position bias on the same inputs, geometric
                # slopes 2^(-8 (h + 1) / Hq); same nominal FLOP counts.
                slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)],
                                      dtype=torch.float32, device=dev)

                def fwd_b():
                    st = fa.fa_fwd_alibi(q, k, v, o, lse, slopes, B, Hq, Hkv, N, d, w.scale,
                                         w.causal, stream.cuda_stream)
                    if st:
                        raise fa.FAError(st, "fa_fwd_alibi")

                row["calls"].append(entry("fa_fwd_alibi", w.fwd_flops(),
                                          time_launches(fwd_b, reps, stream)))
                wsb = fa.fa_bwd_workspace_bytes(B, Hq, Hkv, N, d, fa.BWD_SEPARATE)
                ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

                def bwd_b():
                    st = fa.fa_bwd_alibi(q, k, v, o, lse, do, dq, dk, dv, slopes, B, Hq, Hkv, N,
                                         d, w.scale, w.causal, fa.BWD_SEPARATE, ws, wsb,
                                         stream.cuda_stream)
                    if st:
                        raise fa.FAError(st, "fa_bwd_alibi")

                row["calls"].append(entry("fa_bwd_alibi deterministic", w.bwd_flops(),
                                          time_launches(bwd_b, reps, stream)))
        torch.cuda.synchronize()
        return row

    rows = []
    for w in WORKLOADS.values():
        # The long-context GQA shape also runs its backward (both modes): dO
        # is drawn after V, so Q, K and V are the forward workload's own.
        if w.name == "fwd_causal_gqa_n32768":
            w = replace(w, backward=True)
        rows.append(one(w))  # the workload's tensors are freed on return
    return rows


def cpu_baseline(x_head, threads):
    """The fp64 oracle, as it stands, on bounded samples of every workload:
    whole heads of each forward and whole key/value groups of the backward
    workload, with the inputs those workloads draw.  The headline figure is
    the backward workload's sample (forward + backward); the others are
    listed per workload.  About 20 s on 16 host cores."""
    import numpy as np
    import oracle
    from synth import WORKLOADS, make_inputs
    per = []
    head = None
    samples = {"fwd_small_d64": 2, "fwd_n4096": 16, "fwd_causal_rowscale_n8192": 8,
               "fwd_causal_gqa_n32768": 4, "fwdbwd_causal_n8192": 16}
    for name, n_heads in samples.items():
        w = WORKLOADS[name]
        x = x_head if name == "fwdbwd_causal_n8192" else make_inputs(w)
        heads = list(range(n_heads))
        t0 = time.perf_counter()
        oracle.fwd_heads(x["q"], x["k"], x["v"], w.scale, w.causal, heads, threads=threads)
        secs = time.perf_counter() - t0
        flops = w.fwd_flops() * n_heads / (w.B * w.Hq)
        row = {"workload": name, "call": "forward", "heads": n_heads, "of_heads": w.B * w.Hq,
               "seconds": secs, "tflops": flops / secs / 1e12}
        per.append(row)
        if w.backward:
            groups = list(range(n_heads))   # Hq == Hkv: one head per group
            t0 = time.perf_counter()
            oracle.bwd_groups(x["q"], x["k"], x["v"], x["dout"], w.scale, w.causal, groups,
                              threads=threads)
            bsecs = time.perf_counter() - t0
            # bwd_groups also recomputes the forward of its groups
            bflops = (w.fwd_flops() + w.bwd_flops()) * len(groups) / (w.B * w.Hkv)
            per.append({"workload": name, "call": "forward+backward", "groups": len(groups),
                        "of_groups": w.B * w.Hkv, "seconds": bsecs,
                        "tflops": bflops / bsecs / 1e12})
            head = (bflops / bsecs / 1e12, len(groups), w.B * w.Hkv, bsecs)
        del x
    value, ng, of, secs = head
    return {"value": value, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 forward+backward of {ng} of {of} key/value groups of "
                      f"fwdbwd_causal_n8192 (same inputs), {secs:.1f} s; per_workload lists "
                      f"whole-head forward samples of every workload",
            "per_workload": per}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="fwdbwd_causal_n8192")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--ordered-reps", type=int, default=10,
                   help="timed launches of each of the ordered and the paired-atomic "
                        "backward, reported under parts (0: skip)")
    p.add_argument("--no-per-config", action="store_true",
                   help="skip timing each synthetic workload on its own")
    p.add_argument("--per-config-reps", type=int, default=10)
    p.add_argument("--copy-calibration", action="store_true",
                   help="run one 256 MiB device-to-device copy before the timed region "
                        "(reference kernel for scaling HBM byte counters)")
    return p.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: every workload of "
                                   "the attention hot path fits one MI355X, so --gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import exact_tiled_attention_27_amd as fa
    from synth import WORKLOADS, make_inputs
    from dataclasses import replace

    w = WORKLOADS[args.workload]
    if not w.backward:
        w = replace(w, backward=True)  # the step runs the backward on the same shape
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    x = make_inputs(w)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["dout"])
    B, Hq, Hkv, N, d = w.B, w.Hq, w.Hkv, w.N, w.d
    o = torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    dq = torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev)
    dk = torch.empty((B, Hkv, N, d), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    ws_bytes = max(fa.fa_bwd_workspace_bytes(B, Hq, Hkv, N, d, m)
                   for m in (fa.BWD_ATOMIC, fa.BWD_SEPARATE, fa.BWD_ORDERED,
                             fa.BWD_ATOMIC_PAIRED))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def fwd():
        st = fa.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, w.scale, w.causal, stream.cuda_stream)
        if st:
            raise fa.FAError(st, "fa_fwd")

    def bwd(det):
        st = fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, N, d, w.scale, w.causal, det,
                       ws, ws_bytes, stream.cuda_stream)
        if st:
            raise fa.FAError(st, "fa_bwd")

    calls = [("fwd", fwd), ("bwd_deterministic", lambda: bwd(fa.BWD_SEPARATE)),
             ("bwd_atomic", lambda: bwd(fa.BWD_ATOMIC))]
    print(f"bench: workload {w.name} ({w.note}); warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)
    if args.copy_calibration:
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        for j, (_, fn) in enumerate(calls):
            fn()
            ev[i][j + 1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    f_fwd, f_bwd = w.fwd_flops(), w.bwd_flops()
    flops = {"fwd": f_fwd, "bwd_deterministic": f_bwd, "bwd_atomic": f_bwd}
    value = (f_fwd + 2 * f_bwd) / (ms_step * 1e-3) / 1e12

    parts = {}
    for j, (name, _) in enumerate(calls):
        ms = [e[j].elapsed_time(e[j + 1]) for e in ev]
        parts[f"{name}_ms_avg"] = float(np.mean(ms))
        parts[f"{name}_ms_min"] = float(np.min(ms))
        parts[f"{name}_tflops"] = flops[name] / (np.mean(ms) * 1e-3) / 1e12
        parts[f"{name}_frac_peak"] = parts[f"{name}_tflops"] / PEAK_BF16_TFLOPS

    # The other two dQ modes of the same backward, each back to back after
    # one untimed call.
    for mode, key in ((fa.BWD_ORDERED, "bwd_ordered"), (fa.BWD_ATOMIC_PAIRED, "bwd_atomic_paired")):
        if args.ordered_reps <= 0:
            break
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        bwd(mode)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.ordered_reps):
            bwd(mode)
        e1.record(stream)
        torch.cuda.synchronize()
        at_ms = e0.elapsed_time(e1) / args.ordered_reps
        parts[f"{key}_ms_avg"] = at_ms
        parts[f"{key}_tflops"] = f_bwd / (at_ms * 1e-3) / 1e12

    # Roofline of the dominant launch: the call of the step that takes the
    # longest.  fa_fwd is one kernel; fa_bwd is a short preprocess kernel and
    # the dK/dV kernel (atomic mode: with the dQ atomics), plus the dQ kernel
    # in deterministic mode, timed together by the events around the call.
    # Algorithmic work is the nominal count of the call (the dQ pass's
    # recomputation of S and dP is not counted).
    cz = "true" if w.causal else "false"
    kernels = {
        "fwd": [f"fa::fwd_kernel<{d}, {cz}, 0, false, false>"],
        "bwd_deterministic": [f"fa::bwd_pre_kernel<{d}>",
                              f"fa::bwd_dkdv_split_kernel<{d}, {cz}, 0, false>",
                              f"fa::bwd_dq_kernel<{d}, {cz}, false, false>"],
        "bwd_atomic": [f"fa::bwd_pre_kernel<{d}>",
                       f"fa::bwd_dkdv_split_kernel<{d}, {cz}, 1, false>"],
    }
    dom = max((name for name, _ in calls), key=lambda n: parts[f"{n}_ms_avg"])
    rl_ms = parts[f"{dom}_ms_avg"]
    achieved = flops[dom] / (rl_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "call": dom, "kernel": " + ".join(kernels[dom]),
                "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": measured_traffic(kernels[dom], w.name), "traffic_unit": "bytes",
                "flops_per_launch": flops[dom], "avg_launch_ms": rl_ms}

    configs = None
    if not args.no_per_config:
        configs = per_config(fa, args.per_config_reps, dev, stream)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        cpu = cpu_baseline(x, oracle.default_threads())

    out = {
        "metric": "attention fwd/bwd TFLOP/s (bf16, d=128) and % of MI355X bf16 MFMA peak",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "frac_peak": value / PEAK_BF16_TFLOPS,
        "config": {"workload": w.name, "B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "d": d,
                   "causal": w.causal,
                   "step": "fa_fwd + fa_bwd (deterministic dQ) + fa_bwd (atomic dQ)",
                   "flops_per_step": f_fwd + 2 * f_bwd},
        "parts": parts,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_config": configs,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
