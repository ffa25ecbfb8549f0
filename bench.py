#!/usr/bin/env python3
"""Benchmark of the KDA chunked-prefill forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1] [--no-cpu]

A step is one kda_chunk_prefill_fwd call covering every head of one layer of
the workload (default: 8 sequences x 2048 tokens, 16 heads, head_dim 128, fp32
initial/final state; the 8x2048 shape of vLLM PR #55737's report, "Features
and motivation").  Inputs are seeded synthetic data already resident in HBM.
Two complete buffer sets are rotated so that consecutive steps do not find the
previous step's data in the 256 MB last-level cache.

Prints one JSON line: tokens/s (whole job), microseconds per layer (wall
clock per step, and event median / min / p90 per launch, and the median of the
same call replayed from a captured HIP graph), the HBM roofline of the dominant
kernel (algorithmic bytes / measured launch time against 8 TB/s, and against a
measured device-copy bandwidth), and the fp64 oracle timed on the host cores
as a reported baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s + µs/layer (8x2048, H=16, D=128); % of MFMA/HBM roofline"
CSRC = os.path.join(ROOT, "gated_delta_rule_tok_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, AMD spec
MFMA_BF16_PEAK_TF = 2500.0  # dense bf16, AMD spec


def algorithmic_bytes(T, H, N, state_bytes, has_initial):
    """Bytes the method must move: q, k, v, g (bf16) + beta logit (bf16) + out
    (bf16) per (token, head); the state written once, read once if given."""
    per_token_head = 4 * 128 * 2 + 2 + 128 * 2
    per_seq_head = 128 * 128 * state_bytes * (2 if has_initial else 1)
    return T * H * per_token_head + N * H * per_seq_head


def kernel_source_hash() -> str:
    """sha256 over the kernel sources; traffic figures are only valid for the
    sources they were measured on."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def dominant_kernel(decode: bool, lower_bound: float, seg_len: int = 0, vs: int = 64,
                    duo: bool = False) -> str:
    """The kernels a call's time goes to (the library's automatic choice):
    the token-serial decode kernel for decode-sized calls, else the 16-token
    pipelined kernel for lower_bound >= -5 and the 32-token one below.  A call
    that takes the segment-parallel schedule (seg_len > 0) runs four kernels,
    named "+"-joined as rocprofv3 prints them (vs: the rerun's value slice);
    one that takes the two-workgroup form (duo) runs duo_kernel."""
    if decode:
        return "decode_kernel"
    if lower_bound < -5.0:
        return "fwd32_kernel"
    if seg_len:
        return f"seg_plan_kernel+pipe_kernel<64, true>+seg_combine_kernel+pipe_kernel<{vs}, false>"
    if duo:
        return "duo_kernel"
    return "pipe_kernel"


def plan_vsplit(heads: int, seqs: int, cus: int = 256) -> int:
    """The library's value split (the pages' rule, doubled while it fits)."""
    s = 1
    while s < 8 and 2 * s * heads * seqs <= cus:
        s *= 2
    return s


def call_kernels(args, T: int, H: int, N: int, lower_bound: float) -> str:
    """dominant_kernel for a bench run's call, asking the library whether the
    call takes the segment-parallel schedule."""
    import gated_delta_rule_tok_amd as kda
    decode = bool(args.decode_batch)
    L = 0 if decode or args.checkpoint_interval else kda.kda_debug_segment_length(T, H, N)
    vs = 64
    if L:
        s = args.vsplit or max(2, plan_vsplit(H, N + T // L))
        vs = 128 // s
    duo = (not decode and not args.checkpoint_interval and not L
           and kda.kda_debug_two_workgroups(T, H, N, device_cus()))
    return dominant_kernel(decode, lower_bound, L, vs, duo)


def device_cus() -> int:
    """Compute units of the GPU (256 on MI355X; 256 without a GPU)."""
    import torch
    if torch.cuda.is_available():
        return torch.cuda.get_device_properties(0).multi_processor_count
    return 256


def uniform_dims(spec: str):
    """--uniform N,L,H: N sequences of L tokens, H heads."""
    n, length, h = (int(v) for v in spec.split(","))
    if n <= 0 or length <= 0 or h <= 0:
        raise ValueError(f"--uniform {spec}: sizes must be positive")
    return n, length, h


def traffic_file(workload: str, kernel: str) -> str:
    label = kernel.replace("<", "").replace(">", "").replace(", ", "_")
    return os.path.join(PROFILES, f"traffic__{label}__{workload}.json")


def _pmc_sum(path: str, kernel_sub: str):
    """Mean over dispatches of the per-dispatch counter sum, for one kernel."""
    import collections
    import csv
    per = collections.defaultdict(float)
    for r in csv.DictReader(open(path)):
        if kernel_sub in r["Kernel_Name"]:
            per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    return (sum(per.values()) / len(per), len(per)) if per else (None, 0)


def traffic_from_pmc(pmc_dir: str, workload: str, command: str, kernel: str) -> dict:
    """Turn rocprofv3 FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch) of the
    benchmark and of a plain device copy of known size into HBM bytes per
    launch of the dominant kernel.  Expects pmc_dir/{fetch,write,cal_fetch,cal_write}/
    run_counter_collection.csv; the calibration copy moves 256 MiB."""
    f = lambda d: os.path.join(pmc_dir, d, "run_counter_collection.csv")
    # "a+b": one call launches both kernels; its bytes are the sum of their means
    fetch = write = 0.0
    nf = nw = 0
    for k in kernel.split("+"):
        fk, nfk = _pmc_sum(f("fetch"), k)
        wk, nwk = _pmc_sum(f("write"), k)
        fetch, write, nf, nw = fetch + fk, write + wk, nf + nfk, nw + nwk
    cal_f, _ = _pmc_sum(f("cal_fetch"), "copyBuffer")
    cal_w, _ = _pmc_sum(f("cal_write"), "copyBuffer")
    copy_kib = 256 * 1024
    fs, ws = copy_kib / cal_f, copy_kib / cal_w
    out = {"kernel_source_sha256": kernel_source_hash(), "workload": workload, "kernel": kernel,
           "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
           "dispatches": [nf, nw], "fetch_scale": fs, "write_scale": ws,
           "calibration": "device copy of 256 MiB: FETCH_SIZE %.0f KiB, WRITE_SIZE %.0f KiB"
                          % (cal_f, cal_w),
           "bytes_per_launch": (fetch * fs + write * ws) * 1024.0,
           "read_bytes": fetch * fs * 1024.0, "write_bytes": write * ws * 1024.0,
           "command": command}
    return out


PROJ_KERNELS = "proj_ab_kernel+proj_out_kernel"


def workload_name(args, dims=None):
    """(workload name, dominant kernel, the selecting arguments) of a run;
    dims: the workload's (tokens, heads, sequences) if already known."""
    import kda_inputs as KI
    if getattr(args, "proj", 0):
        return f"proj_{args.proj}x7168_144_1536", PROJ_KERNELS, f"--proj {args.proj}"
    apply_hooks(args)
    if args.decode_batch:
        wl, lb = f"decode_{args.decode_batch}x1_h16", KI.LOWER_BOUND
        sel = f"--decode-batch {args.decode_batch}"
    elif getattr(args, "uniform", None):
        n, length, h = uniform_dims(args.uniform)
        wl, lb = f"uniform_{n}x{length}_h{h}", KI.LOWER_BOUND
        sel = f"--uniform {n},{length},{h}"
        if dims is None:
            dims = (n * length, h, n)
    else:
        wl, lb = KI.CONFIGS[args.config]["name"], KI.LOWER_BOUND
        sel = f"--config {args.config}"
    if args.lower_bound is not None:
        lb = float(args.lower_bound)
        wl += f"_lb{args.lower_bound:g}"
        sel += f" --lower-bound {args.lower_bound:g}"
    if args.segments != "auto":
        sel += f" --segments {args.segments}"
    if getattr(args, "kernel", 0):
        wl += f"_kernel{args.kernel}"
        sel += f" --kernel {args.kernel}"
    if args.vsplit:
        sel += f" --vsplit {args.vsplit}"
    if dims is not None:
        T, H, N = dims
    elif args.decode_batch:
        T, H, N = args.decode_batch, 16, args.decode_batch
    else:
        c = KI.CONFIGS[args.config]
        if c["lengths"] is None:
            x = KI.config_inputs(args.config)
            T, H, N = x.T, x.H, x.N
        else:
            T, H, N = sum(c["lengths"]), c["heads"], len(c["lengths"])
    return wl, call_kernels(args, T, H, N, lb), sel


def apply_hooks(args):
    """The library's test hooks the run asks for: the segment schedule, the
    value split and the kernel family."""
    import gated_delta_rule_tok_amd as kda
    seg = {"auto": 0, "off": 1}.get(args.segments)
    kda.kda_debug_set_segment(int(args.segments) if seg is None else seg)
    kda.kda_debug_set_vsplit(args.vsplit)
    kda.kda_debug_set_kernel(getattr(args, "kernel", 0))


PROJ_K, PROJ_NAB, PROJ_NB = 7168, 144, 1536


def proj_algorithmic_bytes(M, K=PROJ_K, n_ab=PROJ_NAB, n_b=PROJ_NB):
    """Bytes the two projections must move: hidden and both weights read once,
    P and G written once (bf16)."""
    return 2 * (M * K + n_ab * K + n_b * 128 + M * n_ab + M * n_b)


def bench_proj(args):
    """Time kda_gate_proj (both kernels of one call) for args.proj tokens.
    Weight sets are rotated so that the weights come from HBM, as for a layer
    whose weights were last read a whole model pass ago: 128 sets of 2.4 MB
    exceed the 256 MB last-level cache.  The launch time is the call's (both
    kernels, events on the launch stream); the roofline is its algorithmic
    bytes against 8 TB/s."""
    import torch
    import gated_delta_rule_tok_amd as kda
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M, K, NAB, NB = args.proj, PROJ_K, PROJ_NAB, PROJ_NB
    nsets = 128
    rng = np.random.default_rng(11)
    import kda_inputs as KI
    h_np = KI.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    wab_np = KI.f32_to_bf16_bits((K ** -0.5 * rng.standard_normal((NAB, K))).astype(np.float32))
    wb_np = KI.f32_to_bf16_bits((128 ** -0.5 * rng.standard_normal((NB, 128))).astype(np.float32))

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    h0, wab0, wb0 = bf(h_np), bf(wab_np), bf(wb_np)
    sets = []
    for i in range(nsets):
        sets.append(dict(h=h0.clone(), wab=wab0.clone(), wb=wb0.clone(),
                         p=torch.empty(M, NAB, dtype=torch.bfloat16, device=dev),
                         g=torch.empty(M, NB, dtype=torch.bfloat16, device=dev),
                         ws=torch.zeros(kda.kda_gate_proj_workspace_size(M, K, NAB),
                                        dtype=torch.uint8, device=dev)))

    def step(i):
        s = sets[i % nsets]
        kda.kda_gate_proj(s["h"], s["wab"], s["wb"], s["p"], s["g"], s["ws"])

    stream = torch.cuda.current_stream()
    c0, n = time.perf_counter(), 0
    while time.perf_counter() - c0 < args.settle_ms * 1e-3:
        for _ in range(64):
            step(n)
            n += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    call_ms = np.array([a.elapsed_time(b) for a, b in ev])
    # one graph holding 64 calls (64 weight sets): device time per call with no
    # host work and no per-launch submission gap between calls
    graph_us = None
    if not args.no_graph:
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                for i in range(64):
                    s = sets[i]
                    kda.kda_gate_proj(s["h"], s["wab"], s["wb"], s["p"], s["g"], s["ws"],
                                      stream=cap)
        torch.cuda.synchronize()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(10)]
        for a, b in gev:
            a.record(stream)
            graph.replay()
            b.record(stream)
        torch.cuda.synchronize()
        graph_us = float(np.median([a.elapsed_time(b) for a, b in gev])) * 1e3 / 64

    ms_per_step = wall * 1e3 / args.steps
    launch_ms = float(call_ms.mean())
    abytes = proj_algorithmic_bytes(M)
    traffic = None
    wl, _, _ = workload_name(args)
    tf = traffic_file(wl, PROJ_KERNELS)
    if os.path.exists(tf):
        t = json.load(open(tf))
        if t.get("kernel_source_sha256") == kernel_source_hash():
            traffic = t["bytes_per_launch"]
    achieved = abytes / (launch_ms * 1e-3) / 1e9
    result = {
        "metric": "KDA gate / beta projection tokens/s (hidden 7168 -> 144 -> 1536)",
        "value": M / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "us_per_call_event_median": float(np.median(call_ms)) * 1e3,
        "us_per_call_event_min": float(call_ms.min()) * 1e3,
        "us_per_call_graph_replay": graph_us,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl, "tokens": M, "hidden": K,
                   "n_ab": NAB, "n_b": NB, "weight_sets": nsets},
        "roofline": {"bound": "hbm", "kernel": PROJ_KERNELS,
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": abytes, "launch_us": launch_ms * 1e3,
                     "graph_frac": (abytes / (graph_us * 1e-6) / 1e9 / HBM_PEAK_GBS
                                    if graph_us else None)},
    }
    if not args.no_cpu:
        from oracle import proj
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # noqa: BLE001 - thread count is informational
            threads = 1
        times = []
        while len(times) < 50 and sum(times) < 3.0:
            c0 = time.perf_counter()
            proj.gate_proj(h_np, wab_np, wb_np)
            times.append(time.perf_counter() - c0)
        cpu_s = float(np.median(times))
        result["cpu_baseline"] = {
            "value": M / cpu_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole call ({M} tokens), fp64 numpy products; median of "
                      f"{len(times)} calls, {cpu_s * 1e3:.2f} ms each"}
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay timing")
    ap.add_argument("--sets", type=int, default=2, help="buffer sets rotated across steps")
    ap.add_argument("--checkpoint-interval", type=int, default=0,
                    help="also write the state every this many tokens of each sequence "
                         "(kda_chunk_prefill_fwd_checkpoints); 0: off")
    ap.add_argument("--lower-bound", type=float, default=None,
                    help="override the workload's lower_bound (below -5 the 32-token kernel runs; "
                         "not the headline configuration)")
    ap.add_argument("--decode-batch", type=int, default=0,
                    help="instead of --config: this many one-token sequences, 16 heads, fp32 "
                         "state (a decode step; the token-serial decode kernel runs)")
    ap.add_argument("--uniform", metavar="N,L,H", default=None,
                    help="instead of --config: N sequences of L tokens, H heads, fp32 initial "
                         "and final state, the configurations' input distributions")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="run the call this long before the warmup steps (clock ramp; 0: none)")
    ap.add_argument("--traffic-from", metavar="PMC_DIR",
                    help="write the traffic file for --config from rocprofv3 counter runs, then exit")
    ap.add_argument("--segments", default="auto",
                    help="the segment-parallel schedule for long sequences in calls with few "
                         "(sequence, head) pairs: auto, off, or a segment length (multiple of 16)")
    ap.add_argument("--vsplit", type=int, default=0,
                    help="force the value split (1, 2, 4, 8); 0: the library's choice")
    ap.add_argument("--kernel", type=int, default=0,
                    help="force a kernel family (kda_debug_set_kernel: 4 the 16-token kernel, 6 its "
                         "two-workgroup form, ...); 0: the library's choice.  Not the headline number")
    ap.add_argument("--proj", type=int, default=0, metavar="M",
                    help="instead of the forward: time the gate / beta projections (kda_gate_proj) "
                         "for M tokens at hidden 7168, 144 = 128 + 16 rows, 1536 gate columns")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 256 MiB device copy three times (the counter calibration), then exit")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        n = 256 * 1024 * 1024 // 4
        a = torch.ones(n, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(f"copied {4 * n} bytes x3")
        return

    if args.traffic_from:
        wl, kernel, sel = workload_name(args)
        cmd = ("cd /tmp && export TMPDIR=/tmp; for c in FETCH_SIZE WRITE_SIZE: rocprofv3 --pmc $c "
               f"--output-format csv -d <pmc>/<fetch|write> -o run -- python bench.py {sel} "
               "--steps 3 --warmup 1 --settle-ms 0 --no-cpu --no-graph; "
               "rocprofv3 --pmc $c --output-format csv "
               "-d <pmc>/<cal_fetch|cal_write> -o run -- python bench.py --copy-calibration; "
               f"python bench.py {sel} --traffic-from <pmc>")
        t = traffic_from_pmc(args.traffic_from, wl, cmd, kernel)
        os.makedirs(PROFILES, exist_ok=True)
        with open(traffic_file(wl, kernel), "w") as fh:
            json.dump(t, fh, indent=1)
        print(json.dumps(t))
        return

    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (--gpus {args.gpus} requested); "
              "the KDA forward has no cross-GPU path here", file=sys.stderr)
        sys.exit(2)

    if args.proj:
        bench_proj(args)
        return

    import torch
    import kda_inputs as KI
    import gated_delta_rule_tok_amd as kda

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    apply_hooks(args)
    if args.decode_batch:
        x = KI.make_inputs([1] * args.decode_batch, 16, seed=7, init_state="fp32")
    elif args.uniform:
        n, length, h = uniform_dims(args.uniform)
        x = KI.make_inputs([length] * n, h, seed=11, init_state="fp32")
    else:
        x = KI.config_inputs(args.config)
    if args.lower_bound is not None:
        x.lower_bound = float(args.lower_bound)
    x.meta["config"], kernel, _ = workload_name(args, (x.T, x.H, x.N))
    T, H, N = x.T, x.H, x.N
    sbytes = 2 if x.state_bf16 else 4
    sdtype = torch.bfloat16 if x.state_bf16 else torch.float32

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    base = dict(q=bf(x.q), k=bf(x.k), v=bf(x.v), g=bf(x.g), beta=bf(x.beta_logits),
                A_log=torch.from_numpy(x.A_log).to(dev),
                dt_bias=torch.from_numpy(x.dt_bias).to(dev),
                cu=torch.from_numpy(x.cu_seqlens).to(dev))
    if x.initial_state is None:
        base["s0"] = None
    elif x.state_bf16:
        base["s0"] = bf(x.initial_state)
    else:
        base["s0"] = torch.from_numpy(x.initial_state).to(dev)
    sets = []
    for i in range(max(1, args.sets)):
        s = base if i == 0 else {k: (None if v is None else v.clone()) for k, v in base.items()}
        s["out"] = torch.empty(T, H, 128, dtype=torch.bfloat16, device=dev)
        s["fin"] = torch.empty(N, H, 128, 128, dtype=sdtype, device=dev)
        s["ws"] = torch.zeros(max(1, kda.kda_get_workspace_size(T, H, N)), dtype=torch.uint8,
                              device=dev)
        s["ck"] = (torch.empty(T // args.checkpoint_interval, H, 128, 128, dtype=sdtype, device=dev)
                   if args.checkpoint_interval else None)
        sets.append(s)
    lens = np.diff(x.cu_seqlens)
    n_ck = int((lens // args.checkpoint_interval).sum()) if args.checkpoint_interval else 0

    def step(i):
        s = sets[i % len(sets)]
        kda.kda_chunk_prefill_fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], s["A_log"],
                                  s["dt_bias"], x.lower_bound, x.scale, s["s0"], s["cu"],
                                  s["out"], s["fin"], s["ws"], checkpoints=s["ck"],
                                  checkpoint_interval=args.checkpoint_interval)

    # The device's clocks ramp up over the first ~20 ms of this load (one
    # launch went from about 184 to 148 us over its first ~120 calls), so the
    # call runs for a fixed ~200 ms before the warmup steps: the timed steps
    # then see the steady state a serving loop sees.  Reported as
    # "device_settle".
    settle_calls, c0 = 0, time.perf_counter()
    while settle_calls < 5000 and time.perf_counter() - c0 < args.settle_ms * 1e-3:
        for _ in range(20):
            step(settle_calls)
            settle_calls += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - c0) * 1e3
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    # the timed steps (value, ms_per_step): K calls back to back, nothing else
    # queued between them
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the same K calls again, each bracketed by events on its stream (per-launch
    # durations for the roofline; the event records add small gaps between
    # launches, which is why they are not in the loop above)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per_launch_ms = np.array([a.elapsed_time(b) for a, b in ev])

    ms_per_step = wall * 1e3 / args.steps
    launch_ms = float(per_launch_ms.mean())

    # the same call replayed from a captured HIP graph (no host work per call)
    graph_us = graph10_us = None
    if not args.no_graph:
        s0 = sets[0]
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            step(0)  # untimed: settles the stream before capture
            cap.synchronize()
            with torch.cuda.graph(graph, stream=cap):
                kda.kda_chunk_prefill_fwd(s0["q"], s0["k"], s0["v"], s0["g"], s0["beta"],
                                          s0["A_log"], s0["dt_bias"], x.lower_bound, x.scale,
                                          s0["s0"], s0["cu"], s0["out"], s0["fin"], s0["ws"],
                                          checkpoints=s0["ck"],
                                          checkpoint_interval=args.checkpoint_interval)
        torch.cuda.synchronize()
        # the capture left the device idle: settle the clocks again (~100 ms)
        c0 = time.perf_counter()
        while time.perf_counter() - c0 < 0.1:
            for _ in range(20):
                graph.replay()
            torch.cuda.synchronize()
        gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a, b in gev:
            a.record(stream)
            graph.replay()
            b.record(stream)
        torch.cuda.synchronize()
        graph_us = float(np.median([a.elapsed_time(b) for a, b in gev])) * 1e3
        # ten calls in one graph (buffer sets rotated): the time per call
        # without a graph launch per call
        graph10 = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph10, stream=cap):
                for i in range(10):
                    step(i)
        torch.cuda.synchronize()
        c0 = time.perf_counter()  # settle the clocks again after the capture (~100 ms)
        while time.perf_counter() - c0 < 0.1:
            for _ in range(2):
                graph10.replay()
            torch.cuda.synchronize()
        gev10 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(max(3, args.steps // 10))]
        for a, b in gev10:
            a.record(stream)
            graph10.replay()
            b.record(stream)
        torch.cuda.synchronize()
        graph10_us = float(np.median([a.elapsed_time(b) for a, b in gev10])) * 1e3 / 10

    # measured device-copy bandwidth (read + write of 1 GiB), a practical HBM ceiling
    cbuf = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cdst = torch.empty_like(cbuf)
    cdst.copy_(cbuf)
    ce = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(5)]
    for a, b in ce:
        a.record(stream)
        cdst.copy_(cbuf)
        b.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * cbuf.numel() * 4 / (min(a.elapsed_time(b) for a, b in ce) * 1e-3) / 1e9
    del cbuf, cdst
    tokens_per_s = T / (ms_per_step * 1e-3)
    abytes = algorithmic_bytes(T, H, N, sbytes, x.initial_state is not None)
    abytes += n_ck * H * 128 * 128 * sbytes  # checkpoint states written
    achieved_gbs = abytes / (launch_ms * 1e-3) / 1e9

    traffic = None
    tf = traffic_file(x.meta["config"], kernel)
    if os.path.exists(tf) and not args.checkpoint_interval:  # counters of the plain call
        t = json.load(open(tf))
        if t.get("kernel_source_sha256") == kernel_source_hash():
            traffic = t["bytes_per_launch"]

    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "device_settle": {"calls": settle_calls, "ms": settle_ms},
        "ms_per_step": ms_per_step,
        "us_per_layer": ms_per_step * 1e3,
        "us_per_layer_event_median": float(np.median(per_launch_ms)) * 1e3,
        "us_per_layer_event_min": float(per_launch_ms.min()) * 1e3,
        "us_per_layer_event_p90": float(np.percentile(per_launch_ms, 90)) * 1e3,
        "us_per_layer_graph_replay_median": graph_us,
        "us_per_layer_graph_of_10_calls": graph10_us,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": x.meta["config"], "tokens": T, "sequences": N, "heads": H,
                   "head_dim": 128, "state": "bf16" if x.state_bf16 else "fp32",
                   "initial_state": x.initial_state is not None, "buffer_sets": len(sets),
                   **({"checkpoint_interval": args.checkpoint_interval, "checkpoints": n_ck}
                      if args.checkpoint_interval else {})},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": abytes, "launch_us": launch_ms * 1e3,
                     "measured_copy_GBps": copy_gbs,
                     "frac_of_measured_copy": achieved_gbs / copy_gbs},
    }

    if not args.no_cpu:
        import oracle
        # the oracle parallelises over (sequence, head) items: as many threads
        # as it has items, at most the CPUs this process may run on
        host_cpus = os.cpu_count()
        affinity = len(os.sched_getaffinity(0))
        threads = max(1, min(affinity, N * H))
        # whole-workload passes, repeated until about 3 s of wall clock (at most
        # 7 passes); the median pass is reported
        times = []
        while len(times) < 7 and sum(times) < 3.0:
            c0 = time.perf_counter()
            oracle.kda_oracle_fwd(x.q, x.k, x.v, x.g, x.beta_logits, x.A_log, x.dt_bias,
                                  x.lower_bound, x.scale, x.initial_state, x.cu_seqlens,
                                  threads=threads)
            times.append(time.perf_counter() - c0)
        cpu_s = float(np.median(times))
        result["cpu_baseline"] = {
            "value": T / cpu_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host_cpu_count": host_cpus, "affinity_cpus": affinity, "threads_used": threads,
            "sample": f"the whole {x.meta['config']} workload ({T} tokens x {H} heads), "
                      f"fp64 token recurrence, {threads} threads over (sequence, head); "
                      f"median of {len(times)} passes, {cpu_s:.2f} s each"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
