#!/usr/bin/env python3
"""Decode throughput of the 9B-shaped Mamba-2 mixer layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1]

One step = one m2_step call: in_proj GEMV (+conv, dt), SSD state update and
readout (+gate), RMSNorm + out_proj GEMV, for every session of the batch, on
seeded synthetic inputs already resident in HBM. The default workload is the
single-session decode of a 9B-shaped layer (d_model 4480, 128 heads x 80,
d_state 128, 8 groups, bf16 weights, fp32 state), 750 frames of 80 ms.

The layer's weights are held in `--copies` identical device copies used in
turn (default: enough copies for at least 2.5 GB, about ten times the 256 MB
last-level cache, i.e. 9 for bf16 weights and 30 for 4-bit codes), so that no
step is served from the cache by the weights of a recent step, whatever each
load's cache policy, as in a real stack where every other layer's weights
stream through in between. (With two bf16 copies, the two W_out matrices, 184 MB,
fit the cache when in_proj's loads bypass it.)

Prints one JSON line. Besides steps/s it reports the step's algorithmic HBM
bytes and bandwidth, per-kernel durations measured with HIP events on the
stream the kernels run on, the dominant kernel's roofline, a parity check of
the first steps against the CPU oracle, and that oracle's own speed on a
bounded sample (cpu_baseline: a baseline, not a target).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "Mamba-2 decode steps/s + achieved HBM GB/s (% peak), 9B-shaped layer"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", type=int, default=1,
                    help="workload: 1 (default), 2 (32 sessions), 3 (27-layer int8 stack), 4 (prefill + 4 sessions), "
                         "5 (int4 g64 weights, 1 session), 6 (int3 g64 weights, 1 session), "
                         "7 (text and function output heads with greedy argmax, 1 session), "
                         "8 (attention layer with a bf16 KV cache of 1000+ positions, 1 session), "
                         "9 (hybrid stack of 27 Mamba-2 and 4 attention layers, one call per step, 1 session), "
                         "10 (attention layer, 32 sessions)")
    ap.add_argument("--copies", type=int, default=0,
                    help="identical weight copies used in turn (0: enough for >= 2.5 GB)")
    ap.add_argument("--no-graph", action="store_true", help="time plain launches only")
    ap.add_argument("--persistent", action="store_true",
                    help="single-layer decode workloads: plan 2 (the persistent SSD + out_proj kernel); "
                         "stack workloads: each run of mixer layers in one persistent launch")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline and parity")
    ap.add_argument("--prof-steps", type=int, default=200, help="steps of the per-kernel event pass")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run 3 device-to-device copies of MIB MiB (the known-size kernel that "
                         "scales rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def wbytes(dims):
    """Bytes per weight element as stored (4- and 3-bit codes packed)."""
    return {"f32": 4, "bf16": 2, "int8g": 1, "int4g": 0.5, "int3g": 0.375}[dims.wtype]


# phases of m2_step_timed (the same for both step plans of m2_step_plan)
PHASES = ["gemv_in", "ssd_step", "gemv_out"]
# Weight bytes the single-layer workloads rotate through (identical device copies used in
# turn): about ten times the MI355X's 256 MB last-level cache.
ROTATION_BYTES = 2_500_000_000


def kernel_bytes(dims, B):
    """Algorithmic HBM bytes per launch of each phase of the step (in_proj, SSD, out_proj)
    and of the whole step: every weight, state, cache and activation byte the phase must move
    once, nothing for re-reads."""
    d = dims
    f = 4
    wb = wbytes(d)

    def w_rows(rows, K):
        # int8: one fp16 scale per group; low-bit: an fp16 (scale, bias) pair per group
        scales = {"int8g": 2, "int4g": 4, "int3g": 4}.get(d.wtype, 0)
        return int(rows * K * wb) + rows * (K // d.q_group) * scales

    state = 2 * B * d.n_heads * d.head_dim * d.d_state * f
    cache_rd = B * (d.d_conv - 1) * d.conv_dim * f
    conv_par = d.conv_dim * (d.d_conv + 1) * f
    io = B * d.d_model * f
    v = B * d.d_inner * f
    xbc_dt = B * (d.conv_dim + d.n_heads) * f
    # the conv-cache shift (out_proj): rows 1..K-2 and the new raw inputs in, K-1 rows out
    shift = B * ((d.d_conv - 2) + 1 + (d.d_conv - 1)) * d.conv_dim * f
    ssd_core = state + cache_rd + conv_par + xbc_dt + 2 * d.n_heads * f
    k = {"gemv_in": w_rows(d.d_in_proj, d.d_model) + io + B * d.d_in_proj * f + d.n_heads * f,
         "ssd_step": ssd_core + v + v + B * d.n_heads * f + d.d_inner * f,
         "gemv_out": w_rows(d.d_model, d.d_inner) + v + B * d.n_heads * f + io + shift}
    k["step"] = (w_rows(d.d_in_proj, d.d_model) + w_rows(d.d_model, d.d_inner) + state + 2 * cache_rd +
                 conv_par + 3 * d.n_heads * f + d.d_inner * f + 2 * io)
    return k


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


def hip_runtime():
    """The HIP runtime torch has already mapped (same soname), for event timing."""
    import ctypes as C
    hip = C.CDLL("libamdhip64.so.7")
    hip.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
    hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
    hip.hipEventDestroy.argtypes = [C.c_void_p]
    return hip


def hip_event(hip):
    import ctypes as C
    e = C.c_void_p()
    if hip.hipEventCreateWithFlags(C.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
        raise RuntimeError("hipEventCreateWithFlags failed")
    return e.value


def hip_elapsed_ms(hip, a, b):
    import ctypes as C
    ms = C.c_float()
    if hip.hipEventElapsedTime(C.byref(ms), a, b) != 0:
        raise RuntimeError("hipEventElapsedTime failed")
    return ms.value


def hold_gpu(ms: float) -> None:
    """Enqueue a spin kernel of about `ms` milliseconds so that the host can enqueue an
    event-timed pass ahead of the GPU: the events then bracket kernels that run back to back
    instead of kernels that wait for the host's next launch."""
    import torch
    torch.cuda._sleep(int(ms * 2.4e6))          # cycles at 2.4 GHz


REPEATS = 5


def hold_ms(steps):
    """Length of the spin kernel that precedes a timed region: long enough for the host to
    enqueue `steps` steps behind it (about 40 us of host time per step, at least 5 ms)."""
    return max(5.0, 0.04 * steps)


def copy_bandwidth(dev, mib=512, reps=5):
    """A device-to-device copy of `mib` MiB timed with events (median of `reps`), outside any
    timed region: GB/s counting the bytes read and written (2 x the buffer), the box's own
    read-plus-write reference next to the 8 TB/s peak."""
    import numpy as np
    import torch
    src = torch.ones((mib << 20) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * (mib << 20) / (float(np.median(ms)) * 1e-3) / 1e9


def eager_ms_per_step(run, t0, steps, before=None):
    """Median over REPEATS of the milliseconds per step of `steps` plain-launch steps, each
    repeat bracketed by events on torch's current stream (where the steps run), the GPU held
    by a spin kernel while the host enqueues them. Returns (median, all repeats)."""
    import numpy as np
    import torch
    out = []
    for _ in range(REPEATS):
        if before:
            before()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        hold_gpu(hold_ms(steps))
        e0.record()
        run(t0, steps)
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / steps)
    return float(np.median(out)), out


# Launches per captured graph. Capturing 3000 steps of a 31-layer stack as one graph
# (~294k kernel nodes, one dependency chain) ended the process with a host segmentation fault
# during capture, before anything ran on the GPU. Only host-side graph state grows with the
# capture: one node (with a copy of its kernel arguments) and one edge per launch. A fault
# rather than an allocation failure fits a recursive walk over a chain of that length
# exhausting a thread's stack better than memory exhaustion; which one it was is not
# established, and the capture is not repeated. Graphs of at most this many launches (55
# stack steps) capture and replay correctly, so the steps are captured in such graphs and
# replayed in turn, and a single step above the limit is refused with an error.
MAX_GRAPH_LAUNCHES = 16384


def graph_ms_per_step(run, steps, launches_per_step, before_replay=None):
    """Median over REPEATS of the milliseconds per step of `steps` steps replayed from HIP
    graphs. The steps are captured as graphs of at most MAX_GRAPH_LAUNCHES launches
    (replayed as often as they fit) plus one for the remainder. before_replay (untimed) runs
    before the warm replay and before every timed one. Returns (median, all repeats)."""
    import numpy as np
    import torch
    if launches_per_step > MAX_GRAPH_LAUNCHES:
        raise ValueError("one step has %d launches, above the %d a captured graph may hold"
                         % (launches_per_step, MAX_GRAPH_LAUNCHES))
    chunk = max(1, min(steps, MAX_GRAPH_LAUNCHES // max(1, launches_per_step)))
    reps, rem = divmod(steps, chunk)

    def capture(n):
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                run(0, n)
        torch.cuda.current_stream().wait_stream(st)
        return g

    ga = capture(chunk)
    gb = capture(rem) if rem else None

    def replay_all():
        for _ in range(reps):
            ga.replay()
        if gb is not None:
            gb.replay()

    if before_replay:
        before_replay()
    replay_all()
    out = []
    for _ in range(REPEATS):
        if before_replay:
            before_replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        hold_gpu(hold_ms(reps + 1))
        e0.record()
        replay_all()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / steps)
    return float(np.median(out)), out


def traffic_for(kernel_name, workload):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was taken on the
    current kernel source (the summary stores the source hash); else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel_name, workload))
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
        if hashlib.sha256(src).hexdigest() != rec["source_sha256"]:
            return None
        return float(rec["bytes_per_launch"])
    except Exception:
        return None


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(--gpus %d, WORLD_SIZE %d requested)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from full_duplex_speech_mamba2_amd import m2, synth

    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.config in synth.HEAD_WORKLOADS:
        return bench_heads(args, synth.HEAD_WORKLOADS[args.config])
    if args.config in synth.ATTN_WORKLOADS:
        return bench_attn(args, synth.ATTN_WORKLOADS[args.config])
    if args.config in synth.STACK_WORKLOADS:
        return bench_stack(args, synth.STACK_WORKLOADS[args.config])
    wl = synth.workload(args.config)
    dims, B = wl.dims, wl.batch
    print("[bench] workload %s: generating inputs" % wl.name, file=sys.stderr, flush=True)
    xs_np = synth.make_inputs(dims, wl.seed, wl.steps, B)
    ssm0, conv0 = synth.make_state(dims, wl.seed, B, wl.state_var)
    if wl.layers == 1:
        # one layer's weights in identical copies used in turn
        w = synth.make_layer_weights(dims, wl.weight_seed)
        ncopy = args.copies
        if ncopy <= 0:
            per = kernel_bytes(dims, 1)["gemv_in"] + kernel_bytes(dims, 1)["gemv_out"]
            ncopy = max(2, -(-ROTATION_BYTES // per))
        layers = [m2.Layer(dims, w, dev) for _ in range(ncopy)]
        states = [m2.State(layers[0], B, torch.from_numpy(ssm0).to(dev), torch.from_numpy(conv0).to(dev))]
    else:
        # a residual stack: every layer its own seeded weights and zero state
        w = None
        layers, states = [], []
        for l in range(wl.layers):
            layers.append(m2.Layer(dims, synth.make_layer_weights(dims, wl.weight_seed, l), dev))
            states.append(m2.State(layers[-1], B))
    st = states[0]
    prefill_rec = None
    if wl.prefill:
        prefill_rec = time_prefill(args, wl, layers[0], st, dev)
    xs = torch.from_numpy(xs_np).to(dev)
    ys = torch.empty_like(xs)
    ws = layers[0].workspace("step", B)
    nx = xs.shape[0]
    nl = len(layers)

    def run(t0, n):
        for t in range(t0, t0 + n):
            if wl.layers == 1:
                m2.step(layers[t % nl], st, xs[t % nx], ys[t % nx], ws=ws, persistent=args.persistent)
            else:
                u = ys[t % nx]
                u.copy_(xs[t % nx])
                for lay, s_ in zip(layers, states):
                    m2.step(lay, s_, u, u, residual=True, ws=ws)   # y aliases x under M2_RESIDUAL

    torch.cuda.synchronize()
    run(0, args.warmup)
    torch.cuda.synchronize()

    # timed region 1: plain launches on torch's current stream (median of REPEATS)
    ms_eager, rep_eager = eager_ms_per_step(run, args.warmup, args.steps)

    # timed region 2: the same steps captured into HIP graphs and replayed
    ms_graph, rep_graph = None, None
    if not args.no_graph:
        ms_graph, rep_graph = graph_ms_per_step(run, args.steps, 4 * wl.layers)

    ms = min(ms_eager, ms_graph) if ms_graph is not None else ms_eager
    steps_per_s = 1000.0 / ms
    plan = layers[0].step_plan(B, persistent=args.persistent)
    kb = kernel_bytes(dims, B)

    # per-kernel durations: HIP events recorded between the step's kernels on the stream they
    # run on; created without the system-scope fence so that a marker costs little
    kp = max(10, args.prof_steps)
    hip = hip_runtime()
    evs = [[hip_event(hip) for _ in range(4)] for _ in range(kp)]
    torch.cuda.synchronize()
    hold_gpu(150.0)
    for t in range(kp):
        # per-kernel times of one layer (the stack's first layer, residual as in the stack)
        m2.step_timed(layers[t % nl] if wl.layers == 1 else layers[0], st, xs[t % nx], ys[t % nx], evs[t],
                      residual=wl.layers > 1, ws=ws, persistent=args.persistent and wl.layers == 1)
    torch.cuda.synchronize()
    if plan == 2:
        # in_proj, then the SSD and out_proj in one persistent kernel
        names = ["gemv_in", "ssd_out_fused"]
        kb["ssd_out_fused"] = kb["ssd_step"] + kb["gemv_out"]
        dur_us = {"gemv_in": 1000.0 * float(np.mean([hip_elapsed_ms(hip, evs[t][0], evs[t][1]) for t in range(kp)])),
                  "ssd_out_fused": 1000.0 * float(np.mean([hip_elapsed_ms(hip, evs[t][1], evs[t][3])
                                                           for t in range(kp)]))}
    else:
        names = PHASES
        dur_us = {n: 1000.0 * float(np.mean([hip_elapsed_ms(hip, evs[t][i], evs[t][i + 1]) for t in range(kp)]))
                  for i, n in enumerate(names)}
    for row in evs:
        for e in row:
            hip.hipEventDestroy(e)
    dom = max(names, key=lambda n: kb[n])
    copy_gbps = copy_bandwidth(dev)
    achieved = kb[dom] / (dur_us[dom] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic_for(dom, wl.name),
                "algorithmic_bytes": kb[dom], "avg_duration_us": round(dur_us[dom], 2)}

    out = {
        "metric": METRIC, "value": round(steps_per_s, 1), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "d_model": dims.d_model, "n_heads": dims.n_heads,
                   "head_dim": dims.head_dim, "d_state": dims.d_state, "n_groups": dims.n_groups,
                   "d_conv": dims.d_conv, "batch": B, "weight_dtype": dims.wtype,
                   "state_dtype": "f32", "layers": wl.layers, "weight_copies": nl if wl.layers == 1 else 1,
                   "step_plan": plan,
                   "timing": "graph" if (ms_graph is not None and ms_graph <= ms_eager) else "eager"},
        "achieved_GBps": round(wl.layers * kb["step"] * steps_per_s / 1e9, 1),
        "hbm_peak_frac": round(wl.layers * kb["step"] * steps_per_s / 1e9 / HBM_PEAK_GBPS, 4),
        "step_algorithmic_bytes": wl.layers * kb["step"],
        "session_tokens_per_s": round(B * steps_per_s, 1),
        "realtime_sessions": round(B * steps_per_s * 0.08, 1),
        "copy_GBps": round(copy_gbps, 1),
        "copy_frac": round(wl.layers * kb["step"] * steps_per_s / 1e9 / copy_gbps, 4),
        "ms_per_step_eager": round(ms_eager, 5),
        "ms_per_step_graph": None if ms_graph is None else round(ms_graph, 5),
        "repeats_ms_per_step": {"eager": [round(v, 5) for v in rep_eager],
                                "graph": None if rep_graph is None else [round(v, 5) for v in rep_graph],
                                "statistic": "median of %d repeats of %d steps" % (REPEATS, args.steps)},
        "kernel_us": {n: round(v, 2) for n, v in dur_us.items()},
        "kernel_us_source": "HIP events on the kernels' stream, mean over %d steps" % kp,
        "roofline": roofline,
        "cpu_baseline": None,
        "parity": None,
    }
    if prefill_rec is not None:
        out["prefill"] = prefill_rec

    if not args.no_cpu and wl.layers == 1:
        out["cpu_baseline"], out["parity"] = cpu_baseline_and_parity(args, wl, w, xs_np, ssm0, conv0)
    print(json.dumps(out), flush=True)


HEAD_METRIC = "Output-head greedy decode frames/s + achieved HBM GB/s (% peak), text + function head"


def head_bytes(wl):
    """Algorithmic HBM bytes of one head GEMV launch (the weights and the hidden states read
    once, the tokens written) and of one frame (every head)."""
    wb = {"f32": 4, "bf16": 2, "int8g": 1, "int4g": 0.5, "int3g": 0.375}[wl.wtype]
    scales = {"int8g": 2, "int4g": 4, "int3g": 4}.get(wl.wtype, 0)
    w = int(wl.vocab * wl.d_model * wb) + (wl.vocab * (wl.d_model // wl.q_group) * scales if scales else 0)
    launch = w + wl.batch * wl.d_model * 4
    return {"head_wave": launch, "frame": wl.heads * (launch + wl.batch * 4)}


def bench_heads(args, wl):
    """Frames/s of the output heads: per frame every head (text, then function) maps each
    session's hidden state to its greedy token; nothing else runs in the timed region."""
    import numpy as np
    import torch
    import ctypes as C
    from full_duplex_speech_mamba2_amd import m2, synth

    dev = torch.device("cuda:0")
    B, K, V = wl.batch, wl.d_model, wl.vocab
    print("[bench] workload %s: generating inputs" % wl.name, file=sys.stderr, flush=True)
    tags = ["text_head", "func_head"][:wl.heads]
    host_w = [synth.make_head_weights(V, K, wl.wtype, wl.q_group, wl.seed, tag) for tag in tags]
    heads = [m2.Head(K, V, w, s, wtype=wl.wtype, q_group=wl.q_group, device=dev) for w, s in host_w]
    nx = min(wl.steps, 750)
    hs_np = synth.make_head_states(K, nx * B, wl.seed).reshape(nx, B, K)
    hs = torch.from_numpy(hs_np).to(dev)
    toks = torch.empty((nx, wl.heads, B), dtype=torch.int32, device=dev)

    def run(t0, n):
        for t in range(t0, t0 + n):
            for i, hd in enumerate(heads):
                hd.argmax(hs[t % nx], token=toks[t % nx, i])

    run(0, args.warmup)
    torch.cuda.synchronize()
    ms_eager, _ = eager_ms_per_step(run, args.warmup, args.steps)
    ms_graph = None
    if not args.no_graph:
        ms_graph, _ = graph_ms_per_step(run, args.steps, 2 * len(heads))
    ms = min(ms_eager, ms_graph) if ms_graph is not None else ms_eager
    fps = 1000.0 / ms

    # per-kernel durations from HIP events between the two kernels of each head call
    kp = max(10, args.prof_steps)
    hip = hip_runtime()
    evs = [[hip_event(hip) for _ in range(3)] for _ in range(kp)]
    tok1 = torch.empty(B, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    hold_gpu(150.0)
    for t in range(kp):
        heads[t % len(heads)].argmax_timed(hs[t % nx], tok1, evs[t])
    torch.cuda.synchronize()
    wave_us = 1000.0 * float(np.mean([hip_elapsed_ms(hip, e[0], e[1]) for e in evs]))
    red_us = 1000.0 * float(np.mean([hip_elapsed_ms(hip, e[1], e[2]) for e in evs]))
    for row in evs:
        for e in row:
            hip.hipEventDestroy(e)
    hb = head_bytes(wl)
    achieved = hb["head_wave"] / (wave_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": "head_wave", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic_for("head_wave", wl.name),
                "algorithmic_bytes": hb["head_wave"], "avg_duration_us": round(wave_us, 2)}
    out = {
        "metric": HEAD_METRIC, "value": round(fps, 1), "unit": "frames/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "d_model": K, "vocab": V, "heads": wl.heads, "batch": B,
                   "weight_dtype": wl.wtype,
                   "timing": "graph" if (ms_graph is not None and ms_graph <= ms_eager) else "eager"},
        "achieved_GBps": round(hb["frame"] * fps / 1e9, 1),
        "hbm_peak_frac": round(hb["frame"] * fps / 1e9 / HBM_PEAK_GBPS, 4),
        "step_algorithmic_bytes": hb["frame"],
        "ms_per_step_eager": round(ms_eager, 5),
        "ms_per_step_graph": None if ms_graph is None else round(ms_graph, 5),
        "kernel_us": {"head_wave": round(wave_us, 2), "head_reduce": round(red_us, 2)},
        "roofline": roofline, "cpu_baseline": None, "parity": None,
    }
    if not args.no_cpu:
        out["cpu_baseline"], out["parity"] = head_cpu_baseline_and_parity(args, wl, host_w, hs_np, toks)
    print(json.dumps(out), flush=True)


def head_cpu_baseline_and_parity(args, wl, host_w, hs_np, toks):
    """Time the oracle on the first frames (bounded by --cpu-seconds) and compare the GPU
    tokens of those frames with its greedy tokens: equal, or within fp32 rounding of a tie."""
    import numpy as np
    import oracle
    gpu = toks.cpu().numpy()
    t0 = time.perf_counter()
    n, same, worst = 0, 0, 0.0
    while n < hs_np.shape[0] and (n < 1 or time.perf_counter() - t0 < args.cpu_seconds):
        for i, (w, s) in enumerate(host_w):
            lo, to = oracle.head_argmax(wl.wtype, w, hs_np[n], s, wl.q_group)
            g = gpu[n, i]
            same += int(np.sum(g == to))
            gap = (lo[np.arange(wl.batch), to] - lo[np.arange(wl.batch), np.maximum(g, 0)]) / np.max(np.abs(lo))
            worst = max(worst, float(np.max(np.where(g < 0, np.inf, gap))))
        n += 1
    wall = time.perf_counter() - t0
    base = {"value": round(n / wall, 4), "unit": "frames/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "first %d frames of %s (%d heads, batch %d), fp64 C oracle, %.1f s wall"
                      % (n, wl.name, wl.heads, wl.batch, wall)}
    total = n * wl.heads * wl.batch
    return base, {"frames": n, "tokens_equal": same, "tokens": total, "worst_rel_logit_gap": worst,
                  "tol_rel_logit_gap": 1e-5, "ok": bool(worst <= 1e-5)}


ATTN_METRIC = "Attention-layer decode steps/s + achieved HBM GB/s (% peak), 9B-shaped layer, bf16 KV cache"
ATTN_PHASES = ["qkv_gemv", "attn_split", "attn_combine", "o_gemv"]


def attn_bytes(wl, mean_len):
    """Algorithmic HBM bytes per launch of each kernel of the attention step and of the whole
    step at a mean of `mean_len` attended positions: weights, cache rows read once, the new
    rows written, activations in and out; the chunk partials are scratch."""
    d, B = wl.dims, wl.batch
    wb = {"f32": 4, "bf16": 2, "int8g": 1, "int4g": 0.5, "int3g": 0.375}[d.wtype]
    scales = {"int8g": 2, "int4g": 4, "int3g": 4}.get(d.wtype, 0)

    def w(rows, K):
        return int(rows * K * wb) + (rows * (K // d.q_group) * scales if scales else 0)

    qkv = w(d.qkv_rows, d.d_model) + B * d.d_model * 4 + B * d.qkv_rows * 4
    cache = int(2 * B * d.n_kv * mean_len * d.head_dim * 2)
    split = B * d.qkv_rows * 4 + cache + 2 * B * d.n_kv * d.head_dim * 2
    combine = B * d.o_dim * 4
    o = w(d.d_model, d.o_dim) + B * d.o_dim * 4 + 2 * B * d.d_model * 4
    step = (w(d.qkv_rows, d.d_model) + w(d.d_model, d.o_dim) + cache + 2 * B * d.n_kv * d.head_dim * 2 +
            2 * B * d.d_model * 4)
    return {"qkv_gemv": qkv, "attn_split": split, "attn_combine": combine, "o_gemv": o, "step": step}


def bench_attn(args, wl):
    """Steps/s of the attention layer: per step one token for `batch` sessions (QKV GEMV, the
    cache append and grouped-query attention over the cached positions, O GEMV + residual)."""
    import numpy as np
    import torch
    from full_duplex_speech_mamba2_amd import m2, synth

    dev = torch.device("cuda:0")
    d, B, S = wl.dims, wl.batch, wl.slot_sets
    print("[bench] workload %s: generating inputs" % wl.name, file=sys.stderr, flush=True)
    w = synth.make_attn_weights(d, wl.seed)
    pos0_np = np.full(B * S, wl.start_pos, np.int32)
    kc_np, vc_np = synth.make_kv_cache(d, wl.seed, pos0_np)
    ncopy = args.copies
    if ncopy <= 0:
        per = attn_bytes(wl, 0)["qkv_gemv"] + attn_bytes(wl, 0)["o_gemv"]
        ncopy = max(2, -(-ROTATION_BYTES // per))
    layers = [m2.Attn(d, w, dev) for _ in range(ncopy)]
    kc = torch.from_numpy(kc_np.view(np.int16)).to(dev)
    vc = torch.from_numpy(vc_np.view(np.int16)).to(dev)
    pos0 = torch.from_numpy(pos0_np).to(dev)
    pos = pos0.clone()
    sets = torch.arange(B * S, dtype=torch.int32, device=dev).reshape(S, B).contiguous()
    xs_np = synth.make_attn_inputs(d, wl.seed, wl.steps, B)
    xs = torch.from_numpy(xs_np).to(dev)
    ys = torch.empty_like(xs)
    ws = layers[0].workspace(B)
    nx, nl = xs.shape[0], len(layers)
    if args.steps // S > d.max_len - wl.start_pos:
        raise SystemExit("--steps %d would fill the caches (at most %d)" % (args.steps, S * (d.max_len - wl.start_pos)))

    def run(t0, n):
        for t in range(t0, t0 + n):
            layers[t % nl].step(kc, vc, pos, xs[t % nx], ys[t % nx], slot_ids=sets[t % S], residual=True, ws=ws)

    run(0, min(args.warmup, S * (d.max_len - wl.start_pos)))
    pos.copy_(pos0)
    torch.cuda.synchronize()
    ms_eager, _ = eager_ms_per_step(run, 0, args.steps, before=lambda: pos.copy_(pos0))
    if not bool(torch.isfinite(ys[:min(nx, args.steps)]).all()):
        raise SystemExit("attention bench: a session ran out of cache positions (NaN outputs)")
    ms_graph = None
    if not args.no_graph:
        ms_graph, _ = graph_ms_per_step(run, args.steps, 4, before_replay=lambda: pos.copy_(pos0))
    ms = min(ms_eager, ms_graph) if ms_graph is not None else ms_eager
    sps = 1000.0 / ms
    mean_len = wl.start_pos + 1 + (args.steps / S - 1) / 2.0

    kp = min(max(10, args.prof_steps), S * (d.max_len - wl.start_pos))
    hip = hip_runtime()
    evs = [[hip_event(hip) for _ in range(5)] for _ in range(kp)]
    pos.copy_(pos0)
    torch.cuda.synchronize()
    hold_gpu(150.0)
    for t in range(kp):
        layers[t % nl].step_timed(kc, vc, pos, xs[t % nx], ys[t % nx], evs[t], slot_ids=sets[t % S], residual=True,
                                  ws=ws)
    torch.cuda.synchronize()
    dur_us = {n: 1000.0 * float(np.mean([hip_elapsed_ms(hip, e[i], e[i + 1]) for e in evs]))
              for i, n in enumerate(ATTN_PHASES)}
    for row in evs:
        for e in row:
            hip.hipEventDestroy(e)
    kb = attn_bytes(wl, mean_len)
    kb_prof = attn_bytes(wl, wl.start_pos + 1 + (kp / S - 1) / 2.0)
    dom = max(ATTN_PHASES, key=lambda n: kb_prof[n])
    achieved = kb_prof[dom] / (dur_us[dom] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic_for(dom, wl.name),
                "algorithmic_bytes": kb_prof[dom], "avg_duration_us": round(dur_us[dom], 2)}
    out = {
        "metric": ATTN_METRIC, "value": round(sps, 1), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "d_model": d.d_model, "n_q": d.n_q, "n_kv": d.n_kv,
                   "head_dim": d.head_dim, "max_len": d.max_len, "batch": B, "weight_dtype": d.wtype,
                   "kv_dtype": "bf16", "start_positions": wl.start_pos, "mean_attended": round(mean_len, 1),
                   "slot_sets": S, "weight_copies": nl,
                   "timing": "graph" if (ms_graph is not None and ms_graph <= ms_eager) else "eager"},
        "achieved_GBps": round(kb["step"] * sps / 1e9, 1),
        "hbm_peak_frac": round(kb["step"] * sps / 1e9 / HBM_PEAK_GBPS, 4),
        "step_algorithmic_bytes": kb["step"],
        "ms_per_step_eager": round(ms_eager, 5),
        "ms_per_step_graph": None if ms_graph is None else round(ms_graph, 5),
        "kernel_us": {n: round(v, 2) for n, v in dur_us.items()},
        "roofline": roofline, "cpu_baseline": None, "parity": None,
    }
    if not args.no_cpu:
        out["cpu_baseline"], out["parity"] = attn_cpu_baseline_and_parity(args, wl, w, kc_np, vc_np, pos0_np, xs_np)
    print(json.dumps(out), flush=True)


def attn_cpu_baseline_and_parity(args, wl, w, kc_np, vc_np, pos0_np, xs_np):
    """Time the oracle on the first steps (bounded by --cpu-seconds) and compare the GPU
    path's outputs for the same steps, from the same caches, with it."""
    import numpy as np
    import torch
    import oracle
    from full_duplex_speech_mamba2_amd import m2
    d, B, S = wl.dims, wl.batch, wl.slot_sets
    lay = oracle.AttnLayer(d, w)
    kc, vc, pos = kc_np.copy(), vc_np.copy(), pos0_np.copy()
    ys_o = []
    t0 = time.perf_counter()
    n = 0
    while n < xs_np.shape[0] and (n < 2 or time.perf_counter() - t0 < args.cpu_seconds):
        ys_o.append(lay.step(kc, vc, pos, xs_np[n], slot_ids=np.arange(B, dtype=np.int32) + (n % S) * B,
                             residual=True))
        n += 1
    wall = time.perf_counter() - t0
    base = {"value": round(n / wall, 3), "unit": "steps/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "first %d steps of %s (batch %d), fp64 C oracle, %.1f s wall" % (n, wl.name, B, wall)}
    at = m2.Attn(d, w)
    kd = torch.from_numpy(kc_np.view(np.int16)).cuda()
    vd = torch.from_numpy(vc_np.view(np.int16)).cuda()
    pd = torch.from_numpy(pos0_np.copy()).cuda()
    xd = torch.from_numpy(xs_np[:n]).cuda()
    yd = torch.empty_like(xd)
    for t in range(n):
        sl = torch.arange(B, dtype=torch.int32, device="cuda") + (t % S) * B
        at.step(kd, vd, pd, xd[t], yd[t], slot_ids=sl, residual=True)
    torch.cuda.synchronize()
    yg = yd.cpu().numpy().astype(np.float64)
    yo = np.array(ys_o)
    e_out = float(np.max(np.max(np.abs(yg - yo), axis=-1) / np.max(np.abs(yo), axis=-1)))
    return base, {"steps": n, "e_out": e_out, "tol_out": 1e-3, "ok": bool(e_out <= 1e-3),
                  "positions_equal": bool(np.array_equal(pd.cpu().numpy(), pos))}


STACK_METRIC = "Hybrid stack decode steps/s + achieved HBM GB/s (% peak), 27 Mamba-2 + 4 attention layers, 9B-shaped"


def bench_stack(args, wl):
    """Steps/s of a hybrid stack stepped by m2_stack_step: per step one token for `batch`
    sessions through every layer of the pattern (residual chain)."""
    import numpy as np
    import torch
    from full_duplex_speech_mamba2_amd import m2, synth

    dev = torch.device("cuda:0")
    B, S = wl.batch, wl.slot_sets
    n_slots = B * S
    print("[bench] workload %s: generating %d layers" % (wl.name, len(wl.pattern)), file=sys.stderr, flush=True)
    pos0_np = np.full(n_slots, wl.start_pos, np.int32)
    entries, pos_list, pos0 = [], [], torch.from_numpy(pos0_np).to(dev)
    for i, k in enumerate(wl.pattern):
        if k == "M":
            lay = m2.Layer(wl.mixer, synth.make_layer_weights(wl.mixer, wl.seed, i), dev)
            entries.append((lay, m2.State(lay, n_slots)))
        else:
            at = m2.Attn(wl.attn, synth.make_attn_weights(wl.attn, wl.seed, i), dev)
            kc, vc = synth.make_kv_cache(wl.attn, wl.seed, pos0_np, i)
            st = (torch.from_numpy(kc.view(np.int16)).to(dev), torch.from_numpy(vc.view(np.int16)).to(dev),
                  pos0.clone())
            pos_list.append(st[2])
            entries.append((at, st))
    stack = m2.Stack(entries, n_slots)
    print("[bench] layers on the device; warming up", file=sys.stderr, flush=True)
    sets = torch.arange(n_slots, dtype=torch.int32, device=dev).reshape(S, B).contiguous()
    xs = torch.from_numpy(synth.make_inputs(wl.mixer, wl.seed, wl.steps, B)).to(dev)
    ys = torch.empty_like(xs)
    persistent = bool(args.persistent)
    runs = stack.persistent_runs(B) if persistent else 0
    if persistent and runs == 0:
        raise SystemExit("--persistent: the persistent stack step does not apply to %s" % wl.name)
    ws = stack.workspace(B, persistent)
    nx = xs.shape[0]
    if args.steps // S > wl.attn.max_len - wl.start_pos:
        raise SystemExit("--steps %d would fill the caches" % args.steps)

    def reset():
        for p_ in pos_list:
            p_.copy_(pos0)

    def run(t0, n):
        for t in range(t0, t0 + n):
            stack.step(xs[t % nx], ys[t % nx], slot_ids=sets[t % S], ws=ws, persistent=persistent)

    run(0, min(args.warmup, S * (wl.attn.max_len - wl.start_pos)))
    reset()
    torch.cuda.synchronize()
    ms_eager, _ = eager_ms_per_step(run, 0, args.steps, before=reset)
    if not bool(torch.isfinite(ys[:min(nx, args.steps)]).all()):
        raise SystemExit("stack bench: non-finite outputs")
    print("[bench] eager %.3f ms/step; capturing graphs" % ms_eager, file=sys.stderr, flush=True)
    ms_graph = None
    if not args.no_graph:
        ms_graph, _ = graph_ms_per_step(run, args.steps, 4 * len(wl.pattern) + 1, before_replay=reset)
    print("[bench] graph %s ms/step" % ms_graph, file=sys.stderr, flush=True)
    ms = min(ms_eager, ms_graph) if ms_graph is not None else ms_eager
    sps = 1000.0 / ms
    mean_len = wl.start_pos + 1 + (args.steps / S - 1) / 2.0
    n_m, n_a = wl.pattern.count("M"), wl.pattern.count("A")
    awl = synth.AttnWorkload(wl.name, wl.attn, B, wl.steps, wl.start_pos, S)
    step_bytes = n_m * kernel_bytes(wl.mixer, B)["step"] + n_a * attn_bytes(awl, mean_len)["step"]

    # per-kernel durations of the first mixer layer, residual as in the stack (HIP events)
    kp = max(10, args.prof_steps)
    hip = hip_runtime()
    evs = [[hip_event(hip) for _ in range(4)] for _ in range(kp)]
    lay0, st0 = entries[0]
    ws = stack.workspace(B)
    torch.cuda.synchronize()
    hold_gpu(150.0)
    for t in range(kp):
        m2.step_timed(lay0, st0, xs[t % nx], ys[t % nx], evs[t], slot_ids=sets[t % S], residual=True, ws=ws)
    torch.cuda.synchronize()
    dur_us = {n: 1000.0 * float(np.mean([hip_elapsed_ms(hip, e[i], e[i + 1]) for e in evs]))
              for i, n in enumerate(PHASES)}
    for row in evs:
        for e in row:
            hip.hipEventDestroy(e)
    kb = kernel_bytes(wl.mixer, B)
    achieved = kb["gemv_in"] / (dur_us["gemv_in"] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": "gemv_in", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic_for("gemv_in", "mamba2_9b_bf16_b1_decode750"),
                "algorithmic_bytes": kb["gemv_in"], "avg_duration_us": round(dur_us["gemv_in"], 2)}
    out = {
        "metric": STACK_METRIC, "value": round(sps, 2), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "pattern": wl.pattern, "mixer_layers": n_m, "attention_layers": n_a,
                   "d_model": wl.mixer.d_model, "batch": B, "weight_dtype": wl.mixer.wtype, "kv_dtype": "bf16",
                   "start_positions": wl.start_pos, "mean_attended": round(mean_len, 1), "slot_sets": S,
                   "persistent_runs": runs,
                   "timing": "graph" if (ms_graph is not None and ms_graph <= ms_eager) else "eager"},
        "achieved_GBps": round(step_bytes * sps / 1e9, 1),
        "hbm_peak_frac": round(step_bytes * sps / 1e9 / HBM_PEAK_GBPS, 4),
        "step_algorithmic_bytes": step_bytes,
        "frame_budget_ms": 80.0,
        "realtime_sessions": round(B * sps * 0.08, 1),
        "ms_per_step_eager": round(ms_eager, 4),
        "ms_per_step_graph": None if ms_graph is None else round(ms_graph, 4),
        "kernel_us_first_mixer": {n: round(v, 2) for n, v in dur_us.items()},
        "roofline": roofline, "cpu_baseline": None, "parity": None,
    }
    print(json.dumps(out), flush=True)


def prefill_flops(dims, B, T, Q):
    """Algorithmic flops of one prefill: the two projections and the chunked scan."""
    d = dims
    proj = 2.0 * B * T * (d.d_in_proj * d.d_model + d.d_model * d.d_inner)
    nch = -(-T // Q)
    cb = 2.0 * B * nch * d.n_groups * Q * Q * d.d_state
    diag = 2.0 * B * nch * d.n_heads * (Q * (Q + 1) / 2) * d.head_dim
    states = 2.0 * B * nch * d.n_heads * Q * d.head_dim * d.d_state
    off = 2.0 * B * nch * d.n_heads * Q * d.d_state * d.head_dim
    return proj, cb + diag + states + off


def time_prefill(args, wl, layer, st, dev):
    """Time m2_prefill of the workload's prompt from a zero state (events around each call)."""
    import numpy as np
    import torch
    from full_duplex_speech_mamba2_amd import m2, synth
    dims, B, T, Q = wl.dims, wl.batch, wl.prefill, wl.chunk
    x = torch.from_numpy(synth.make_prompt(dims, wl.seed, B, T)).to(dev)
    y = torch.empty_like(x)
    ws = layer.workspace("prefill", B, T, Q)
    times = []
    for it in range(5):
        st.zero()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        m2.prefill(layer, st, x, y, chunk=Q, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        if it >= 2:
            times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    proj, scan = prefill_flops(dims, B, T, Q)
    executed = 2 * proj + scan          # hi/lo activations: two MFMAs per projection product
    return {"batch": B, "seqlen": T, "chunk": Q, "ms": round(ms, 4),
            "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "algorithmic_tflop": round((proj + scan) / 1e12, 4),
            "algorithmic_tflops_per_s": round((proj + scan) / (ms * 1e-3) / 1e12, 2),
            "executed_tflops_per_s": round(executed / (ms * 1e-3) / 1e12, 2),
            "mfma_bf16_peak_tflops": 2500.0,
            "workspace_bytes": int(ws.numel())}


def cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def single_thread_oracle(lay, wl, xs_np, ssm0, conv0):
    """The oracle on one thread: the whole tiny workload (16 steps) and one step of this
    workload, each timed once; the thread count is restored afterwards."""
    import numpy as np
    import oracle
    from full_duplex_speech_mamba2_amd import synth
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        tw = synth.workload(0)
        tl = oracle.Layer(tw.dims, synth.make_layer_weights(tw.dims, tw.weight_seed))
        ts, tc = tl.new_state(tw.batch)
        txs = synth.make_inputs(tw.dims, tw.seed, tw.steps, tw.batch)
        t0 = time.perf_counter()
        for t in range(tw.steps):
            tl.step(ts, tc, txs[t])
        tiny = time.perf_counter() - t0
        so, co = lay.new_state(wl.batch, ssm0, conv0)
        t0 = time.perf_counter()
        lay.step(so, co, xs_np[0])
        one = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(threads)
    return {"tiny_16_steps_s": round(tiny, 5), "tiny_steps_per_s": round(tw.steps / tiny, 1),
            "one_step_s": round(one, 4), "steps_per_s": round(1.0 / one, 3), "threads": 1}


def cpu_baseline_and_parity(args, wl, w, xs_np, ssm0, conv0):
    """Time the oracle on the first steps of the workload (bounded by --cpu-seconds) and compare
    the GPU path's outputs for those steps, from the same initial state, with it."""
    import numpy as np
    import torch
    import oracle
    from full_duplex_speech_mamba2_amd import m2
    from full_duplex_speech_mamba2_amd.synth import workload  # noqa: F401

    dims, B = wl.dims, wl.batch
    lay = oracle.Layer(dims, w)
    so, co = lay.new_state(B, ssm0, conv0)
    ys_o = []
    t0 = time.perf_counter()
    n = 0
    while n < xs_np.shape[0] and (n < 2 or time.perf_counter() - t0 < args.cpu_seconds):
        ys_o.append(lay.step(so, co, xs_np[n]))
        n += 1
    wall = time.perf_counter() - t0
    base = {"value": round(n / wall, 3), "unit": "steps/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "first %d decode steps of %s (batch %d), fp64 C oracle, %.1f s wall"
                      % (n, wl.name, B, wall)}
    base["single_thread"] = single_thread_oracle(lay, wl, xs_np, ssm0, conv0)

    gl = m2.Layer(dims, w)
    gs = m2.State(gl, B, torch.from_numpy(ssm0).cuda(), torch.from_numpy(conv0).cuda())
    xd = torch.from_numpy(xs_np[:n]).cuda()
    yd = torch.empty_like(xd)
    for t in range(n):
        m2.step(gl, gs, xd[t], yd[t])
    torch.cuda.synchronize()
    yg = yd.cpu().numpy().astype(np.float64)
    yo = np.array(ys_o)
    e_out = float(np.max(np.max(np.abs(yg - yo), axis=-1) / np.max(np.abs(yo), axis=-1)))
    sg = gs.ssm.cpu().numpy().astype(np.float64)
    floor = 1e-6 * float(np.max(np.abs(so)))
    e_state = float(np.max(np.max(np.abs(sg - so), axis=(-2, -1)) /
                           np.maximum(np.max(np.abs(so), axis=(-2, -1)), floor)))
    return base, {"steps": n, "e_out": e_out, "e_state": e_state, "tol_out": 2e-3, "tol_state": 1e-3,
                  "ok": bool(e_out <= 2e-3 and e_state <= 1e-3)}


if __name__ == "__main__":
    main()
