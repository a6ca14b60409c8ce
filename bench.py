"""Benchmark: fused selective-scan forward (ssm_scan_fwd) on one MI355X.

One step = one ssm_scan_fwd call over the whole Mamba-2.8B-shaped layer
(batch 4, d_inner 5120, N 16, L 2048, bf16 x/dt/z/Bm/Cm, fp32 A/Dskip/dt_bias,
fp32 y and final state), inputs already resident in HBM.  Prints one JSON line:

  value       scan elements (batch*dim*L*N) per second, whole job
  roofline    the dominant (only) kernel against the VALU issue-rate peak it is
              bound by; the algorithmic HBM rate is reported beside it
  cpu_baseline the fp64 CPU oracle on the host cores, same workload
  decode      the 256-step ssm_state_update loop of the decode workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload I]
       [--no-cpu-baseline] [--no-decode]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# ---------------------------------------------------------------- chip model
# MI355X: 256 CUs at 2.4 GHz.  fp32 VALU: 128 lanes/clk/CU (157.3 TFLOP/s with
# FMA = 2 flops) = 78.6 T lane-op issue slots/s.  Transcendentals (exp2, log2,
# rcp) issue at a quarter of that rate, i.e. 4 slots each.  HBM3E: 8 TB/s.
CUS, CLOCK_HZ = 256, 2.4e9
PEAK_SLOTS = CUS * 128 * CLOCK_HZ          # 7.864e13 fp32 lane-op slots / s
TRANS_SLOTS = 4
PEAK_HBM = 8.0e12                          # B/s

# Algorithmic work (the method's minimum, no scan overhead):
#  per (b,d,l,n): Delta*A (1), exp (4), Delta*x*B (1), state fma (1), readout fma (1)
#  per (b,d,l):   dt + bias (1), softplus = exp + add + log (9), Delta*x (1),
#                 skip fma (1), silu = exp + add + rcp + mul (10), gate mul (1)
SLOTS_PER_ELEM = 1 + TRANS_SLOTS + 1 + 1 + 1
SLOTS_PER_ROW_STEP = 1 + (TRANS_SLOTS + 1 + TRANS_SLOTS) + 1 + 1 + (TRANS_SLOTS + 1 + TRANS_SLOTS + 1) + 1


COUNTERS = os.path.join(ROOT, "profiles", "scan_fwd_counters.json")
KERNEL_SOURCES = ("selective_state_space_64_amd/csrc/scan_fwd.hip",
                  "selective_state_space_64_amd/csrc/scan_common.hpp",
                  "selective_state_space_64_amd/csrc/ssm_device.hpp")


def counter_traffic(workload_name):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE
    summary, or None when it was taken on other kernel sources or another
    workload."""
    try:
        with open(COUNTERS) as f:
            rec = json.load(f)
        digest = kernel_sources_sha256()
    except OSError:
        return None
    if rec.get("kernel_sources_sha256") != digest or rec.get("workload") != workload_name:
        return None
    return rec["traffic_bytes_per_launch"]


def kernel_sources_sha256():
    h = hashlib.sha256()
    for src in KERNEL_SOURCES:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


SCAN_KERNEL = "scan_fwd_kernel<ssm::bf16_t, float, 16, 8, false, false, false, true>"


def ingest_counters(fetch_dir, write_dir, copyf_dir, copyw_dir, copy_mib=256, workload=None):
    """Per-dispatch mean of FETCH_SIZE / WRITE_SIZE (KiB) for the scan kernel,
    scaled by what the same counters read for a plain device copy of copy_mib
    MiB, written with the hash of the kernel sources they were taken on."""
    import csv

    def mean(d, counter, kernel):
        vals = []
        for root, _, files in os.walk(d):
            for f in files:
                if f.endswith("counter_collection.csv"):
                    with open(os.path.join(root, f)) as fh:
                        for r in csv.DictReader(fh):
                            if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
                                vals.append(float(r["Counter_Value"]))
        if not vals:
            raise SystemExit("no %s samples for %s under %s" % (counter, kernel, d))
        return sum(vals) / len(vals)

    copy_kib = copy_mib * 1024.0
    fetch = mean(fetch_dir, "FETCH_SIZE", SCAN_KERNEL)
    write = mean(write_dir, "WRITE_SIZE", SCAN_KERNEL)
    cf = mean(copyf_dir, "FETCH_SIZE", "copyBuffer")
    cw = mean(copyw_dir, "WRITE_SIZE", "copyBuffer")
    fs, ws = copy_kib / cf, copy_kib / cw
    rec = {
        "kernel": SCAN_KERNEL,
        "workload": workload,
        "kernel_sources_sha256": kernel_sources_sha256(),
        "fetch_size_kib_per_dispatch": fetch,
        "write_size_kib_per_dispatch": write,
        "copy_calibration": {"bytes_each_way": int(copy_kib * 1024), "fetch_size_kib": cf,
                             "write_size_kib": cw, "fetch_scale": fs, "write_scale": ws},
        "read_bytes_per_launch": fetch * fs * 1024,
        "write_bytes_per_launch": write * ws * 1024,
        "traffic_bytes_per_launch": (fetch * fs + write * ws) * 1024,
    }
    with open(COUNTERS, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def algorithmic_slots(batch, dim, L, N):
    return batch * dim * L * (N * SLOTS_PER_ELEM + SLOTS_PER_ROW_STEP)


def algorithmic_bytes(batch, dim, L, N, in_bytes, out_bytes, gate=True):
    per_row_step = (3 if gate else 2) * in_bytes + out_bytes          # x, dt, (z) in; y out
    bc = 2 * batch * N * L * in_bytes                                 # Bm, Cm
    params = dim * N * 4 + 2 * dim * 4                                # A, Dskip, dt_bias
    state = batch * dim * N * 4                                       # hL out
    return batch * dim * L * per_row_step + bc + params + state


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="before the W warm-up steps, run the step for at least this long "
                         "(untimed): the GPU's clocks ramp up under sustained load, and a "
                         "cold first second reads 10-20%% slower than steady state")
    ap.add_argument("--workload", type=int, default=2, help="index into synth.WORKLOADS")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPYF_DIR", "COPYW_DIR"),
                    help="write profiles/scan_fwd_counters.json from four rocprofv3 --pmc output "
                         "directories (scan FETCH_SIZE, scan WRITE_SIZE, copy FETCH_SIZE, copy "
                         "WRITE_SIZE; csv output) and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times) and exit; "
                         "used to scale the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def to_dev(inp, name):
    import torch
    a = getattr(inp, name)
    if name in inp.stored and inp.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def cpu_baseline(inp, block=512, min_seconds=10.0):
    """The fp64 oracle as it stands, on all host cores, over whole passes of the
    workload (channel blocks bound host memory), repeated until about
    min_seconds of oracle time have been measured."""
    import oracle
    wl = inp.wl
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    A, Dk, bias = (inp.A.astype(np.float64), inp.Dskip.astype(np.float64),
                   inp.dt_bias.astype(np.float64))
    Bm, Cm = inp.values("Bm"), inp.values("Cm")
    blocks = []
    for d0 in range(0, wl.dim, block):
        d1 = min(wl.dim, d0 + block)
        blocks.append((d0, d1, synth_vals(inp, "x", d0, d1), synth_vals(inp, "dt", d0, d1),
                       synth_vals(inp, "z", d0, d1)))
    elapsed, passes = 0.0, 0
    while passes == 0 or elapsed < min_seconds:
        for d0, d1, x, dt, z in blocks:
            t0 = time.perf_counter()
            oracle.scan_fwd(x, dt, A[d0:d1], Bm, Cm, dt_bias=bias[d0:d1], Dskip=Dk[d0:d1], z=z,
                            threads=threads)
            elapsed += time.perf_counter() - t0
        passes += 1
    elems = wl.batch * wl.dim * wl.seqlen * wl.dstate * passes
    return {"value": elems / elapsed, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": "%d passes over the whole workload (%d x %d x %d x %d), fp64 sequential "
                      "recurrence, %.2f s" % (passes, wl.batch, wl.dim, wl.seqlen, wl.dstate, elapsed)}


def synth_vals(inp, name, d0, d1):
    from selective_state_space_64_amd import synth
    a = getattr(inp, name)[:, d0:d1]
    if inp.dtype == "bf16":
        return synth.bf16_values(a).astype(np.float64)
    return a.astype(np.float64)


def bench_decode(torch, ssm, synth, steps_cap=256):
    wl = synth.WORKLOADS[4]
    inp = synth.make_inputs(wl)
    perm = lambda t: t.permute(2, 0, 1).contiguous()
    xs, dts, zs = perm(to_dev(inp, "x")), perm(to_dev(inp, "dt")), perm(to_dev(inp, "z"))
    Bs, Cs = perm(to_dev(inp, "Bm")), perm(to_dev(inp, "Cm"))
    A, Dk, bias = to_dev(inp, "A"), to_dev(inp, "Dskip"), to_dev(inp, "dt_bias")
    state0 = torch.from_numpy(inp.h0).cuda()
    state = state0.clone()
    ys = torch.empty((wl.seqlen, wl.batch, wl.dim), device="cuda")
    steps = min(steps_cap, wl.seqlen)

    def loop():
        for s in range(steps):
            ssm.ssm_state_update(state, xs[s], dts[s], A, Bs[s], Cs[s], dt_bias=bias, Dskip=Dk,
                                 z=zs[s], y=ys[s])

    loop()
    state.copy_(state0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    loop()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps

    # the same loop captured once in a HIP graph and replayed (no launch
    # overhead per token); checked against the eager loop before timing
    ref_state, ref_y = state.clone(), ys[:steps].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        state.copy_(state0)
        loop()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    state.copy_(state0)
    with torch.cuda.graph(graph):
        loop()
    state.copy_(state0)
    graph.replay()
    torch.cuda.synchronize()
    graph_ok = bool(torch.equal(state, ref_state) and torch.equal(ys[:steps], ref_y))
    state.copy_(state0)
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / steps
    per_call_bytes = (2 * wl.batch * wl.dim * wl.dstate * 4 + 3 * wl.batch * wl.dim * 2
                      + 2 * wl.batch * wl.dstate * 2 + wl.dim * wl.dstate * 4 + 2 * wl.dim * 4
                      + wl.batch * wl.dim * 4)
    elems = wl.batch * wl.dim * wl.dstate
    return {"workload": wl.name, "calls": steps, "us_per_call": ms * 1e3,
            "elements_per_s": elems / (ms * 1e-3),
            "hbm_gbps_algorithmic": per_call_bytes / (ms * 1e-3) / 1e9,
            "bytes_per_call": per_call_bytes,
            "graph_us_per_call": graph_ms * 1e3, "graph_matches_eager": graph_ok,
            "graph_hbm_gbps_algorithmic": per_call_bytes / (graph_ms * 1e-3) / 1e9,
            "roofline": {"bound": "hbm", "achieved": per_call_bytes / (graph_ms * 1e-3) / 1e9,
                         "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                         "frac": per_call_bytes / (graph_ms * 1e-3) / PEAK_HBM, "traffic": None,
                         "algorithmic_bytes": per_call_bytes,
                         "timing": "per step of the graph replay (launch gaps included)"},
            "note": "one launch per token, state fp32 in place; 21 MB state can stay in the 256 MB MALL"}


def bench_conv(torch, ssm, synth, wl, x, launches=20):
    """Causal depthwise conv (W 4, silu, bf16 in and out) over the layer's x,
    and its decode step on the decode workload's shape; HBM-bound."""
    w, b = synth.conv_parameters(wl, 4)
    wt, bt = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        ssm.ssm_conv1d_fwd(x, wt, bias=bt, y=y, return_final_state=False)
    # launches back to back between two events (the roofline's time base),
    # then events around each launch for the per-launch mean
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    for _ in range(launches):
        ssm.ssm_conv1d_fwd(x, wt, bias=bt, y=y, return_final_state=False)
    r1.record(stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(launches)]
    for e0, e1 in evs:
        e0.record(stream)
        ssm.ssm_conv1d_fwd(x, wt, bias=bt, y=y, return_final_state=False)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = r0.elapsed_time(r1) / launches
    per_launch = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    nbytes = 2 * x.numel() * x.element_size() + wl.dim * 5 * 4
    achieved = nbytes / (ms * 1e-3)
    out = {"workload": "conv1d W4 silu, %s" % wl.name, "kernel_ms_mean": ms,
           "per_launch_events_ms_mean": per_launch,
           "outputs_per_s": x.numel() / (ms * 1e-3),
           "roofline": {"bound": "hbm", "achieved": achieved / 1e9, "peak": PEAK_HBM / 1e9,
                        "unit": "GB/s", "frac": achieved / PEAK_HBM, "traffic": None,
                        "algorithmic_bytes": nbytes,
                        "model": "x read once (2 B) + y written once (2 B) per output, plus taps"}}
    dwl = synth.WORKLOADS[4]
    state = torch.zeros((dwl.batch, dwl.dim, 3), device="cuda")
    xs = torch.randn((64, dwl.batch, dwl.dim), device="cuda").to(torch.bfloat16)
    ys = torch.empty((64, dwl.batch, dwl.dim), device="cuda", dtype=torch.bfloat16)
    wd, bd = synth.conv_parameters(dwl, 4)
    wd, bd = torch.from_numpy(wd).cuda(), torch.from_numpy(bd).cuda()
    for s in range(8):
        ssm.ssm_conv1d_update(state, xs[s], wd, bias=bd, y=ys[s])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(64):
        ssm.ssm_conv1d_update(state, xs[s], wd, bias=bd, y=ys[s])
    e1.record(stream)
    torch.cuda.synchronize()
    out["decode_us_per_call"] = e0.elapsed_time(e1) / 64 * 1e3
    out["decode_workload"] = "conv1d update W4, batch %d dim %d" % (dwl.batch, dwl.dim)
    return out


BWD_SLOTS_PER_ELEM = 17      # recompute 8 + adjoint 2 + dBm, dCm 2 + dA 3 + dx/dDelta sums 2
BWD_SLOTS_PER_ROW_STEP = 40  # softplus 9, sigmoid(u) 9, silu + silu' 14, gradient assembly 8


def bench_bwd(torch, ssm, wl, t, launches=10):
    """Backward pass (all launches of one ssm_scan_bwd call: checkpoint
    recompute, zero-fill, reverse pass, sum of partial copies) on the layer,
    dy ~ N(0, 1) fp32, gradients fp32, outputs and workspace preallocated;
    also in training order after a forward that writes the checkpoints, and
    for the exact zero-order-hold form."""
    dy = torch.randn((wl.batch, wl.dim, wl.seqlen), device="cuda")
    ws = torch.empty(ssm.lib().ssm_scan_bwd_workspace_bytes(wl.batch, wl.dim, wl.seqlen, wl.dstate),
                     dtype=torch.uint8, device="cuda")
    L = ssm.lib()
    f32 = torch.float32
    g = {k: torch.empty(shape, dtype=f32, device="cuda") for k, shape in (
        ("dx", (wl.batch, wl.dim, wl.seqlen)), ("ddt", (wl.batch, wl.dim, wl.seqlen)),
        ("dz", (wl.batch, wl.dim, wl.seqlen)), ("dBm", (wl.batch, wl.dstate, wl.seqlen)),
        ("dCm", (wl.batch, wl.dstate, wl.seqlen)), ("dA", (wl.dim, wl.dstate)),
        ("dDskip", (wl.dim,)), ("ddt_bias", (wl.dim,)))}
    stream = torch.cuda.current_stream()
    ptr = lambda k: t[k].data_ptr()

    ind = 1 if wl.dtype == "bf16" else 0

    def call(flags=0):
        st = L.ssm_scan_bwd(wl.batch, wl.dim, wl.seqlen, wl.dstate, ind, flags, ptr("x"), ptr("dt"),
                            ptr("dt_bias"), ptr("A"), ptr("Bm"), ptr("Cm"), ptr("Dskip"), ptr("z"),
                            None, 0, dy.data_ptr(), None, g["dx"].data_ptr(), g["ddt"].data_ptr(),
                            g["dz"].data_ptr(), g["dBm"].data_ptr(), g["dCm"].data_ptr(),
                            g["dA"].data_ptr(), g["dDskip"].data_ptr(), g["ddt_bias"].data_ptr(),
                            None, ws.data_ptr(), ws.numel(), stream.cuda_stream)
        if st != 0:
            raise RuntimeError("ssm_scan_bwd failed with status %d" % st)

    def timed(fn):
        # calls back to back between two events on the launch stream
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / launches

    ms = timed(call)
    # training order: the forward writes the checkpoints (SSM_FLAG_CHECKPOINTS)
    # into the backward's workspace, the backward reads them
    y = torch.empty((wl.batch, wl.dim, wl.seqlen), device="cuda")

    def fwd_ckpt():
        st = L.ssm_scan_fwd(wl.batch, wl.dim, wl.seqlen, wl.dstate, ind, 2, ptr("x"), ptr("dt"),
                            ptr("dt_bias"), ptr("A"), ptr("Bm"), ptr("Cm"), ptr("Dskip"), ptr("z"),
                            None, 0, y.data_ptr(), None, ws.data_ptr(), ws.numel(),
                            stream.cuda_stream)
        if st != 0:
            raise RuntimeError("ssm_scan_fwd failed with status %d" % st)

    fwd_ckpt_ms = timed(fwd_ckpt)
    fwd_ckpt()
    bwd_ckpt_ms = timed(lambda: call(2))
    zoh_ms = timed(lambda: call(1))  # SSM_FLAG_ZOH_B, checkpoints recomputed
    elems = wl.batch * wl.dim * wl.seqlen * wl.dstate
    slots = elems * BWD_SLOTS_PER_ELEM + wl.batch * wl.dim * wl.seqlen * BWD_SLOTS_PER_ROW_STEP
    achieved = slots / (ms * 1e-3) / 1e12
    return {"workload": "scan backward, %s" % wl.name, "ms_mean": ms,
            "elements_per_s": elems / (ms * 1e-3),
            "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_SLOTS / 1e12,
                         "unit": "TOP/s", "frac": achieved / (PEAK_SLOTS / 1e12), "traffic": None,
                         "model": "fp32 VALU issue slots (transcendental = 4), %.2f slots/element"
                                  % (slots / elems)},
            "with_forward_checkpoints": {"forward_ms": fwd_ckpt_ms, "backward_ms": bwd_ckpt_ms},
            "zoh_ms_mean": zoh_ms,
            "note": "checkpoint recompute + zero-fill + reverse pass + partial-copy sum; "
                    "with_forward_checkpoints: the forward writes the checkpoints and the "
                    "backward skips its recomputation pass; zoh: the exact zero-order-hold "
                    "form of B-bar"}


def main():
    args = parse()
    if args.ingest_counters:
        from selective_state_space_64_amd import synth
        rec = ingest_counters(*args.ingest_counters, workload=synth.WORKLOADS[args.workload].name)
        print(json.dumps(rec))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the scan is benchmarked on a single device, "
              "and runs over several GPUs are not part of this library (--gpus %d is not "
              "supported)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    import selective_state_space_64_amd as ssm
    from selective_state_space_64_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n * 4, "launches": 3}), flush=True)
        return
    wl = synth.WORKLOADS[args.workload]
    inp = synth.make_inputs(wl)
    t = {k: to_dev(inp, k) for k in ("x", "dt", "z", "Bm", "Cm", "A", "Dskip", "dt_bias")}
    y = torch.empty((wl.batch, wl.dim, wl.seqlen), device="cuda")
    hL = torch.empty((wl.batch, wl.dim, wl.dstate), device="cuda")

    def step():
        ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                         Dskip=t["Dskip"], z=t["z"], y=y, hL=hL)

    t_end = time.perf_counter() + args.warmup_seconds
    while time.perf_counter() < t_end:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # The timed region: K steps back to back between two HIP events on the
    # launch stream (their mean is the kernel's average launch duration, the
    # roofline's time base); the wall clock around it gives ms_per_step.
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record(stream)
    for _ in range(args.steps):
        step()
    r1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = r0.elapsed_time(r1) / args.steps
    # the spread per launch, from events around each launch of a second loop
    # (the event packets between launches add about a microsecond each)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    launch_ms = np.array([a.elapsed_time(b) for a, b in evs])
    ms_step = wall * 1e3 / args.steps
    kern_s = region_ms * 1e-3
    elems = wl.batch * wl.dim * wl.seqlen * wl.dstate
    in_bytes = 2 if wl.dtype == "bf16" else 4
    slots = algorithmic_slots(wl.batch, wl.dim, wl.seqlen, wl.dstate)
    nbytes = algorithmic_bytes(wl.batch, wl.dim, wl.seqlen, wl.dstate, in_bytes, 4)
    achieved = slots / kern_s / 1e12
    peak = PEAK_SLOTS / 1e12
    result = {
        "metric": "selective-scan elems/s (B·D·L·N) fwd + achieved HBM GB/s, 1 MI355X",
        "value": elems / (ms_step * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "dim": wl.dim, "dstate": wl.dstate,
                   "seqlen": wl.seqlen, "input_dtype": wl.dtype, "output_dtype": "f32",
                   "parallelism": "single GPU"},
        "kernel_ms": {"mean": region_ms, "timing": "K launches back to back between two events",
                      "per_launch_mean": float(launch_ms.mean()), "per_launch_min": float(launch_ms.min()),
                      "per_launch_median": float(np.median(launch_ms)),
                      "per_launch_p90": float(np.percentile(launch_ms, 90))},
        "hbm_gbps_algorithmic": nbytes / kern_s / 1e9,
        "roofline": {"bound": "alu", "achieved": achieved, "peak": peak, "unit": "TOP/s",
                     "frac": achieved / peak, "traffic": counter_traffic(wl.name),
                     "model": "fp32 VALU issue slots (transcendental = 4), %.4f slots/element algorithmic"
                              % (slots / elems),
                     "hbm": {"achieved": nbytes / kern_s / 1e9, "peak": PEAK_HBM / 1e9,
                             "unit": "GB/s", "frac": nbytes / kern_s / PEAK_HBM,
                             "algorithmic_bytes": nbytes}},
    }
    # exact zero-order-hold B-bar variant of the same step (SSM_FLAG_ZOH_B)
    for _ in range(2):
        ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                         Dskip=t["Dskip"], z=t["z"], y=y, hL=hL, zoh=True)
    z0, z1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    z0.record(stream)
    for _ in range(10):
        ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                         Dskip=t["Dskip"], z=t["z"], y=y, hL=hL, zoh=True)
    z1.record(stream)
    torch.cuda.synchronize()
    zms = z0.elapsed_time(z1) / 10
    result["zoh_variant"] = {"kernel_ms_mean": zms, "elements_per_s": elems / (zms * 1e-3)}
    if not args.no_decode:
        result["decode"] = bench_decode(torch, ssm, synth)
        result["conv1d"] = bench_conv(torch, ssm, synth, wl, t["x"])
        result["backward"] = bench_bwd(torch, ssm, wl, t)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
