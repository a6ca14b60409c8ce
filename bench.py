"""Benchmark: fused selective-scan forward (ssm_scan_fwd) on one MI355X.

One step = one ssm_scan_fwd call over the whole Mamba-2.8B-shaped layer
(batch 4, d_inner 5120, N 16, L 2048, bf16 x/dt/z/Bm/Cm, fp32 A/Dskip/dt_bias,
fp32 y and final state), inputs already resident in HBM.  Prints one JSON line:

  value        scan elements (batch*dim*L*N) per second, whole job
  roofline     the step's kernel against its binding roof (the fp32 VALU issue
               rate here; the HBM view beside it), algorithmic work / kernel time
  configs      the other scan workloads (tiny, Mamba-130M layer, 2^20-step
               sequence), each with kernel time, elements/s and its own roofline
  cache        the same launches timed with a 512 MiB write before each one
               (L2 and the 256 MB MALL flushed) against the warm figure
  peaks        the chip's issue rates measured by a probe kernel, beside the
               nominal ones the rooflines use
  decode       the ssm_state_update step of the decode workload: a state
               rotating over 16 buffers (336 MB, past the MALL) in a HIP graph,
               the single cached state, and an eager per-token loop
  cpu_baseline the fp64 CPU oracle on the host cores, same workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload I]
       [--no-configs] [--no-cpu-baseline] [--no-decode] [--no-peaks]
"""
import argparse
import hashlib
import json
import os
import platform
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
FLUSH_BYTES = 512 << 20                    # > the 256 MB MALL and every L2

COUNTERS = os.path.join(ROOT, "profiles", "scan_fwd_counters.json")
KERNEL_SOURCES = ("selective_state_space_64_amd/csrc/scan_fwd.hip",
                  "selective_state_space_64_amd/csrc/scan_common.hpp",
                  "selective_state_space_64_amd/csrc/ssm_device.hpp")


def scan_kernel_name(in_dtype, agg=False):
    """The scan kernel's instantiation for a workload (rocprofv3 prints it in
    the kernel name): Tin, Tout, N, K, kZoh, kCkpt, kAgg, kOut.  The split's
    aggregate pass folds 16 steps per lane, the main pass 8."""
    tin = "ssm::bf16_t" if in_dtype == "bf16" else "float"
    return "scan_fwd_kernel<%s, float, 16, %d, false, false, %s, true>" % (
        tin, 16 if agg else 8, "true" if agg else "false")


SCAN_KERNEL = scan_kernel_name("bf16")


def kernel_sources_sha256():
    h = hashlib.sha256()
    for src in KERNEL_SOURCES:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _load_counters():
    try:
        with open(COUNTERS) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return {}
    return rec if isinstance(rec, dict) else {}


def counter_traffic(workload_name):
    """HBM bytes per step from the committed FETCH_SIZE / WRITE_SIZE summary
    for this workload, or None when none was taken or it was taken on other
    kernel sources."""
    rec = _load_counters().get(workload_name)
    if not rec:
        return None
    try:
        digest = kernel_sources_sha256()
    except OSError:
        return None
    if rec.get("kernel_sources_sha256") != digest:
        return None
    return rec["traffic_bytes_per_launch"]


def ingest_counters(fetch_dir, write_dir, copyf_dir, copyw_dir, copy_mib=256, workload=None,
                    kernels=(SCAN_KERNEL,)):
    """Per-dispatch means of FETCH_SIZE / WRITE_SIZE (KiB) for each kernel of
    one step (summed over the kernels), scaled by what the same counters read
    for a plain device copy of copy_mib MiB, stored under the workload's name
    with the hash of the kernel sources they were taken on."""
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
    fetch = {k: mean(fetch_dir, "FETCH_SIZE", k) for k in kernels}
    write = {k: mean(write_dir, "WRITE_SIZE", k) for k in kernels}
    cf = mean(copyf_dir, "FETCH_SIZE", "copyBuffer")
    cw = mean(copyw_dir, "WRITE_SIZE", "copyBuffer")
    fs, ws = copy_kib / cf, copy_kib / cw
    f_tot, w_tot = sum(fetch.values()), sum(write.values())
    rec = {
        "kernels": list(kernels),
        "workload": workload,
        "kernel_sources_sha256": kernel_sources_sha256(),
        "fetch_size_kib_per_dispatch": fetch,
        "write_size_kib_per_dispatch": write,
        "copy_calibration": {"bytes_each_way": int(copy_kib * 1024), "fetch_size_kib": cf,
                             "write_size_kib": cw, "fetch_scale": fs, "write_scale": ws},
        "read_bytes_per_launch": f_tot * fs * 1024,
        "write_bytes_per_launch": w_tot * ws * 1024,
        "traffic_bytes_per_launch": (f_tot * fs + w_tot * ws) * 1024,
    }
    allrec = _load_counters()
    allrec[workload] = rec
    with open(COUNTERS, "w") as f:
        json.dump(allrec, f, indent=1)
    return rec


def algorithmic_slots(batch, dim, L, N):
    return batch * dim * L * (N * SLOTS_PER_ELEM + SLOTS_PER_ROW_STEP)


def algorithmic_bytes(batch, dim, L, N, in_bytes, out_bytes, gate=True):
    per_row_step = (3 if gate else 2) * in_bytes + out_bytes          # x, dt, (z) in; y out
    bc = 2 * batch * N * L * in_bytes                                 # Bm, Cm
    params = dim * N * 4 + 2 * dim * 4                                # A, Dskip, dt_bias
    state = batch * dim * N * 4                                       # hL out
    return batch * dim * L * per_row_step + bc + params + state


def roofline(batch, dim, L, N, in_bytes, seconds, traffic=None):
    """Both roofs for one forward step of `seconds`; `bound` is the one whose
    minimum time is the larger (the binding roof), and the top-level fields
    are that roof's."""
    slots = algorithmic_slots(batch, dim, L, N)
    nbytes = algorithmic_bytes(batch, dim, L, N, in_bytes, 4)
    alu = {"achieved": slots / seconds / 1e12, "peak": PEAK_SLOTS / 1e12, "unit": "TOP/s",
           "frac": slots / seconds / PEAK_SLOTS, "min_seconds": slots / PEAK_SLOTS,
           "model": "fp32 VALU issue slots (transcendental = 4), %.4f slots/element algorithmic"
                    % (slots / (batch * dim * L * N))}
    hbm = {"achieved": nbytes / seconds / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
           "frac": nbytes / seconds / PEAK_HBM, "min_seconds": nbytes / PEAK_HBM,
           "algorithmic_bytes": nbytes}
    if alu["min_seconds"] >= hbm["min_seconds"]:
        out = {"bound": "alu", **{k: alu[k] for k in ("achieved", "peak", "unit", "frac")},
               "traffic": traffic, "model": alu["model"], "hbm": hbm}
    else:
        out = {"bound": "hbm", **{k: hbm[k] for k in ("achieved", "peak", "unit", "frac")},
               "traffic": traffic, "algorithmic_bytes": nbytes, "alu": alu}
    return out


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="before the W warm-up steps, run the step for at least this long "
                         "(untimed): the GPU's clocks ramp up under sustained load, and a "
                         "cold first second reads 10-20%% slower than steady state")
    ap.add_argument("--workload", type=int, default=2, help="index into synth.WORKLOADS")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other scan workloads (tiny, 130M layer, long sequence)")
    ap.add_argument("--configs", default="0,1,3",
                    help="comma-separated synth.WORKLOADS indices measured beside the step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPYF_DIR", "COPYW_DIR"),
                    help="store the --workload's FETCH_SIZE / WRITE_SIZE in "
                         "profiles/scan_fwd_counters.json from four rocprofv3 --pmc output "
                         "directories (scan FETCH_SIZE, scan WRITE_SIZE, copy FETCH_SIZE, copy "
                         "WRITE_SIZE; csv output) and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times) and exit; "
                         "used to scale the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--only-backward", action="store_true",
                    help="time only ssm_scan_bwd on --workload (for profiler passes)")
    ap.add_argument("--only-workload", action="store_true",
                    help="time only --workload (for profiling one configuration) and exit")
    return ap.parse_args(argv)


def to_dev(inp, name):
    import torch
    a = getattr(inp, name)
    if name in inp.stored and inp.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def host_threads():
    return len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()


def cpu_baseline(inp, block=512, min_seconds=10.0, threads=None):
    """The fp64 oracle as it stands, on all host cores, over whole passes of the
    workload (channel blocks bound host memory), repeated until about
    min_seconds of oracle time have been measured."""
    import oracle
    wl = inp.wl
    threads = threads or host_threads()
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
            "cpu_model": cpu_model(),
            "sample": "%d passes over the whole workload (%d x %d x %d x %d), fp64 sequential "
                      "recurrence, %.2f s" % (passes, wl.batch, wl.dim, wl.seqlen, wl.dstate, elapsed)}


def cpu_single_thread(synth, wl, channels=48, min_seconds=4.0):
    """The oracle on one thread over the first `channels` channels of every
    batch row of a workload (its elements/s: rows are independent, so the
    whole workload takes elements / rate seconds on one core)."""
    import dataclasses
    import oracle
    sub = dataclasses.replace(wl, dim=channels)
    inp = synth.make_inputs(sub)
    A, Dk, bias = (inp.A.astype(np.float64), inp.Dskip.astype(np.float64),
                   inp.dt_bias.astype(np.float64))
    args = [inp.values(k) for k in ("x", "dt", "Bm", "Cm", "z")]
    elapsed, passes = 0.0, 0
    while passes == 0 or elapsed < min_seconds:
        t0 = time.perf_counter()
        oracle.scan_fwd(args[0], args[1], A, args[2], args[3], dt_bias=bias, Dskip=Dk, z=args[4],
                        threads=1)
        elapsed += time.perf_counter() - t0
        passes += 1
    elems = sub.batch * sub.dim * sub.seqlen * sub.dstate * passes
    rate = elems / elapsed
    return {"value": rate, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "workload": wl.name,
            "whole_workload_seconds": wl.batch * wl.dim * wl.seqlen * wl.dstate / rate,
            "sample": "%d passes over %d x %d x %d x %d (the first %d channels of every batch "
                      "row), %.2f s" % (passes, sub.batch, sub.dim, sub.seqlen, sub.dstate,
                                        channels, elapsed)}


def synth_vals(inp, name, d0, d1):
    from selective_state_space_64_amd import synth
    a = getattr(inp, name)[:, d0:d1]
    if inp.dtype == "bf16":
        return synth.bf16_values(a).astype(np.float64)
    return a.astype(np.float64)


class Flusher:
    """Writes a FLUSH_BYTES buffer: afterwards no input of the next launch is
    left in the L2 caches or the MALL."""

    def __init__(self, torch):
        self.buf = torch.empty(FLUSH_BYTES // 4, device="cuda")

    def __call__(self):
        self.buf.fill_(1.0)


def time_launches(torch, fn, launches, stream, flusher=None):
    """(ms back to back between two events, per-launch event times) on `stream`;
    with a flusher, only per-launch times, each launch after a flush."""
    E = lambda: torch.cuda.Event(enable_timing=True)
    region = None
    if flusher is None:
        r0, r1 = E(), E()
        r0.record(stream)
        for _ in range(launches):
            fn()
        r1.record(stream)
    evs = [(E(), E()) for _ in range(launches)]
    for a, b in evs:
        if flusher is not None:
            flusher()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    if flusher is None:
        region = r0.elapsed_time(r1) / launches
    return region, np.array([a.elapsed_time(b) for a, b in evs])


def measure_scan(torch, ssm, synth, wl, launches, flusher, warmup_seconds=0.5, warmup=3):
    """One workload's forward: kernel time (launches back to back), the spread
    per launch, the same with a cache flush before each launch, and the
    rooflines.  Inputs come from the seeded generator the parity tests use."""
    t0 = time.perf_counter()
    inp = synth.make_inputs(wl)
    t = {k: to_dev(inp, k) for k in ("x", "dt", "z", "Bm", "Cm", "A", "Dskip", "dt_bias")}
    del inp
    gen_s = time.perf_counter() - t0
    y = torch.empty((wl.batch, wl.dim, wl.seqlen), device="cuda")
    hL = torch.empty((wl.batch, wl.dim, wl.dstate), device="cuda")
    need = ssm.lib().ssm_scan_fwd_workspace_bytes(wl.batch, wl.dim, wl.seqlen, wl.dstate)
    ws = torch.empty(max(1, need), dtype=torch.uint8, device="cuda")

    def step():
        ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                         Dskip=t["Dskip"], z=t["z"], y=y, hL=hL, workspace=ws)

    step()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + warmup_seconds
    while time.perf_counter() < t_end:
        step()
        torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    wall0 = time.perf_counter()
    region, per = time_launches(torch, step, launches, stream)
    wall = time.perf_counter() - wall0
    _, cold = time_launches(torch, step, max(3, launches // 2), stream, flusher)
    in_bytes = 2 if wl.dtype == "bf16" else 4
    elems = wl.batch * wl.dim * wl.seqlen * wl.dstate
    rf = roofline(wl.batch, wl.dim, wl.seqlen, wl.dstate, in_bytes, region * 1e-3,
                  counter_traffic(wl.name))
    split = need > 0
    out = {
        "workload": wl.name,
        "kernel_ms": {"mean": region, "timing": "%d launches back to back between two events"
                                                % launches,
                      "per_launch_mean": float(per.mean()), "per_launch_min": float(per.min()),
                      "per_launch_median": float(np.median(per)),
                      "per_launch_p90": float(np.percentile(per, 90))},
        "elements_per_s": elems / (region * 1e-3),
        "roofline": rf,
        "cache": {"flushed_per_launch_median_ms": float(np.median(cold)),
                  "warm_per_launch_median_ms": float(np.median(per)),
                  "flushed_over_warm": float(np.median(cold) / np.median(per)),
                  "flush": "%d MiB written before each launch" % (FLUSH_BYTES >> 20)},
        "sequence_split": split,
        "launches_per_step": 2 if split else 1,
        "input_generation_s": gen_s,
    }
    if split:
        out["note"] = ("split along the sequence: an aggregate pass over every segment but the "
                       "last, then the main pass; the kernel time is both launches")
    del t, y, hL, ws
    torch.cuda.empty_cache()
    return out, (region, wall, per)


def bench_decode(torch, ssm, synth, steps_cap=256, layers=16):
    """The decode workload's step (batch 64, dim 5120, N 16): 256 per-token
    launches, timed three ways.
      rotating: in a HIP graph, token s updates the state of layer s mod 16,
        16 distinct 21 MB states (336 MB with their inputs past the 256 MB
        MALL), as a multi-layer model's decode reads each layer's state from
        HBM: the roofline;
      cached: in a HIP graph, one state updated 256 times (it stays in the
        MALL between steps);
      eager: one launch per token from Python through StateUpdateSteps (the
        arguments checked once, per step a pointer offset and one C call)."""
    wl = synth.WORKLOADS[4]
    inp = synth.make_inputs(wl)
    perm = lambda t: t.permute(2, 0, 1).contiguous()
    xs, dts, zs = perm(to_dev(inp, "x")), perm(to_dev(inp, "dt")), perm(to_dev(inp, "z"))
    Bs, Cs = perm(to_dev(inp, "Bm")), perm(to_dev(inp, "Cm"))
    A, Dk, bias = to_dev(inp, "A"), to_dev(inp, "Dskip"), to_dev(inp, "dt_bias")
    state0 = torch.from_numpy(inp.h0).cuda()
    states = state0.unsqueeze(0).repeat(layers, 1, 1, 1)
    state = state0.clone()
    ys = torch.empty((wl.seqlen, wl.batch, wl.dim), device="cuda")
    steps = min(steps_cap, wl.seqlen)
    E = lambda: torch.cuda.Event(enable_timing=True)

    def bind(stream):
        """The step objects, bound to `stream` (the current one when eager,
        the capture stream inside a graph)."""
        run = ssm.StateUpdateSteps(state, A, xs, dts, Bs, Cs, ys=ys, dt_bias=bias, Dskip=Dk, zs=zs,
                                   stream=stream)
        layer_runs = [ssm.StateUpdateSteps(states[k], A, xs, dts, Bs, Cs, ys=ys, dt_bias=bias,
                                           Dskip=Dk, zs=zs, stream=stream) for k in range(layers)]

        def loop():
            for s in range(steps):
                run(s)

        def rotating():
            for s in range(steps):
                layer_runs[s % layers](s)

        return loop, rotating

    loop, rotating = bind(torch.cuda.current_stream())

    # eager: the per-token Python loop
    loop()
    state.copy_(state0)
    torch.cuda.synchronize()
    e0, e1 = E(), E()
    h0 = time.perf_counter()
    e0.record()
    loop()
    e1.record()
    host_us = (time.perf_counter() - h0) / steps * 1e6
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    ref_state, ref_y = state.clone(), ys[:steps].clone()

    def capture(which):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            bind(side)[which]()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            bind(torch.cuda.current_stream())[which]()
        return g

    g_cached = capture(0)
    state.copy_(state0)
    g_cached.replay()
    torch.cuda.synchronize()
    graph_ok = bool(torch.equal(state, ref_state) and torch.equal(ys[:steps], ref_y))
    g_rot = capture(1)

    def replay(g, reset, n=3):
        out = []
        for _ in range(n):
            reset()
            torch.cuda.synchronize()
            a, b = E(), E()
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) / steps)
        return float(np.median(out))

    graph_ms = replay(g_cached, lambda: state.copy_(state0))
    flusher = Flusher(torch)

    def reset_rot():
        states.copy_(state0.unsqueeze(0).expand_as(states))
        flusher()

    rot_ms = replay(g_rot, reset_rot)

    # measured ceiling for a pass over the same rotating states: one torch
    # in-place add per token on the layer's state (read + write of the state,
    # no inputs), captured and replayed the same way
    g_add = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        states[0].add_(1.0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g_add):
        for s in range(steps):
            states[s % layers].add_(1.0)
    add_ms = replay(g_add, reset_rot)
    add_bytes = 2 * wl.batch * wl.dim * wl.dstate * 4
    del g_add
    per_call_bytes = (2 * wl.batch * wl.dim * wl.dstate * 4 + 3 * wl.batch * wl.dim * 2
                      + 2 * wl.batch * wl.dstate * 2 + wl.dim * wl.dstate * 4 + 2 * wl.dim * 4
                      + wl.batch * wl.dim * 4)
    elems = wl.batch * wl.dim * wl.dstate
    gbps = lambda t_ms: per_call_bytes / (t_ms * 1e-3) / 1e9
    del flusher
    return {"workload": wl.name, "calls": steps,
            "us_per_call": ms * 1e3, "host_us_per_call": host_us,
            "elements_per_s": elems / (rot_ms * 1e-3),
            "hbm_gbps_algorithmic": gbps(rot_ms),
            "bytes_per_call": per_call_bytes,
            "rotating_graph_us_per_call": rot_ms * 1e3,
            "cached_graph_us_per_call": graph_ms * 1e3, "graph_matches_eager": graph_ok,
            "cached_graph_hbm_gbps_algorithmic": gbps(graph_ms),
            "roofline": {"bound": "hbm", "achieved": gbps(rot_ms), "peak": PEAK_HBM / 1e9,
                         "unit": "GB/s", "frac": gbps(rot_ms) * 1e9 / PEAK_HBM, "traffic": None,
                         "algorithmic_bytes": per_call_bytes,
                         "timing": "per step of a graph replay, state rotating over %d "
                                   "buffers (launch gaps included)" % layers,
                         "cached_state": {"achieved": gbps(graph_ms),
                                          "frac": gbps(graph_ms) * 1e9 / PEAK_HBM},
                         "measured_ceiling": {
                             "what": "torch in-place add over the same 16 rotating states, "
                                     "one per token in a graph replay",
                             "us_per_step": add_ms * 1e3,
                             "achieved": add_bytes / (add_ms * 1e-3) / 1e9,
                             "decode_frac_of_ceiling": gbps(rot_ms) / (add_bytes / (add_ms * 1e-3) / 1e9)}},
            "note": "one launch per token, state fp32 in place; eager: StateUpdateSteps loop"}


def bench_conv(torch, ssm, synth, wl, x, launches=20):
    """Causal depthwise conv (W 4, silu, bf16 in and out) over the layer's x,
    and its decode step on the decode workload's shape; HBM-bound."""
    w, b = synth.conv_parameters(wl, 4)
    wt, bt = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    fn = lambda: ssm.ssm_conv1d_fwd(x, wt, bias=bt, y=y, return_final_state=False)
    for _ in range(3):
        fn()
    ms, per = time_launches(torch, fn, launches, stream)
    nbytes = 2 * x.numel() * x.element_size() + wl.dim * 5 * 4
    achieved = nbytes / (ms * 1e-3)
    out = {"workload": "conv1d W4 silu, %s" % wl.name, "kernel_ms_mean": ms,
           "per_launch_events_ms_mean": float(per.mean()),
           "outputs_per_s": x.numel() / (ms * 1e-3),
           "roofline": {"bound": "hbm", "achieved": achieved / 1e9, "peak": PEAK_HBM / 1e9,
                        "unit": "GB/s", "frac": achieved / PEAK_HBM, "traffic": None,
                        "algorithmic_bytes": nbytes,
                        "model": "x read once (2 B) + y written once (2 B) per output, plus taps"}}
    # the same conv on (batch, L, dim)-ordered tensors (ssm_conv1d_fwd_bld)
    xt = x.transpose(1, 2).contiguous()
    yt = torch.empty_like(xt)
    fb = lambda: ssm.ssm_conv1d_fwd_bld(xt, wt, bias=bt, y=yt, return_final_state=False)
    for _ in range(3):
        fb()
    ms_b, _ = time_launches(torch, fb, launches, stream)
    out["bld_layout"] = {"kernel_ms_mean": ms_b, "achieved": nbytes / (ms_b * 1e-3) / 1e9,
                         "frac": nbytes / (ms_b * 1e-3) / PEAK_HBM,
                         "note": "x, y as [batch, L, dim]; same algorithmic bytes"}
    del xt, yt
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


def bench_bwd(torch, ssm, wl, t, launches=10, warmup_seconds=1.0):
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

    def timed(fn, seconds=0.0):
        # the clock ramps up under sustained load: the first timing of the
        # call runs it untimed for `seconds` first, as the forward's does
        t_end = time.perf_counter() + seconds
        for _ in range(2):
            fn()
        while time.perf_counter() < t_end:
            fn()
            torch.cuda.synchronize()
        ms, _ = time_launches(torch, fn, launches, stream)
        return ms

    ms = timed(call, warmup_seconds)
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
    # the same backward on (batch, L, dim) tensors (ssm_scan_bwd_bld): inputs
    # transposed into its workspace, outputs transposed back
    del ws
    tb = lambda k: t[k].transpose(1, 2).contiguous()
    bt = {k: tb(k) for k in ("x", "dt", "z", "Bm", "Cm")}
    dyb = dy.transpose(1, 2).contiguous()
    gb = {k: torch.empty((wl.batch, wl.seqlen, wl.dim), device="cuda") for k in ("dx", "ddt", "dz")}
    wsb = torch.empty(ssm.lib().ssm_scan_bwd_bld_workspace_bytes(wl.batch, wl.dim, wl.seqlen,
                                                                 wl.dstate),
                      dtype=torch.uint8, device="cuda")
    bld_ms = timed(lambda: ssm.ssm_scan_bwd_bld(
        bt["x"], bt["dt"], t["A"], bt["Bm"], bt["Cm"], dyb, dt_bias=t["dt_bias"],
        Dskip=t["Dskip"], z=bt["z"], workspace=wsb, dx=gb["dx"], ddt=gb["ddt"], dz=gb["dz"]))
    del bt, dyb, gb, wsb
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
            "zoh_ms_mean": zoh_ms, "bld_layout_ms_mean": bld_ms,
            "note": "checkpoint recompute + zero-fill + reverse pass + partial-copy sum, "
                    "timed after %.1f s of untimed calls; " % warmup_seconds +
                    "bld_layout: ssm_scan_bwd_bld on (batch, L, dim) tensors, transposes "
                    "included; "
                    "with_forward_checkpoints: the forward writes the checkpoints and the "
                    "backward skips its recomputation pass; zoh: the exact zero-order-hold "
                    "form of B-bar"}


def main():
    args = parse()
    if args.ingest_counters:
        import selective_state_space_64_amd as ssm
        from selective_state_space_64_amd import synth
        wl = synth.WORKLOADS[args.workload]
        split = ssm.lib().ssm_scan_fwd_workspace_bytes(wl.batch, wl.dim, wl.seqlen, wl.dstate) > 0
        kernels = [scan_kernel_name(wl.dtype)] + ([scan_kernel_name(wl.dtype, agg=True)]
                                                  if split else [])
        rec = ingest_counters(*args.ingest_counters, workload=wl.name, kernels=kernels)
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
    flusher = Flusher(torch)
    wl = synth.WORKLOADS[args.workload]
    if args.only_workload:
        res, _ = measure_scan(torch, ssm, synth, wl, args.steps, flusher,
                              warmup_seconds=args.warmup_seconds, warmup=args.warmup)
        print(json.dumps(res), flush=True)
        return
    if args.only_backward:
        inp = synth.make_inputs(wl)
        t = {k: to_dev(inp, k) for k in ("x", "dt", "z", "Bm", "Cm", "A", "Dskip", "dt_bias")}
        del inp
        print(json.dumps(bench_bwd(torch, ssm, wl, t, launches=args.steps,
                                   warmup_seconds=args.warmup_seconds)), flush=True)
        return
    inp = synth.make_inputs(wl)
    t = {k: to_dev(inp, k) for k in ("x", "dt", "z", "Bm", "Cm", "A", "Dskip", "dt_bias")}
    y = torch.empty((wl.batch, wl.dim, wl.seqlen), device="cuda")
    hL = torch.empty((wl.batch, wl.dim, wl.dstate), device="cuda")
    need = ssm.lib().ssm_scan_fwd_workspace_bytes(wl.batch, wl.dim, wl.seqlen, wl.dstate)
    ws = torch.empty(max(1, need), dtype=torch.uint8, device="cuda")

    def step():
        ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                         Dskip=t["Dskip"], z=t["z"], y=y, hL=hL, workspace=ws)

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
    # (the event packets between launches add about a microsecond each), and
    # the same with the caches flushed before each launch
    _, launch_ms = time_launches(torch, step, args.steps, stream)
    _, cold_ms = time_launches(torch, step, max(3, args.steps // 2), stream, flusher)
    ms_step = wall * 1e3 / args.steps
    kern_s = region_ms * 1e-3
    elems = wl.batch * wl.dim * wl.seqlen * wl.dstate
    in_bytes = 2 if wl.dtype == "bf16" else 4
    rf = roofline(wl.batch, wl.dim, wl.seqlen, wl.dstate, in_bytes, kern_s, counter_traffic(wl.name))
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
        "hbm_gbps_algorithmic": rf["hbm"]["achieved"] if "hbm" in rf else rf["achieved"],
        "roofline": rf,
        "cache": {"flushed_per_launch_median_ms": float(np.median(cold_ms)),
                  "warm_per_launch_median_ms": float(np.median(launch_ms)),
                  "flushed_over_warm": float(np.median(cold_ms) / np.median(launch_ms)),
                  "flush": "%d MiB written before each launch" % (FLUSH_BYTES >> 20)},
    }
    # exact zero-order-hold B-bar variant of the same step (SSM_FLAG_ZOH_B)
    zfn = lambda: ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                                   Dskip=t["Dskip"], z=t["z"], y=y, hL=hL, zoh=True)
    for _ in range(2):
        zfn()
    zms, _ = time_launches(torch, zfn, 10, stream)
    result["zoh_variant"] = {"kernel_ms_mean": zms, "elements_per_s": elems / (zms * 1e-3)}
    # the same step on (batch, L, dim)-ordered copies of the inputs (ssm_scan_fwd_bld)
    tb = {k: t[k].transpose(1, 2).contiguous() for k in ("x", "dt", "z", "Bm", "Cm")}
    yb = torch.empty((wl.batch, wl.seqlen, wl.dim), device="cuda")
    wsb = torch.empty(ssm.lib().ssm_scan_fwd_bld_workspace_bytes(wl.batch, wl.dim, wl.seqlen,
                                                                 wl.dstate),
                      dtype=torch.uint8, device="cuda")
    bfn = lambda: ssm.ssm_scan_fwd_bld(tb["x"], tb["dt"], t["A"], tb["Bm"], tb["Cm"],
                                       dt_bias=t["dt_bias"], Dskip=t["Dskip"], z=tb["z"], y=yb,
                                       hL=hL, workspace=wsb)
    for _ in range(3):
        bfn()
    bms, _ = time_launches(torch, bfn, 20, stream)
    brf = roofline(wl.batch, wl.dim, wl.seqlen, wl.dstate, in_bytes, bms * 1e-3)
    result["bld_layout"] = {"kernel_ms_mean": bms, "elements_per_s": elems / (bms * 1e-3),
                            "over_bdl_time": bms / region_ms, "roofline_frac": brf["frac"],
                            "note": "x, dt, z, y as [batch, L, dim], Bm, Cm as [batch, L, N]: "
                                    "aggregate, combine and main launches"}
    del tb, yb, wsb
    if not args.no_peaks:
        from selective_state_space_64_amd import peaks
        result["peaks"] = peaks.measure(torch)
    if not args.no_decode:
        result["decode"] = bench_decode(torch, ssm, synth)
        result["conv1d"] = bench_conv(torch, ssm, synth, wl, t["x"])
        result["backward"] = bench_bwd(torch, ssm, wl, t, warmup_seconds=args.warmup_seconds)
    del t, y, hL, ws
    torch.cuda.empty_cache()
    if not args.no_configs:
        result["configs"] = {}
        for idx in [int(i) for i in args.configs.split(",") if i.strip()]:
            cwl = synth.WORKLOADS[idx]
            n = 5 if cwl.seqlen >= (1 << 20) else 20
            res, _ = measure_scan(torch, ssm, synth, cwl, n, flusher)
            result["configs"][cwl.name] = res
            print("# measured %s: %.4f ms" % (cwl.name, res["kernel_ms"]["mean"]), file=sys.stderr,
                  flush=True)
    if "peaks" in result:
        # the ALU rooflines against the measured practical rate of the
        # scan's instruction mix as well as against the nominal peak
        mix = result["peaks"]["scan_mix"]["slots_per_s"] / 1e12
        rfs = [result["roofline"]] + [c["roofline"] for c in result.get("configs", {}).values()]
        for rf in rfs:
            alu = rf if rf["bound"] == "alu" else rf["alu"]
            alu["measured_peak"] = mix
            alu["frac_of_measured_peak"] = alu["achieved"] / mix
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp)
        result["cpu_baseline"]["single_thread"] = cpu_single_thread(synth, synth.WORKLOADS[1])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
