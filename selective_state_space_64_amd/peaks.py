"""Measured issue rates of the chip (csrc/peaks.hip), reported by bench.py
beside the nominal peaks its rooflines use.

measure(torch) times each probe kernel with HIP events on the current stream
and returns, per probe, lane operations per second and per clock per CU (at
the nominal 2.4 GHz), plus the scan mix (one exp2 and four plain fp32 ops per
step, the per-element work of the recurrence) in the rooflines' unit: issue
slots per second with a transcendental counted as 4 slots."""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssm_peaks.so")
CUS, CLOCK_HZ = 256, 2.4e9
NOMINAL_SLOTS = CUS * 128 * CLOCK_HZ
KINDS = {0: "fma", 1: "exp2", 2: "scan_mix", 3: "fma_sgpr_operand"}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libssm_peaks.so is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.ssm_peaks_ops_per_thread.restype = ctypes.c_longlong
        L.ssm_peaks_ops_per_thread.argtypes = [ctypes.c_int, ctypes.c_int]
        L.ssm_peaks_launch.restype = ctypes.c_int
        L.ssm_peaks_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]
        _lib = L
    return _lib


def measure(torch, blocks=CUS * 8, iters=(4096, 1024, 1024, 4096), repeats=5):
    """Median over `repeats` launches of each probe, 2048 workgroups of 256
    threads (8 waves per SIMD) by default."""
    L = lib()
    out = torch.empty(blocks * 256, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}
    for kind, name in KINDS.items():
        it = iters[kind]
        run = lambda: L.ssm_peaks_launch(kind, blocks, it, out.data_ptr(), stream.cuda_stream)
        for _ in range(2):
            if run() != 0:
                raise RuntimeError("peaks probe %d failed to launch" % kind)
        times = []
        for _ in range(repeats):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e-3)
        t = sorted(times)[len(times) // 2]
        ops = L.ssm_peaks_ops_per_thread(kind, it) * blocks * 256
        res[name] = {"lane_ops_per_s": ops / t, "lanes_per_clk_per_cu": ops / t / CUS / CLOCK_HZ,
                     "seconds": t}
    mix = res["scan_mix"]
    # the mix has 4 plain ops and 1 transcendental per 5 counted lane ops:
    # 8 slots per 5 ops
    mix["slots_per_s"] = mix["lane_ops_per_s"] * 8.0 / 5.0
    res["nominal_slots_per_s"] = NOMINAL_SLOTS
    res["measured_over_nominal"] = {
        "fma": res["fma"]["lane_ops_per_s"] / NOMINAL_SLOTS,
        "exp2_x4": 4.0 * res["exp2"]["lane_ops_per_s"] / NOMINAL_SLOTS,
        "scan_mix": mix["slots_per_s"] / NOMINAL_SLOTS,
        "fma_sgpr_operand": res["fma_sgpr_operand"]["lane_ops_per_s"] / NOMINAL_SLOTS,
    }
    res["note"] = ("probe kernels built like the library (no packed fp32); slots count a "
                   "transcendental as 4, as the rooflines do")
    return res
