"""GPU parity of ssm_scan_bwd (through the C ABI) against the fp64 backward
oracle (itself pinned to the forward oracle by exact directional derivatives
and finite differences).

Full-tensor comparisons of every gradient at small shapes (several chunks,
ragged tails, channel counts that leave part of a workgroup empty, every
supported state size, with and without gate / skip / bias / h0 / dhL), the
whole Mamba-130M-shaped layer (batch 8, dim 1536, L 2048, bf16 inputs) and
the whole Mamba-2.8B-shaped layer (batch 4, dim 5120, L 2048), bf16 gradient
outputs, and the long sequence (L = 2^20) on sampled channels for
the per-channel gradients.

Tolerances (metric of tests/helpers.py): the gradients are fp32 chains of the
same kind as the forward (exp2 / rcp / fma), plus fp32 atomic sums over
channels, batch and time; observed errors are 1e-7..1e-5 relative, gated at
the fp32 bar 1e-4.  bf16 gradient outputs add one rounding (2^-8 + 1e-4).
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_64_amd as ssm
from selective_state_space_64_amd import synth
from helpers import TOL_BF16_OUT, TOL_F32, rel_err, to_dev, workload

pytestmark = pytest.mark.gpu

GRADS = ("dx", "ddt", "dz", "dBm", "dCm", "dA", "dDskip", "ddt_bias", "dh0")


def _dy(rng, shape, gdt):
    """dy on the device and as the fp32 values it holds (exact for bf16)."""
    dy = rng.standard_normal(shape, dtype=np.float32)
    if gdt == torch.bfloat16:
        bits = synth.bf16_bits(dy)
        return (torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16),
                synth.bf16_values(bits))
    return torch.from_numpy(dy).cuda(), dy


def _compare(inp, gate=True, skip=True, bias=True, use_h0=True, use_dhL=True,
             gdt=torch.float32, seed=3, rows=None):
    """Run both sides; `rows` restricts the oracle to the listed channels of
    batch row 0 (per-channel gradients only)."""
    batch, dim, L = inp.x.shape
    N = inp.A.shape[1]
    rng = np.random.default_rng(seed)
    dyt, dyv = _dy(rng, (batch, dim, L), gdt)
    dhL = rng.standard_normal((batch, dim, N)).astype(np.float32) if use_dhL else None
    h0 = inp.h0 if use_h0 else None
    g = ssm.ssm_scan_bwd(
        to_dev(inp, "x"), to_dev(inp, "dt"), to_dev(inp, "A"), to_dev(inp, "Bm"), to_dev(inp, "Cm"),
        dyt, dt_bias=to_dev(inp, "dt_bias") if bias else None,
        Dskip=to_dev(inp, "Dskip") if skip else None, z=to_dev(inp, "z") if gate else None,
        h0=torch.from_numpy(h0).cuda() if use_h0 else None,
        dhL=torch.from_numpy(dhL).cuda() if use_dhL else None, grad_dtype=gdt)
    torch.cuda.synchronize()
    g = {k: (None if v is None else v.float().cpu().numpy()) for k, v in g.items()}
    sel = slice(None) if rows is None else rows
    bsel = slice(None) if rows is None else slice(0, 1)

    def vals(name, per_channel=True):
        a = getattr(inp, name)[bsel]
        if per_channel:
            a = a[:, sel]
        return synth.bf16_values(a).astype(np.float64) if inp.dtype == "bf16" else a.astype(np.float64)

    r = oracle.scan_bwd(
        vals("x"), vals("dt"), inp.A[sel], vals("Bm", False), vals("Cm", False),
        dyv[bsel][:, sel].astype(np.float64), dt_bias=inp.dt_bias[sel] if bias else None,
        Dskip=inp.Dskip[sel] if skip else None, z=vals("z") if gate else None,
        h0=None if h0 is None else h0[bsel][:, sel],
        dhL=None if dhL is None else dhL[bsel][:, sel])
    if rows is not None:
        g = {k: (None if v is None else
                 (v[rows] if k in ("dA", "dDskip", "ddt_bias") else
                  (None if k in ("dBm", "dCm") else v[0:1][:, rows])))
             for k, v in g.items()}
    return g, r


def _errors(g, r):
    out = {}
    for k in GRADS:
        if g.get(k) is None or r.get(k) is None:
            continue
        gg, rr = g[k], r[k]
        if gg.ndim == 1:
            gg, rr = gg[None], rr[None]
        out[k] = rel_err(gg, rr)
    return out


def _check(errs, gdt, shape):
    for k, e in errs.items():
        tol = TOL_BF16_OUT if (gdt == torch.bfloat16 and k in ("dx", "ddt", "dz")) else TOL_F32
        assert e <= tol, (shape, k, e, errs)


SMALL = [
    # (batch, dim, N, L, dtype)
    (1, 4, 4, 64, "f32"), (2, 16, 16, 256, "f32"), (2, 16, 16, 257, "bf16"),
    (1, 17, 16, 1000, "f32"), (3, 33, 8, 511, "bf16"), (2, 5, 4, 4099, "f32"),
    (1, 16, 2, 300, "bf16"), (2, 20, 1, 777, "f32"), (1, 1, 16, 1, "f32"), (1, 3, 16, 7, "bf16"),
    (2, 48, 16, 2048, "bf16"),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "b%d_d%d_N%d_L%d_%s" % s)
def test_bwd_small_full(shape):
    batch, dim, N, L, dt = shape
    print("bwd small", shape, flush=True)
    inp = synth.make_inputs(workload("bwd", batch, dim, N, L, dt, seed=3), with_h0=True)
    for opts in (dict(), dict(gate=False, skip=False, bias=False),
                 dict(use_h0=False, use_dhL=False)):
        g, r = _compare(inp, **opts)
        _check(_errors(g, r), torch.float32, (shape, opts))


def test_bwd_bf16_gradients():
    inp = synth.make_inputs(workload("bwd16", 2, 48, 16, 2048, "bf16", seed=4), with_h0=True)
    g, r = _compare(inp, gdt=torch.bfloat16)
    _check(_errors(g, r), torch.bfloat16, "bf16 grads")


def test_bwd_130m_layer_full():
    """Mamba-130M-shaped layer (batch 8, dim 1536, N 16, L 2048, bf16 in),
    every gradient against the oracle."""
    wl = synth.WORKLOADS[1]
    print("bwd", wl.name, flush=True)
    inp = synth.make_inputs(wl, with_h0=True)
    g, r = _compare(inp)
    errs = _errors(g, r)
    print("  " + " ".join("%s %.1e" % kv for kv in errs.items()), flush=True)
    _check(errs, torch.float32, wl.name)


def test_bwd_2p8b_layer_full():
    """Mamba-2.8B-shaped layer (batch 4, dim 5120, N 16, L 2048, bf16 in, fp32
    gradients) in the configuration the benchmark times (gate, skip and bias,
    no h0 or dhL): every gradient against the oracle, in full."""
    wl = synth.WORKLOADS[2]
    print("bwd", wl.name, flush=True)
    inp = synth.make_inputs(wl)
    g, r = _compare(inp, use_h0=False, use_dhL=False, seed=6)
    errs = _errors(g, r)
    print("  " + " ".join("%s %.1e" % kv for kv in errs.items()), flush=True)
    _check(errs, torch.float32, wl.name)


def test_bwd_long_sequence_sampled():
    """L = 2^20, 1536 channels (fp32): the per-channel gradients (dx, ddt, dz,
    dh0, dA, dDskip, ddt_bias) of sampled channels against the oracle run on
    those channels alone (dBm and dCm sum over every channel and are covered
    at the shorter shapes)."""
    base = synth.WORKLOADS[3]
    print("bwd", base.name, flush=True)
    inp = synth.make_inputs(base, with_h0=True)
    rows = [0, 15, 16, 777, 1535]
    g, r = _compare(inp, rows=rows)
    for k in ("dBm", "dCm"):
        r.pop(k)
    errs = _errors(g, r)
    print("  " + " ".join("%s %.1e" % kv for kv in errs.items()), flush=True)
    _check(errs, torch.float32, base.name)


def test_bwd_deterministic_per_row_outputs():
    """dx, ddt, dz and dh0 involve no atomics: two calls agree bit for bit."""
    inp = synth.make_inputs(workload("bwdd", 2, 24, 16, 600, "bf16", seed=5), with_h0=True)
    dy = torch.randn(2, 24, 600, device="cuda")
    args = (to_dev(inp, "x"), to_dev(inp, "dt"), to_dev(inp, "A"), to_dev(inp, "Bm"),
            to_dev(inp, "Cm"), dy)
    kw = dict(dt_bias=to_dev(inp, "dt_bias"), Dskip=to_dev(inp, "Dskip"), z=to_dev(inp, "z"),
              h0=torch.from_numpy(inp.h0).cuda())
    g1 = ssm.ssm_scan_bwd(*args, **kw)
    g2 = ssm.ssm_scan_bwd(*args, **kw)
    torch.cuda.synchronize()
    for k in ("dx", "ddt", "dz", "dh0"):
        assert torch.equal(g1[k], g2[k]), k


def test_bwd_argument_errors():
    inp = synth.make_inputs(workload("bwde", 1, 8, 4, 40, "f32", seed=6))
    dy = torch.randn(1, 8, 40, device="cuda")
    x, dt, A, Bm, Cm = (to_dev(inp, k) for k in ("x", "dt", "A", "Bm", "Cm"))
    with pytest.raises(ssm.SSMError) as e:
        ssm.ssm_scan_bwd(x, dt, A, Bm, Cm, dy, workspace=torch.empty(16, dtype=torch.uint8,
                                                                      device="cuda"))
    assert e.value.status == 7  # workspace too small
    L = ssm.lib()
    f = lambda t: t.data_ptr()
    outs = [torch.full((1, 8, 40), 7.0, device="cuda") for _ in range(3)]
    dB, dC = torch.full((1, 4, 40), 7.0, device="cuda"), torch.full((1, 4, 40), 7.0, device="cuda")
    dAo = torch.full((8, 4), 7.0, device="cuda")
    ws = torch.empty(L.ssm_scan_bwd_workspace_bytes(1, 8, 40, 4), dtype=torch.uint8, device="cuda")

    zt = to_dev(inp, "z")

    def call(**o):
        a = dict(flags=0, z=f(zt), dz=f(outs[2]), dx=f(outs[0]), dBm=f(dB))
        a.update(o)
        return L.ssm_scan_bwd(1, 8, 40, 4, 0, a["flags"], f(x), f(dt), None, f(A), f(Bm), f(Cm),
                              None, a["z"], None, 0, f(dy), None, a["dx"], f(outs[1]), a["dz"],
                              a["dBm"], f(dC), f(dAo), None, None, None, f(ws), ws.numel(), None)

    assert call(flags=4) == 6          # an unknown flag bit
    assert call(dz=None) == 1          # z given without dz
    assert call(dx=f(x)) == 5          # output over an input
    assert call(dBm=f(dC)) == 5        # two outputs overlapping
    torch.cuda.synchronize()
    assert all((t == 7.0).all() for t in outs + [dB, dC, dAo])


def _offset_copy(t, off=1):
    buf = torch.empty(t.numel() + off, dtype=t.dtype, device=t.device)
    v = buf[off:off + t.numel()].view(t.shape)
    v.copy_(t)
    return v


def test_bwd_unaligned_pointers_and_guard_bands():
    """Inputs, dy and the per-step gradients one element off a 16-byte
    boundary (every run takes the element path) at L = 1024 whose rows would
    otherwise be vector-aligned; NaN guard bands around every output stay
    untouched."""
    batch, dim, N, L = 2, 21, 16, 1024
    inp = synth.make_inputs(workload("bwdu", batch, dim, N, L, "bf16", seed=11), with_h0=True)
    rng = np.random.default_rng(11)
    dy = rng.standard_normal((batch, dim, L), dtype=np.float32)
    G = 64
    nan_bits = torch.tensor([0x7FC0DEAD], dtype=torch.int32).view(torch.float32).item()
    shapes = {"dx": (batch, dim, L), "ddt": (batch, dim, L), "dz": (batch, dim, L),
              "dBm": (batch, N, L), "dCm": (batch, N, L), "dA": (dim, N), "dDskip": (dim,),
              "ddt_bias": (dim,), "dh0": (batch, dim, N)}
    bigs, outs = {}, {}
    for k, shp in shapes.items():
        n = int(np.prod(shp))
        off = 1 if k in ("dx", "ddt", "dz") else 0
        bigs[k] = (torch.full((n + 2 * G + off,), nan_bits, device="cuda"), G + off, n)
        outs[k] = bigs[k][0][G + off:G + off + n].view(shp)
    args = [_offset_copy(to_dev(inp, k)) for k in ("x", "dt")] + [to_dev(inp, "A")] + \
           [_offset_copy(to_dev(inp, k)) for k in ("Bm", "Cm")]
    z = _offset_copy(to_dev(inp, "z"))
    dyt = _offset_copy(torch.from_numpy(dy).cuda())
    h0 = torch.from_numpy(inp.h0).cuda()
    L_ = ssm.lib()
    ws = torch.empty(L_.ssm_scan_bwd_workspace_bytes(batch, dim, L, N), dtype=torch.uint8,
                     device="cuda")
    p = lambda t: None if t is None else t.data_ptr()
    bias, skip = to_dev(inp, "dt_bias"), to_dev(inp, "Dskip")  # kept alive across the call
    st = L_.ssm_scan_bwd(batch, dim, L, N, 1, 0, p(args[0]), p(args[1]), p(bias),
                         p(args[2]), p(args[3]), p(args[4]), p(skip), p(z), p(h0),
                         0, p(dyt), None, p(outs["dx"]), p(outs["ddt"]), p(outs["dz"]),
                         p(outs["dBm"]), p(outs["dCm"]), p(outs["dA"]), p(outs["dDskip"]),
                         p(outs["ddt_bias"]), p(outs["dh0"]), p(ws), ws.numel(), None)
    assert st == 0
    torch.cuda.synchronize()
    r = oracle.scan_bwd(inp.values("x"), inp.values("dt"), inp.A, inp.values("Bm"),
                        inp.values("Cm"), dy.astype(np.float64), dt_bias=inp.dt_bias,
                        Dskip=inp.Dskip, z=inp.values("z"), h0=inp.h0)
    g = {k: v.cpu().numpy() for k, v in outs.items()}
    _check(_errors(g, r), torch.float32, "unaligned")
    for k, (big, lo, n) in bigs.items():
        bits = big.view(torch.int32).cpu().numpy()
        assert (bits[:lo] == 0x7FC0DEAD).all() and (bits[lo + n:] == 0x7FC0DEAD).all(), k


@pytest.mark.parametrize("shape", [(2, 48, 16, 2048, "bf16"), (1, 17, 8, 1000, "f32"),
                                   (2, 5, 1, 777, "f32"), (1, 3, 16, 7, "bf16"),
                                   (2, 20, 4, 64, "bf16")],
                         ids=lambda s: "b%d_d%d_N%d_L%d_%s" % s)
def test_bwd_checkpoints_from_forward(shape):
    """SSM_FLAG_CHECKPOINTS: the forward writes the state entering every
    64-step chunk into the backward's workspace without changing its own
    outputs, and the backward that reads them matches the one that
    recomputes them.  Not bit for bit: the recomputation folds 16 steps per
    lane where the forward folds 8, so the two sets of checkpoints differ in
    the order of their fp32 roundings."""
    batch, dim, N, L, dt = shape
    inp = synth.make_inputs(workload("ckpt", batch, dim, N, L, dt, seed=13), with_h0=True)
    t = {k: to_dev(inp, k) for k in ("x", "dt", "A", "Bm", "Cm", "dt_bias", "Dskip", "z")}
    h0 = torch.from_numpy(inp.h0).cuda()
    kw = dict(dt_bias=t["dt_bias"], Dskip=t["Dskip"], z=t["z"], h0=h0)
    need = ssm.lib().ssm_scan_bwd_workspace_bytes(batch, dim, L, N)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    y0, hL0 = ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], **kw)
    y1, hL1 = ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], checkpoints=ws, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(hL0, hL1)
    dy = torch.from_numpy(np.random.default_rng(13).standard_normal((batch, dim, L),
                                                                    dtype=np.float32)).cuda()
    g0 = ssm.ssm_scan_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dy, **kw)
    g1 = ssm.ssm_scan_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dy, workspace=ws,
                          checkpoints_in_workspace=True, **kw)
    torch.cuda.synchronize()
    for k in ("dx", "ddt", "dz", "dh0", "dBm", "dCm", "dA", "dDskip", "ddt_bias"):
        assert float((g0[k] - g1[k]).abs().max()) <= 1e-5 * float(g0[k].abs().max()) + 1e-30, k
