"""GPU parity of the backward pass on (batch, L, dim)-ordered tensors
(ssm_scan_bwd_bld, through the C ABI).

Every gradient is compared in full with the fp64 backward oracle (which works
in [batch][dim][L] order; the tensors are transposed on the host), and with
ssm_scan_bwd on the same values in [batch][dim][L] order: the per-step
gradients dx, ddt, dz (no atomic sums) bit for bit, the sums over channels,
batch and time within fp32 rounding.  Shapes: ragged sequences, channel
counts that leave part of a workgroup empty, N = 1 to 16, both input dtypes,
bf16 gradients, the exact zero-order-hold form, a sequence long enough to be
split inside the GPU, projection halves as inputs and outputs, and the
Mamba-2.8B-shaped layer.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_64_amd as ssm
from selective_state_space_64_amd import synth
from helpers import TOL_BF16_OUT, TOL_F32, rel_err, to_dev, workload

pytestmark = pytest.mark.gpu

PER_STEP = ("dx", "ddt", "dz")
SUMS = ("dBm", "dCm", "dA", "dDskip", "ddt_bias", "dh0")


def _bld(t):
    """[batch, c, L] -> [batch, L, c], contiguous."""
    return t.transpose(1, 2).contiguous()


def _run(inp, gdt=torch.float32, zoh=False, seed=3, gate=True):
    batch, dim, L = inp.x.shape
    N = inp.A.shape[1]
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal((batch, dim, L), dtype=np.float32)
    if gdt == torch.bfloat16:
        bits = synth.bf16_bits(dy)
        dyt = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        dyv = synth.bf16_values(bits)
    else:
        dyt, dyv = torch.from_numpy(dy).cuda(), dy
    dhL = rng.standard_normal((batch, dim, N)).astype(np.float32)
    dev = {k: to_dev(inp, k) for k in ("x", "dt", "z", "Bm", "Cm", "A", "Dskip", "dt_bias")}
    h0, dhLt = torch.from_numpy(inp.h0).cuda(), torch.from_numpy(dhL).cuda()
    kw = dict(dt_bias=dev["dt_bias"], Dskip=dev["Dskip"], h0=h0, dhL=dhLt, grad_dtype=gdt, zoh=zoh)
    g = ssm.ssm_scan_bwd_bld(_bld(dev["x"]), _bld(dev["dt"]), dev["A"], _bld(dev["Bm"]),
                             _bld(dev["Cm"]), _bld(dyt), z=_bld(dev["z"]) if gate else None, **kw)
    r = ssm.ssm_scan_bwd(dev["x"], dev["dt"], dev["A"], dev["Bm"], dev["Cm"], dyt,
                         z=dev["z"] if gate else None, **kw)
    torch.cuda.synchronize()
    return g, r, dyv, dhL


def _check(inp, g, r, dyv, dhL, gdt, zoh=False, gate=True):
    # per-step gradients: the same kernels on exact copies, bit for bit
    for k in PER_STEP:
        if g[k] is None:
            assert r[k] is None
            continue
        assert torch.equal(g[k], _bld(r[k])), k
    # sums through fp32 atomics: the same values up to their rounding
    for k in SUMS:
        gv = g[k].cpu().numpy()
        rv = r[k].cpu().numpy()
        if k in ("dBm", "dCm"):
            rv = rv.transpose(0, 2, 1)
        assert rel_err(gv, rv) <= 1e-5, (k, rel_err(gv, rv))

    def vals(name):
        a = getattr(inp, name)
        return synth.bf16_values(a).astype(np.float64) if inp.dtype == "bf16" else a.astype(np.float64)

    ro = oracle.scan_bwd(vals("x"), vals("dt"), inp.A, vals("Bm"), vals("Cm"),
                         dyv.astype(np.float64), dt_bias=inp.dt_bias, Dskip=inp.Dskip,
                         z=vals("z") if gate else None, h0=inp.h0, dhL=dhL, zoh=zoh)
    for k in PER_STEP + SUMS:
        if ro.get(k) is None or g[k] is None:
            continue
        gv = g[k].float().cpu().numpy()
        if k in PER_STEP:
            gv = gv.transpose(0, 2, 1)
        elif k in ("dBm", "dCm"):
            gv = gv.transpose(0, 2, 1)
        tol = TOL_BF16_OUT if (gdt == torch.bfloat16 and k in PER_STEP) else TOL_F32
        assert rel_err(gv, ro[k]) <= tol, (k, rel_err(gv, ro[k]))


SHAPES = [
    # (batch, dim, N, L, dtype, grad dtype, zoh, gate)
    (1, 4, 4, 64, "f32", torch.float32, False, True),
    (2, 20, 16, 777, "bf16", torch.float32, False, True),
    (3, 17, 8, 300, "f32", torch.bfloat16, False, False),
    (2, 33, 1, 129, "bf16", torch.bfloat16, False, True),
    (1, 24, 16, 1000, "f32", torch.float32, True, True),
    (2, 48, 2, 70, "bf16", torch.float32, True, False),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b%d_d%d_N%d_L%d_%s_g%s_zoh%d_gate%d" % (
    s[0], s[1], s[2], s[3], s[4], "bf16" if s[5] == torch.bfloat16 else "f32", s[6], s[7]))
def test_bwd_bld_full(shape):
    batch, dim, N, L, dt, gdt, zoh, gate = shape
    print("bwd bld", shape, flush=True)
    inp = synth.make_inputs(workload("bwd bld", batch, dim, N, L, dt, seed=31), with_h0=True)
    g, r, dyv, dhL = _run(inp, gdt, zoh, gate=gate)
    _check(inp, g, r, dyv, dhL, gdt, zoh, gate)


def test_bwd_bld_split_sequence():
    """Few channels and a long sequence: the backward kernels split the
    sequence inside the GPU under the transposes."""
    inp = synth.make_inputs(workload("bwd bld split", 1, 16, 16, 20000, "f32", seed=33),
                            with_h0=True)
    g, r, dyv, dhL = _run(inp)
    _check(inp, g, r, dyv, dhL, torch.float32)


def test_bwd_bld_projection_halves():
    """x and z as the two halves of one [batch, L, 2 dim] projection output,
    dz into the second half of a [batch, L, 2 dim] gradient buffer whose first
    half is left alone: the same bits as dense tensors."""
    batch, dim, N, L = 2, 40, 16, 300
    inp = synth.make_inputs(workload("bwd bld proj", batch, dim, N, L, "bf16", seed=35),
                            with_h0=True)
    dev = {k: to_dev(inp, k) for k in ("x", "dt", "z", "Bm", "Cm", "A", "Dskip", "dt_bias")}
    xz = torch.cat([_bld(dev["x"]), _bld(dev["z"])], dim=2)
    dy = torch.randn(batch, L, dim, device="cuda")
    gbuf = torch.full((batch, L, 2 * dim), 7.0, device="cuda")
    kw = dict(dt_bias=dev["dt_bias"], Dskip=dev["Dskip"])
    g = ssm.ssm_scan_bwd_bld(xz[:, :, :dim], _bld(dev["dt"]), dev["A"], _bld(dev["Bm"]),
                             _bld(dev["Cm"]), dy, z=xz[:, :, dim:], dz=gbuf[:, :, dim:], **kw)
    gd = ssm.ssm_scan_bwd_bld(_bld(dev["x"]), _bld(dev["dt"]), dev["A"], _bld(dev["Bm"]),
                              _bld(dev["Cm"]), dy, z=_bld(dev["z"]), **kw)
    torch.cuda.synchronize()
    assert torch.equal(gbuf[:, :, dim:], gd["dz"])
    assert (gbuf[:, :, :dim] == 7.0).all()
    assert torch.equal(g["dx"], gd["dx"]) and torch.equal(g["ddt"], gd["ddt"])


def test_bwd_bld_layer():
    """The Mamba-2.8B-shaped layer (batch 4, dim 5120, N 16, L 2048, bf16
    inputs, fp32 gradients) in (batch, L, dim) order: per-step gradients bit
    for bit against the [batch][dim][L] call, every gradient against the
    oracle."""
    wl = synth.WORKLOADS[2]
    print("bwd bld layer", wl.name, flush=True)
    inp = synth.make_inputs(wl, with_h0=True)
    g, r, dyv, dhL = _run(inp)
    _check(inp, g, r, dyv, dhL, torch.float32)


def test_bwd_bld_argument_errors_write_nothing():
    inp = synth.make_inputs(workload("bwd bld err", 2, 8, 4, 40, "f32", seed=37))
    dev = {k: _bld(to_dev(inp, k)) if k in ("x", "dt", "z", "Bm", "Cm") else to_dev(inp, k)
           for k in ("x", "dt", "z", "Bm", "Cm", "A")}
    dy = torch.randn(2, 40, 8, device="cuda")
    outs = {k: torch.full(s, 7.0, device="cuda") for k, s in (
        ("dx", (2, 40, 8)), ("ddt", (2, 40, 8)), ("dz", (2, 40, 8)), ("dBm", (2, 40, 4)),
        ("dCm", (2, 40, 4)), ("dA", (8, 4)))}
    need = ssm.lib().ssm_scan_bwd_bld_workspace_bytes(2, 8, 40, 4)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    L = ssm.lib()
    p = lambda t: t.data_ptr()

    def call(layout=None, flags=0, wsb=need, **over):
        a = dict(x=p(dev["x"]), dt=p(dev["dt"]), A=p(dev["A"]), Bm=p(dev["Bm"]), Cm=p(dev["Cm"]),
                 z=p(dev["z"]), dy=p(dy), dx=p(outs["dx"]), ddt=p(outs["ddt"]), dz=p(outs["dz"]),
                 dBm=p(outs["dBm"]), dCm=p(outs["dCm"]), dA=p(outs["dA"]), ws=p(ws), ind=0, gd=0,
                 N=4)
        a.update(over)
        lay = ssm.BwdBldLayout(*layout) if layout else None
        return L.ssm_scan_bwd_bld(2, 8, 40, a["N"], a["ind"], flags, a["x"], a["dt"], None, a["A"],
                                  a["Bm"], a["Cm"], None, a["z"], None, a["gd"], a["dy"], None,
                                  a["dx"], a["ddt"], a["dz"], a["dBm"], a["dCm"], a["dA"], None,
                                  None, None, a["ws"], wsb,
                                  ctypes.byref(lay) if lay is not None else None, None)

    seven = ctypes.c_longlong * 7
    assert call(dy=None) == 1
    assert call(z=p(dev["z"]), dz=None) == 1
    assert call(ind=3) == 3
    assert call(layout=(seven(7, 0, 0, 0, 0, 0, 0), seven(), 0, 0, 0, 0)) == 2
    assert call(layout=(seven(), seven(0, 0, 0, 0, 319, 0, 0), 0, 0, 0, 0)) == 2
    assert call(layout=(seven(), seven(), 3, 0, 0, 0)) == 2
    assert call(N=3) == 6
    assert call(flags=2) == 6     # checkpoints: the (B, L, D) forward writes none
    assert call(dx=p(dy)) == 5
    assert call(dBm=p(outs["dCm"]) + 4) == 5
    assert call(ws=p(outs["dA"])) == 5
    assert call(wsb=need - 1) == 7
    torch.cuda.synchronize()
    assert all((t == 7.0).all() for t in outs.values())
