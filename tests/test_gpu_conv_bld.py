"""GPU parity of the causal depthwise conv on (batch, L, dim)-ordered tensors
(ssm_conv1d_fwd_bld, through the C ABI).

Every output is compared with the fp64 oracle on the same values (the oracle
works in [batch][dim][L] order; the tensors are transposed on the host), and
with the [batch][dim][L] kernel, which sums in the same order, bit for bit.
Shapes cover both channel mappings (4 channels per lane when dim and every
stride allow it, else 1), sequences shorter than the window, ragged pieces,
every width, both dtypes, the conv state handed over in place, the input as
one half of a projection output, and the Mamba-2.8B-shaped layer.
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_64_amd as ssm
from selective_state_space_64_amd import synth
from helpers import TOL_BF16_OUT, TOL_F32, rel_err, to_dev, workload

pytestmark = pytest.mark.gpu

TOL = {torch.float32: TOL_F32, torch.bfloat16: TOL_BF16_OUT}


def _inputs(batch, dim, L, W, dtype, seed=11):
    wl = workload("conv bld", batch, dim, 16, L, dtype, seed=seed)
    inp = synth.make_inputs(wl)
    w, b = synth.conv_parameters(wl, W)
    s0 = synth.conv_state(wl, W)
    return inp, w, b, s0


def _bld(t):
    """[batch, dim, L] -> [batch, L, dim], contiguous."""
    return t.transpose(1, 2).contiguous()


SHAPES = [
    # (batch, dim, L, W, in dtype): dim % 4 != 0 takes one channel per lane
    (1, 3, 1, 4, "f32"), (2, 5, 2, 4, "bf16"), (1, 8, 3, 4, "f32"), (2, 7, 8, 3, "bf16"),
    (3, 4, 9, 2, "f32"), (2, 6, 63, 4, "bf16"), (1, 12, 130, 4, "bf16"), (2, 33, 517, 3, "f32"),
    (2, 300, 1000, 4, "bf16"), (1, 1028, 700, 2, "f32"), (4, 64, 4099, 4, "bf16"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b%d_d%d_L%d_W%d_%s" % s)
def test_conv_bld_full_tensor(shape):
    batch, dim, L, W, dt = shape
    print("conv bld", shape, flush=True)
    inp, w, b, s0 = _inputs(batch, dim, L, W, dt)
    x = to_dev(inp, "x")
    xt = _bld(x)
    wt, bt, st = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda(), torch.from_numpy(s0).cuda()
    for silu, bias, state, outd in [(True, True, True, torch.float32),
                                    (False, False, False, torch.float32),
                                    (True, True, False, torch.bfloat16),
                                    (False, True, True, torch.bfloat16)]:
        kw = dict(bias=bt if bias else None, state0=st if state else None, silu=silu,
                  out_dtype=outd)
        y, sL = ssm.ssm_conv1d_fwd_bld(xt, wt, **kw)
        yr, sr = ssm.ssm_conv1d_fwd(x, wt, **kw)
        torch.cuda.synchronize()
        assert torch.equal(y, _bld(yr)), (shape, silu, bias, state, outd)
        assert torch.equal(sL, sr), (shape, silu, bias, state, outd)
        ry, rs = oracle.conv1d(inp.values("x"), w, bias=b if bias else None,
                               state0=s0 if state else None, silu=silu)
        gy = y.float().cpu().numpy().transpose(0, 2, 1)
        assert rel_err(gy, ry) <= TOL[outd], (shape, silu, bias, state, outd, rel_err(gy, ry))
        assert np.array_equal(sL.cpu().numpy(), rs.astype(np.float32))


def test_conv_bld_projection_half_and_padded_output():
    """x as the first half of a [batch, L, 2 dim] projection output, y into
    the first half of a [batch, L, 2 dim + 8] buffer: the same bits as the
    dense call, and the rest of y's buffer untouched."""
    batch, dim, L, W = 2, 96, 333, 4
    inp, w, b, s0 = _inputs(batch, dim, L, W, "bf16")
    x = _bld(to_dev(inp, "x"))
    proj = torch.randn(batch, L, 2 * dim, device="cuda").to(torch.bfloat16)
    proj[:, :, :dim] = x
    ybuf = torch.full((batch, L, 2 * dim + 8), 7.0, device="cuda")
    wt, bt, st = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda(), torch.from_numpy(s0).cuda()
    y, sL = ssm.ssm_conv1d_fwd_bld(proj[:, :, :dim], wt, bias=bt, state0=st,
                                   out_dtype=torch.float32, y=ybuf[:, :, :dim])
    yd, sd = ssm.ssm_conv1d_fwd_bld(x, wt, bias=bt, state0=st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(ybuf[:, :, :dim], yd)
    assert torch.equal(sL, sd)
    assert (ybuf[:, :, dim:] == 7.0).all()
    # odd strides (one channel per lane): the second half of the projection
    # starts at an element offset of dim, so dim = 95 leaves 4-element vectors
    # misaligned
    dim2 = 95
    x2 = torch.randn(batch, L, 2 * dim2, device="cuda")
    y2, _ = ssm.ssm_conv1d_fwd_bld(x2[:, :, dim2:], wt[:dim2], bias=bt[:dim2], silu=True)
    yr2, _ = ssm.ssm_conv1d_fwd(x2[:, :, dim2:].transpose(1, 2).contiguous(), wt[:dim2],
                                bias=bt[:dim2], silu=True)
    torch.cuda.synchronize()
    assert torch.equal(y2, _bld(yr2))


def test_conv_bld_state_in_place_many_pieces():
    """stateL may be the state0 buffer also when the sequence is walked in
    many pieces by separate workgroups (only the first piece's lanes read
    state0, and they write stateL after reading it)."""
    inp, w, b, s0 = _inputs(3, 40, 2000, 4, "bf16")
    st = torch.from_numpy(s0).cuda()
    x = _bld(to_dev(inp, "x"))
    y, sL = ssm.ssm_conv1d_fwd_bld(x, torch.from_numpy(w).cuda(), bias=torch.from_numpy(b).cuda(),
                                   state0=st, stateL=st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ry, rs = oracle.conv1d(inp.values("x"), w, bias=b, state0=s0)
    assert sL.data_ptr() == st.data_ptr()
    assert rel_err(y.cpu().numpy().transpose(0, 2, 1), ry) <= TOL_F32
    assert np.array_equal(st.cpu().numpy(), rs.astype(np.float32))


def test_conv_bld_layer_full():
    """The Mamba-2.8B-shaped layer in (batch, L, dim) order (batch 4, L 2048,
    dim 5120, bf16 in and out, W 4, silu): every output against the oracle and
    bit-identical to the [batch][dim][L] kernel."""
    wl = synth.WORKLOADS[2]
    print("conv bld layer", wl.name, flush=True)
    inp = synth.make_inputs(wl)
    w, b = synth.conv_parameters(wl, 4)
    x = to_dev(inp, "x")
    wt, bt = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
    y, sL = ssm.ssm_conv1d_fwd_bld(_bld(x), wt, bias=bt, silu=True)
    yr, sr = ssm.ssm_conv1d_fwd(x, wt, bias=bt, silu=True)
    torch.cuda.synchronize()
    assert torch.equal(y, _bld(yr)) and torch.equal(sL, sr)
    ry, _ = oracle.conv1d(inp.values("x"), w, bias=b, silu=True)
    err = rel_err(y.float().cpu().numpy().transpose(0, 2, 1), ry)
    print("  err y %.3e" % err, flush=True)
    assert err <= TOL_BF16_OUT


def test_conv_bld_feeds_scan_bld():
    """The block's front half in (batch, L, dim) order: conv over the x half
    of one projection output, then the selective scan on the conv output and
    the z half, against the same two steps in [batch][dim][L] order."""
    batch, dim, N, L = 2, 64, 16, 600
    wl = workload("block bld", batch, dim, N, L, "bf16", seed=21)
    inp = synth.make_inputs(wl)
    w, b = synth.conv_parameters(wl, 4)
    x, z, dt = to_dev(inp, "x"), to_dev(inp, "z"), to_dev(inp, "dt")
    Bm, Cm = to_dev(inp, "Bm"), to_dev(inp, "Cm")
    A, Dk, bias = to_dev(inp, "A"), to_dev(inp, "Dskip"), to_dev(inp, "dt_bias")
    wt, bt = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
    proj = torch.cat([_bld(x), _bld(z)], dim=2)  # [batch, L, 2 dim]
    xc, _ = ssm.ssm_conv1d_fwd_bld(proj[:, :, :dim], wt, bias=bt, silu=True)
    y, hL = ssm.ssm_scan_fwd_bld(xc, _bld(dt), A, _bld(Bm), _bld(Cm), dt_bias=bias, Dskip=Dk,
                                 z=proj[:, :, dim:])
    xr, _ = ssm.ssm_conv1d_fwd(x, wt, bias=bt, silu=True)
    yr, hr = ssm.ssm_scan_fwd(xr, dt, A, Bm, Cm, dt_bias=bias, Dskip=Dk, z=z)
    torch.cuda.synchronize()
    assert torch.equal(xc, _bld(xr))
    assert rel_err(y.cpu().numpy().transpose(0, 2, 1), yr.cpu().numpy()) <= 1e-5
    assert rel_err(hL.cpu().numpy(), hr.cpu().numpy()) <= 1e-5


def test_conv_bld_argument_errors_write_nothing():
    g = torch.Generator().manual_seed(2)
    x = torch.randn(2, 40, 8, generator=g).to(torch.bfloat16).cuda()
    w = torch.randn(8, 4, generator=g).cuda()
    s0 = torch.randn(2, 8, 3, generator=g).cuda()
    y = torch.full((2, 40, 8), 7.0, device="cuda")
    sL = torch.full((2, 8, 3), 7.0, device="cuda")
    L = ssm.lib()

    def call(layout=None, **over):
        a = dict(batch=2, dim=8, seqlen=40, width=4, ind=1, flags=1, x=x.data_ptr(),
                 w=w.data_ptr(), bias=None, s0=s0.data_ptr(), outd=0, y=y.data_ptr(),
                 sL=sL.data_ptr())
        a.update(over)
        lay = ssm.ConvBldLayout(*layout) if layout else None
        return L.ssm_conv1d_fwd_bld(a["batch"], a["dim"], a["seqlen"], a["width"], a["ind"],
                                    a["flags"], a["x"], a["w"], a["bias"], a["s0"], a["outd"],
                                    a["y"], a["sL"], ctypes_byref(lay), None)

    assert call(x=None) == 1
    assert call(seqlen=0) == 2
    assert call(layout=(7, 0, 0, 0)) == 2          # step below dim
    assert call(layout=(0, 0, 0, 319)) == 2        # batch stride below seqlen * step
    assert call(ind=4) == 3
    assert call(x=x.data_ptr() + 1) == 4
    assert call(y=x.data_ptr()) == 5
    assert call(sL=s0.data_ptr() + 4) == 5
    assert call(width=5) == 6
    assert call(flags=2) == 6
    torch.cuda.synchronize()
    assert (y == 7.0).all() and (sL == 7.0).all()


def ctypes_byref(lay):
    import ctypes
    return ctypes.byref(lay) if lay is not None else None
