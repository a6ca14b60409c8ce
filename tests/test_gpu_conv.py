"""GPU parity of the causal depthwise conv (ssm_conv1d_fwd, ssm_conv1d_update,
through the C ABI) against the fp64 oracle.

Full-tensor comparisons at small shapes (ragged tails, sequences shorter than
the conv window, every supported width, both dtypes, with and without the
initial conv state and activation), the whole Mamba-2.8B-shaped layer
(batch 4, dim 5120, L 2048, bf16) compared in full, the final conv state
bit-exact (it is a copy of inputs), decode steps against the whole-sequence
oracle, and the conv feeding the scan as in the Mamba block.
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_64_amd as ssm
from selective_state_space_64_amd import synth
from helpers import TOL_BF16_OUT, TOL_F32, rel_err, to_dev, workload

pytestmark = pytest.mark.gpu

# fp32 output: W fma + silu in fp32 against fp64 (well inside the fp32 gate);
# bf16 output adds one rounding to an 8-bit significand.
TOL = {"f32": TOL_F32, "bf16": TOL_BF16_OUT}


def _conv_inputs(batch, dim, L, W, dtype, seed=5):
    wl = workload("conv", batch, dim, 16, L, dtype, seed=seed)
    inp = synth.make_inputs(wl)
    w, b = synth.conv_parameters(wl, W)
    s0 = synth.conv_state(wl, W)
    return inp, w, b, s0


def _gpu(inp, w, b, s0, silu, out_dtype, bias=True, state=True):
    y, sL = ssm.ssm_conv1d_fwd(to_dev(inp, "x"), torch.from_numpy(w).cuda(),
                               bias=torch.from_numpy(b).cuda() if bias else None,
                               state0=torch.from_numpy(s0).cuda() if state else None,
                               silu=silu, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), sL.cpu().numpy()


SMALL = [
    # (batch, dim, L, W, in dtype)
    (1, 3, 1, 4, "f32"), (2, 5, 2, 4, "bf16"), (1, 2, 3, 4, "f32"), (2, 7, 8, 4, "bf16"),
    (3, 4, 9, 3, "f32"), (2, 6, 63, 2, "bf16"), (1, 9, 64, 4, "bf16"), (2, 33, 517, 4, "f32"),
    (2, 17, 1000, 3, "bf16"), (1, 300, 2048, 4, "bf16"), (4, 2, 4099, 2, "f32"),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "b%d_d%d_L%d_W%d_%s" % s)
def test_conv_small_full_tensor(shape):
    batch, dim, L, W, dt = shape
    print("conv small", shape, flush=True)
    inp, w, b, s0 = _conv_inputs(batch, dim, L, W, dt)
    x = inp.values("x")
    for silu, bias, state, outd in [(True, True, True, torch.float32),
                                    (False, False, False, torch.float32),
                                    (True, True, False, torch.bfloat16),
                                    (False, True, True, torch.bfloat16)]:
        gy, gs = _gpu(inp, w, b, s0, silu, outd, bias, state)
        ry, rs = oracle.conv1d(x, w.astype(np.float64), bias=b.astype(np.float64) if bias else None,
                               state0=s0.astype(np.float64) if state else None, silu=silu)
        tol = TOL["bf16" if outd == torch.bfloat16 else "f32"]
        assert rel_err(gy, ry) <= tol, (shape, silu, bias, state, outd, rel_err(gy, ry))
        # the final conv state is a copy of inputs: exact
        assert np.array_equal(gs, rs.astype(np.float32)), (shape, silu, bias, state)


def test_conv_state_in_place_alias():
    """stateL may be the state0 buffer (chunked prefill keeps one state)."""
    inp, w, b, s0 = _conv_inputs(2, 24, 37, 4, "bf16")
    st = torch.from_numpy(s0).cuda()
    y, sL = ssm.ssm_conv1d_fwd(to_dev(inp, "x"), torch.from_numpy(w).cuda(),
                               bias=torch.from_numpy(b).cuda(), state0=st, stateL=st,
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    ry, rs = oracle.conv1d(inp.values("x"), w, bias=b, state0=s0)
    assert sL.data_ptr() == st.data_ptr()
    assert rel_err(y.cpu().numpy(), ry) <= TOL_F32
    assert np.array_equal(st.cpu().numpy(), rs.astype(np.float32))


def test_conv_chunked_prefill_matches_whole():
    """Two calls chained through the conv state equal one call over the whole
    sequence, bit for bit (each output depends only on its own window)."""
    inp, w, b, s0 = _conv_inputs(2, 40, 300, 4, "bf16")
    x = to_dev(inp, "x")
    wt, bt, st = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda(), torch.from_numpy(s0).cuda()
    y, sL = ssm.ssm_conv1d_fwd(x, wt, bias=bt, state0=st, out_dtype=torch.float32)
    y1, s1 = ssm.ssm_conv1d_fwd(x[:, :, :123].contiguous(), wt, bias=bt, state0=st,
                                out_dtype=torch.float32)
    y2, s2 = ssm.ssm_conv1d_fwd(x[:, :, 123:].contiguous(), wt, bias=bt, state0=s1,
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([y1, y2], dim=2), y)
    assert torch.equal(s2, sL)


def test_conv_layer_full():
    """The Mamba-2.8B-shaped layer (batch 4, dim 5120, L 2048, bf16 in and
    out, W 4, silu), every output against the oracle."""
    wl = synth.WORKLOADS[2]
    print("conv layer", wl.name, flush=True)
    inp = synth.make_inputs(wl)
    w, b = synth.conv_parameters(wl, 4)
    gy, gs = _gpu(inp, w, b, None, True, torch.bfloat16, state=False)
    ry, rs = oracle.conv1d(inp.values("x"), w, bias=b, silu=True)
    err = rel_err(gy, ry)
    print("  err y %.3e" % err, flush=True)
    assert err <= TOL_BF16_OUT
    assert np.array_equal(gs, rs.astype(np.float32))


@pytest.mark.parametrize("W,dt,outd", [(4, "bf16", torch.float32), (3, "f32", torch.float32),
                                       (2, "bf16", torch.bfloat16)])
def test_conv_decode_steps(W, dt, outd):
    batch, dim, steps = 3, 70, 6
    inp, w, b, s0 = _conv_inputs(batch, dim, steps, W, dt)
    x = to_dev(inp, "x")
    st = torch.from_numpy(s0).cuda()
    wt, bt = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
    ys = []
    for t in range(steps):
        ys.append(ssm.ssm_conv1d_update(st, x[:, :, t].contiguous(), wt, bias=bt, out_dtype=outd))
    torch.cuda.synchronize()
    gy = torch.stack(ys, dim=2).float().cpu().numpy()
    ry, rs = oracle.conv1d(inp.values("x"), w, bias=b, state0=s0)
    assert rel_err(gy, ry) <= TOL["bf16" if outd == torch.bfloat16 else "f32"]
    assert np.array_equal(st.cpu().numpy(), rs.astype(np.float32))


def test_conv_feeds_scan():
    """The block's order: conv (fp32 out) then the selective scan on its
    output, against the oracle conv followed by the oracle scan."""
    wl = workload("block", 2, 48, 16, 700, "bf16", seed=9)
    inp = synth.make_inputs(wl)
    w, b = synth.conv_parameters(wl, 4)
    xc, _ = ssm.ssm_conv1d_fwd(to_dev(inp, "x"), torch.from_numpy(w).cuda(),
                               bias=torch.from_numpy(b).cuda(), out_dtype=torch.float32)
    f32 = lambda name: torch.from_numpy(inp.values(name).astype(np.float32)).cuda()
    y, hL = ssm.ssm_scan_fwd(xc, f32("dt"), to_dev(inp, "A"), f32("Bm"), f32("Cm"),
                             dt_bias=to_dev(inp, "dt_bias"), Dskip=to_dev(inp, "Dskip"), z=f32("z"))
    torch.cuda.synchronize()
    rc, _ = oracle.conv1d(inp.values("x"), w, bias=b)
    ry, rh = oracle.scan_fwd(rc, inp.values("dt"), inp.A, inp.values("Bm"), inp.values("Cm"),
                             dt_bias=inp.dt_bias, Dskip=inp.Dskip, z=inp.values("z"))
    assert rel_err(y.cpu().numpy(), ry) <= TOL_F32
    assert rel_err(hL.cpu().numpy(), rh) <= TOL_F32


def _offset_copy(t, off=1):
    """A contiguous copy of t whose data starts `off` elements into a larger
    buffer: element-aligned but not 16-byte aligned."""
    buf = torch.empty(t.numel() + off, dtype=t.dtype, device=t.device)
    v = buf[off:off + t.numel()].view(t.shape)
    v.copy_(t)
    return v


def test_conv_unaligned_pointers_and_guard_bands():
    """x and y one element off a 16-byte boundary (every run takes the
    element path) at a shape whose rows would otherwise be vector-aligned;
    NaN guard bands around y and the final state stay untouched."""
    inp, w, b, s0 = _conv_inputs(2, 37, 2048, 4, "bf16")
    x = _offset_copy(to_dev(inp, "x"))
    G = 64
    nan_bits = torch.tensor([0x7FC0DEAD], dtype=torch.int32).view(torch.float32).item()
    n_y, n_s = 2 * 37 * 2048, 2 * 37 * 3
    ybig = torch.full((n_y + 2 * G + 1,), nan_bits, device="cuda")
    sbig = torch.full((n_s + 2 * G,), nan_bits, device="cuda")
    y = ybig[G + 1:G + 1 + n_y].view(2, 37, 2048)
    sL = sbig[G:G + n_s].view(2, 37, 3)
    ssm.ssm_conv1d_fwd(x, torch.from_numpy(w).cuda(), bias=torch.from_numpy(b).cuda(),
                       state0=torch.from_numpy(s0).cuda(), y=y, stateL=sL,
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    ry, rs = oracle.conv1d(inp.values("x"), w, bias=b, state0=s0)
    assert rel_err(y.cpu().numpy(), ry) <= TOL_F32
    assert np.array_equal(sL.cpu().numpy(), rs.astype(np.float32))
    for big, lo, n in ((ybig, G + 1, n_y), (sbig, G, n_s)):
        bits = big.view(torch.int32).cpu().numpy()
        assert (bits[:lo] == 0x7FC0DEAD).all() and (bits[lo + n:] == 0x7FC0DEAD).all()


def test_conv_strided_x_from_projection_halves():
    """x as the first half of the input projection's [batch, 2 dim, L]
    output (vector path), and again with rows padded by 3 elements and y
    written into a padded view (element path): both equal to the dense call
    bit for bit, the padding of y untouched."""
    batch, dim, L = 2, 37, 2048
    inp, w, b, s0 = _conv_inputs(batch, dim, L, 4, "bf16")
    x = to_dev(inp, "x")
    wt, bt, st = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda(), torch.from_numpy(s0).cuda()
    y0, s0d = ssm.ssm_conv1d_fwd(x, wt, bias=bt, state0=st, out_dtype=torch.float32)
    xz = torch.cat([x, torch.randn(batch, dim, L, device="cuda").to(torch.bfloat16)], dim=1)
    y1, s1 = ssm.ssm_conv1d_fwd(xz[:, :dim], wt, bias=bt, state0=st, out_dtype=torch.float32)
    xp = torch.zeros(batch, dim, L + 3, dtype=torch.bfloat16, device="cuda")
    xp[:, :, :L] = x
    ybuf = torch.full((batch, dim + 1, L + 3), 777.0, device="cuda")
    y2, s2 = ssm.ssm_conv1d_fwd(xp[:, :, :L], wt, bias=bt, state0=st, out_dtype=torch.float32,
                                y=ybuf[:, 1:, :L])
    torch.cuda.synchronize()
    assert torch.equal(y1, y0) and torch.equal(s1, s0d)
    assert torch.equal(y2, y0) and torch.equal(s2, s0d)
    assert bool((ybuf[:, 0] == 777.0).all()) and bool((ybuf[:, :, L:] == 777.0).all())
    ry, rs = oracle.conv1d(inp.values("x"), w, bias=b, state0=s0)
    assert rel_err(y1.cpu().numpy(), ry) <= TOL_F32


def test_block_order_on_projection_halves():
    """The Mamba block's order on one bf16 projection buffer xz: the conv
    reads the x half and writes bf16, the scan reads that output and the z
    half in place.  The conv output against the oracle conv (bf16 output
    gate); the scan against the oracle scan run on the conv output the GPU
    produced."""
    wl = workload("block_xz", 2, 40, 16, 900, "bf16", seed=10)
    inp = synth.make_inputs(wl)
    w, b = synth.conv_parameters(wl, 4)
    xz = torch.cat([to_dev(inp, "x"), to_dev(inp, "z")], dim=1)
    xc, _ = ssm.ssm_conv1d_fwd(xz[:, :40], torch.from_numpy(w).cuda(),
                               bias=torch.from_numpy(b).cuda(), out_dtype=torch.bfloat16)
    y, hL = ssm.ssm_scan_fwd(xc, to_dev(inp, "dt"), to_dev(inp, "A"), to_dev(inp, "Bm"),
                             to_dev(inp, "Cm"), dt_bias=to_dev(inp, "dt_bias"),
                             Dskip=to_dev(inp, "Dskip"), z=xz[:, 40:])
    torch.cuda.synchronize()
    xcv = xc.float().cpu().numpy().astype(np.float64)
    rc, _ = oracle.conv1d(inp.values("x"), w, bias=b)
    assert rel_err(xcv, rc) <= TOL_BF16_OUT
    ry, rh = oracle.scan_fwd(xcv, inp.values("dt"), inp.A, inp.values("Bm"), inp.values("Cm"),
                             dt_bias=inp.dt_bias, Dskip=inp.Dskip, z=inp.values("z"))
    assert rel_err(y.cpu().numpy(), ry) <= 2e-3
    assert rel_err(hL.cpu().numpy(), rh) <= 2e-3
