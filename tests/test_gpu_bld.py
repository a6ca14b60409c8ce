"""GPU parity of ssm_scan_fwd_bld, the scan on (batch, L, dim)-ordered tensors
(through the C ABI), against the fp64 oracle on the same values transposed
to the oracle's [batch][dim][L] order: full tensors over ragged lengths,
channel counts that leave a wave partly empty, every state size, both input
dtypes, bf16 output, the exact zero-order-hold form, with and without gate,
skip, bias and h0, and the Mamba-2.8B-shaped layer in full; projection halves
and padded rows equal the dense call bit for bit; hL written over h0."""
import numpy as np
import pytest
import torch

import selective_state_space_64_amd as ssm
from selective_state_space_64_amd import synth
from helpers import TOL_BF16_OUT, oracle_full, rel_err, to_dev, tol_for, workload

pytestmark = pytest.mark.gpu


def _bld(t):
    """[batch, X, L] -> [batch, L, X] contiguous."""
    return t.transpose(1, 2).contiguous()


def _inputs(inp):
    d = {k: _bld(to_dev(inp, k)) for k in ("x", "dt", "z", "Bm", "Cm")}
    d.update({k: to_dev(inp, k) for k in ("A", "Dskip", "dt_bias")})
    return d


def _state_err(g, r):
    """Final-state error over (b, d, :) rows of states; with fewer than 4
    states such a row degenerates to an elementwise relative error on values
    that may cancel to near zero, so those shapes are compared over rows of
    channels, (b, :, n), as the decode tests compare states."""
    if g.shape[-1] >= 4:
        return rel_err(g, r)
    return rel_err(np.swapaxes(g, 1, 2), np.swapaxes(r, 1, 2))


def _run(t, gate=True, skip=True, bias=True, h0=None, **kw):
    y, hL = ssm.ssm_scan_fwd_bld(
        t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"] if bias else None,
        Dskip=t["Dskip"] if skip else None, z=t["z"] if gate else None,
        h0=None if h0 is None else torch.from_numpy(np.asarray(h0, np.float32)).cuda(), **kw)
    torch.cuda.synchronize()
    return y, hL


SHAPES = [
    # (batch, dim, N, L, dtype)
    (1, 4, 4, 64, "f32"), (2, 64, 16, 300, "bf16"), (1, 65, 16, 1000, "f32"),
    (3, 20, 8, 7, "bf16"), (2, 200, 1, 777, "f32"), (1, 1, 16, 1, "f32"),
    (2, 130, 2, 2048, "bf16"), (1, 16, 16, 5000, "f32"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b%d_d%d_N%d_L%d_%s" % s)
def test_bld_full_tensor(shape):
    batch, dim, N, L, dt = shape
    print("bld", shape, flush=True)
    inp = synth.make_inputs(workload("bld", batch, dim, N, L, dt, seed=51), with_h0=True)
    t = _inputs(inp)
    tol = tol_for(dt)
    for gate, skip, bias, use_h0 in [(True, True, True, True), (False, False, False, False),
                                     (True, False, True, False)]:
        h0 = inp.h0 if use_h0 else None
        y, hL = _run(t, gate, skip, bias, h0)
        ry, rh = oracle_full(inp, gate, skip, bias, h0)
        ey = rel_err(y.transpose(1, 2).cpu().numpy(), ry)
        eh = _state_err(hL.cpu().numpy(), rh)
        assert ey <= tol and eh <= tol, (shape, gate, skip, bias, use_h0, ey, eh)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_bld_zoh_and_bf16_out(dt):
    inp = synth.make_inputs(workload("bld_zoh", 2, 96, 16, 900, dt, seed=52), with_h0=True)
    t = _inputs(inp)
    y, hL = _run(t, h0=inp.h0, zoh=True)
    ry, rh = oracle_full(inp, h0=inp.h0, zoh=True)
    tol = tol_for(dt)
    assert rel_err(y.transpose(1, 2).cpu().numpy(), ry) <= tol
    assert rel_err(hL.cpu().numpy(), rh) <= tol
    yb, _ = _run(t, h0=inp.h0, out_dtype=torch.bfloat16)
    ry, _ = oracle_full(inp, h0=inp.h0)
    assert yb.dtype == torch.bfloat16
    assert rel_err(yb.float().transpose(1, 2).cpu().numpy(), ry) <= TOL_BF16_OUT


def test_bld_views_equal_dense_bitwise():
    """x and z as the two halves of one [batch, L, 2 dim] projection output,
    Bm and Cm as parts of one [batch, L, dt_rank + 2 N] output, y into the
    first half of a [batch, L, 2 dim] buffer: the same bits as dense inputs,
    and the other half of y's buffer untouched."""
    batch, dim, N, L = 2, 96, 16, 700
    inp = synth.make_inputs(workload("bld_views", batch, dim, N, L, "bf16", seed=53))
    t = _inputs(inp)
    y_ref, h_ref = _run(t)
    xz = torch.cat([t["x"], t["z"]], dim=2)
    proj = torch.cat([torch.zeros(batch, L, 5, dtype=t["Bm"].dtype, device="cuda"), t["Bm"], t["Cm"]],
                     dim=2)
    ybuf = torch.full((batch, L, 2 * dim), 7.0, device="cuda")
    v = dict(t, x=xz[..., :dim], z=xz[..., dim:], Bm=proj[..., 5:5 + N], Cm=proj[..., 5 + N:])
    y, hL = _run(v, y=ybuf[..., :dim])
    assert y.data_ptr() == ybuf.data_ptr()
    assert torch.equal(y, y_ref) and torch.equal(hL, h_ref)
    assert bool((ybuf[..., dim:] == 7.0).all())


def test_bld_matches_bdl_path_and_in_place_state():
    """The (batch, L, dim) call agrees with the [batch, dim, L] call on the
    same values (within fp32 rounding: the two association orders differ),
    and hL may be written over h0."""
    batch, dim, N, L = 2, 80, 16, 3000
    inp = synth.make_inputs(workload("bld_vs", batch, dim, N, L, "f32", seed=54), with_h0=True)
    t = _inputs(inp)
    h0 = torch.from_numpy(inp.h0).cuda()
    yb, hb = ssm.ssm_scan_fwd(to_dev(inp, "x"), to_dev(inp, "dt"), t["A"], to_dev(inp, "Bm"),
                              to_dev(inp, "Cm"), dt_bias=t["dt_bias"], Dskip=t["Dskip"],
                              z=to_dev(inp, "z"), h0=h0)
    st = h0.clone()
    y, hL = ssm.ssm_scan_fwd_bld(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                                 Dskip=t["Dskip"], z=t["z"], h0=st, hL=st)
    torch.cuda.synchronize()
    assert hL.data_ptr() == st.data_ptr()
    assert rel_err(y.transpose(1, 2).cpu().numpy(), yb.cpu().numpy()) <= 1e-5
    assert rel_err(st.cpu().numpy(), hb.cpu().numpy()) <= 1e-5


def test_bld_layer_workload_full():
    """The Mamba-2.8B-shaped layer (batch 4, dim 5120, N 16, L 2048, bf16) in
    (batch, L, dim) order, every y and hL value against the oracle."""
    wl = synth.WORKLOADS[2]
    print("workload", wl.name, "(batch, L, dim)", flush=True)
    inp = synth.make_inputs(wl)
    t = _inputs(inp)
    y, hL = _run(t)
    gy = y.transpose(1, 2).cpu().numpy()
    gh = hL.cpu().numpy()
    del y, hL, t
    ry, rh = oracle_full(inp)
    ey, eh = rel_err(gy, ry), rel_err(gh, rh)
    print("  err y %.3e hL %.3e" % (ey, eh), flush=True)
    assert ey <= tol_for(wl.dtype) and eh <= tol_for(wl.dtype)


def test_bld_argument_errors_write_nothing():
    batch, dim, N, L = 2, 8, 16, 40
    x = torch.randn(batch, L, dim, device="cuda")
    B = torch.randn(batch, L, N, device="cuda")
    A = -torch.rand(dim, N, device="cuda")
    y = torch.full((batch, L, dim), 7.0, device="cuda")
    ws = torch.empty(ssm.lib().ssm_scan_fwd_bld_workspace_bytes(batch, dim, L, N), dtype=torch.uint8,
                     device="cuda")
    L_ = ssm.lib()
    p = lambda t: t.data_ptr()
    base = dict(x=p(x), dt=p(x), A=p(A), B=p(B), C=p(B), y=p(y), ws=p(ws), wsb=ws.numel(),
                flags=0, lay=None)

    def call(**over):
        a = dict(base, **over)
        return L_.ssm_scan_fwd_bld(batch, dim, L, N, 0, a["flags"], a["x"], a["dt"], None, a["A"],
                                   a["B"], a["C"], None, None, None, 0, a["y"], None, a["ws"],
                                   a["wsb"], a["lay"], None)

    assert call(ws=None) == 1
    assert call(wsb=ws.numel() - 4) == 7
    assert call(flags=ssm.SSM_FLAG_CHECKPOINTS) == 6
    assert call(y=p(x)) == 5
    assert call(ws=p(x)) == 5
    bad = ssm.BldLayout()
    bad.x_step = dim - 1
    assert call(lay=ctypes_ref(bad)) == 2
    bad = ssm.BldLayout()
    bad.C_batch = L * N - 1
    assert call(lay=ctypes_ref(bad)) == 2
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())


def ctypes_ref(s):
    import ctypes
    return ctypes.byref(s)
