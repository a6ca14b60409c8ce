"""GPU parity of ssm_state_update (through the C ABI) against the fp64 oracle:
the 256-step decode workload on a [64, 5120, 16] fp32 state updated in place
(in full),
small shapes compared in full, and shapes that take the four-rows-per-lane
launch compared in full.  The oracle side runs the same steps as
one scan from the initial state (the decode recurrence and the scan are the
same function; the oracle's own pins show it)."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_64_amd as ssm
from selective_state_space_64_amd import synth
from helpers import TOL_BF16_OUT, oracle_full, rel_err, sample_rows, to_dev, tol_for, workload

pytestmark = pytest.mark.gpu


def _steps(t):
    """[batch, X, steps] -> [steps, batch, X] contiguous per-step slices."""
    return t.permute(2, 0, 1).contiguous()


def _run_decode(inp, steps, gate=True, out_dtype=torch.float32, zoh=False):
    state = torch.from_numpy(inp.h0.astype(np.float32)).cuda()
    xs, dts, zs = _steps(to_dev(inp, "x")), _steps(to_dev(inp, "dt")), _steps(to_dev(inp, "z"))
    Bs, Cs = _steps(to_dev(inp, "Bm")), _steps(to_dev(inp, "Cm"))
    A, Dk, bias = to_dev(inp, "A"), to_dev(inp, "Dskip"), to_dev(inp, "dt_bias")
    ys = torch.empty((steps,) + tuple(state.shape[:2]), dtype=out_dtype, device="cuda")
    for s in range(steps):
        ssm.ssm_state_update(state, xs[s], dts[s], A, Bs[s], Cs[s], dt_bias=bias, Dskip=Dk,
                             z=zs[s] if gate else None, y=ys[s], out_dtype=out_dtype, zoh=zoh)
    torch.cuda.synchronize()
    return ys, state


def _oracle_decode(inp, rows, gate=True):
    ys, hs = [], []
    for b, d in rows:
        y, hL = oracle.scan_fwd(
            inp.values("x")[b:b + 1, d:d + 1], inp.values("dt")[b:b + 1, d:d + 1],
            inp.A[d:d + 1].astype(np.float64), inp.values("Bm")[b:b + 1], inp.values("Cm")[b:b + 1],
            dt_bias=inp.dt_bias[d:d + 1].astype(np.float64),
            Dskip=inp.Dskip[d:d + 1].astype(np.float64),
            z=inp.values("z")[b:b + 1, d:d + 1] if gate else None,
            h0=inp.h0[b:b + 1, d:d + 1].astype(np.float64))
        ys.append(y[0, 0])
        hs.append(hL[0, 0])
    return np.stack(ys), np.stack(hs)


def test_decode_workload_full():
    """The decode workload in full: 256 steps on the [64, 5120, 16] state,
    every y of every step and every final state value against the oracle
    (the steps run there as one scan from the initial state).  y is compared
    over rows of channels (b, :) per step, the state over (b, d, :)."""
    wl = synth.WORKLOADS[4]
    print("workload", wl.name, flush=True)
    inp = synth.make_inputs(wl)
    ys, state = _run_decode(inp, wl.seqlen)
    gy, gh = ys.cpu().numpy(), state.cpu().numpy()    # [steps, batch, dim], [batch, dim, N]
    del ys, state
    assert np.isfinite(gy).all() and np.isfinite(gh).all()
    ry, rh = oracle_full(inp, h0=inp.h0)             # [batch, dim, steps], [batch, dim, N]
    ey = rel_err(gy, np.transpose(ry, (2, 0, 1)))
    eh = rel_err(gh, rh)
    print("  %d x %d rows x %d steps: err y %.3e state %.3e"
          % (wl.batch, wl.dim, wl.seqlen, ey, eh), flush=True)
    assert ey <= tol_for("bf16") and eh <= tol_for("bf16")


def test_decode_steps_object_matches_calls():
    """StateUpdateSteps (arguments checked once, per step a pointer offset)
    gives the same bits as ssm_state_update called per step, also with some
    inputs given once for every step and x / z as projection halves."""
    inp = synth.make_inputs(workload("decobj", 5, 300, 16, 6, "bf16", seed=41), with_h0=True)
    ys_ref, st_ref = _run_decode(inp, 6)
    state = torch.from_numpy(inp.h0.astype(np.float32)).cuda()
    xz = torch.cat([_steps(to_dev(inp, "x")), _steps(to_dev(inp, "z"))], dim=2)  # [steps, b, 2d]
    xs, zs = xz[..., :300], xz[..., 300:]
    dts = _steps(to_dev(inp, "dt"))
    Bs, Cs = _steps(to_dev(inp, "Bm")), _steps(to_dev(inp, "Cm"))
    A, Dk, bias = to_dev(inp, "A"), to_dev(inp, "Dskip"), to_dev(inp, "dt_bias")
    ys = torch.empty((6, 5, 300), device="cuda")
    run = ssm.StateUpdateSteps(state, A, xs, dts, Bs, Cs, ys=ys, dt_bias=bias, Dskip=Dk, zs=zs)
    for s in range(6):
        run(s)
    torch.cuda.synchronize()
    assert torch.equal(ys, ys_ref) and torch.equal(state, st_ref)
    with pytest.raises(IndexError):
        run(6)
    # Bm given once for every step: equals calls passing the same Bm each time
    state2 = torch.from_numpy(inp.h0.astype(np.float32)).cuda()
    state3 = state2.clone()
    ys2, ys3 = torch.empty_like(ys), torch.empty_like(ys)
    run2 = ssm.StateUpdateSteps(state2, A, xs, dts, Bs[0], Cs, ys=ys2, dt_bias=bias, Dskip=Dk, zs=zs)
    for s in range(6):
        run2(s)
        ssm.ssm_state_update(state3, xs[s], dts[s], A, Bs[0], Cs[s], dt_bias=bias, Dskip=Dk, z=zs[s],
                             y=ys3[s])
    torch.cuda.synchronize()
    assert torch.equal(ys2, ys3) and torch.equal(state2, state3)


@pytest.mark.parametrize("shape", [(3, 7, 16, 5, "f32"), (2, 70, 4, 9, "bf16"), (1, 1, 1, 3, "f32"),
                                   (4, 33, 2, 4, "bf16"), (2, 64, 8, 6, "f32")],
                         ids=lambda s: "b%d_d%d_N%d_steps%d_%s" % s)
def test_decode_small_full(shape):
    batch, dim, N, steps, dt = shape
    inp = synth.make_inputs(workload("dec", batch, dim, N, steps, dt), with_h0=True)
    for gate in (True, False):
        ys, state = _run_decode(inp, steps, gate)
        rows = [(b, d) for b in range(batch) for d in range(dim)]
        ry, rh = _oracle_decode(inp, rows, gate)
        gy = ys.permute(1, 2, 0).reshape(batch * dim, steps).cpu().numpy()
        gh = state.reshape(batch * dim, N).cpu().numpy()
        tol = tol_for(dt)
        assert rel_err(gy, ry) <= tol and rel_err(gh, rh) <= tol, (shape, gate)


@pytest.mark.parametrize("shape", [(300, 1000, 16, 3, "bf16", False), (600, 1000, 8, 3, "f32", False),
                                   (1100, 1000, 4, 2, "bf16", False), (1100, 1000, 1, 2, "f32", False),
                                   (300, 1000, 16, 3, "bf16", True)],
                         ids=lambda s: "b%d_d%d_N%d_steps%d_%s_zoh%d" % s)
def test_decode_four_rows_per_lane_full(shape):
    """Shapes large enough for the launch that gives each lane four (b, d)
    rows, with a dim that leaves rows of the last workgroup dead, one of them
    with the exact zero-order-hold B-bar: every y and state value against the
    oracle (the steps run as one scan)."""
    batch, dim, N, steps, dt, zoh = shape
    inp = synth.make_inputs(workload("dec4", batch, dim, N, steps, dt, seed=31), with_h0=True)
    ys, state = _run_decode(inp, steps, zoh=zoh)
    ry, rh = oracle_full(inp, h0=inp.h0, zoh=zoh)
    # y and the state are compared over rows of channels, (b, :) per step and
    # (b, :, n) per state: a row over only 2-3 steps or N = 1 states would turn
    # the rounding of a value that cancels to near zero into a relative error
    gy = ys.cpu().numpy()                      # [steps, batch, dim]
    tol = tol_for(dt)
    ey = rel_err(gy, np.transpose(ry, (2, 0, 1)))
    eh = rel_err(state.transpose(1, 2).cpu().numpy(), np.transpose(rh, (0, 2, 1)))
    print("  %s: err y %.3e state %.3e" % (shape, ey, eh), flush=True)
    assert ey <= tol and eh <= tol
    if N == 16 and not zoh:
        # the same steps on projection halves (x, z of one [batch, 2 dim] row,
        # y into half of another): equal bit for bit to the dense calls
        state2 = torch.from_numpy(inp.h0.astype(np.float32)).cuda()
        xz = torch.cat([_steps(to_dev(inp, "x")), _steps(to_dev(inp, "z"))], dim=2)
        dts, Bs, Cs = _steps(to_dev(inp, "dt")), _steps(to_dev(inp, "Bm")), _steps(to_dev(inp, "Cm"))
        A, Dk, bias = to_dev(inp, "A"), to_dev(inp, "Dskip"), to_dev(inp, "dt_bias")
        ybuf = torch.full((steps, batch, 2 * dim), 555.0, device="cuda")
        for st in range(steps):
            ssm.ssm_state_update(state2, xz[st, :, :dim], dts[st], A, Bs[st], Cs[st], dt_bias=bias,
                                 Dskip=Dk, z=xz[st, :, dim:], y=ybuf[st, :, :dim])
        torch.cuda.synchronize()
        assert torch.equal(ybuf[:, :, :dim], ys) and torch.equal(state2, state)
        assert bool((ybuf[:, :, dim:] == 555.0).all())


def test_decode_bf16_output():
    inp = synth.make_inputs(workload("dec16", 2, 40, 16, 4, "bf16"), with_h0=True)
    ys, state = _run_decode(inp, 4, out_dtype=torch.bfloat16)
    rows = [(b, d) for b in range(2) for d in range(40)]
    ry, rh = _oracle_decode(inp, rows)
    gy = ys.float().permute(1, 2, 0).reshape(80, 4).cpu().numpy()
    assert rel_err(gy, ry) <= TOL_BF16_OUT


def test_decode_steps_in_hip_graph():
    """The decode step allocates nothing and issues no memset, so a loop of
    steps can be captured once in a HIP graph and replayed; every replay
    (from the same initial state, reset eagerly in between) matches the eager
    loop bit for bit."""
    inp = synth.make_inputs(workload("decg", 4, 96, 16, 8, "bf16"), with_h0=True)
    steps = 8
    state0 = torch.from_numpy(inp.h0.astype(np.float32)).cuda()
    state = state0.clone()
    xs, dts, zs = _steps(to_dev(inp, "x")), _steps(to_dev(inp, "dt")), _steps(to_dev(inp, "z"))
    Bs, Cs = _steps(to_dev(inp, "Bm")), _steps(to_dev(inp, "Cm"))
    A, Dk, bias = to_dev(inp, "A"), to_dev(inp, "Dskip"), to_dev(inp, "dt_bias")
    ys = torch.empty((steps, 4, 96), device="cuda")

    def loop():
        for s in range(steps):
            ssm.ssm_state_update(state, xs[s], dts[s], A, Bs[s], Cs[s], dt_bias=bias, Dskip=Dk,
                                 z=zs[s], y=ys[s])

    loop()
    torch.cuda.synchronize()
    ref_y, ref_state = ys.clone(), state.clone()

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
    for _ in range(3):
        state.copy_(state0)
        ys.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys, ref_y) and torch.equal(state, ref_state)


def test_decode_on_projection_slices():
    """The decode step's inputs as slices of its projection rows: x and z
    halves of one [batch, 2 dim] row per step, Bm and Cm parts of one
    [batch, r + 2N] row per step, y into half of a [batch, 2 dim] buffer,
    and the conv's decode step reading the same x half.  Equal bit for bit
    to the dense calls, y's other half untouched, and against the oracle."""
    batch, dim, N, steps, r = 5, 70, 16, 6, 12
    inp = synth.make_inputs(workload("decode_slices", batch, dim, N, steps, "bf16", seed=41),
                            with_h0=True)
    ys0, st0 = _run_decode(inp, steps)
    state = torch.from_numpy(inp.h0.astype(np.float32)).cuda()
    xs, dts, zs = _steps(to_dev(inp, "x")), _steps(to_dev(inp, "dt")), _steps(to_dev(inp, "z"))
    Bs, Cs = _steps(to_dev(inp, "Bm")), _steps(to_dev(inp, "Cm"))
    xz = torch.cat([xs, zs], dim=2)                                   # [steps, batch, 2 dim]
    pad = torch.zeros(steps, batch, r, dtype=torch.bfloat16, device="cuda")
    xdbl = torch.cat([pad, Bs, Cs], dim=2)                            # [steps, batch, r + 2N]
    A, Dk, bias = to_dev(inp, "A"), to_dev(inp, "Dskip"), to_dev(inp, "dt_bias")
    ybuf = torch.full((steps, batch, 2 * dim), 555.0, device="cuda")
    for s in range(steps):
        ssm.ssm_state_update(state, xz[s, :, :dim], dts[s], A, xdbl[s, :, r:r + N],
                             xdbl[s, :, r + N:], dt_bias=bias, Dskip=Dk, z=xz[s, :, dim:],
                             y=ybuf[s, :, dim:])
    torch.cuda.synchronize()
    assert torch.equal(ybuf[:, :, dim:], ys0) and torch.equal(state, st0)
    assert bool((ybuf[:, :, :dim] == 555.0).all())
    rows = [(b, d) for b in range(batch) for d in (0, 1, 33, dim - 1)]
    ry, rh = _oracle_decode(inp, rows)
    gy = torch.stack([ybuf[:, b, dim + d] for b, d in rows]).cpu().numpy()
    assert rel_err(gy, ry) <= tol_for("bf16")
    # the conv's decode step on the same x half
    W = 4
    w, cb = synth.conv_parameters(inp.wl, W)
    wt, bt = torch.from_numpy(w).cuda(), torch.from_numpy(cb).cuda()
    cs0 = torch.zeros(batch, dim, W - 1, device="cuda")
    cs1 = torch.zeros(batch, dim, W - 1, device="cuda")
    for s in range(steps):
        a = ssm.ssm_conv1d_update(cs0, xs[s], wt, bias=bt, out_dtype=torch.float32)
        ob = torch.full((batch, 2 * dim), 9.0, device="cuda")
        b_ = ssm.ssm_conv1d_update(cs1, xz[s, :, :dim], wt, bias=bt, out_dtype=torch.float32,
                                   y=ob[:, :dim])
        torch.cuda.synchronize()
        assert torch.equal(a, b_) and bool((ob[:, dim:] == 9.0).all())
    assert torch.equal(cs0, cs1)
