"""GPU parity of the exact zero-order-hold B-bar (SSM_FLAG_ZOH_B) against the
fp64 oracle's ZOH mode, which the hand-derived L = 1 example and the
gated-RNN identity pin ("Method" and "The selection mechanism (S6)" sections
of "Mamba: Linear-Time Sequence Modeling with Selective State Spaces")."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_64_amd as ssm
from selective_state_space_64_amd import synth
from helpers import oracle_full, oracle_rows, rel_err, sample_rows, to_dev, tol_for, workload

pytestmark = pytest.mark.gpu


def _scan(inp, h0=None, **kw):
    y, hL = ssm.ssm_scan_fwd(
        to_dev(inp, "x"), to_dev(inp, "dt"), to_dev(inp, "A"), to_dev(inp, "Bm"), to_dev(inp, "Cm"),
        dt_bias=to_dev(inp, "dt_bias"), Dskip=to_dev(inp, "Dskip"), z=to_dev(inp, "z"),
        h0=None if h0 is None else torch.from_numpy(h0).cuda(), zoh=True, **kw)
    torch.cuda.synchronize()
    return y, hL


@pytest.mark.parametrize("shape", [(2, 16, 16, 300, "f32"), (1, 21, 8, 1031, "bf16"),
                                   (2, 5, 1, 77, "f32"), (1, 3, 16, 5, "bf16")],
                         ids=lambda s: "b%d_d%d_N%d_L%d_%s" % s)
def test_zoh_scan_full(shape):
    batch, dim, N, L, dt = shape
    inp = synth.make_inputs(workload("zoh", batch, dim, N, L, dt), with_h0=True)
    y, hL = _scan(inp, h0=inp.h0)
    ry, rh = oracle_full(inp, h0=inp.h0, zoh=True)
    tol = tol_for(dt)
    assert rel_err(y.cpu().numpy(), ry) <= tol and rel_err(hL.cpu().numpy(), rh) <= tol


def test_zoh_zero_A_equals_delta_form():
    """A = 0: the ZOH factor is exactly 1 (limit Delta B), both modes agree."""
    inp = synth.make_inputs(workload("zohA0", 2, 20, 16, 400, "f32"))
    inp.A[:] = 0.0
    y1, h1 = _scan(inp)
    y2, h2 = ssm.ssm_scan_fwd(
        to_dev(inp, "x"), to_dev(inp, "dt"), to_dev(inp, "A"), to_dev(inp, "Bm"), to_dev(inp, "Cm"),
        dt_bias=to_dev(inp, "dt_bias"), Dskip=to_dev(inp, "Dskip"), z=to_dev(inp, "z"))
    torch.cuda.synchronize()
    assert torch.isfinite(y1).all() and torch.isfinite(h1).all()
    assert rel_err(y1.cpu().numpy(), y2.cpu().numpy()) <= 1e-6


def test_zoh_layer_sampled():
    wl = synth.WORKLOADS[1]
    inp = synth.make_inputs(wl)
    y, hL = _scan(inp)
    rows = sample_rows(wl.batch, wl.dim, per_batch=6, seed=9)
    bi = torch.tensor([r[0] for r in rows], device="cuda")
    di = torch.tensor([r[1] for r in rows], device="cuda")
    ys, hs = [], []
    for b, d in rows:
        from helpers import row_problem
        yy, hh = oracle.scan_fwd(**row_problem(inp, b, d), zoh=True)
        ys.append(yy[0, 0]); hs.append(hh[0, 0])
    ey = rel_err(y[bi, di].cpu().numpy(), np.stack(ys))
    eh = rel_err(hL[bi, di].cpu().numpy(), np.stack(hs))
    print("zoh %s: err y %.3e hL %.3e" % (wl.name, ey, eh), flush=True)
    assert ey <= tol_for("bf16") and eh <= tol_for("bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zoh_decode_matches_oracle(dtype):
    inp = synth.make_inputs(workload("zohdec", 3, 40, 16, 6, dtype), with_h0=True)
    state = torch.from_numpy(inp.h0).cuda()
    ref = inp.values("h0")
    for s in range(6):
        sl = lambda name: to_dev(inp, name)[..., s].contiguous()
        y = ssm.ssm_state_update(state, sl("x"), sl("dt"), to_dev(inp, "A"), sl("Bm"), sl("Cm"),
                                 dt_bias=to_dev(inp, "dt_bias"), Dskip=to_dev(inp, "Dskip"),
                                 z=sl("z"), zoh=True)
        ry, ref = oracle.state_update(ref, inp.values("x")[..., s], inp.values("dt")[..., s],
                                      inp.values("A"), inp.values("Bm")[..., s],
                                      inp.values("Cm")[..., s], dt_bias=inp.values("dt_bias"),
                                      Dskip=inp.values("Dskip"), z=inp.values("z")[..., s], zoh=True)
        torch.cuda.synchronize()
        assert rel_err(y.cpu().numpy(), ry) <= tol_for(dtype), s
    assert rel_err(state.cpu().numpy(), ref) <= tol_for(dtype)


# ------------------------------------------------------------ backward pass
ZOH_BWD = [
    # (batch, dim, N, L, dtype)
    (2, 16, 16, 300, "f32"), (1, 17, 8, 1000, "bf16"), (2, 5, 4, 777, "f32"),
    (1, 20, 16, 5000, "f32"),  # split along the sequence
]


@pytest.mark.parametrize("shape", ZOH_BWD, ids=lambda s: "b%d_d%d_N%d_L%d_%s" % s)
def test_zoh_bwd_full_tensor(shape):
    """The backward of the exact ZOH form (SSM_FLAG_ZOH_B) against the oracle's
    ZOH backward, every gradient in full; the checkpoints are recomputed in
    the call and, again, handed over by a ZOH forward with
    SSM_FLAG_CHECKPOINTS (the two must agree)."""
    import oracle
    batch, dim, N, L, dt = shape
    print("zoh bwd", shape, flush=True)
    inp = synth.make_inputs(workload("zoh_bwd", batch, dim, N, L, dt, seed=71), with_h0=True)
    rng = np.random.default_rng(8)
    dyv = rng.standard_normal((batch, dim, L)).astype(np.float32)
    dhL = rng.standard_normal((batch, dim, N)).astype(np.float32)
    t = {k: to_dev(inp, k) for k in ("x", "dt", "z", "Bm", "Cm", "A", "Dskip", "dt_bias")}
    h0 = torch.from_numpy(inp.h0.astype(np.float32)).cuda()
    kw = dict(dt_bias=t["dt_bias"], Dskip=t["Dskip"], z=t["z"], h0=h0)
    dy = torch.from_numpy(dyv).cuda()
    g = ssm.ssm_scan_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dy,
                         dhL=torch.from_numpy(dhL).cuda(), zoh=True, **kw)
    ws = torch.zeros(ssm.lib().ssm_scan_bwd_workspace_bytes(batch, dim, L, N), dtype=torch.uint8,
                     device="cuda")
    y, _ = ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], zoh=True, checkpoints=ws,
                            **kw)
    g2 = ssm.ssm_scan_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dy,
                          dhL=torch.from_numpy(dhL).cuda(), zoh=True, workspace=ws,
                          checkpoints_in_workspace=True, **kw)
    torch.cuda.synchronize()
    r = oracle.scan_bwd(inp.values("x"), inp.values("dt"), inp.A.astype(np.float64),
                        inp.values("Bm"), inp.values("Cm"), dyv.astype(np.float64),
                        dt_bias=inp.dt_bias.astype(np.float64), Dskip=inp.Dskip.astype(np.float64),
                        z=inp.values("z"), h0=inp.h0.astype(np.float64),
                        dhL=dhL.astype(np.float64), zoh=True)
    ry, _ = oracle_full(inp, h0=inp.h0, zoh=True)
    assert rel_err(y.cpu().numpy(), ry) <= tol_for(dt)
    for k in ("dx", "ddt", "dz", "dBm", "dCm", "dh0"):
        e = rel_err(g[k].cpu().numpy(), r[k])
        assert e <= 1e-4, (shape, k, e)
        assert rel_err(g2[k].cpu().numpy(), g[k].cpu().numpy()) <= 1e-5, k
    for k in ("dA", "dDskip", "ddt_bias"):
        e = rel_err(g[k].cpu().numpy()[None], r[k][None])
        assert e <= 1e-4, (shape, k, e)
