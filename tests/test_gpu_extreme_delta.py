"""Step sizes at both ends of softplus, against the fp64 oracle: channels with
dt_bias = -40 (Delta ~ 4e-18: the state is frozen, y = (C h0 + D x) silu(z)),
channels with dt_bias = +40 (Delta ~ 40: the state resets to Delta B x at
every step) and ordinary channels side by side, for the forward in both forms
of B-bar, the backward pass and decode steps (the oracle's own pins fix both
limits)."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_64_amd as ssm
from selective_state_space_64_amd import synth
from helpers import TOL_F32, oracle_full, rel_err, to_dev, workload

pytestmark = pytest.mark.gpu


def _inputs(batch, dim, N, L, seed):
    inp = synth.make_inputs(workload("extremeDelta", batch, dim, N, L, "f32", seed=seed), with_h0=True)
    bias = inp.dt_bias.copy()
    bias[0::3] = -40.0
    bias[1::3] = 40.0
    inp.dt_bias[:] = bias
    return inp


def _dev_h0(inp):
    return torch.from_numpy(inp.h0.astype(np.float32)).cuda()


@pytest.mark.parametrize("zoh", [False, True], ids=["delta_b", "zoh"])
def test_forward_extreme_delta(zoh):
    batch, dim, N, L = 2, 33, 16, 400
    inp = _inputs(batch, dim, N, L, seed=91)
    y, hL = ssm.ssm_scan_fwd(
        to_dev(inp, "x"), to_dev(inp, "dt"), to_dev(inp, "A"), to_dev(inp, "Bm"), to_dev(inp, "Cm"),
        dt_bias=to_dev(inp, "dt_bias"), Dskip=to_dev(inp, "Dskip"), z=to_dev(inp, "z"), h0=_dev_h0(inp),
        zoh=zoh)
    torch.cuda.synchronize()
    ry, rh = oracle_full(inp, h0=inp.h0, zoh=zoh)
    assert rel_err(y.cpu().numpy(), ry) <= TOL_F32 and rel_err(hL.cpu().numpy(), rh) <= TOL_F32
    # the frozen channels keep h0 exactly: Delta A rounds to an exponent of 0
    # and Delta B x vanishes next to h0
    frozen = slice(0, dim, 3)
    assert torch.equal(hL[:, frozen], _dev_h0(inp)[:, frozen])


@pytest.mark.parametrize("zoh", [False, True], ids=["delta_b", "zoh"])
def test_backward_extreme_delta(zoh):
    batch, dim, N, L = 2, 33, 16, 300
    inp = _inputs(batch, dim, N, L, seed=92)
    dy = np.random.default_rng(93).standard_normal((batch, dim, L)).astype(np.float32)
    g = ssm.ssm_scan_bwd(to_dev(inp, "x"), to_dev(inp, "dt"), to_dev(inp, "A"), to_dev(inp, "Bm"),
                         to_dev(inp, "Cm"), torch.from_numpy(dy).cuda(), dt_bias=to_dev(inp, "dt_bias"),
                         Dskip=to_dev(inp, "Dskip"), z=to_dev(inp, "z"), h0=_dev_h0(inp), zoh=zoh)
    torch.cuda.synchronize()
    r = oracle.scan_bwd(inp.values("x"), inp.values("dt"), inp.A.astype(np.float64), inp.values("Bm"),
                        inp.values("Cm"), dy.astype(np.float64), dt_bias=inp.dt_bias.astype(np.float64),
                        Dskip=inp.Dskip.astype(np.float64), z=inp.values("z"),
                        h0=inp.h0.astype(np.float64), zoh=zoh)
    errs = {k: rel_err(g[k].cpu().numpy(), r[k]) for k in ("dx", "ddt", "dz", "dBm", "dCm", "dA", "dh0")}
    errs.update({k: rel_err(g[k].cpu().numpy()[None], r[k][None]) for k in ("dDskip", "ddt_bias")})
    print("  " + " ".join("%s %.1e" % kv for kv in errs.items()), flush=True)
    for k, e in errs.items():
        assert e <= TOL_F32, (k, errs)


@pytest.mark.parametrize("zoh", [False, True], ids=["delta_b", "zoh"])
def test_decode_extreme_delta(zoh):
    batch, dim, N, steps = 3, 33, 16, 5
    inp = _inputs(batch, dim, N, steps, seed=94)
    state = _dev_h0(inp)
    t = {k: to_dev(inp, k) for k in ("x", "dt", "z", "Bm", "Cm", "A", "Dskip", "dt_bias")}
    ys = []
    for s in range(steps):
        ys.append(ssm.ssm_state_update(state, t["x"][:, :, s].contiguous(), t["dt"][:, :, s].contiguous(),
                                       t["A"], t["Bm"][:, :, s].contiguous(), t["Cm"][:, :, s].contiguous(),
                                       dt_bias=t["dt_bias"], Dskip=t["Dskip"], z=t["z"][:, :, s].contiguous(),
                                       zoh=zoh))
    torch.cuda.synchronize()
    ry, rh = oracle_full(inp, h0=inp.h0, zoh=zoh)
    gy = torch.stack(ys).cpu().numpy()  # [steps, batch, dim]: rows over channels
    assert rel_err(gy, np.transpose(ry, (2, 0, 1))) <= TOL_F32
    assert rel_err(state.transpose(1, 2).cpu().numpy(), np.transpose(rh, (0, 2, 1))) <= TOL_F32
