"""GPU parity of the sequence-split forward scan against the fp64 oracle.

Shapes with few batch rows and channels and a long sequence are split into
segments scanned by separate workgroups: an aggregate pass gives every
segment but the last its end state and Delta sum, and the main pass enters
each segment with the earlier ones composed.  Full-tensor comparisons at
split shapes (ragged last segments, every state size, both dtypes, with and
without gate, skip, bias and h0, hL written over h0, exact ZOH, strided
views), the checkpoints a split forward writes for the backward pass, and the
workspace rules through the binding.
"""
import numpy as np
import pytest
import torch

import selective_state_space_64_amd as ssm
from selective_state_space_64_amd import synth
from helpers import oracle_full, rel_err, to_dev, tol_for, workload

pytestmark = pytest.mark.gpu


def _nseg(batch, dim, L):
    need = ssm.lib().ssm_scan_fwd_workspace_bytes(batch, dim, L, 16)
    return need // (batch * dim * 17 * 4)


def _run(inp, gate=True, skip=True, bias=True, h0=None, **kw):
    y, hL = ssm.ssm_scan_fwd(
        to_dev(inp, "x"), to_dev(inp, "dt"), to_dev(inp, "A"), to_dev(inp, "Bm"), to_dev(inp, "Cm"),
        dt_bias=to_dev(inp, "dt_bias") if bias else None,
        Dskip=to_dev(inp, "Dskip") if skip else None,
        z=to_dev(inp, "z") if gate else None,
        h0=None if h0 is None else torch.from_numpy(np.asarray(h0, np.float32)).cuda(), **kw)
    torch.cuda.synchronize()
    return y, hL


SPLIT = [
    # (batch, dim, N, L, dtype): all split by the library's rule
    (1, 16, 16, 4096, "bf16"), (1, 20, 16, 5000, "f32"), (2, 3, 8, 3001, "bf16"),
    (1, 5, 4, 10000, "f32"), (1, 40, 2, 2048, "bf16"), (3, 7, 1, 6000, "f32"),
    (1, 1, 16, 20000, "bf16"),
]


@pytest.mark.parametrize("shape", SPLIT, ids=lambda s: "b%d_d%d_N%d_L%d_%s" % s)
def test_split_full_tensor(shape):
    batch, dim, N, L, dt = shape
    print("split", shape, flush=True)
    assert ssm.lib().ssm_scan_fwd_workspace_bytes(batch, dim, L, N) > 0
    inp = synth.make_inputs(workload("split", batch, dim, N, L, dt, seed=21), with_h0=True)
    for gate, skip, bias, use_h0 in [(True, True, True, True), (False, False, False, False),
                                     (True, False, True, False)]:
        h0 = inp.h0 if use_h0 else None
        y, hL = _run(inp, gate, skip, bias, h0)
        ry, rh = oracle_full(inp, gate, skip, bias, h0)
        ey, eh = rel_err(y.cpu().numpy(), ry), rel_err(hL.cpu().numpy(), rh)
        assert ey <= tol_for(dt) and eh <= tol_for(dt), (shape, gate, skip, bias, use_h0, ey, eh)


def test_split_segment_count():
    """The shapes above really are split, into the expected segment counts."""
    assert _nseg(1, 16, 4096) == 4           # 1 workgroup, 1024-step segments
    assert _nseg(1, 1536, 1 << 20) == 164    # 96 workgroups, 6400-step segments
    assert _nseg(4, 5120, 2048) == 0         # 1280 workgroups: not split


def test_split_hL_over_h0_in_place():
    """hL may be the h0 buffer: the main pass reads a copy of h0 made by the
    aggregate pass, so the last segment's hL cannot race with the first
    segment's read of h0."""
    batch, dim, N, L = 2, 24, 16, 8192
    inp = synth.make_inputs(workload("split_inplace", batch, dim, N, L, "bf16", seed=22),
                            with_h0=True)
    st = torch.from_numpy(inp.h0.astype(np.float32)).cuda()
    y, hL = ssm.ssm_scan_fwd(to_dev(inp, "x"), to_dev(inp, "dt"), to_dev(inp, "A"),
                             to_dev(inp, "Bm"), to_dev(inp, "Cm"), dt_bias=to_dev(inp, "dt_bias"),
                             Dskip=to_dev(inp, "Dskip"), z=to_dev(inp, "z"), h0=st, hL=st)
    torch.cuda.synchronize()
    assert hL.data_ptr() == st.data_ptr()
    ry, rh = oracle_full(inp, h0=inp.h0)
    assert rel_err(y.cpu().numpy(), ry) <= tol_for("bf16")
    assert rel_err(st.cpu().numpy(), rh) <= tol_for("bf16")


def test_split_chained_calls_match_whole():
    """Two split calls chained through h0/hL match the oracle over the whole
    sequence (sequence sharding across calls on top of the split inside)."""
    batch, dim, N, L = 1, 32, 16, 12288
    inp = synth.make_inputs(workload("split_chain", batch, dim, N, L, "f32", seed=23))
    t = {k: to_dev(inp, k) for k in ("x", "dt", "z", "Bm", "Cm", "A", "Dskip", "dt_bias")}
    cut = 5120
    part = lambda k, a, b: t[k][:, :, a:b].contiguous()
    y1, h1 = ssm.ssm_scan_fwd(part("x", 0, cut), part("dt", 0, cut), t["A"], part("Bm", 0, cut),
                              part("Cm", 0, cut), dt_bias=t["dt_bias"], Dskip=t["Dskip"],
                              z=part("z", 0, cut))
    y2, h2 = ssm.ssm_scan_fwd(part("x", cut, L), part("dt", cut, L), t["A"], part("Bm", cut, L),
                              part("Cm", cut, L), dt_bias=t["dt_bias"], Dskip=t["Dskip"],
                              z=part("z", cut, L), h0=h1)
    torch.cuda.synchronize()
    ry, rh = oracle_full(inp)
    assert rel_err(torch.cat([y1, y2], dim=2).cpu().numpy(), ry) <= tol_for("f32")
    assert rel_err(h2.cpu().numpy(), rh) <= tol_for("f32")


def test_split_zoh():
    batch, dim, N, L = 1, 12, 16, 6144
    inp = synth.make_inputs(workload("split_zoh", batch, dim, N, L, "bf16", seed=24), with_h0=True)
    y, hL = _run(inp, h0=inp.h0, zoh=True)
    ry, rh = oracle_full(inp, h0=inp.h0, zoh=True)
    assert rel_err(y.cpu().numpy(), ry) <= tol_for("bf16")
    assert rel_err(hL.cpu().numpy(), rh) <= tol_for("bf16")


def test_split_strided_views():
    """x/z halves of one buffer and y into half of a larger one, at a split
    shape; the other half of y's buffer stays untouched."""
    batch, dim, N, L = 2, 10, 16, 4096
    inp = synth.make_inputs(workload("split_strided", batch, dim, N, L, "bf16", seed=25))
    xz = torch.cat([to_dev(inp, "x"), to_dev(inp, "z")], dim=1)
    ybuf = torch.full((batch, 2 * dim, L), 12345.0, device="cuda")
    y, hL = ssm.ssm_scan_fwd(xz[:, :dim], to_dev(inp, "dt"), to_dev(inp, "A"), to_dev(inp, "Bm"),
                             to_dev(inp, "Cm"), dt_bias=to_dev(inp, "dt_bias"),
                             Dskip=to_dev(inp, "Dskip"), z=xz[:, dim:], y=ybuf[:, dim:])
    torch.cuda.synchronize()
    ry, rh = oracle_full(inp)
    assert rel_err(y.cpu().numpy(), ry) <= tol_for("bf16")
    assert rel_err(hL.cpu().numpy(), rh) <= tol_for("bf16")
    assert bool((ybuf[:, :dim] == 12345.0).all())


def test_split_forward_checkpoints_feed_backward():
    """A split forward with SSM_FLAG_CHECKPOINTS writes the same checkpoints
    the backward pass computes itself (within rounding: the split composes
    segments), and the backward from them matches the oracle's gradients."""
    import oracle
    batch, dim, N, L = 1, 16, 16, 4096
    assert _nseg(batch, dim, L) > 1
    inp = synth.make_inputs(workload("split_ck", batch, dim, N, L, "f32", seed=26), with_h0=True)
    t = {k: to_dev(inp, k) for k in ("x", "dt", "z", "Bm", "Cm", "A", "Dskip", "dt_bias")}
    h0 = torch.from_numpy(inp.h0.astype(np.float32)).cuda()
    nbytes = ssm.lib().ssm_scan_bwd_workspace_bytes(batch, dim, L, N)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    y, _ = ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                            Dskip=t["Dskip"], z=t["z"], h0=h0, checkpoints=ws)
    ry, _ = oracle_full(inp, h0=inp.h0)
    assert rel_err(y.cpu().numpy(), ry) <= tol_for("f32")
    g = np.random.default_rng(3).standard_normal((batch, dim, L)).astype(np.float32)
    dy = torch.from_numpy(g).cuda()
    kw = dict(dt_bias=t["dt_bias"], Dskip=t["Dskip"], z=t["z"], h0=h0)
    ga = ssm.ssm_scan_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dy, workspace=ws,
                          checkpoints_in_workspace=True, **kw)
    gb = ssm.ssm_scan_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dy, **kw)
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(inp.values("x"), inp.values("dt"), inp.A.astype(np.float64),
                          inp.values("Bm"), inp.values("Cm"), g.astype(np.float64),
                          dt_bias=inp.dt_bias.astype(np.float64), Dskip=inp.Dskip.astype(np.float64),
                          z=inp.values("z"), h0=inp.h0.astype(np.float64))
    for k in ("dx", "ddt", "dz", "dBm", "dCm", "dA", "dh0"):
        a, b = ga[k].cpu().numpy(), gb[k].cpu().numpy()
        assert rel_err(a, ref[k]) <= 1e-4, (k, rel_err(a, ref[k]))
        assert rel_err(a, b) <= 1e-4, k


def test_split_workspace_given_and_rejected():
    """A caller-provided workspace is used as is; one too small is rejected
    with nothing written."""
    batch, dim, N, L = 1, 16, 16, 4096
    inp = synth.make_inputs(workload("split_ws", batch, dim, N, L, "bf16", seed=27))
    need = ssm.lib().ssm_scan_fwd_workspace_bytes(batch, dim, L, N)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y, hL = _run(inp, workspace=ws)
    ry, rh = oracle_full(inp)
    assert rel_err(y.cpu().numpy(), ry) <= tol_for("bf16")
    y0 = torch.full((batch, dim, L), 7.0, device="cuda")
    with pytest.raises(ssm.SSMError) as e:
        _run(inp, workspace=ws[:need - 4], y=y0)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert bool((y0 == 7.0).all())


# ------------------------------------------------------------ backward pass
SPLIT_BWD = [
    # (batch, dim, N, L, dtype): split by the library's rule
    (1, 16, 16, 4096, "f32"), (2, 3, 8, 3001, "bf16"), (1, 20, 16, 5000, "f32"),
    (1, 5, 4, 10000, "bf16"),
]


@pytest.mark.parametrize("shape", SPLIT_BWD, ids=lambda s: "b%d_d%d_N%d_L%d_%s" % s)
def test_split_bwd_full_tensor(shape):
    """The backward pass at split shapes: checkpoints from the split forward
    kernel, adjoint aggregates of the later segments, every segment's reverse
    pass at once; every gradient against the oracle, with h0, dhL and the gate."""
    import oracle
    batch, dim, N, L, dt = shape
    print("split bwd", shape, flush=True)
    assert ssm.lib().ssm_scan_fwd_workspace_bytes(batch, dim, L, N) > 0
    inp = synth.make_inputs(workload("split_bwd", batch, dim, N, L, dt, seed=28), with_h0=True)
    rng = np.random.default_rng(6)
    dyv = rng.standard_normal((batch, dim, L)).astype(np.float32)
    dhL = rng.standard_normal((batch, dim, N)).astype(np.float32)
    g = ssm.ssm_scan_bwd(to_dev(inp, "x"), to_dev(inp, "dt"), to_dev(inp, "A"), to_dev(inp, "Bm"),
                         to_dev(inp, "Cm"), torch.from_numpy(dyv).cuda(),
                         dt_bias=to_dev(inp, "dt_bias"), Dskip=to_dev(inp, "Dskip"),
                         z=to_dev(inp, "z"), h0=torch.from_numpy(inp.h0.astype(np.float32)).cuda(),
                         dhL=torch.from_numpy(dhL).cuda())
    torch.cuda.synchronize()
    r = oracle.scan_bwd(inp.values("x"), inp.values("dt"), inp.A.astype(np.float64),
                        inp.values("Bm"), inp.values("Cm"), dyv.astype(np.float64),
                        dt_bias=inp.dt_bias.astype(np.float64), Dskip=inp.Dskip.astype(np.float64),
                        z=inp.values("z"), h0=inp.h0.astype(np.float64),
                        dhL=dhL.astype(np.float64))
    for k in ("dx", "ddt", "dz", "dBm", "dCm", "dh0"):
        e = rel_err(g[k].cpu().numpy(), r[k])
        assert e <= 1e-4, (shape, k, e)
    for k in ("dA", "dDskip", "ddt_bias"):
        e = rel_err(g[k].cpu().numpy()[None], r[k][None])
        assert e <= 1e-4, (shape, k, e)
