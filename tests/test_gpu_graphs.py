"""The compute entry points inside HIP graphs (captured through torch's
graph API on the caller's stream).

None of the kernels allocates, and no entry point issues a memset (the
backward pass clears its sums with a kernel), so whole steps can be captured
once and replayed.  Each test runs the step eagerly, captures it, and
replays it several times with eager work and synchronisations in between;
every replay must match the eager result: bit for bit where no atomics are
involved, within fp32 rounding for the sums the backward accumulates with
atomic adds (their order is not fixed).
"""
import numpy as np
import pytest
import torch

import selective_state_space_64_amd as ssm
from selective_state_space_64_amd import synth
from helpers import rel_err, to_dev, workload

pytestmark = pytest.mark.gpu


def _capture(step):
    """Eager reference, then a graph of the same step (warm-up on a side
    stream first, as torch's capture requires)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = step()
    return graph, out


def test_training_step_in_graph():
    """Forward writing the checkpoints, then the backward reading them, as one
    captured step."""
    batch, dim, N, L = 2, 48, 16, 1000
    inp = synth.make_inputs(workload("graph_train", batch, dim, N, L, "bf16", seed=61),
                            with_h0=True)
    t = {k: to_dev(inp, k) for k in ("x", "dt", "z", "Bm", "Cm", "A", "Dskip", "dt_bias")}
    h0 = torch.from_numpy(inp.h0.astype(np.float32)).cuda()
    dy = torch.randn(batch, dim, L, device="cuda")
    ws = torch.zeros(ssm.lib().ssm_scan_bwd_workspace_bytes(batch, dim, L, N), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty(batch, dim, L, device="cuda")
    hL = torch.empty(batch, dim, N, device="cuda")
    grads = {k: torch.empty(batch, dim, L, device="cuda") for k in ("dx", "ddt", "dz")}
    kw = dict(dt_bias=t["dt_bias"], Dskip=t["Dskip"], z=t["z"], h0=h0)

    def step():
        ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], y=y, hL=hL, checkpoints=ws, **kw)
        return ssm.ssm_scan_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dy, workspace=ws,
                                checkpoints_in_workspace=True, **grads, **kw)

    g_ref = {k: v.clone() for k, v in step().items() if v is not None}
    y_ref, hL_ref = y.clone(), hL.clone()
    graph, g_cap = _capture(step)
    for _ in range(3):
        for v in (y, hL, *grads.values(), *[v for v in g_cap.values() if v is not None]):
            v.fill_(float("nan"))
        ws.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(hL, hL_ref)
        for k in ("dx", "ddt", "dz", "dh0"):
            assert torch.equal(g_cap[k], g_ref[k]), k
        for k in ("dBm", "dCm", "dA", "dDskip", "ddt_bias"):
            assert rel_err(g_cap[k].cpu().numpy(), g_ref[k].cpu().numpy()) <= 1e-6, k


def test_split_forward_in_graph():
    """A shape the library splits along the sequence (aggregate pass + main
    pass), with its workspace given, captured and replayed."""
    batch, dim, N, L = 1, 32, 16, 8192
    assert ssm.lib().ssm_scan_fwd_workspace_bytes(batch, dim, L, N) > 0
    inp = synth.make_inputs(workload("graph_split", batch, dim, N, L, "f32", seed=62),
                            with_h0=True)
    t = {k: to_dev(inp, k) for k in ("x", "dt", "z", "Bm", "Cm", "A", "Dskip", "dt_bias")}
    h0 = torch.from_numpy(inp.h0.astype(np.float32)).cuda()
    ws = torch.empty(ssm.lib().ssm_scan_fwd_workspace_bytes(batch, dim, L, N), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty(batch, dim, L, device="cuda")
    hL = torch.empty(batch, dim, N, device="cuda")

    def step():
        return ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                                Dskip=t["Dskip"], z=t["z"], h0=h0, y=y, hL=hL, workspace=ws)

    step()
    torch.cuda.synchronize()
    y_ref, hL_ref = y.clone(), hL.clone()
    graph, _ = _capture(step)
    for _ in range(3):
        y.fill_(float("nan"))
        hL.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(hL, hL_ref)


def test_conv_then_scan_in_graph():
    """The block's conv and scan on one projection buffer, captured."""
    batch, dim, N, L = 2, 40, 16, 700
    wl = workload("graph_block", batch, dim, N, L, "bf16", seed=63)
    inp = synth.make_inputs(wl)
    w, b = synth.conv_parameters(wl, 4)
    xz = torch.cat([to_dev(inp, "x"), to_dev(inp, "z")], dim=1)
    wt, bt = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
    xc = torch.empty(batch, dim, L, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(batch, dim, L, device="cuda")
    hL = torch.empty(batch, dim, N, device="cuda")
    t = {k: to_dev(inp, k) for k in ("dt", "Bm", "Cm", "A", "Dskip", "dt_bias")}

    def step():
        ssm.ssm_conv1d_fwd(xz[:, :dim], wt, bias=bt, y=xc, out_dtype=torch.bfloat16,
                           return_final_state=False)
        ssm.ssm_scan_fwd(xc, t["dt"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                         Dskip=t["Dskip"], z=xz[:, dim:], y=y, hL=hL)

    step()
    torch.cuda.synchronize()
    y_ref, hL_ref = y.clone(), hL.clone()
    graph, _ = _capture(step)
    for _ in range(3):
        y.zero_()
        xc.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(hL, hL_ref)
