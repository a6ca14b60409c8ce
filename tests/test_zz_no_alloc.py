"""The allocation-free forward entry point (ssm_scan_fwd_noalloc), for callers
that cannot allocate device memory.  Called through the C ABI, its outputs
must equal those of ssm_scan_fwd_strided on the same inputs (the same kernels,
so bit for bit) on two calls in a row, the second with a smaller input, both
split along the sequence so that the library's scratch array is used; and
they must agree with the oracle within the parity gates."""
import ctypes

import numpy as np
import pytest
import torch

import selective_state_space_64_amd as ssm
from selective_state_space_64_amd import synth
from helpers import oracle_full, rel_err, to_dev, tol_for, workload

pytestmark = pytest.mark.gpu

SHAPES = [  # (name, batch, dim, N, L, dtype); the second is smaller than the first
    ("noalloc_a b1 d40 N16 L9000 f32", 1, 40, 16, 9000, "f32"),
    ("noalloc_b b1 d20 N8 L5000 bf16", 1, 20, 8, 5000, "bf16"),
]


def _inputs(name, batch, dim, N, L, dtype, seed):
    inp = synth.make_inputs(workload(name, batch, dim, N, L, dtype, seed=seed), with_h0=True)
    t = {k: to_dev(inp, k) for k in ("x", "dt", "z", "Bm", "Cm", "A", "Dskip", "dt_bias")}
    t["h0"] = torch.from_numpy(inp.h0).cuda()
    return inp, t


def _noalloc(t, y, hL, flags=0):
    batch, dim, L = t["x"].shape
    N = t["A"].shape[1]
    ind = ssm.SSM_BF16 if t["x"].dtype == torch.bfloat16 else ssm.SSM_F32
    p = lambda k: t[k].data_ptr()
    return ssm.lib().ssm_scan_fwd_noalloc(
        batch, dim, L, N, ind, flags, p("x"), p("dt"), p("dt_bias"), p("A"), p("Bm"), p("Cm"),
        p("Dskip"), p("z"), p("h0"), ssm.SSM_F32, y.data_ptr(), hL.data_ptr(),
        ctypes.cast(None, ctypes.POINTER(ssm.ScanLayout)),
        torch.cuda.current_stream().cuda_stream)


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    cases = [_inputs(*s, seed=90 + i) for i, s in enumerate(SHAPES)]
    outs = []
    for inp, t in cases:  # the first library call of the process may be this one
        batch, dim, L = t["x"].shape
        N = t["A"].shape[1]
        assert ssm.lib().ssm_scan_fwd_workspace_bytes(batch, dim, L, N) > 0  # split: scratch used
        y = torch.full((batch, dim, L), 7.0, device="cuda")
        hL = torch.full((batch, dim, N), 7.0, device="cuda")
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        assert _noalloc(t, y, hL) == 0
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        outs.append((y.clone(), hL.clone()))
    for (inp, t), (y, hL) in zip(cases, outs):
        ry, rh = ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                                  Dskip=t["Dskip"], z=t["z"], h0=t["h0"])
        torch.cuda.synchronize()
        assert torch.equal(y, ry) and torch.equal(hL, rh)
        oy, oh = oracle_full(inp, h0=inp.h0)
        tol = tol_for(inp.dtype)
        assert rel_err(y.cpu().numpy(), oy) <= tol
        assert rel_err(hL.cpu().numpy(), oh) <= tol


def test_noalloc_unsplit_shape_and_errors():
    inp, t = _inputs("noalloc_c b2 d24 N16 L700 bf16", 2, 24, 16, 700, "bf16", seed=95)
    assert ssm.lib().ssm_scan_fwd_workspace_bytes(2, 24, 700, 16) == 0
    y = torch.full((2, 24, 700), 7.0, device="cuda")
    hL = torch.full((2, 24, 16), 7.0, device="cuda")
    # checkpoints need the backward's workspace: refused, nothing written
    assert _noalloc(t, y, hL, flags=ssm.SSM_FLAG_CHECKPOINTS) == 6
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()) and bool((hL == 7.0).all())
    assert _noalloc(t, y, hL) == 0
    ry, rh = ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                              Dskip=t["Dskip"], z=t["z"], h0=t["h0"])
    torch.cuda.synchronize()
    assert torch.equal(y, ry) and torch.equal(hL, rh)


def test_noalloc_binding_wrapper():
    inp, t = _inputs("noalloc_d b1 d16 N16 L4096 f32", 1, 16, 16, 4096, "f32", seed=96)
    y = torch.empty((1, 16, 4096), device="cuda")
    hL = torch.empty((1, 16, 16), device="cuda")
    ssm.ssm_scan_fwd_noalloc(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], y=y, hL=hL,
                             dt_bias=t["dt_bias"], Dskip=t["Dskip"], z=t["z"], h0=t["h0"])
    ry, rh = ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                              Dskip=t["Dskip"], z=t["z"], h0=t["h0"])
    torch.cuda.synchronize()
    assert torch.equal(y, ry) and torch.equal(hL, rh)
