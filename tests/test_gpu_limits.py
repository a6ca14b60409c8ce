"""GPU parity at the supported maxima (through the C ABI) against the fp64
oracle.

- batch = 65535, the largest grid y dimension, for the scan, the backward
  pass, the decode step and the conv, compared in full;
- seqlen = 2^28 - 4096, the longest sequence the scan accepts: four
  channels (the fourth sits at the largest in-wave row offset), split into
  1024 segments, the last channel's whole row against the oracle, for the
  forward and for the per-channel gradients of the backward pass;
- one past each limit is rejected before launch (also covered without a GPU
  in test_abi.py).
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_64_amd as ssm
from selective_state_space_64_amd import synth
from helpers import TOL_F32, oracle_full, rel_err, to_dev, tol_for, workload

pytestmark = pytest.mark.gpu

MAX_BATCH = 65535
MAX_SEQLEN = (1 << 28) - (1 << 12)


def test_scan_max_batch_full():
    wl = workload("max_batch", MAX_BATCH, 3, 16, 70, "bf16", seed=51)
    print("scan max batch", flush=True)
    inp = synth.make_inputs(wl, with_h0=True)
    h0 = torch.from_numpy(inp.h0.astype(np.float32)).cuda()
    y, hL = ssm.ssm_scan_fwd(to_dev(inp, "x"), to_dev(inp, "dt"), to_dev(inp, "A"),
                             to_dev(inp, "Bm"), to_dev(inp, "Cm"), dt_bias=to_dev(inp, "dt_bias"),
                             Dskip=to_dev(inp, "Dskip"), z=to_dev(inp, "z"), h0=h0)
    torch.cuda.synchronize()
    ry, rh = oracle_full(inp, h0=inp.h0)
    assert rel_err(y.cpu().numpy(), ry) <= tol_for("bf16")
    assert rel_err(hL.cpu().numpy(), rh) <= tol_for("bf16")
    with pytest.raises(ssm.SSMError) as e:
        x1 = torch.zeros(MAX_BATCH + 1, 1, 1, device="cuda")
        ssm.ssm_scan_fwd(x1, x1, torch.zeros(1, 16, device="cuda"),
                         torch.zeros(MAX_BATCH + 1, 16, 1, device="cuda"),
                         torch.zeros(MAX_BATCH + 1, 16, 1, device="cuda"))
    assert e.value.status == 2


def test_bwd_max_batch_full():
    wl = workload("max_batch_bwd", MAX_BATCH, 1, 4, 64, "f32", seed=52)
    print("bwd max batch", flush=True)
    inp = synth.make_inputs(wl)
    dyv = np.random.default_rng(5).standard_normal((MAX_BATCH, 1, 64)).astype(np.float32)
    g = ssm.ssm_scan_bwd(to_dev(inp, "x"), to_dev(inp, "dt"), to_dev(inp, "A"), to_dev(inp, "Bm"),
                         to_dev(inp, "Cm"), torch.from_numpy(dyv).cuda(),
                         dt_bias=to_dev(inp, "dt_bias"), Dskip=to_dev(inp, "Dskip"),
                         z=to_dev(inp, "z"))
    torch.cuda.synchronize()
    r = oracle.scan_bwd(inp.values("x"), inp.values("dt"), inp.A.astype(np.float64),
                        inp.values("Bm"), inp.values("Cm"), dyv.astype(np.float64),
                        dt_bias=inp.dt_bias.astype(np.float64), Dskip=inp.Dskip.astype(np.float64),
                        z=inp.values("z"))
    for k in ("dx", "ddt", "dz", "dBm", "dCm", "dh0"):
        assert rel_err(g[k].cpu().numpy(), r[k]) <= TOL_F32, k
    for k in ("dA", "dDskip", "ddt_bias"):  # sums over 65535 x 64 terms
        assert rel_err(g[k].cpu().numpy()[None], r[k][None]) <= TOL_F32, k


def test_decode_and_conv_max_batch():
    wl = workload("max_batch_dec", MAX_BATCH, 64, 16, 1, "bf16", seed=53)
    print("decode/conv max batch", flush=True)
    inp = synth.make_inputs(wl, with_h0=True)
    st = torch.from_numpy(inp.h0.astype(np.float32)).cuda()
    y = ssm.ssm_state_update(st, to_dev(inp, "x")[:, :, 0], to_dev(inp, "dt")[:, :, 0],
                             to_dev(inp, "A"), to_dev(inp, "Bm")[:, :, 0].contiguous(),
                             to_dev(inp, "Cm")[:, :, 0].contiguous(),
                             dt_bias=to_dev(inp, "dt_bias"), Dskip=to_dev(inp, "Dskip"),
                             z=to_dev(inp, "z")[:, :, 0])
    torch.cuda.synchronize()
    ry, rh = oracle_full(inp, h0=inp.h0)
    # the decode step's y is compared over the (b, :) row of channels
    assert rel_err(y.cpu().numpy(), ry[:, :, 0]) <= tol_for("bf16")
    assert rel_err(st.cpu().numpy(), rh) <= tol_for("bf16")
    wlc = workload("max_batch_conv", MAX_BATCH, 3, 16, 70, "bf16", seed=54)
    w, b = synth.conv_parameters(wlc, 4)
    xs = synth.make_inputs(wlc)
    yc, sc = ssm.ssm_conv1d_fwd(to_dev(xs, "x"), torch.from_numpy(w).cuda(),
                                bias=torch.from_numpy(b).cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    rc, rs = oracle.conv1d(xs.values("x"), w, bias=b)
    assert rel_err(yc.cpu().numpy(), rc) <= TOL_F32
    assert np.array_equal(sc.cpu().numpy(), rs.astype(np.float32))


def test_scan_max_seqlen():
    """The longest supported sequence, fp32, four channels of one batch row
    (the fourth at the largest row offset of a wave), N = 1.  The library
    splits it into 1024 segments; the fourth channel's whole row (y and hL)
    against the oracle, and one step more is rejected."""
    L, dim = MAX_SEQLEN, 4
    assert ssm.lib().ssm_scan_fwd_workspace_bytes(1, dim, L, 1) == 1024 * dim * 2 * 4
    wl = workload("max_seqlen", 1, dim, 1, L, "f32", seed=55)
    print("scan max seqlen", flush=True)
    inp = synth.make_inputs(wl)
    t = {k: to_dev(inp, k) for k in ("x", "dt", "z", "Bm", "Cm", "A", "Dskip", "dt_bias")}
    y, hL = ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                             Dskip=t["Dskip"], z=t["z"])
    torch.cuda.synchronize()
    yg = y[0, dim - 1].cpu().numpy()
    hg = hL[0, dim - 1].cpu().numpy()
    del y, t
    torch.cuda.empty_cache()
    d = dim - 1
    row = lambda a: np.ascontiguousarray(a[:, d:d + 1], dtype=np.float64)  # fp32 values, exact
    ry, rh = oracle.scan_fwd(row(inp.x), row(inp.dt), inp.A[d:d + 1].astype(np.float64),
                             inp.Bm.astype(np.float64), inp.Cm.astype(np.float64),
                             dt_bias=inp.dt_bias[d:d + 1].astype(np.float64),
                             Dskip=inp.Dskip[d:d + 1].astype(np.float64), z=row(inp.z))
    del inp
    assert rel_err(yg[None], ry[0]) <= tol_for("f32")
    assert rel_err(hg[None], rh[0]) <= tol_for("f32")
    with pytest.raises(ssm.SSMError) as e:
        one = torch.zeros(1, 1, L + 1, device="cuda")
        ssm.ssm_scan_fwd(one, one, torch.zeros(1, 1, device="cuda"), one, one)
    assert e.value.status == 2


def test_bwd_max_seqlen():
    """The backward pass at the longest supported sequence (fp32, four
    channels, N = 1, split into 1024 segments): the fourth channel's
    per-channel gradients (dx, ddt, dz over the whole row, dA, dDskip,
    ddt_bias) against the oracle run on that channel alone (dBm and dCm sum
    over channels and are covered at the shorter shapes)."""
    L, dim = MAX_SEQLEN, 4
    wl = workload("max_seqlen_bwd", 1, dim, 1, L, "f32", seed=56)
    print("bwd max seqlen", flush=True)
    inp = synth.make_inputs(wl)
    dyv = np.random.default_rng(57).standard_normal((1, dim, L), dtype=np.float32)
    t = {k: to_dev(inp, k) for k in ("x", "dt", "z", "Bm", "Cm", "A", "Dskip", "dt_bias")}
    g = ssm.ssm_scan_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], torch.from_numpy(dyv).cuda(),
                         dt_bias=t["dt_bias"], Dskip=t["Dskip"], z=t["z"])
    torch.cuda.synchronize()
    d = dim - 1
    got = {k: g[k][0, d].cpu().numpy() for k in ("dx", "ddt", "dz")}
    got.update({k: g[k][d].cpu().numpy() for k in ("dA", "dDskip", "ddt_bias")})
    del g, t
    torch.cuda.empty_cache()
    row = lambda a: np.ascontiguousarray(a[:, d:d + 1], dtype=np.float64)
    r = oracle.scan_bwd(row(inp.x), row(inp.dt), inp.A[d:d + 1].astype(np.float64),
                        inp.Bm.astype(np.float64), inp.Cm.astype(np.float64), row(dyv),
                        dt_bias=inp.dt_bias[d:d + 1].astype(np.float64),
                        Dskip=inp.Dskip[d:d + 1].astype(np.float64), z=row(inp.z))
    del inp
    for k in ("dx", "ddt", "dz"):
        assert rel_err(got[k][None], r[k][0]) <= TOL_F32, k
    # dA, dDskip and ddt_bias are sums over the 2.7e8 steps, accumulated in
    # fp32 (per lane over its chunks, a 16-lane butterfly, then one atomic add
    # per segment in whatever order the 1024 segments finish).  They cancel:
    # ddt_bias here is 18.84, 3e-6 of the sum of its terms' magnitudes (5.9e6).
    # Summing the oracle's own per-step ddt, rounded to fp32, in that order
    # gives 2.1e-5 to 6.4e-5 relative error over 20 segment orders (CPU), and
    # the per-step fp32 errors of the kernel add to it; observed on the GPU up
    # to 1.15e-4 for ddt_bias.  Gate: three times the fp32 bar for these sums.
    for k in ("dA", "dDskip", "ddt_bias"):
        e = rel_err(np.atleast_1d(got[k])[None], np.atleast_1d(r[k][0])[None])
        assert e <= 3 * TOL_F32, (k, e)
