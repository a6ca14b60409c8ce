"""GPU parity of the scan on strided views (ssm_scan_fwd_strided, through the
C ABI) against the fp64 oracle and against the dense call.

The Mamba block takes the SSM branch x and the gate z from one input
projection, so x and z arrive as the two halves of one [batch, 2 dim, L]
buffer (and Bm, Cm as parts of one projection).  Cases: x/z and Bm/Cm as
halves of one buffer, y written into half of a larger buffer whose other
half is a NaN guard band, rows padded past L (element path, and a padding
that keeps rows on 16-byte boundaries), size-1 batch and channel counts,
the exact-ZOH variant, the checkpoints for the backward pass, the
Mamba-2.8B-shaped layer in full, and the binding's rejection of views the
library cannot take.
"""
import numpy as np
import pytest
import torch

import selective_state_space_64_amd as ssm
from selective_state_space_64_amd import synth
from helpers import oracle_full, rel_err, to_dev, tol_for, workload

pytestmark = pytest.mark.gpu

NAN_BITS = 0x7FC0DEAD


def _nan_fill(shape, dtype):
    if dtype == torch.float32:
        return torch.full(shape, NAN_BITS, dtype=torch.int32, device="cuda").view(torch.float32)
    return torch.full(shape, 0x7FC1, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def _untouched(t):
    if t.dtype == torch.float32:
        return bool((t.view(torch.int32) == NAN_BITS).all())
    return bool((t.view(torch.int16) == 0x7FC1).all())


def _halves(a, b):
    """a and b as the two halves (along the row index) of one new buffer; the
    buffer is returned too so that the views stay alive."""
    buf = torch.cat([a, b], dim=1)
    return buf[:, :a.shape[1]], buf[:, a.shape[1]:], buf


def _padded(t, pad):
    """t copied into a view whose rows are L + pad elements apart."""
    B, R, L = t.shape
    buf = _nan_fill((B, R, L + pad), t.dtype)
    v = buf[:, :, :L]
    v.copy_(t)
    return v, buf


def _dense(inp, h0=True):
    return dict(x=to_dev(inp, "x"), dt=to_dev(inp, "dt"), z=to_dev(inp, "z"),
                Bm=to_dev(inp, "Bm"), Cm=to_dev(inp, "Cm"), A=to_dev(inp, "A"),
                Dskip=to_dev(inp, "Dskip"), dt_bias=to_dev(inp, "dt_bias"),
                h0=torch.from_numpy(inp.h0.astype(np.float32)).cuda() if h0 else None)


def _scan(t, **kw):
    return ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dt_bias=t["dt_bias"],
                            Dskip=t["Dskip"], z=t["z"], h0=t["h0"], **kw)


XZ = [
    # (batch, dim, N, L, dtype)
    (2, 40, 16, 517, "bf16"), (3, 33, 16, 1024, "bf16"), (2, 20, 8, 300, "f32"),
    (1, 7, 4, 129, "bf16"), (2, 1, 16, 256, "f32"), (1, 18, 2, 4099, "bf16"),
]


@pytest.mark.parametrize("shape", XZ, ids=lambda s: "b%d_d%d_N%d_L%d_%s" % s)
def test_projection_halves(shape):
    """x, z halves of one xz buffer; Bm, Cm halves of one buffer; y into the
    first half of a [batch, 2 dim, L] buffer.  Equal to the dense call bit for
    bit (same vector/element path decisions), within the gate of the oracle,
    and the other half of y's buffer untouched."""
    batch, dim, N, L, dt = shape
    print("strided halves", shape, flush=True)
    inp = synth.make_inputs(workload("strided", batch, dim, N, L, dt, seed=11), with_h0=True)
    d = _dense(inp)
    y0, h0 = _scan(d)
    s = dict(d)
    s["x"], s["z"], xz = _halves(d["x"], d["z"])
    s["Bm"], s["Cm"], bc = _halves(d["Bm"], d["Cm"])
    ybuf = _nan_fill((batch, 2 * dim, L), torch.float32)
    y1, h1 = _scan(s, y=ybuf[:, :dim])
    torch.cuda.synchronize()
    assert y1.data_ptr() == ybuf.data_ptr()
    assert torch.equal(y1, y0) and torch.equal(h1, h0)
    assert _untouched(ybuf[:, dim:])
    ry, rh = oracle_full(inp, h0=inp.h0)
    assert rel_err(y1.cpu().numpy(), ry) <= tol_for(dt)
    assert rel_err(h1.cpu().numpy(), rh) <= tol_for(dt)
    del xz, bc


@pytest.mark.parametrize("pad,dt", [(3, "bf16"), (8, "bf16"), (1, "f32"), (4, "f32")])
def test_padded_rows(pad, dt):
    """Rows L + pad apart for x, dt, z and y (and Bm, Cm with another
    padding): an odd padding forces the element path, a padding of 16 bytes
    keeps the vector path; both against the oracle and the dense call, with
    the padding of y left untouched."""
    batch, dim, N, L = 2, 37, 16, 640
    print("strided padded", pad, dt, flush=True)
    inp = synth.make_inputs(workload("padded", batch, dim, N, L, dt, seed=12), with_h0=True)
    d = _dense(inp)
    y0, h0 = _scan(d)
    s, keep = dict(d), []
    for k in ("x", "dt", "z"):
        s[k], b = _padded(d[k], pad)
        keep.append(b)
    for k in ("Bm", "Cm"):
        s[k], b = _padded(d[k], 2 * pad)
        keep.append(b)
    y, ybuf = _padded(torch.empty((batch, dim, L), device="cuda"), pad)
    ybuf.view(torch.int32).fill_(NAN_BITS)
    y1, h1 = _scan(s, y=y)
    torch.cuda.synchronize()
    assert rel_err(y1.cpu().numpy(), y0.cpu().numpy()) <= 1e-6
    assert torch.equal(h1, h0) or rel_err(h1.cpu().numpy(), h0.cpu().numpy()) <= 1e-6
    assert _untouched(ybuf[:, :, L:])
    ry, rh = oracle_full(inp, h0=inp.h0)
    assert rel_err(y1.cpu().numpy(), ry) <= tol_for(dt)
    assert rel_err(h1.cpu().numpy(), rh) <= tol_for(dt)


def test_bf16_output_and_no_gate_strided():
    """bf16 y into a strided view, no gate, no skip, no h0."""
    batch, dim, N, L = 3, 24, 16, 800
    inp = synth.make_inputs(workload("strided_bf16", batch, dim, N, L, "bf16", seed=13))
    d = _dense(inp, h0=False)
    d["z"] = d["Dskip"] = None
    y0, h0 = _scan(d, out_dtype=torch.bfloat16)
    s = dict(d)
    s["x"], s["dt"], xdt = _halves(d["x"], d["dt"])
    ybuf = _nan_fill((batch, dim + 5, L), torch.bfloat16)
    y1, h1 = _scan(s, y=ybuf[:, 5:], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y1, y0) and torch.equal(h1, h0)
    assert _untouched(ybuf[:, :5])
    del xdt


def test_zoh_strided_matches_dense():
    batch, dim, N, L = 2, 30, 16, 700
    inp = synth.make_inputs(workload("strided_zoh", batch, dim, N, L, "bf16", seed=14))
    d = _dense(inp, h0=False)
    y0, h0 = _scan(d, zoh=True)
    s = dict(d)
    s["x"], s["z"], xz = _halves(d["x"], d["z"])
    y1, h1 = _scan(s, zoh=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y0) and torch.equal(h1, h0)
    ry, rh = oracle_full(inp, zoh=True)
    assert rel_err(y1.cpu().numpy(), ry) <= tol_for("bf16")
    del xz


def test_checkpoints_from_strided_forward():
    """The backward pass's checkpoints written by a forward on strided views
    equal those of the dense forward, bit for bit."""
    batch, dim, N, L = 2, 20, 16, 333
    inp = synth.make_inputs(workload("strided_ck", batch, dim, N, L, "bf16", seed=15), with_h0=True)
    d = _dense(inp)
    nbytes = ssm.lib().ssm_scan_bwd_workspace_bytes(batch, dim, L, N)
    w0 = torch.zeros(nbytes // 4, device="cuda")
    w1 = torch.ones(nbytes // 4, device="cuda")
    y0, _ = _scan(d, checkpoints=w0)
    s = dict(d)
    s["x"], s["z"], xz = _halves(d["x"], d["z"])
    y1, _ = _scan(s, checkpoints=w1)
    torch.cuda.synchronize()
    assert torch.equal(y1, y0)
    nck = batch * dim * ((L + 63) // 64) * N
    assert torch.equal(w0[:nck], w1[:nck])
    del xz


def test_layer_projection_halves_full():
    """The Mamba-2.8B-shaped layer (batch 4, dim 5120, N 16, L 2048, bf16)
    with x/z and Bm/Cm as halves of their projection buffers: every output
    equal to the dense call's."""
    wl = synth.WORKLOADS[2]
    print("strided layer", wl.name, flush=True)
    inp = synth.make_inputs(wl)
    d = _dense(inp, h0=False)
    y0, h0 = _scan(d)
    s = dict(d)
    s["x"], s["z"], xz = _halves(d["x"], d["z"])
    s["Bm"], s["Cm"], bc = _halves(d["Bm"], d["Cm"])
    y1, h1 = _scan(s)
    torch.cuda.synchronize()
    assert torch.equal(y1, y0) and torch.equal(h1, h0)
    del xz, bc


def test_binding_rejects_unsupported_views():
    batch, dim, N, L = 2, 8, 16, 40
    inp = synth.make_inputs(workload("strided_err", batch, dim, N, L, "bf16", seed=16))
    d = _dense(inp, h0=False)
    # time index not contiguous
    s = dict(d)
    s["x"] = d["x"].transpose(1, 2).contiguous().transpose(1, 2)
    with pytest.raises(ValueError):
        _scan(s)
    # x and dt with different row strides
    s = dict(d)
    s["x"], xb = _padded(d["x"], 8)
    with pytest.raises(ValueError):
        _scan(s)
    # batch entries closer than dim rows: the library's own check
    s = dict(d)
    big = d["x"].transpose(0, 1).contiguous().transpose(0, 1)  # strides (L, batch L, 1)
    for k in ("x", "dt", "z"):
        s[k] = d[k].transpose(0, 1).contiguous().transpose(0, 1)
    y = torch.empty((dim, batch, L), device="cuda").transpose(0, 1)
    with pytest.raises(ssm.SSMError) as e:
        _scan(s, y=y)
    assert e.value.status == 2
    del xb, big


# ------------------------------------------------------------ backward pass
BWD_PER_ROW = ("dx", "ddt", "dz", "dh0")  # no atomics: bit-identical between calls


def _bwd_dense(t, dy, **kw):
    return ssm.ssm_scan_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], dy, dt_bias=t["dt_bias"],
                            Dskip=t["Dskip"], z=t["z"], h0=t["h0"], **kw)


@pytest.mark.parametrize("shape", [(2, 24, 16, 517, "bf16"), (3, 17, 8, 1024, "f32"),
                                   (1, 40, 16, 2048, "bf16")],
                         ids=lambda s: "b%d_d%d_N%d_L%d_%s" % s)
def test_bwd_projection_halves(shape):
    """Training layout: x and z halves of one xz buffer, Bm and Cm halves of
    one buffer, dz written into the second half of the projection's dxz
    gradient buffer (whose first half, the conv's input gradient, is left
    alone), dt, dy and ddt as halves of buffers of their own (one shared row
    stride).  The per-row gradients equal the dense call bit for bit, the
    summed ones within rounding, and all match the oracle."""
    import oracle
    batch, dim, N, L, dt = shape
    print("strided bwd", shape, flush=True)
    inp = synth.make_inputs(workload("strided_bwd", batch, dim, N, L, dt, seed=31), with_h0=True)
    d = _dense(inp)
    rng = np.random.default_rng(4)
    dyv = rng.standard_normal((batch, dim, L)).astype(np.float32)
    dy = torch.from_numpy(dyv).cuda()
    g0 = _bwd_dense(d, dy)
    s = dict(d)
    s["x"], s["z"], xz = _halves(d["x"], d["z"])
    s["Bm"], s["Cm"], bc = _halves(d["Bm"], d["Cm"])
    # x and z have rows L apart (halves of xz); dt and dy need the same row
    # stride, so they are halves of buffers of their own
    s["dt"], _, dtb = _halves(d["dt"], torch.zeros_like(d["dt"]))
    dys, _, dyb = _halves(dy, torch.zeros_like(dy))
    dxz = _nan_fill((batch, 2 * dim, L), torch.float32)
    ddtb = _nan_fill((batch, 2 * dim, L), torch.float32)
    g1 = ssm.ssm_scan_bwd(s["x"], s["dt"], s["A"], s["Bm"], s["Cm"], dys, dt_bias=s["dt_bias"],
                          Dskip=s["Dskip"], z=s["z"], h0=s["h0"], dz=dxz[:, dim:],
                          ddt=ddtb[:, dim:])
    torch.cuda.synchronize()
    assert g1["dz"].data_ptr() == dxz[:, dim:].data_ptr()
    assert _untouched(dxz[:, :dim])
    for k in BWD_PER_ROW:
        assert torch.equal(g1[k], g0[k]), k
    for k in ("dBm", "dCm", "dA", "dDskip", "ddt_bias"):
        assert rel_err(g1[k].cpu().numpy(), g0[k].cpu().numpy()) <= 1e-5, k
    assert _untouched(ddtb[:, :dim])
    r = oracle.scan_bwd(inp.values("x"), inp.values("dt"), inp.A.astype(np.float64),
                        inp.values("Bm"), inp.values("Cm"), dyv.astype(np.float64),
                        dt_bias=inp.dt_bias.astype(np.float64), Dskip=inp.Dskip.astype(np.float64),
                        z=inp.values("z"), h0=inp.h0.astype(np.float64))
    for k in ("dx", "ddt", "dz", "dBm", "dCm", "dA", "dh0"):
        e = rel_err(g1[k].cpu().numpy(), r[k])
        assert e <= 1e-4, (k, e)
    del xz, bc, dtb, dyb


def test_bwd_padded_rows_element_path():
    """Rows L + 3 apart (bf16 runs then never sit on 8-byte boundaries): the
    element path, against the dense call."""
    batch, dim, N, L = 2, 20, 16, 400
    inp = synth.make_inputs(workload("strided_bwd_pad", batch, dim, N, L, "bf16", seed=32),
                            with_h0=True)
    d = _dense(inp)
    dy = torch.randn(batch, dim, L, device="cuda")
    g0 = _bwd_dense(d, dy)
    s, keep = dict(d), []
    for k in ("x", "dt", "z"):
        s[k], b = _padded(d[k], 3)
        keep.append(b)
    dys, b = _padded(dy, 3)
    keep.append(b)
    outs = {}
    for k in ("dx", "ddt", "dz"):
        outs[k], b = _padded(torch.empty((batch, dim, L), device="cuda"), 3)
        b.view(torch.int32).fill_(NAN_BITS)
        keep.append(b)
    g1 = ssm.ssm_scan_bwd(s["x"], s["dt"], s["A"], s["Bm"], s["Cm"], dys, dt_bias=s["dt_bias"],
                          Dskip=s["Dskip"], z=s["z"], h0=s["h0"], **outs)
    torch.cuda.synchronize()
    for k in BWD_PER_ROW:
        assert torch.equal(g1[k], g0[k]), k
    for k in ("dBm", "dCm", "dA"):
        assert rel_err(g1[k].cpu().numpy(), g0[k].cpu().numpy()) <= 1e-5, k
    for b in keep[-3:]:
        assert _untouched(b[:, :, L:])
