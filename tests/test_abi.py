"""The C-ABI boundary: exported symbols (CPU), and the documented status for
every argument error with nothing written (GPU, real device buffers)."""
import ctypes
import os
import re

import pytest
import torch

import selective_state_space_64_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            with open(os.path.join(inc, h)) as f:
                text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
            names |= set(re.findall(r"\b(ssm_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert set(names) == set(ssm.EXPORTS)
    lib = ctypes.CDLL(ssm.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def _declared_signatures():
    """{name: [parameter types]} from the prototypes in include/*.h."""
    sigs = {}
    inc = os.path.join(ROOT, "include")
    for h in sorted(os.listdir(inc)):
        if not h.endswith(".h"):
            continue
        with open(os.path.join(inc, h)) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        for m in re.finditer(r"\b(ssm_[a-z_0-9]+)\s*\(([^)]*)\)\s*;", text):
            params = [p.strip() for p in m.group(2).split(",") if p.strip() and p.strip() != "void"]
            sigs[m.group(1)] = params
    return sigs


def test_binding_argtypes_match_prototypes():
    """Every ctypes prototype has the header's parameter count, and each
    pointer parameter is passed as a pointer (a mismatch would hand an
    unconverted Python int to the C side)."""
    L = ssm.lib()
    sigs = _declared_signatures()
    assert set(sigs) == set(ssm.EXPORTS)
    for name, params in sigs.items():
        argtypes = getattr(L, name).argtypes
        assert len(argtypes) == len(params), (name, len(argtypes), len(params))
        for decl, at in zip(params, argtypes):
            if "ssm_scan_bwd_bld_layout_t" in decl:
                assert at == ctypes.POINTER(ssm.BwdBldLayout), (name, decl, at)
            elif "ssm_scan_layout_t" in decl:
                assert at == ctypes.POINTER(ssm.ScanLayout), (name, decl, at)
            elif "ssm_scan_bwd_layout_t" in decl:
                assert at == ctypes.POINTER(ssm.BwdLayout), (name, decl, at)
            elif "ssm_conv_layout_t" in decl:
                assert at == ctypes.POINTER(ssm.ConvLayout), (name, decl, at)
            elif "ssm_conv_bld_layout_t" in decl:
                assert at == ctypes.POINTER(ssm.ConvBldLayout), (name, decl, at)
            elif "ssm_update_layout_t" in decl:
                assert at == ctypes.POINTER(ssm.UpdateLayout), (name, decl, at)
            elif "ssm_bld_layout_t" in decl:
                assert at == ctypes.POINTER(ssm.BldLayout), (name, decl, at)
            elif "*" in decl:
                assert at in (ctypes.c_void_p, ctypes.c_char_p), (name, decl, at)
            elif decl.startswith("size_t"):
                assert at == ctypes.c_size_t, (name, decl, at)
            elif decl.startswith("long long"):
                assert at == ctypes.c_longlong, (name, decl, at)
            else:
                assert at in (ctypes.c_int, ctypes.c_uint), (name, decl, at)


def test_host_only_entry_points():
    L = ssm.lib()
    assert L.ssm_abi_version() == 1
    for s in range(9):
        assert L.ssm_status_string(s).decode()
    assert L.ssm_status_string(99).decode() == "unknown status"
    assert L.ssm_scan_fwd_workspace_bytes(4, 5120, 2048, 16) == 0


# ---------------------------------------------------------------- CPU: broadcast views
# The C ABI reads a stride of 0 as "dense default", so a broadcast view (an
# expand()-ed tensor: stride 0 on a dimension of size > 1) passed through
# unchanged would make the kernels read past its one stored copy.  The binding
# must refuse such views before anything reaches the library.  CPU tensors
# suffice: the view checks come before the device check.
def _scan_inputs(batch=2, dim=8, L=40, N=4, dtype=torch.float32):
    g = torch.Generator().manual_seed(0)
    r = lambda *s: torch.randn(*s, generator=g).to(dtype)
    return dict(x=r(batch, dim, L), dt=r(batch, dim, L), A=-torch.rand(dim, N), Bm=r(batch, N, L),
                Cm=r(batch, N, L), z=r(batch, dim, L))


@pytest.mark.parametrize("which", ["Bm_batch", "Cm_state", "x_batch", "x_channel", "z_channel",
                                   "dt_batch"])
def test_binding_rejects_broadcast_views_scan(which):
    t = _scan_inputs()
    name, how = which.split("_")
    full = t[name]
    if how == "batch":
        t[name] = full[:1].expand(*full.shape)
    elif how == "channel" or how == "state":
        t[name] = full[:, :1].expand(*full.shape)
    assert 0 in t[name].stride()
    with pytest.raises(ValueError, match="broadcast"):
        ssm.ssm_scan_fwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], z=t["z"], y=torch.empty(2, 8, 40),
                         hL=torch.empty(2, 8, 4))
    with pytest.raises(ValueError, match="broadcast"):
        ssm.ssm_scan_bwd(t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], torch.randn(2, 8, 40), z=t["z"],
                         dx=torch.empty(2, 8, 40), ddt=torch.empty(2, 8, 40), dz=torch.empty(2, 8, 40),
                         workspace=torch.empty(1, dtype=torch.uint8))


@pytest.mark.parametrize("which", ["x", "Bm", "Cm", "z", "dt"])
def test_binding_rejects_broadcast_views_decode(which):
    batch, dim, N = 3, 8, 4
    t = {k: torch.randn(batch, n) for k, n in (("x", dim), ("dt", dim), ("z", dim), ("Bm", N),
                                                ("Cm", N))}
    t[which] = t[which][:1].expand(batch, t[which].shape[1])
    assert t[which].stride(0) == 0
    with pytest.raises(ValueError, match="broadcast"):
        ssm.ssm_state_update(torch.zeros(batch, dim, N), t["x"], t["dt"], -torch.rand(dim, N),
                             t["Bm"], t["Cm"], z=t["z"], y=torch.empty(batch, dim))


def test_binding_rejects_broadcast_views_conv():
    x = torch.randn(1, 8, 40).expand(3, 8, 40)
    with pytest.raises(ValueError, match="broadcast"):
        ssm.ssm_conv1d_fwd(x, torch.randn(8, 4), y=torch.empty(3, 8, 40), return_final_state=False)
    with pytest.raises(ValueError, match="broadcast"):
        ssm.ssm_conv1d_update(torch.zeros(3, 8, 3), torch.randn(1, 8).expand(3, 8), torch.randn(8, 4),
                              y=torch.empty(3, 8))


def test_binding_accepts_size_one_strides():
    """A size-1 dimension may carry any stride (it is never stepped over):
    such views pass the view checks and only fail the device check here."""
    x = torch.randn(1, 8, 40).expand(1, 8, 40)
    x2 = torch.randn(8, 1, 40).transpose(0, 1)  # batch 1, odd strides
    for v in (x, x2):
        with pytest.raises(TypeError, match="CUDA"):
            ssm.ssm_scan_fwd(v, v, -torch.rand(8, 4), torch.randn(1, 4, 40), torch.randn(1, 4, 40),
                             y=torch.empty(1, 8, 40), hL=torch.empty(1, 8, 4))


# ---------------------------------------------------------------- GPU: errors
def _bufs(batch=2, dim=8, L=40, N=16, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(0)
    r = lambda *s: torch.randn(*s, generator=g).to(dtype).cuda()
    f = lambda *s: torch.randn(*s, generator=g).cuda()
    return dict(batch=batch, dim=dim, L=L, N=N, x=r(batch, dim, L), dt=r(batch, dim, L),
                z=r(batch, dim, L), Bm=r(batch, N, L), Cm=r(batch, N, L), A=-f(dim, N).abs(),
                Dskip=f(dim), dt_bias=f(dim), h0=f(batch, dim, N),
                y=torch.full((batch, dim, L), 7.0, device="cuda"),
                hL=torch.full((batch, dim, N), 7.0, device="cuda"))


def _call(b, **over):
    a = dict(batch=b["batch"], dim=b["dim"], seqlen=b["L"], dstate=b["N"], in_dtype=1, flags=0,
             x=b["x"].data_ptr(), dt=b["dt"].data_ptr(), dt_bias=b["dt_bias"].data_ptr(),
             A=b["A"].data_ptr(), Bm=b["Bm"].data_ptr(), Cm=b["Cm"].data_ptr(),
             Dskip=b["Dskip"].data_ptr(), z=b["z"].data_ptr(), h0=b["h0"].data_ptr(), out_dtype=0,
             y=b["y"].data_ptr(), hL=b["hL"].data_ptr(), ws=None, wsb=0, stream=None)
    a.update(over)
    return ssm.lib().ssm_scan_fwd(a["batch"], a["dim"], a["seqlen"], a["dstate"], a["in_dtype"],
                                  a["flags"], a["x"], a["dt"], a["dt_bias"], a["A"], a["Bm"],
                                  a["Cm"], a["Dskip"], a["z"], a["h0"], a["out_dtype"], a["y"],
                                  a["hL"], a["ws"], a["wsb"], a["stream"])


ERRORS = [
    ("null_x", dict(x=None), 1), ("null_A", dict(A=None), 1), ("null_y", dict(y=None), 1),
    ("batch0", dict(batch=0), 2), ("dim_neg", dict(dim=-1), 2), ("L0", dict(seqlen=0), 2),
    ("batch_huge", dict(batch=70000), 2), ("L_huge", dict(seqlen=(1 << 28) - 4095), 2),
    ("in_dtype", dict(in_dtype=7), 3), ("out_dtype", dict(out_dtype=-1), 3),
    ("N3", dict(dstate=3), 6), ("N32", dict(dstate=32), 6), ("flag_bit2", dict(flags=4), 6),
    ("flag_other", dict(flags=0x81), 6), ("zoh_checkpoints_without_workspace", dict(flags=3), 1),
    ("checkpoints_without_workspace", dict(flags=2), 1),
]


@pytest.mark.gpu
@pytest.mark.parametrize("name,over,status", ERRORS, ids=[e[0] for e in ERRORS])
def test_scan_argument_errors_write_nothing(name, over, status):
    b = _bufs()
    assert _call(b, **over) == status
    torch.cuda.synchronize()
    assert (b["y"] == 7.0).all() and (b["hL"] == 7.0).all()


@pytest.mark.gpu
def test_scan_misaligned_and_alias():
    b = _bufs()
    assert _call(b, x=b["x"].data_ptr() + 1) == 4
    assert _call(b, hL=b["hL"].data_ptr() + 2) == 4
    assert _call(b, y=b["x"].data_ptr()) == 5                       # y over x (bf16 vs f32 sizes)
    assert _call(b, hL=b["Dskip"].data_ptr()) == 5                  # hL over a parameter
    assert _call(b, hL=b["y"].data_ptr()) == 5                      # hL over y
    big = torch.empty(4096, device="cuda")
    assert _call(b, y=big.data_ptr(), hL=big.data_ptr() + 64) == 5  # hL inside y
    torch.cuda.synchronize()
    assert (b["y"] == 7.0).all() and (b["hL"] == 7.0).all()
    # hL exactly equal to h0 is allowed
    assert _call(b, hL=b["h0"].data_ptr()) == 0
    torch.cuda.synchronize()


@pytest.mark.gpu
def test_state_update_argument_errors():
    b = _bufs()
    st = b["h0"]
    keep = st.clone()
    L = ssm.lib()
    x1, dt1 = b["x"][:, :, 0].contiguous(), b["dt"][:, :, 0].contiguous()
    B1, C1 = b["Bm"][:, :, 0].contiguous(), b["Cm"][:, :, 0].contiguous()
    y = torch.full((2, 8), 7.0, device="cuda")

    def call(**o):
        a = dict(batch=2, dim=8, N=16, ind=1, flags=0, state=st.data_ptr(), x=x1.data_ptr(),
                 dt=dt1.data_ptr(), bias=b["dt_bias"].data_ptr(), A=b["A"].data_ptr(),
                 B=B1.data_ptr(), C=C1.data_ptr(), D=b["Dskip"].data_ptr(), z=None, outd=0,
                 y=y.data_ptr())
        a.update(o)
        return L.ssm_state_update(a["batch"], a["dim"], a["N"], a["ind"], a["flags"], a["state"],
                                  a["x"], a["dt"], a["bias"], a["A"], a["B"], a["C"], a["D"],
                                  a["z"], a["outd"], a["y"], None)

    assert call(state=None) == 1
    assert call(batch=0) == 2
    assert call(ind=5) == 3
    assert call(x=x1.data_ptr() + 1) == 4
    assert call(state=st.data_ptr() + 4) == 4
    assert call(y=st.data_ptr()) == 5
    assert call(state=b["A"].data_ptr()) == 5
    assert call(N=5) == 6
    assert call(flags=2) == 6
    torch.cuda.synchronize()
    assert torch.equal(st, keep) and (y == 7.0).all()
    with pytest.raises(ssm.SSMError):
        ssm.ssm_scan_fwd(b["x"], b["dt"], b["A"][:, :3].contiguous(), b["Bm"][:, :3].contiguous(),
                         b["Cm"][:, :3].contiguous())


# ---------------------------------------------------------------- CPU: validation
# Fake, 16-byte-aligned addresses that are never dereferenced: every case below
# must be rejected before any launch.  Skipped where a GPU is present so that a
# validation bug could never launch a kernel on them.
_FAKE = {k: 0x10000000 * (i + 1) for i, k in enumerate(
    ["x", "dt", "z", "Bm", "Cm", "A", "Dskip", "dt_bias", "h0", "y", "hL"])}


def _fake_call(**over):
    a = dict(batch=2, dim=8, seqlen=40, dstate=16, in_dtype=1, flags=0, out_dtype=0,
             ws=None, wsb=0, **_FAKE)
    a.update(over)
    return ssm.lib().ssm_scan_fwd(a["batch"], a["dim"], a["seqlen"], a["dstate"], a["in_dtype"],
                                  a["flags"], a["x"], a["dt"], a["dt_bias"], a["A"], a["Bm"],
                                  a["Cm"], a["Dskip"], a["z"], a["h0"], a["out_dtype"], a["y"],
                                  a["hL"], a["ws"], a["wsb"], None)


no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer checks run only without a GPU")


@no_gpu
@pytest.mark.parametrize("name,over,status", ERRORS, ids=[e[0] for e in ERRORS])
def test_validation_rejects_before_launch(name, over, status):
    assert _fake_call(**over) == status


@no_gpu
def test_validation_alignment_and_alias():
    assert _fake_call(x=_FAKE["x"] + 1) == 4
    assert _fake_call(z=_FAKE["z"] + 3) == 4
    assert _fake_call(A=_FAKE["A"] + 2) == 4
    assert _fake_call(out_dtype=1, y=_FAKE["y"] + 1) == 4
    assert _fake_call(x=_FAKE["x"] + 2, dt=_FAKE["dt"] + 2) == 8  # bf16 element alignment suffices
    assert _fake_call(y=_FAKE["x"]) == 5
    assert _fake_call(y=_FAKE["x"] + 1280 - 16) == 5      # tail of x (2*8*40 bf16 = 1280 B)
    assert _fake_call(y=_FAKE["x"] + 1280) != 5           # just past x: no overlap with x
    assert _fake_call(hL=_FAKE["Dskip"]) == 5
    assert _fake_call(hL=_FAKE["y"] + 2560 - 16) == 5     # last bytes of y (fp32)
    assert _fake_call(hL=_FAKE["h0"] + 16) == 5           # partial overlap with h0
    # valid arguments reach the launch, which fails without a device
    assert _fake_call() == 8
    assert _fake_call(hL=_FAKE["h0"]) == 8                # hL == h0 exactly is allowed
    assert _fake_call(z=None, h0=None, hL=None, Dskip=None, dt_bias=None) == 8
    assert _fake_call(flags=1) == 8  # SSM_FLAG_ZOH_B is accepted
    # SSM_FLAG_CHECKPOINTS: the backward's workspace size, no overlap, aligned
    need = ssm.lib().ssm_scan_bwd_workspace_bytes(2, 8, 40, 16)
    ws = 0x200000000  # clear of every fake buffer above
    assert _fake_call(flags=2, ws=ws, wsb=need - 4) == 7
    assert _fake_call(flags=2, ws=ws + 2, wsb=need) == 4
    assert _fake_call(flags=2, ws=_FAKE["y"], wsb=need) == 5
    assert _fake_call(flags=2, ws=ws, wsb=need) == 8


def _strided_call(layout, **over):
    a = dict(batch=2, dim=8, seqlen=40, dstate=16, in_dtype=1, flags=0, out_dtype=0,
             ws=None, wsb=0, **_FAKE)
    a.update(over)
    lay = None
    if layout is not None:
        lay = ssm.ScanLayout(layout.get("seq_row", 0),
                             (ctypes.c_longlong * 4)(*layout.get("seq_batch", (0, 0, 0, 0))),
                             layout.get("bc_row", 0),
                             (ctypes.c_longlong * 2)(*layout.get("bc_batch", (0, 0))))
    return ssm.lib().ssm_scan_fwd_strided(
        a["batch"], a["dim"], a["seqlen"], a["dstate"], a["in_dtype"], a["flags"], a["x"], a["dt"],
        a["dt_bias"], a["A"], a["Bm"], a["Cm"], a["Dskip"], a["z"], a["h0"], a["out_dtype"], a["y"],
        a["hL"], a["ws"], a["wsb"], ctypes.byref(lay) if lay is not None else None, None)


STRIDE_ERRORS = [
    ("row_below_L", dict(seq_row=39)), ("row_negative", dict(seq_row=-40)),
    ("row_huge", dict(seq_row=(1 << 28) - 4095)),
    ("x_batch_below", dict(seq_row=48, seq_batch=(8 * 48 - 1, 0, 0, 0))),
    ("y_batch_below", dict(seq_batch=(0, 0, 0, 8 * 40 - 1))),
    ("batch_negative", dict(seq_batch=(0, -1, 0, 0))),
    ("bc_row_below_L", dict(bc_row=39)), ("bc_row_huge", dict(bc_row=1 << 28)),
    ("Cm_batch_below", dict(bc_batch=(0, 16 * 40 - 1))),
    ("span_2_56", dict(seq_batch=(1 << 56, 0, 0, 0))),
]


@no_gpu
@pytest.mark.parametrize("name,layout", STRIDE_ERRORS, ids=[e[0] for e in STRIDE_ERRORS])
def test_strided_validation_rejects_bad_strides(name, layout):
    assert _strided_call(layout) == 2


@no_gpu
def test_strided_validation_spans_and_defaults():
    # a NULL layout, or all strides 0, is the dense call (reaches the launch)
    assert _strided_call(None) == 8
    assert _strided_call({}) == 8
    assert _strided_call(None, flags=1) == 8
    assert _strided_call(None, batch=0) == 2
    # strides equal to the dense ones, given explicitly
    assert _strided_call(dict(seq_row=40, seq_batch=(320,) * 4, bc_row=40, bc_batch=(640, 640))) == 8
    # x and z as halves of one [2, 16, 40] bf16 buffer: batch stride 640, and
    # x's span runs to the end of its second batch entry (640 + 320 elements)
    xz = dict(seq_batch=(640, 0, 640, 0))
    assert _strided_call(xz, z=_FAKE["x"] + 320 * 2) == 8          # inputs may interleave
    assert _strided_call(xz, y=_FAKE["x"] + 1280) == 5             # dense-free byte, inside the span
    assert _strided_call(xz, y=_FAKE["x"] + 960 * 2) == 8          # just past x's span
    # y strided: its span (fp32) is what hL must avoid
    assert _strided_call(dict(seq_batch=(0, 0, 0, 1000)), hL=_FAKE["y"] + (1000 + 320) * 4 - 4) == 5
    assert _strided_call(dict(seq_batch=(0, 0, 0, 1000)), hL=_FAKE["y"] + (1000 + 320) * 4) == 8
    # padded rows: every row 48 apart
    assert _strided_call(dict(seq_row=48, bc_row=41)) == 8
    # Bm/Cm spans follow bc strides
    bc = dict(bc_batch=(2 * 640, 2 * 640))
    assert _strided_call(bc, y=_FAKE["Bm"] + (640 + 640) * 2 - 4) == 5
    assert _strided_call(bc, y=_FAKE["Bm"] + (1280 + 640) * 2) == 8


def _split_bytes(batch, dim, L, N):
    """The documented split rule, restated: split when batch * ceil(dim / 16)
    < 256, into whole multiples of that many workgroups up to 16384, segments
    >= 1024 steps and a multiple of 256 (whole chunks of the aggregate pass's
    16-step lanes), at most 1024 segments."""
    wgs = batch * ((dim + 15) // 16)
    if wgs >= 256:
        return 0
    nseg = min(16384 // wgs, L // 1024, 1024)
    if nseg < 2:
        return 0
    seg = -(-(-(-L // nseg)) // 256) * 256
    nseg = -(-L // seg)
    return 0 if nseg < 2 else nseg * batch * dim * (N + 1) * 4


@pytest.mark.parametrize("shape", [(4, 5120, 2048, 16), (8, 1536, 2048, 16), (1, 1536, 1 << 20, 16),
                                   (1, 16, 2048, 16), (1, 16, 2047, 16), (2, 20, 5000, 8),
                                   (1, 1, 1 << 20, 1), (256, 16, 4096, 4), (255, 16, 4096, 4),
                                   (1, 8185, 4096, 16)])
def test_fwd_workspace_bytes_follow_the_split_rule(shape):
    assert ssm.lib().ssm_scan_fwd_workspace_bytes(*shape) == _split_bytes(*shape)


def test_fwd_workspace_bytes_examples():
    L = ssm.lib()
    assert L.ssm_scan_fwd_workspace_bytes(4, 5120, 2048, 16) == 0      # 1280 workgroups
    assert L.ssm_scan_fwd_workspace_bytes(1, 16, 2048, 16) == 2 * 16 * 17 * 4
    # the long sequence: 96 workgroups -> 164 segments of 6400 steps
    assert L.ssm_scan_fwd_workspace_bytes(1, 1536, 1 << 20, 16) == 164 * 1536 * 17 * 4
    assert L.ssm_scan_fwd_workspace_bytes(2, 2560, 2048, 16) == 0      # 320 workgroups
    assert L.ssm_scan_fwd_workspace_bytes(0, 16, 4096, 16) == 0
    assert L.ssm_scan_fwd_workspace_bytes(1, 16, 4096, 3) == 0
    # the backward's workspace also covers the forward's split planes
    for shape in [(1, 16, 4096, 16), (1, 4096, 1 << 14, 16), (1, 8, 1 << 20, 1)]:
        bw = L.ssm_scan_bwd_workspace_bytes(*shape)
        b, d, n_l, n = shape
        ck = b * d * (-(-n_l // 64)) * n * 4
        # checkpoints, partial sums (or the forward's split planes), adjoint planes
        assert bw == ck + max(8 * 2 * b * n * n_l * 4, _split_bytes(*shape)) + _split_bytes(*shape)


@no_gpu
def test_split_workspace_validation():
    shape = dict(batch=1, dim=16, seqlen=4096, dstate=16)
    need = _split_bytes(1, 16, 4096, 16)
    assert need > 0
    ws = 0x200000000
    assert _fake_call(**shape) == 7                                  # no workspace
    assert _fake_call(**shape, ws=ws, wsb=need - 4) == 7
    assert _fake_call(**shape, ws=ws + 2, wsb=need) == 4
    assert _fake_call(**shape, ws=_FAKE["dt"] + 16, wsb=need) == 5   # inside dt
    assert _fake_call(**shape, ws=_FAKE["hL"] - need + 4, wsb=need) == 5
    assert _fake_call(**shape, ws=ws, wsb=need) == 8
    # with checkpoints the backward's workspace is what is checked
    bw = ssm.lib().ssm_scan_bwd_workspace_bytes(1, 16, 4096, 16)
    assert _fake_call(**shape, flags=2, ws=ws, wsb=bw - 4) == 7
    assert _fake_call(**shape, flags=2, ws=ws, wsb=bw) == 8


_BWD_FAKE = {k: 0x10000000 * (i + 20) for i, k in enumerate(
    ["dy", "dx", "ddt", "dz", "dBm", "dCm", "dA", "dDskip", "ddt_bias", "dh0", "dhL"])}


def _bwd_call(layout=None, **over):
    """ssm_scan_bwd_strided on fake, never dereferenced addresses."""
    a = dict(batch=2, dim=8, seqlen=40, dstate=16, in_dtype=1, flags=0, grad_dtype=0,
             ws=0x300000000, wsb=None, **_FAKE, **_BWD_FAKE)
    a.update(over)
    if a["wsb"] is None:
        a["wsb"] = ssm.lib().ssm_scan_bwd_workspace_bytes(a["batch"], a["dim"], a["seqlen"],
                                                          a["dstate"])
    lay = None
    if layout is not None:
        lay = ssm.BwdLayout(layout.get("seq_row", 0),
                            (ctypes.c_longlong * 7)(*layout.get("seq_batch", (0,) * 7)),
                            layout.get("bc_row", 0),
                            (ctypes.c_longlong * 2)(*layout.get("bc_batch", (0, 0))))
    return ssm.lib().ssm_scan_bwd_strided(
        a["batch"], a["dim"], a["seqlen"], a["dstate"], a["in_dtype"], a["flags"], a["x"], a["dt"],
        a["dt_bias"], a["A"], a["Bm"], a["Cm"], a["Dskip"], a["z"], a["h0"], a["grad_dtype"],
        a["dy"], a["dhL"], a["dx"], a["ddt"], a["dz"], a["dBm"], a["dCm"], a["dA"], a["dDskip"],
        a["ddt_bias"], a["dh0"], a["ws"], a["wsb"], ctypes.byref(lay) if lay is not None else None,
        None)


@no_gpu
def test_bwd_strided_validation():
    assert _bwd_call() == 8                                        # dense: reaches the launch
    assert _bwd_call({}) == 8
    assert _bwd_call({"seq_row": 39}) == 2
    assert _bwd_call({"seq_row": -1}) == 2
    assert _bwd_call({"seq_batch": (0, 0, 0, 0, 0, 8 * 40 - 1, 0)}) == 2   # ddt batch too small
    assert _bwd_call({"bc_row": 39}) == 2
    assert _bwd_call({"bc_batch": (0, 16 * 40 - 1)}) == 2
    # z and dz as halves of [2, 16, 40] fp32 / bf16 buffers
    half = dict(seq_batch=(0, 0, 640, 0, 0, 0, 640))
    assert _bwd_call(half) == 8
    # dz's span (fp32, 960 elements) now reaches past the dense 320 * 2 ...
    assert _bwd_call(half, dCm=_BWD_FAKE["dz"] + 2 * 320 * 4) == 5
    assert _bwd_call(half, dCm=_BWD_FAKE["dz"] + 960 * 4) == 8
    # an input's span: z (bf16) spans 960 elements
    assert _bwd_call(half, dh0=_FAKE["z"] + 900 * 2) == 5
    assert _bwd_call(half, dh0=_FAKE["z"] + 960 * 2) == 8
    # outputs may not interleave with each other either
    assert _bwd_call(dict(seq_batch=(0, 0, 0, 0, 640, 640, 0)), ddt=_BWD_FAKE["dx"] + 320 * 4) == 5


@no_gpu
def test_decode_strided_validation():
    L = ssm.lib()

    def upd(layout, **o):
        a = dict(batch=2, dim=8, N=16, state=_FAKE["h0"], x=_FAKE["x"], dt=_FAKE["dt"],
                 z=_FAKE["z"], B=_FAKE["Bm"], C=_FAKE["Cm"], y=_FAKE["y"])
        a.update(o)
        lay = None if layout is None else ssm.UpdateLayout(*layout)
        return L.ssm_state_update_strided(a["batch"], a["dim"], a["N"], 1, 0, a["state"], a["x"],
                                          a["dt"], _FAKE["dt_bias"], _FAKE["A"], a["B"], a["C"],
                                          _FAKE["Dskip"], a["z"], 0, a["y"],
                                          ctypes.byref(lay) if lay is not None else None, None)

    assert upd(None) == 8
    assert upd((0,) * 6) == 8
    assert upd((16, 0, 16, 0, 44, 44)) == 8                # x/z halves, Bm/Cm parts of x_dbl
    assert upd((7, 0, 0, 0, 0, 0)) == 2                    # below dim
    assert upd((0, 0, 0, 0, 15, 0)) == 2                   # below dstate
    assert upd((0, 0, 0, -8, 0, 0)) == 2
    # y (fp32) with batch stride 16 spans 16 + 8 elements; the state must avoid it
    assert upd((0, 0, 0, 16, 0, 0), state=_FAKE["y"] + 96 - 16) == 5
    assert upd((0, 0, 0, 16, 0, 0), state=_FAKE["y"] + 96) == 8

    def cupd(xb, yb, **o):
        a = dict(state=_CFAKE["s0"], x=_CFAKE["x"], y=_CFAKE["y"])
        a.update(o)
        return L.ssm_conv1d_update_strided(2, 8, 4, 1, 1, a["state"], a["x"], _CFAKE["w"],
                                           _CFAKE["bias"], 0, a["y"], xb, yb, None)

    assert cupd(0, 0) == 8
    assert cupd(16, 0) == 8
    assert cupd(7, 0) == 2
    assert cupd(0, -1) == 2
    assert cupd(16, 0, y=_CFAKE["x"] + 2 * 20) == 5         # y inside x's strided span
    assert cupd(16, 0, y=_CFAKE["x"] + 2 * 24) == 8


@no_gpu
def test_state_update_validation():
    L = ssm.lib()

    def call(**o):
        a = dict(batch=2, dim=8, N=16, ind=1, flags=0, state=_FAKE["h0"], x=_FAKE["x"],
                 dt=_FAKE["dt"], bias=_FAKE["dt_bias"], A=_FAKE["A"], B=_FAKE["Bm"], C=_FAKE["Cm"],
                 D=_FAKE["Dskip"], z=_FAKE["z"], outd=0, y=_FAKE["y"])
        a.update(o)
        return L.ssm_state_update(a["batch"], a["dim"], a["N"], a["ind"], a["flags"], a["state"],
                                  a["x"], a["dt"], a["bias"], a["A"], a["B"], a["C"], a["D"],
                                  a["z"], a["outd"], a["y"], None)

    assert call(state=None) == 1
    assert call(y=None) == 1
    assert call(batch=0) == 2
    assert call(ind=5) == 3
    assert call(outd=2) == 3
    assert call(x=_FAKE["x"] + 1) == 4
    assert call(state=_FAKE["h0"] + 4) == 4
    assert call(x=_FAKE["x"] + 2) == 8
    assert call(y=_FAKE["h0"]) == 5
    assert call(state=_FAKE["A"]) == 5
    assert call(N=5) == 6
    assert call(flags=2) == 6
    assert call() == 8
    assert call(flags=1) == 8  # SSM_FLAG_ZOH_B is accepted


# ---------------------------------------------------------------- conv entry points
_CFAKE = {k: 0x10000000 * (i + 1) for i, k in enumerate(["x", "w", "bias", "s0", "y", "sL"])}


def _conv_call(L, **over):
    a = dict(batch=2, dim=8, seqlen=40, width=4, ind=1, flags=1, outd=1, **_CFAKE)
    a.update(over)
    return L.ssm_conv1d_fwd(a["batch"], a["dim"], a["seqlen"], a["width"], a["ind"], a["flags"],
                            a["x"], a["w"], a["bias"], a["s0"], a["outd"], a["y"], a["sL"], None)


def _conv_strided_call(layout, **over):
    a = dict(batch=2, dim=8, seqlen=40, width=4, ind=1, flags=1, outd=1, **_CFAKE)
    a.update(over)
    lay = None if layout is None else ssm.ConvLayout(*layout)
    return ssm.lib().ssm_conv1d_fwd_strided(
        a["batch"], a["dim"], a["seqlen"], a["width"], a["ind"], a["flags"], a["x"], a["w"],
        a["bias"], a["s0"], a["outd"], a["y"], a["sL"],
        ctypes.byref(lay) if lay is not None else None, None)


@no_gpu
def test_conv_strided_validation():
    assert _conv_strided_call(None) == 8
    assert _conv_strided_call((0, 0, 0, 0)) == 8
    assert _conv_strided_call((40, 320, 40, 320)) == 8       # the dense strides, explicit
    assert _conv_strided_call((39, 0, 0, 0)) == 2
    assert _conv_strided_call((0, 0, -40, 0)) == 2
    assert _conv_strided_call((0, 319, 0, 0)) == 2
    assert _conv_strided_call((48, 8 * 48 - 1, 0, 0)) == 2
    assert _conv_strided_call((0, 1 << 56, 0, 0)) == 2
    # x as the first half of a [2, 16, 40] bf16 projection output: its span is
    # 640 + 320 elements, so y (bf16) may start right after it but not before
    xz = (0, 640, 0, 0)
    assert _conv_strided_call(xz, y=_CFAKE["x"] + 900 * 2) == 5
    assert _conv_strided_call(xz, y=_CFAKE["x"] + 960 * 2) == 8
    # y strided: stateL must avoid y's span
    assert _conv_strided_call((0, 0, 50, 1000), sL=_CFAKE["y"] + (1000 + 7 * 50 + 40) * 2 - 4) == 5
    assert _conv_strided_call((0, 0, 50, 1000), sL=_CFAKE["y"] + (1000 + 7 * 50 + 40) * 2) == 8


def _conv_bld_call(layout, **over):
    a = dict(batch=2, dim=8, seqlen=40, width=4, ind=1, flags=1, outd=1, **_CFAKE)
    a.update(over)
    lay = None if layout is None else ssm.ConvBldLayout(*layout)
    return ssm.lib().ssm_conv1d_fwd_bld(
        a["batch"], a["dim"], a["seqlen"], a["width"], a["ind"], a["flags"], a["x"], a["w"],
        a["bias"], a["s0"], a["outd"], a["y"], a["sL"],
        ctypes.byref(lay) if lay is not None else None, None)


@no_gpu
def test_conv_bld_validation():
    """ssm_conv1d_fwd_bld: x, y as [batch][L][dim] with step and batch strides."""
    assert _conv_bld_call(None) == 8
    assert _conv_bld_call((0, 0, 0, 0)) == 8
    assert _conv_bld_call((8, 320, 8, 320)) == 8          # the dense strides, explicit
    assert _conv_bld_call((7, 0, 0, 0)) == 2              # step below dim
    assert _conv_bld_call((0, 0, -8, 0)) == 2
    assert _conv_bld_call((0, 319, 0, 0)) == 2            # batch stride below seqlen * step
    assert _conv_bld_call(((1 << 40) + 8, 0, 0, 0)) == 2  # step stride above 2^40
    assert _conv_bld_call((0, 1 << 56, 0, 0)) == 2
    for over, status in [(dict(x=None), 1), (dict(batch=0), 2), (dict(seqlen=0), 2),
                         (dict(ind=2), 3), (dict(width=1), 6), (dict(flags=2), 6),
                         (dict(x=_CFAKE["x"] + 1), 4), (dict(sL=_CFAKE["sL"] + 2), 4),
                         (dict(sL=_CFAKE["s0"]), 8), (dict(sL=_CFAKE["s0"] + 4), 5)]:
        assert _conv_bld_call(None, **over) == status, over
    # x as the first half of a [2, 40, 16] bf16 projection output: its span is
    # 640 + 39 * 16 + 8 elements, so y (bf16) may start right after it, not before
    xz = (16, 640, 0, 0)
    span = 640 + 39 * 16 + 8
    assert _conv_bld_call(xz, y=_CFAKE["x"] + (span - 1) * 2) == 5
    assert _conv_bld_call(xz, y=_CFAKE["x"] + span * 2) == 8


@no_gpu
def test_scan_bwd_bld_validation():
    """ssm_scan_bwd_bld: (batch, L, dim) strides checked before any launch."""
    L = ssm.lib()
    f = {k: 0x10000000 * (i + 1) for i, k in enumerate(
        ["x", "dt", "A", "Bm", "Cm", "z", "dy", "dx", "ddt", "dz", "dBm", "dCm", "dA", "ws"])}
    need = L.ssm_scan_bwd_bld_workspace_bytes(2, 8, 40, 4)
    assert need >= 7 * 2560 + 4 * 1280 + L.ssm_scan_bwd_workspace_bytes(2, 8, 40, 4)
    assert L.ssm_scan_bwd_bld_workspace_bytes(2, 8, 40, 3) == 0
    # 65535 x 2^30 x 4096 elements: within the product limit of the other
    # entry points, but the transposed planes would take 2^62 bytes or more
    assert L.ssm_scan_bwd_bld_workspace_bytes(65535, 1 << 30, 4096, 16) == 0
    seven = ctypes.c_longlong * 7

    def call(layout=None, flags=0, wsb=need, **over):
        a = dict(f, ind=1, gd=0)
        a.update(over)
        lay = ssm.BwdBldLayout(*layout) if layout else None
        return L.ssm_scan_bwd_bld(2, 8, 40, 4, a["ind"], flags, a["x"], a["dt"], None, a["A"],
                                  a["Bm"], a["Cm"], None, a["z"], None, a["gd"], a["dy"], None,
                                  a["dx"], a["ddt"], a["dz"], a["dBm"], a["dCm"], a["dA"], None,
                                  None, None, a["ws"], wsb,
                                  ctypes.byref(lay) if lay is not None else None, None)

    assert call() == 8
    assert call(layout=(seven(), seven(), 0, 0, 0, 0)) == 8
    assert call(flags=1) == 8                                   # exact ZOH accepted
    assert call(flags=2) == 6                                   # checkpoints refused
    assert call(ws=None) == 1
    assert call(layout=(seven(0, 7, 0, 0, 0, 0, 0), seven(), 0, 0, 0, 0)) == 2
    assert call(layout=(seven(), seven(0, 0, 0, 0, 0, 0, 319), 0, 0, 0, 0)) == 2
    assert call(layout=(seven(), seven(), 0, 3, 0, 0)) == 2
    assert call(layout=(seven(), seven(), 0, 0, 0, 159)) == 2
    assert call(wsb=need - 1) == 7
    assert L.ssm_scan_bwd_bld(65535, 1 << 30, 4096, 4, 1, 0, f["x"], f["dt"], None, f["A"], f["Bm"],
                              f["Cm"], None, f["z"], None, 0, f["dy"], None, f["dx"], f["ddt"],
                              f["dz"], f["dBm"], f["dCm"], f["dA"], None, None, None, f["ws"],
                              1 << 62, None, None) == 2
    assert call(x=f["x"] + 1) == 4
    # dz as the second half of a [2, 40, 16] fp32 gradient buffer whose first
    # half is dx: interleaved halves of one buffer overlap by address range
    assert call(layout=(seven(0, 0, 0, 0, 16, 0, 16), seven(0, 0, 0, 0, 640, 0, 640), 0, 0, 0, 0),
                dz=f["dx"] + 8 * 4) == 5
    assert call(layout=(seven(0, 0, 0, 0, 0, 0, 16), seven(0, 0, 0, 0, 0, 0, 640), 0, 0, 0, 0)) == 8


def _conv_update_call(L, **over):
    a = dict(batch=2, dim=8, width=4, ind=1, flags=1, state=_CFAKE["s0"], x=_CFAKE["x"],
             w=_CFAKE["w"], bias=_CFAKE["bias"], outd=0, y=_CFAKE["y"])
    a.update(over)
    return L.ssm_conv1d_update(a["batch"], a["dim"], a["width"], a["ind"], a["flags"], a["state"],
                               a["x"], a["w"], a["bias"], a["outd"], a["y"], None)


CONV_ERRORS = [
    ("null_x", dict(x=None), 1), ("null_w", dict(w=None), 1), ("null_y", dict(y=None), 1),
    ("batch0", dict(batch=0), 2), ("dim0", dict(dim=0), 2), ("L0", dict(seqlen=0), 2),
    ("in_dtype", dict(ind=2), 3), ("out_dtype", dict(outd=9), 3),
    ("width1", dict(width=1), 6), ("width5", dict(width=5), 6), ("flag2", dict(flags=2), 6),
]


@no_gpu
@pytest.mark.parametrize("name,over,status", CONV_ERRORS, ids=[e[0] for e in CONV_ERRORS])
def test_conv_validation_rejects_before_launch(name, over, status):
    assert _conv_call(ssm.lib(), **over) == status


@no_gpu
def test_conv_validation_alignment_alias_and_update():
    L = ssm.lib()
    assert _conv_call(L, x=_CFAKE["x"] + 1) == 4
    assert _conv_call(L, w=_CFAKE["w"] + 2) == 4
    assert _conv_call(L, sL=_CFAKE["sL"] + 2) == 4
    assert _conv_call(L, outd=0, y=_CFAKE["y"] + 2) == 4
    assert _conv_call(L, y=_CFAKE["x"] + 1280 - 2) == 5      # y over the tail of x
    assert _conv_call(L, sL=_CFAKE["bias"]) == 5
    assert _conv_call(L, sL=_CFAKE["s0"] + 4) == 5           # partial overlap with state0
    assert _conv_call(L, sL=_CFAKE["y"] + 16) == 5
    assert _conv_call(L) == 8                                 # valid: reaches the launch
    assert _conv_call(L, sL=_CFAKE["s0"]) == 8                # stateL == state0 allowed
    assert _conv_call(L, bias=None, s0=None, sL=None, flags=0, width=2) == 8
    assert _conv_update_call(L, state=None) == 1
    assert _conv_update_call(L, dim=-3) == 2
    assert _conv_update_call(L, width=7) == 6
    assert _conv_update_call(L, state=_CFAKE["s0"] + 2) == 4
    assert _conv_update_call(L, y=_CFAKE["s0"]) == 5
    assert _conv_update_call(L, state=_CFAKE["w"]) == 5
    assert _conv_update_call(L) == 8


@pytest.mark.gpu
def test_conv_argument_errors_write_nothing():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(2, 8, 40, generator=g).to(torch.bfloat16).cuda()
    w = torch.randn(8, 4, generator=g).cuda()
    s0 = torch.randn(2, 8, 3, generator=g).cuda()
    y = torch.full((2, 8, 40), 7.0, device="cuda")
    sL = torch.full((2, 8, 3), 7.0, device="cuda")
    L = ssm.lib()
    base = dict(x=x.data_ptr(), w=w.data_ptr(), bias=None, s0=s0.data_ptr(), outd=0,
                y=y.data_ptr(), sL=sL.data_ptr())
    for name, over, status in CONV_ERRORS:
        assert _conv_call(L, **{**base, **over}) == status, name
    assert _conv_call(L, **{**base, "sL": s0.data_ptr() + 4}) == 5
    assert _conv_call(L, **{**base, "y": x.data_ptr()}) == 5
    torch.cuda.synchronize()
    assert (y == 7.0).all() and (sL == 7.0).all()
