"""Selective state-space (S6) scan for AMD MI355X (gfx950).

Thin Python binding over the C ABI in ``include/ssm.h``, ``include/ssm_bwd.h``
and ``include/ssm_conv.h`` (``libssm.so``):
argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``csrc/``; PyTorch only provides device memory and the stream.
There is no CPU fallback: if the library is missing or no GPU is present the
calls raise.

    y, hL = ssm_scan_fwd(x, dt, A, Bm, Cm, dt_bias=..., Dskip=..., z=..., h0=...)
    y = ssm_state_update(state, x, dt, A, Bm, Cm, dt_bias=..., Dskip=..., z=...)
    grads = ssm_scan_bwd(x, dt, A, Bm, Cm, dy, dt_bias=..., Dskip=..., z=..., h0=..., dhL=...)
    y, stateL = ssm_conv1d_fwd(x, weight, bias=..., state0=..., silu=True)
    y = ssm_conv1d_update(state, x, weight, bias=..., silu=True)

Layouts: x, dt, z, y [batch, dim, L]; Bm, Cm [batch, N, L]; A [dim, N];
Dskip, dt_bias [dim]; h0, hL, state [batch, dim, N] (decode: drop L);
conv weight [dim, W], bias [dim], conv state [batch, dim, W-1].
"""
import ctypes
import functools
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssm.so")

SSM_F32, SSM_BF16 = 0, 1
SSM_FLAG_ZOH_B = 0x1
SSM_FLAG_CHECKPOINTS = 0x2
SSM_CONV_SILU = 0x1
STATUS = {
    0: "SSM_OK", 1: "SSM_ERR_NULL_ARG", 2: "SSM_ERR_BAD_SHAPE", 3: "SSM_ERR_BAD_DTYPE",
    4: "SSM_ERR_MISALIGNED", 5: "SSM_ERR_ALIAS", 6: "SSM_ERR_UNSUPPORTED",
    7: "SSM_ERR_WORKSPACE", 8: "SSM_ERR_HIP",
}
EXPORTS = ["ssm_abi_version", "ssm_status_string", "ssm_scan_fwd_workspace_bytes",
           "ssm_scan_fwd", "ssm_scan_fwd_strided", "ssm_scan_fwd_noalloc",
           "ssm_scan_fwd_bld_workspace_bytes", "ssm_scan_fwd_bld",
           "ssm_state_update", "ssm_state_update_strided",
           "ssm_conv1d_fwd", "ssm_conv1d_fwd_strided", "ssm_conv1d_fwd_bld", "ssm_conv1d_update",
           "ssm_conv1d_update_strided",
           "ssm_scan_bwd_workspace_bytes", "ssm_scan_bwd", "ssm_scan_bwd_strided",
           "ssm_scan_bwd_bld_workspace_bytes", "ssm_scan_bwd_bld"]


class ScanLayout(ctypes.Structure):
    """ssm_scan_layout_t: strides in elements, 0 = dense default."""
    _fields_ = [("seq_row", ctypes.c_longlong), ("seq_batch", ctypes.c_longlong * 4),
                ("bc_row", ctypes.c_longlong), ("bc_batch", ctypes.c_longlong * 2)]


class BldLayout(ctypes.Structure):
    """ssm_bld_layout_t: step and batch strides in elements, 0 = dense default."""
    _fields_ = [(n, ctypes.c_longlong) for n in (
        "x_step", "dt_step", "z_step", "y_step", "x_batch", "dt_batch", "z_batch", "y_batch",
        "B_step", "C_step", "B_batch", "C_batch")]


class BwdLayout(ctypes.Structure):
    """ssm_scan_bwd_layout_t: strides in elements, 0 = dense default."""
    _fields_ = [("seq_row", ctypes.c_longlong), ("seq_batch", ctypes.c_longlong * 7),
                ("bc_row", ctypes.c_longlong), ("bc_batch", ctypes.c_longlong * 2)]


class BwdBldLayout(ctypes.Structure):
    """ssm_scan_bwd_bld_layout_t: step and batch strides in elements (x, dt, z,
    dy, dx, ddt, dz; then Bm, Cm), 0 = dense default."""
    _fields_ = [("step", ctypes.c_longlong * 7), ("batch_stride", ctypes.c_longlong * 7),
                ("B_step", ctypes.c_longlong), ("C_step", ctypes.c_longlong),
                ("B_batch", ctypes.c_longlong), ("C_batch", ctypes.c_longlong)]


class ConvLayout(ctypes.Structure):
    """ssm_conv_layout_t: strides in elements, 0 = dense default."""
    _fields_ = [("x_row", ctypes.c_longlong), ("x_batch", ctypes.c_longlong),
                ("y_row", ctypes.c_longlong), ("y_batch", ctypes.c_longlong)]


class ConvBldLayout(ctypes.Structure):
    """ssm_conv_bld_layout_t: step and batch strides in elements, 0 = dense default."""
    _fields_ = [(n, ctypes.c_longlong) for n in ("x_step", "x_batch", "y_step", "y_batch")]


class UpdateLayout(ctypes.Structure):
    """ssm_update_layout_t: batch strides in elements, 0 = dense default."""
    _fields_ = [("x_batch", ctypes.c_longlong), ("dt_batch", ctypes.c_longlong),
                ("z_batch", ctypes.c_longlong), ("y_batch", ctypes.c_longlong),
                ("B_batch", ctypes.c_longlong), ("C_batch", ctypes.c_longlong)]


class SSMError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s (%d): %s" % (STATUS.get(status, "?"), status, message))
        self.status = status


_lib = None


def lib():
    """The loaded libssm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libssm.so is not built (run __graft_entry__.build() or "
                               "python -m selective_state_space_64_amd._build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, u, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t
        L.ssm_abi_version.restype = i
        L.ssm_abi_version.argtypes = []
        L.ssm_status_string.restype = ctypes.c_char_p
        L.ssm_status_string.argtypes = [i]
        L.ssm_scan_fwd_workspace_bytes.restype = sz
        L.ssm_scan_fwd_workspace_bytes.argtypes = [i, i, i, i]
        L.ssm_scan_fwd.restype = i
        L.ssm_scan_fwd.argtypes = [i, i, i, i, i, u] + [vp] * 9 + [i, vp, vp, vp, sz, vp]
        L.ssm_scan_fwd_strided.restype = i
        L.ssm_scan_fwd_strided.argtypes = ([i, i, i, i, i, u] + [vp] * 9 +
                                           [i, vp, vp, vp, sz, ctypes.POINTER(ScanLayout), vp])
        L.ssm_scan_fwd_noalloc.restype = i
        L.ssm_scan_fwd_noalloc.argtypes = ([i, i, i, i, i, u] + [vp] * 9 +
                                           [i, vp, vp, ctypes.POINTER(ScanLayout), vp])
        L.ssm_scan_fwd_bld_workspace_bytes.restype = sz
        L.ssm_scan_fwd_bld_workspace_bytes.argtypes = [i, i, i, i]
        L.ssm_scan_fwd_bld.restype = i
        L.ssm_scan_fwd_bld.argtypes = ([i, i, i, i, i, u] + [vp] * 9 +
                                       [i, vp, vp, vp, sz, ctypes.POINTER(BldLayout), vp])
        L.ssm_state_update_strided.restype = i
        L.ssm_state_update_strided.argtypes = ([i, i, i, i, u] + [vp] * 9 +
                                               [i, vp, ctypes.POINTER(UpdateLayout), vp])
        L.ssm_conv1d_update_strided.restype = i
        L.ssm_conv1d_update_strided.argtypes = ([i, i, i, i, u] + [vp] * 4 +
                                                [i, vp, ctypes.c_longlong, ctypes.c_longlong, vp])
        L.ssm_state_update.restype = i
        L.ssm_state_update.argtypes = [i, i, i, i, u] + [vp] * 9 + [i, vp, vp]
        L.ssm_scan_bwd_workspace_bytes.restype = sz
        L.ssm_scan_bwd_workspace_bytes.argtypes = [i, i, i, i]
        L.ssm_scan_bwd.restype = i
        L.ssm_scan_bwd.argtypes = [i, i, i, i, i, u] + [vp] * 9 + [i] + [vp] * 12 + [sz, vp]
        L.ssm_scan_bwd_strided.restype = i
        L.ssm_scan_bwd_strided.argtypes = ([i, i, i, i, i, u] + [vp] * 9 + [i] + [vp] * 12 +
                                           [sz, ctypes.POINTER(BwdLayout), vp])
        L.ssm_scan_bwd_bld_workspace_bytes.restype = sz
        L.ssm_scan_bwd_bld_workspace_bytes.argtypes = [i, i, i, i]
        L.ssm_scan_bwd_bld.restype = i
        L.ssm_scan_bwd_bld.argtypes = ([i, i, i, i, i, u] + [vp] * 9 + [i] + [vp] * 12 +
                                       [sz, ctypes.POINTER(BwdBldLayout), vp])
        L.ssm_conv1d_fwd.restype = i
        L.ssm_conv1d_fwd.argtypes = [i, i, i, i, i, u] + [vp] * 4 + [i, vp, vp, vp]
        L.ssm_conv1d_fwd_strided.restype = i
        L.ssm_conv1d_fwd_strided.argtypes = ([i, i, i, i, i, u] + [vp] * 4 +
                                             [i, vp, vp, ctypes.POINTER(ConvLayout), vp])
        L.ssm_conv1d_fwd_bld.restype = i
        L.ssm_conv1d_fwd_bld.argtypes = ([i, i, i, i, i, u] + [vp] * 4 +
                                         [i, vp, vp, ctypes.POINTER(ConvBldLayout), vp])
        L.ssm_conv1d_update.restype = i
        L.ssm_conv1d_update.argtypes = [i, i, i, i, u] + [vp] * 4 + [i, vp, vp]
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise SSMError(status, lib().ssm_status_string(status).decode())


def _dtype_code(t):
    if t == torch.float32:
        return SSM_F32
    if t == torch.bfloat16:
        return SSM_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t)


def _ptr(t, name, shape=None, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and t.shape != shape:
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


def _rows(ts, names, shape, dtype):
    """Pointers, shared row stride and batch strides of [batch, rows, L]
    tensors whose time index is contiguous (views such as halves of one
    projection output).  Strides of size-1 dimensions are free and read as the
    dense default (0).  Broadcast views (stride 0 on a dimension of size > 1,
    e.g. from expand()) are rejected: the C ABI reads a stride of 0 as the
    dense default, so passing one through would index past the allocation."""
    batch, rows, L = shape
    ptrs, bstrides, rstride = [], [], None
    for t, name in zip(ts, names):
        if t is None:
            ptrs.append(None)
            bstrides.append(0)
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a CUDA (HIP) tensor" % name)
        if t.shape != shape:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
        want = dtype[name] if isinstance(dtype, dict) else dtype
        if t.dtype != want:
            raise TypeError("%s must be %s, got %s" % (name, want, t.dtype))
        _no_broadcast(t, name)
        if L > 1 and t.stride(2) != 1:
            raise ValueError("%s must have a contiguous time index (stride 1)" % name)
        if not t.is_cuda:
            raise TypeError("%s must be a CUDA (HIP) tensor" % name)
        if rows > 1:
            if rstride is None:
                rstride = t.stride(1)
            elif t.stride(1) != rstride:
                raise ValueError("%s must share the row stride of %s (%d, got %d)"
                                 % (name, "/".join(names), rstride, t.stride(1)))
        ptrs.append(t.data_ptr())
        bstrides.append(t.stride(0) if batch > 1 else 0)
    return ptrs, (rstride if rstride is not None else 0), bstrides


def _no_broadcast(t, name):
    """Raise for a view that repeats memory along a dimension (stride 0 on a
    dimension of size > 1): the kernels would read it at dense offsets."""
    for k in range(t.dim()):
        if t.shape[k] > 1 and t.stride(k) == 0:
            raise ValueError("%s is a broadcast view (stride 0 along dimension %d); "
                             "pass a materialised tensor (.contiguous())" % (name, k))


def _no_broadcast_args(**tensors):
    """_no_broadcast over every tensor argument of a call, before any other
    check, so that such a view is reported as what it is."""
    for name, t in tensors.items():
        if isinstance(t, torch.Tensor):
            _no_broadcast(t, name)


def _bptr(t, name, shape, dtype):
    """Pointer and batch stride (elements; 0 = dense) of a [batch, n] tensor
    whose last index is contiguous, e.g. one half of a projection row.
    Broadcast views (stride 0 on a dimension of size > 1) are rejected."""
    if t is None:
        return None, 0
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if t.shape != shape:
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    _no_broadcast(t, name)
    if shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("%s must have a contiguous last index" % name)
    if not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    sb = t.stride(0)
    return t.data_ptr(), (sb if shape[0] > 1 and sb != shape[1] else 0)


def _on_caller_stream(fn):
    """Run the call with `stream` (when given) as the current stream, so that
    every tensor allocated inside it (outputs, workspace) belongs to the stream
    the kernels are enqueued on: the caching allocator then cannot hand such a
    block to work on another stream while these kernels still use it."""
    @functools.wraps(fn)
    def call(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kw)
    return call


def _stream(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


@_on_caller_stream
def ssm_scan_fwd(x, dt, A, Bm, Cm, *, dt_bias=None, Dskip=None, z=None, h0=None,
                 out_dtype=torch.float32, return_final_state=True, y=None, hL=None,
                 zoh=False, checkpoints=None, workspace=None, stream=None):
    """Fused selective scan; returns (y, hL) (hL is None unless requested).
    x, dt, z, y (and Bm, Cm) may be strided views with a contiguous time
    index and one row stride shared among them, e.g. x and z as the two
    halves of one [batch, 2 dim, L] projection output.
    zoh=True selects the exact zero-order-hold B-bar (SSM_FLAG_ZOH_B).
    checkpoints: a device buffer of ssm_scan_bwd_workspace_bytes(...) bytes
    that receives the backward pass's checkpoints (SSM_FLAG_CHECKPOINTS); pass
    it to ssm_scan_bwd with checkpoints_in_workspace=True.
    workspace: device scratch of ssm_scan_fwd_workspace_bytes(...) bytes for
    shapes whose sequence the library splits across workgroups (few batch
    rows and channels, long L); allocated here when not given."""
    _no_broadcast_args(x=x, dt=dt, A=A, Bm=Bm, Cm=Cm, dt_bias=dt_bias, Dskip=Dskip, z=z, h0=h0,
                       y=y, hL=hL)
    if x.dim() != 3:
        raise ValueError("x must be [batch, dim, L]")
    batch, dim, L = x.shape
    N = A.shape[-1]
    ind = x.dtype
    if y is None:
        y = torch.empty((batch, dim, L), dtype=out_dtype, device=x.device)
    if hL is None and return_final_state:
        hL = torch.empty((batch, dim, N), dtype=torch.float32, device=x.device)
    f32 = torch.float32
    (xp, dtp, zp, yp), row, seq_b = _rows(
        (x, dt, z, y), ("x", "dt", "z", "y"), (batch, dim, L),
        {"x": ind, "dt": ind, "z": ind, "y": out_dtype})
    (Bp, Cp), bc_row, bc_b = _rows((Bm, Cm), ("Bm", "Cm"), (batch, N, L), ind)
    layout = ScanLayout(row, (ctypes.c_longlong * 4)(*seq_b), bc_row,
                        (ctypes.c_longlong * 2)(*bc_b))
    args = [
        xp, dtp, _ptr(dt_bias, "dt_bias", (dim,), f32), _ptr(A, "A", (dim, N), f32),
        Bp, Cp, _ptr(Dskip, "Dskip", (dim,), f32), zp, _ptr(h0, "h0", (batch, dim, N), f32),
    ]
    hp = _ptr(hL, "hL", (batch, dim, N), f32)
    flags = SSM_FLAG_ZOH_B if zoh else 0
    wp, wb = None, 0
    if checkpoints is not None:
        flags |= SSM_FLAG_CHECKPOINTS
        wp, wb = _ptr(checkpoints, "checkpoints"), checkpoints.numel() * checkpoints.element_size()
    else:
        need = lib().ssm_scan_fwd_workspace_bytes(batch, dim, L, N)
        if workspace is None and need:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        if workspace is not None:
            wp, wb = _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size()
    st = lib().ssm_scan_fwd_strided(batch, dim, L, N, _dtype_code(ind), flags, *args,
                                    _dtype_code(y.dtype), yp, hp, wp, wb, ctypes.byref(layout),
                                    _stream(stream, x.device))
    _check(st)
    return y, hL


def _steps(ts, names, shape, dtype):
    """Pointers, step strides and batch strides (elements; 0 = dense default)
    of [batch, L, n] tensors whose last index is contiguous."""
    batch, L, n = shape
    ptrs, st, sb = [], [], []
    for t, name in zip(ts, names):
        if t is None:
            ptrs.append(None)
            st.append(0)
            sb.append(0)
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a CUDA (HIP) tensor" % name)
        if t.shape != shape:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
        want = dtype[name] if isinstance(dtype, dict) else dtype
        if t.dtype != want:
            raise TypeError("%s must be %s, got %s" % (name, want, t.dtype))
        _no_broadcast(t, name)
        if n > 1 and t.stride(2) != 1:
            raise ValueError("%s must have a contiguous last (channel) index" % name)
        if not t.is_cuda:
            raise TypeError("%s must be a CUDA (HIP) tensor" % name)
        ptrs.append(t.data_ptr())
        st.append(t.stride(1) if L > 1 else 0)
        sb.append(t.stride(0) if batch > 1 else 0)
    return ptrs, st, sb


@_on_caller_stream
def ssm_scan_fwd_bld(x, dt, A, Bm, Cm, *, dt_bias=None, Dskip=None, z=None, h0=None,
                     out_dtype=torch.float32, return_final_state=True, y=None, hL=None, zoh=False,
                     workspace=None, stream=None):
    """The selective scan on (batch, L, dim)-ordered tensors: x, dt, z, y are
    [batch, L, dim] and Bm, Cm [batch, L, N], each with a contiguous last
    index (views such as x and z as halves of one [batch, L, 2 dim]
    projection output are taken as they are).  Returns (y, hL); y is
    [batch, L, dim].  workspace: ssm_scan_fwd_bld_workspace_bytes(...) bytes,
    allocated here when not given."""
    _no_broadcast_args(x=x, dt=dt, A=A, Bm=Bm, Cm=Cm, dt_bias=dt_bias, Dskip=Dskip, z=z, h0=h0,
                       y=y, hL=hL)
    if x.dim() != 3:
        raise ValueError("x must be [batch, L, dim]")
    batch, L, dim = x.shape
    N = A.shape[-1]
    ind, f32 = x.dtype, torch.float32
    if y is None:
        y = torch.empty((batch, L, dim), dtype=out_dtype, device=x.device)
    if hL is None and return_final_state:
        hL = torch.empty((batch, dim, N), dtype=f32, device=x.device)
    (xp, dtp, zp, yp), st, sb = _steps((x, dt, z, y), ("x", "dt", "z", "y"), (batch, L, dim),
                                       {"x": ind, "dt": ind, "z": ind, "y": y.dtype})
    (Bp, Cp), bst, bsb = _steps((Bm, Cm), ("Bm", "Cm"), (batch, L, N), ind)
    layout = BldLayout(*st, *sb, *bst, *bsb)
    need = lib().ssm_scan_fwd_bld_workspace_bytes(batch, dim, L, N)
    if workspace is None:
        workspace = torch.empty(max(1, need), dtype=torch.uint8, device=x.device)
    st_ = lib().ssm_scan_fwd_bld(
        batch, dim, L, N, _dtype_code(ind), SSM_FLAG_ZOH_B if zoh else 0, xp, dtp,
        _ptr(dt_bias, "dt_bias", (dim,), f32), _ptr(A, "A", (dim, N), f32), Bp, Cp,
        _ptr(Dskip, "Dskip", (dim,), f32), zp, _ptr(h0, "h0", (batch, dim, N), f32),
        _dtype_code(y.dtype), yp, _ptr(hL, "hL", (batch, dim, N), f32), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), ctypes.byref(layout),
        _stream(stream, x.device))
    _check(st_)
    return y, hL


def ssm_scan_fwd_noalloc(x, dt, A, Bm, Cm, *, y, hL=None, dt_bias=None, Dskip=None, z=None,
                         h0=None, zoh=False, stream=None):
    """ssm_scan_fwd through the allocation-free entry point: nothing is
    allocated, here or in the library (y, and hL if wanted, are given by the
    caller; a sequence split uses the library's per-GPU scratch array, so
    calls overlapping in time on one GPU must be serialised).  Returns (y, hL)."""
    _no_broadcast_args(x=x, dt=dt, A=A, Bm=Bm, Cm=Cm, dt_bias=dt_bias, Dskip=Dskip, z=z, h0=h0,
                       y=y, hL=hL)
    if x.dim() != 3:
        raise ValueError("x must be [batch, dim, L]")
    batch, dim, L = x.shape
    N = A.shape[-1]
    ind, f32 = x.dtype, torch.float32
    (xp, dtp, zp, yp), row, seq_b = _rows(
        (x, dt, z, y), ("x", "dt", "z", "y"), (batch, dim, L),
        {"x": ind, "dt": ind, "z": ind, "y": y.dtype})
    (Bp, Cp), bc_row, bc_b = _rows((Bm, Cm), ("Bm", "Cm"), (batch, N, L), ind)
    layout = ScanLayout(row, (ctypes.c_longlong * 4)(*seq_b), bc_row,
                        (ctypes.c_longlong * 2)(*bc_b))
    st = lib().ssm_scan_fwd_noalloc(
        batch, dim, L, N, _dtype_code(ind), SSM_FLAG_ZOH_B if zoh else 0, xp, dtp,
        _ptr(dt_bias, "dt_bias", (dim,), f32), _ptr(A, "A", (dim, N), f32), Bp, Cp,
        _ptr(Dskip, "Dskip", (dim,), f32), zp, _ptr(h0, "h0", (batch, dim, N), f32),
        _dtype_code(y.dtype), yp, _ptr(hL, "hL", (batch, dim, N), f32), ctypes.byref(layout),
        _stream(stream, x.device))
    _check(st)
    return y, hL


@_on_caller_stream
def ssm_state_update(state, x, dt, A, Bm, Cm, *, dt_bias=None, Dskip=None, z=None,
                     out_dtype=torch.float32, y=None, zoh=False, stream=None):
    """One decode step; updates `state` in place and returns y [batch, dim].
    zoh=True selects the exact zero-order-hold B-bar (SSM_FLAG_ZOH_B).
    x, dt, z, y, Bm and Cm may be batch-strided views with a contiguous last
    index (x and z as halves of the step's [batch, 2 dim] projection row)."""
    _no_broadcast_args(state=state, x=x, dt=dt, A=A, Bm=Bm, Cm=Cm, dt_bias=dt_bias, Dskip=Dskip,
                       z=z, y=y)
    batch, dim, N = state.shape
    ind = x.dtype
    if y is None:
        y = torch.empty((batch, dim), dtype=out_dtype, device=x.device)
    f32 = torch.float32
    xp, xb = _bptr(x, "x", (batch, dim), ind)
    dtp, dtb = _bptr(dt, "dt", (batch, dim), ind)
    zp, zb = _bptr(z, "z", (batch, dim), ind)
    yp, yb = _bptr(y, "y", (batch, dim), out_dtype)
    Bp, Bb = _bptr(Bm, "Bm", (batch, N), ind)
    Cp, Cb = _bptr(Cm, "Cm", (batch, N), ind)
    # a layout only when some tensor is strided (keeps the per-token call lean)
    layout = UpdateLayout(xb, dtb, zb, yb, Bb, Cb) if (xb or dtb or zb or yb or Bb or Cb) else None
    args = [
        _ptr(state, "state", (batch, dim, N), f32), xp, dtp,
        _ptr(dt_bias, "dt_bias", (dim,), f32), _ptr(A, "A", (dim, N), f32), Bp, Cp,
        _ptr(Dskip, "Dskip", (dim,), f32), zp,
    ]
    flags = SSM_FLAG_ZOH_B if zoh else 0
    st = lib().ssm_state_update_strided(batch, dim, N, _dtype_code(ind), flags, *args,
                                        _dtype_code(y.dtype), yp,
                                        None if layout is None else ctypes.byref(layout),
                                        _stream(stream, x.device))
    _check(st)
    return y


class StateUpdateSteps:
    """Token-by-token decode over step-major buffers with the arguments
    checked once: the per-token call is a pointer offset and one C call.

        steps = StateUpdateSteps(state, A, xs, dts, Bs, Cs, ys=ys, dt_bias=..., Dskip=..., zs=...)
        for s in range(n): steps(s)      # = ssm_state_update(state, xs[s], ..., y=ys[s])

    xs, dts, zs, ys are [steps, batch, dim] and Bs, Cs [steps, batch, N]
    tensors (any of them may instead be [batch, dim] / [batch, N], reused
    for every step), each step's slice a batch-strided view as
    ssm_state_update accepts.  The buffers must stay alive and in place while
    the object is used; the stream is fixed at construction (the current one
    by default).  The library still validates every call."""

    def __init__(self, state, A, xs, dts, Bs, Cs, *, ys, dt_bias=None, Dskip=None, zs=None,
                 zoh=False, stream=None):
        _no_broadcast_args(state=state, A=A, xs=xs, dts=dts, Bs=Bs, Cs=Cs, ys=ys, dt_bias=dt_bias,
                           Dskip=Dskip, zs=zs)
        batch, dim, N = state.shape
        ind, f32 = xs.dtype, torch.float32
        self.nsteps = None
        per = []   # (base pointer, bytes per step) of x, dt, z, y, Bm, Cm
        bstr = []  # batch strides (0 = dense)
        for t, name, n, dtype in ((xs, "xs", dim, ind), (dts, "dts", dim, ind), (zs, "zs", dim, ind),
                                  (ys, "ys", dim, None), (Bs, "Bs", N, ind), (Cs, "Cs", N, ind)):
            if t is None:
                per.append((None, 0))
                bstr.append(0)
                continue
            if dtype is not None and t.dtype != dtype:
                raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
            one = t[0] if t.dim() == 3 else t
            p, sb = _bptr(one, name, (batch, n), t.dtype)
            if t.dim() == 3:
                if self.nsteps is not None and t.shape[0] != self.nsteps:
                    raise ValueError("%s has %d steps, expected %d" % (name, t.shape[0], self.nsteps))
                self.nsteps = t.shape[0]
                per.append((p, t.stride(0) * t.element_size()))
            else:
                per.append((p, 0))
            bstr.append(sb)
        self._per = per
        self._layout = UpdateLayout(*bstr) if any(bstr) else None
        self._lp = None if self._layout is None else ctypes.byref(self._layout)
        self._fixed = (batch, dim, N, _dtype_code(ind), SSM_FLAG_ZOH_B if zoh else 0,
                       _ptr(state, "state", (batch, dim, N), f32))
        self._bias = _ptr(dt_bias, "dt_bias", (dim,), f32)
        self._A = _ptr(A, "A", (dim, N), f32)
        self._D = _ptr(Dskip, "Dskip", (dim,), f32)
        self._out = _dtype_code(ys.dtype)
        self._stream = _stream(stream, state.device)
        self._fn = lib().ssm_state_update_strided
        self._keep = (state, A, xs, dts, Bs, Cs, ys, dt_bias, Dskip, zs)

    def __call__(self, s):
        if self.nsteps is not None and not 0 <= s < self.nsteps:
            raise IndexError("step %d of %d" % (s, self.nsteps))
        (x, xs), (d, ds), (z, zs), (y, ys), (b, bs), (c, cs) = self._per
        st = self._fn(*self._fixed, x + s * xs, d + s * ds, self._bias, self._A, b + s * bs,
                      c + s * cs, self._D, None if z is None else z + s * zs, self._out, y + s * ys,
                      self._lp, self._stream)
        if st != 0:
            _check(st)


@_on_caller_stream
def ssm_scan_bwd(x, dt, A, Bm, Cm, dy, *, dt_bias=None, Dskip=None, z=None, h0=None, dhL=None,
                 grad_dtype=torch.float32, workspace=None, checkpoints_in_workspace=False,
                 dx=None, ddt=None, dz=None, zoh=False, stream=None):
    """Gradients of sum(dy * y) + sum(dhL * hL) through ssm_scan_fwd (Delta*B
    form, or the exact zero-order-hold form with zoh=True).  Returns a dict:
    dx, ddt, dz (None without z) in grad_dtype; dBm, dCm, dA, dDskip,
    ddt_bias, dh0 in fp32 (dDskip / ddt_bias / dh0 are computed for every
    call).  checkpoints_in_workspace=True: `workspace`
    holds the checkpoints a forward call wrote (SSM_FLAG_CHECKPOINTS).
    x, dt, z, dy and the outputs dx, ddt, dz (given here, else allocated
    dense) may be strided views with a contiguous time index and one shared
    row stride, e.g. z and dz as halves of the projection's buffers; Bm and
    Cm likewise with their own row stride."""
    _no_broadcast_args(x=x, dt=dt, A=A, Bm=Bm, Cm=Cm, dy=dy, dt_bias=dt_bias, Dskip=Dskip, z=z,
                       h0=h0, dhL=dhL, dx=dx, ddt=ddt, dz=dz)
    if x.dim() != 3:
        raise ValueError("x must be [batch, dim, L]")
    batch, dim, L = x.shape
    N = A.shape[-1]
    ind, dev, f32 = x.dtype, x.device, torch.float32
    shape = (batch, dim, L)
    g = {
        "dx": dx if dx is not None else torch.empty(shape, dtype=grad_dtype, device=dev),
        "ddt": ddt if ddt is not None else torch.empty(shape, dtype=grad_dtype, device=dev),
        "dz": (dz if dz is not None else torch.empty(shape, dtype=grad_dtype, device=dev))
              if z is not None else None,
        "dBm": torch.empty((batch, N, L), dtype=f32, device=dev),
        "dCm": torch.empty((batch, N, L), dtype=f32, device=dev),
        "dA": torch.empty((dim, N), dtype=f32, device=dev),
        "dDskip": torch.empty((dim,), dtype=f32, device=dev),
        "ddt_bias": torch.empty((dim,), dtype=f32, device=dev),
        "dh0": torch.empty((batch, dim, N), dtype=f32, device=dev),
    }
    need = lib().ssm_scan_bwd_workspace_bytes(batch, dim, L, N)
    if workspace is None:
        if checkpoints_in_workspace:
            raise ValueError("checkpoints_in_workspace needs the forward's workspace")
        workspace = torch.empty((max(1, need),), dtype=torch.uint8, device=dev)
    names = ("x", "dt", "z", "dy", "dx", "ddt", "dz")
    (xp, dtp, zp, dyp, dxp, ddtp, dzp), row, seq_b = _rows(
        (x, dt, z, dy, g["dx"], g["ddt"], g["dz"]), names, shape,
        {"x": ind, "dt": ind, "z": ind, "dy": grad_dtype, "dx": grad_dtype, "ddt": grad_dtype,
         "dz": grad_dtype})
    (Bp, Cp), bc_row, bc_b = _rows((Bm, Cm), ("Bm", "Cm"), (batch, N, L), ind)
    layout = BwdLayout(row, (ctypes.c_longlong * 7)(*seq_b), bc_row,
                       (ctypes.c_longlong * 2)(*bc_b))
    args = [
        xp, dtp, _ptr(dt_bias, "dt_bias", (dim,), f32), _ptr(A, "A", (dim, N), f32),
        Bp, Cp, _ptr(Dskip, "Dskip", (dim,), f32), zp, _ptr(h0, "h0", (batch, dim, N), f32),
    ]
    gargs = [
        dyp, _ptr(dhL, "dhL", (batch, dim, N), f32), dxp, ddtp, dzp, _ptr(g["dBm"], "dBm"),
        _ptr(g["dCm"], "dCm"), _ptr(g["dA"], "dA"), _ptr(g["dDskip"], "dDskip"),
        _ptr(g["ddt_bias"], "ddt_bias"), _ptr(g["dh0"], "dh0"),
    ]
    flags = SSM_FLAG_CHECKPOINTS if checkpoints_in_workspace else 0
    if zoh:
        flags |= SSM_FLAG_ZOH_B
    st = lib().ssm_scan_bwd_strided(batch, dim, L, N, _dtype_code(ind), flags, *args,
                                    _dtype_code(grad_dtype), *gargs, _ptr(workspace, "workspace"),
                                    workspace.numel() * workspace.element_size(),
                                    ctypes.byref(layout), _stream(stream, dev))
    _check(st)
    return g


@_on_caller_stream
def ssm_scan_bwd_bld(x, dt, A, Bm, Cm, dy, *, dt_bias=None, Dskip=None, z=None, h0=None,
                     dhL=None, grad_dtype=torch.float32, workspace=None, dx=None, ddt=None,
                     dz=None, zoh=False, stream=None):
    """ssm_scan_bwd on (batch, L, dim) tensors: x, dt, z, dy and the outputs
    dx, ddt, dz as [batch, L, dim], Bm, Cm as [batch, L, N] (the layout of
    ssm_scan_fwd_bld; channel index contiguous, e.g. z and dz as halves of
    [batch, L, 2 dim] buffers).  Returns a dict as ssm_scan_bwd, with dBm and
    dCm as [batch, L, N].  workspace: ssm_scan_bwd_bld_workspace_bytes(...)
    bytes (allocated here when not given)."""
    _no_broadcast_args(x=x, dt=dt, A=A, Bm=Bm, Cm=Cm, dy=dy, dt_bias=dt_bias, Dskip=Dskip, z=z,
                       h0=h0, dhL=dhL, dx=dx, ddt=ddt, dz=dz)
    if x.dim() != 3:
        raise ValueError("x must be [batch, L, dim]")
    batch, L, dim = x.shape
    N = A.shape[-1]
    ind, dev, f32 = x.dtype, x.device, torch.float32
    shape = (batch, L, dim)
    g = {
        "dx": dx if dx is not None else torch.empty(shape, dtype=grad_dtype, device=dev),
        "ddt": ddt if ddt is not None else torch.empty(shape, dtype=grad_dtype, device=dev),
        "dz": (dz if dz is not None else torch.empty(shape, dtype=grad_dtype, device=dev))
              if z is not None else None,
        "dBm": torch.empty((batch, L, N), dtype=f32, device=dev),
        "dCm": torch.empty((batch, L, N), dtype=f32, device=dev),
        "dA": torch.empty((dim, N), dtype=f32, device=dev),
        "dDskip": torch.empty((dim,), dtype=f32, device=dev),
        "ddt_bias": torch.empty((dim,), dtype=f32, device=dev),
        "dh0": torch.empty((batch, dim, N), dtype=f32, device=dev),
    }
    need = lib().ssm_scan_bwd_bld_workspace_bytes(batch, dim, L, N)
    if workspace is None:
        workspace = torch.empty((max(1, need),), dtype=torch.uint8, device=dev)
    names = ("x", "dt", "z", "dy", "dx", "ddt", "dz")
    (xp, dtp, zp, dyp, dxp, ddtp, dzp), st, sb = _steps(
        (x, dt, z, dy, g["dx"], g["ddt"], g["dz"]), names, shape,
        {"x": ind, "dt": ind, "z": ind, "dy": grad_dtype, "dx": grad_dtype, "ddt": grad_dtype,
         "dz": grad_dtype})
    (Bp, Cp), bst, bsb = _steps((Bm, Cm), ("Bm", "Cm"), (batch, L, N), ind)
    layout = BwdBldLayout((ctypes.c_longlong * 7)(*st), (ctypes.c_longlong * 7)(*sb),
                          bst[0], bst[1], bsb[0], bsb[1])
    args = [
        xp, dtp, _ptr(dt_bias, "dt_bias", (dim,), f32), _ptr(A, "A", (dim, N), f32),
        Bp, Cp, _ptr(Dskip, "Dskip", (dim,), f32), zp, _ptr(h0, "h0", (batch, dim, N), f32),
    ]
    gargs = [
        dyp, _ptr(dhL, "dhL", (batch, dim, N), f32), dxp, ddtp, dzp, _ptr(g["dBm"], "dBm"),
        _ptr(g["dCm"], "dCm"), _ptr(g["dA"], "dA"), _ptr(g["dDskip"], "dDskip"),
        _ptr(g["ddt_bias"], "ddt_bias"), _ptr(g["dh0"], "dh0"),
    ]
    st_ = lib().ssm_scan_bwd_bld(batch, dim, L, N, _dtype_code(ind), SSM_FLAG_ZOH_B if zoh else 0,
                                 *args, _dtype_code(grad_dtype), *gargs,
                                 _ptr(workspace, "workspace"),
                                 workspace.numel() * workspace.element_size(),
                                 ctypes.byref(layout), _stream(stream, dev))
    _check(st_)
    return g


@_on_caller_stream
def ssm_conv1d_fwd(x, weight, *, bias=None, state0=None, silu=True, out_dtype=None,
                   return_final_state=True, y=None, stateL=None, stream=None):
    """Causal depthwise conv over [batch, dim, L]; returns (y, stateL).
    out_dtype defaults to x's dtype (the conv output feeds the scan's x).
    x and y may be strided views with a contiguous time index (x as the
    first half of the input projection's [batch, 2 dim, L] output)."""
    _no_broadcast_args(x=x, weight=weight, bias=bias, state0=state0, y=y, stateL=stateL)
    if x.dim() != 3:
        raise ValueError("x must be [batch, dim, L]")
    batch, dim, L = x.shape
    W = weight.shape[-1]
    out_dtype = out_dtype or x.dtype
    if y is None:
        y = torch.empty((batch, dim, L), dtype=out_dtype, device=x.device)
    if stateL is None and return_final_state:
        stateL = torch.empty((batch, dim, W - 1), dtype=torch.float32, device=x.device)
    f32 = torch.float32
    (xp,), x_row, (x_b,) = _rows((x,), ("x",), (batch, dim, L), x.dtype)
    (yp,), y_row, (y_b,) = _rows((y,), ("y",), (batch, dim, L), out_dtype)
    layout = ConvLayout(x_row, x_b, y_row, y_b)
    args = [xp, _ptr(weight, "weight", (dim, W), f32),
            _ptr(bias, "bias", (dim,), f32), _ptr(state0, "state0", (batch, dim, W - 1), f32)]
    sp = _ptr(stateL, "stateL", (batch, dim, W - 1), f32)
    st = lib().ssm_conv1d_fwd_strided(batch, dim, L, W, _dtype_code(x.dtype),
                                      SSM_CONV_SILU if silu else 0, *args, _dtype_code(y.dtype), yp,
                                      sp, ctypes.byref(layout), _stream(stream, x.device))
    _check(st)
    return y, stateL


@_on_caller_stream
def ssm_conv1d_fwd_bld(x, weight, *, bias=None, state0=None, silu=True, out_dtype=None,
                       return_final_state=True, y=None, stateL=None, stream=None):
    """The causal depthwise conv on [batch, L, dim] tensors (channels
    contiguous; x may be the first half of a [batch, L, 2 dim] projection
    output); returns (y [batch, L, dim], stateL [batch, dim, W-1]).  The conv
    states are [batch, dim, W-1] as in ssm_conv1d_fwd."""
    _no_broadcast_args(x=x, weight=weight, bias=bias, state0=state0, y=y, stateL=stateL)
    if x.dim() != 3:
        raise ValueError("x must be [batch, L, dim]")
    batch, L, dim = x.shape
    W = weight.shape[-1]
    out_dtype = out_dtype or x.dtype
    if y is None:
        y = torch.empty((batch, L, dim), dtype=out_dtype, device=x.device)
    if stateL is None and return_final_state:
        stateL = torch.empty((batch, dim, W - 1), dtype=torch.float32, device=x.device)
    f32 = torch.float32
    (xp,), (x_t,), (x_b,) = _steps((x,), ("x",), (batch, L, dim), x.dtype)
    (yp,), (y_t,), (y_b,) = _steps((y,), ("y",), (batch, L, dim), out_dtype)
    layout = ConvBldLayout(x_t, x_b, y_t, y_b)
    args = [xp, _ptr(weight, "weight", (dim, W), f32),
            _ptr(bias, "bias", (dim,), f32), _ptr(state0, "state0", (batch, dim, W - 1), f32)]
    sp = _ptr(stateL, "stateL", (batch, dim, W - 1), f32)
    st = lib().ssm_conv1d_fwd_bld(batch, dim, L, W, _dtype_code(x.dtype),
                                  SSM_CONV_SILU if silu else 0, *args, _dtype_code(y.dtype), yp,
                                  sp, ctypes.byref(layout), _stream(stream, x.device))
    _check(st)
    return y, stateL


@_on_caller_stream
def ssm_conv1d_update(state, x, weight, *, bias=None, silu=True, out_dtype=None, y=None,
                      stream=None):
    """One decode step of the conv; shifts `state` [batch, dim, W-1] in place
    and returns y [batch, dim].  x and y may be batch-strided views with a
    contiguous last index (x as the first half of the step's projection row)."""
    _no_broadcast_args(state=state, x=x, weight=weight, bias=bias, y=y)
    batch, dim, H = state.shape
    out_dtype = out_dtype or x.dtype
    if y is None:
        y = torch.empty((batch, dim), dtype=out_dtype, device=x.device)
    f32 = torch.float32
    xp, xb = _bptr(x, "x", (batch, dim), x.dtype)
    yp, yb = _bptr(y, "y", (batch, dim), out_dtype)
    args = [_ptr(state, "state", (batch, dim, H), f32), xp,
            _ptr(weight, "weight", (dim, H + 1), f32), _ptr(bias, "bias", (dim,), f32)]
    st = lib().ssm_conv1d_update_strided(batch, dim, H + 1, _dtype_code(x.dtype),
                                         SSM_CONV_SILU if silu else 0, *args, _dtype_code(y.dtype),
                                         yp, xb, yb, _stream(stream, x.device))
    _check(st)
    return y


scan_fwd = ssm_scan_fwd
scan_bwd = ssm_scan_bwd
scan_bwd_bld = ssm_scan_bwd_bld
state_update = ssm_state_update
conv1d_fwd = ssm_conv1d_fwd
conv1d_fwd_bld = ssm_conv1d_fwd_bld
conv1d_update = ssm_conv1d_update
