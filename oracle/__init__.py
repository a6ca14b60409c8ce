"""fp64 CPU oracle for the selective state-space (S6) scan -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
in ``selective_state_space_64_amd`` and never imports it.

The arithmetic lives in ``ssm_oracle.c`` (plain sequential fp64 recurrence,
threaded over independent (batch, channel) rows); this module only marshals
numpy float64 arrays into it.  Sources and readings are listed in the C file's
header.  Mutant ids for the pin meta-test are listed in ``MUTANTS``.
"""
import ctypes
import os

import numpy as np

from . import _build

_HERE = os.path.dirname(os.path.abspath(__file__))

# Deliberately wrong variants compiled with -DORACLE_MUTANT=k.
MUTANTS = {
    1: "readout from the state before the update",
    2: "skip term D*x dropped",
    3: "gate sigmoid(z) instead of silu(z)",
    4: "sign error in exp(Delta*A)",
    5: "B read with transposed [L][N] indexing",
    6: "dt_bias ignored",
    7: "Delta taken from the neighbouring channel",
    8: "B and C swapped",
    9: "initial state ignored",
    10: "Delta factor dropped from B-bar",
    11: "A read with transposed [N][dim] indexing",
    12: "softplus without its max(u, 0) branch",
    13: "ZOH B-bar without the 1/A factor",
    14: "last entry of the final state not returned",
    15: "conv taps applied in reverse order",
    16: "conv reads one step ahead (not causal)",
    17: "initial conv state ignored",
    18: "conv activation not applied",
    19: "final conv state stored newest first",
    20: "backward: Delta gradient without the A-bar term",
    21: "backward: A gradient without the Delta factor",
    22: "backward: adjoint state not decayed by A-bar",
    23: "backward: gradient of the final state ignored",
    24: "backward: gate derivative sigmoid(z) instead of silu'(z)",
    25: "backward: softplus derivative taken as softplus",
    26: "backward: C gradient paired with the previous state",
    27: "ZOH backward: Delta derivative of B-bar taken from the Delta B form",
    28: "ZOH backward: A gradient without the B-bar term",
}

_dp = ctypes.POINTER(ctypes.c_double)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(_dp)


def _f64(a, shape, name):
    if a is None:
        return None
    arr = np.ascontiguousarray(a, dtype=np.float64)
    if arr.shape != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, arr.shape, tuple(shape)))
    return arr


class Oracle:
    """ctypes handle on one build of the oracle library."""

    def __init__(self, path=None):
        path = path or _build.LIB
        if not os.path.exists(path):
            raise FileNotFoundError("oracle library not built: %s (run oracle/_build.py)" % path)
        self.path = path
        lib = ctypes.CDLL(path)
        lib.ssm_oracle_scan_f64.restype = ctypes.c_int
        lib.ssm_oracle_scan_f64.argtypes = [ctypes.c_int] * 5 + [_dp] * 11 + [ctypes.c_int]
        lib.ssm_oracle_state_update_f64.restype = ctypes.c_int
        lib.ssm_oracle_state_update_f64.argtypes = [ctypes.c_int] * 4 + [_dp] * 10 + [ctypes.c_int]
        lib.ssm_oracle_conv1d_f64.restype = ctypes.c_int
        lib.ssm_oracle_conv1d_f64.argtypes = [ctypes.c_int] * 5 + [_dp] * 6 + [ctypes.c_int]
        lib.ssm_oracle_conv1d_update_f64.restype = ctypes.c_int
        lib.ssm_oracle_conv1d_update_f64.argtypes = [ctypes.c_int] * 4 + [_dp] * 5 + [ctypes.c_int]
        lib.ssm_oracle_scan_bwd_f64.restype = ctypes.c_int
        lib.ssm_oracle_scan_bwd_f64.argtypes = [ctypes.c_int] * 5 + [_dp] * 20 + [ctypes.c_int]
        lib.ssm_oracle_mutant_id.restype = ctypes.c_int
        self._lib = lib
        self.mutant = lib.ssm_oracle_mutant_id()

    def scan_fwd(self, x, dt, A, Bm, Cm, dt_bias=None, Dskip=None, z=None, h0=None,
                 zoh=False, threads=None):
        """y[batch,dim,L], hL[batch,dim,N] from the sequential fp64 recurrence."""
        x = np.asarray(x)
        if x.ndim != 3:
            raise ValueError("x must be [batch, dim, L]")
        batch, dim, L = x.shape
        A = np.asarray(A)
        N = A.shape[1]
        x = _f64(x, (batch, dim, L), "x")
        dt = _f64(dt, (batch, dim, L), "dt")
        A = _f64(A, (dim, N), "A")
        Bm = _f64(Bm, (batch, N, L), "Bm")
        Cm = _f64(Cm, (batch, N, L), "Cm")
        dt_bias = _f64(dt_bias, (dim,), "dt_bias")
        Dskip = _f64(Dskip, (dim,), "Dskip")
        z = _f64(z, (batch, dim, L), "z")
        h0 = _f64(h0, (batch, dim, N), "h0")
        y = np.empty((batch, dim, L), np.float64)
        hL = np.empty((batch, dim, N), np.float64)
        nt = threads or os.cpu_count() or 1
        rc = self._lib.ssm_oracle_scan_f64(
            batch, dim, L, N, 1 if zoh else 0, _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A),
            _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z), _ptr(h0), _ptr(y), _ptr(hL), int(nt))
        if rc != 0:
            raise RuntimeError("oracle scan failed with code %d" % rc)
        return y, hL

    def state_update(self, state, x, dt, A, Bm, Cm, dt_bias=None, Dskip=None, z=None,
                     zoh=False, threads=None):
        """One decode step; returns (y[batch,dim], new_state[batch,dim,N])."""
        state = np.array(state, dtype=np.float64, order="C", copy=True)
        batch, dim, N = state.shape
        x = _f64(x, (batch, dim), "x")
        dt = _f64(dt, (batch, dim), "dt")
        A = _f64(A, (dim, N), "A")
        Bm = _f64(Bm, (batch, N), "Bm")
        Cm = _f64(Cm, (batch, N), "Cm")
        dt_bias = _f64(dt_bias, (dim,), "dt_bias")
        Dskip = _f64(Dskip, (dim,), "Dskip")
        z = _f64(z, (batch, dim), "z")
        y = np.empty((batch, dim), np.float64)
        nt = threads or os.cpu_count() or 1
        rc = self._lib.ssm_oracle_state_update_f64(
            batch, dim, N, 1 if zoh else 0, _ptr(state), _ptr(x), _ptr(dt), _ptr(dt_bias),
            _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dskip), _ptr(z), _ptr(y), int(nt))
        if rc != 0:
            raise RuntimeError("oracle state update failed with code %d" % rc)
        return y, state

    def scan_bwd(self, x, dt, A, Bm, Cm, dy, dt_bias=None, Dskip=None, z=None, h0=None,
                 dhL=None, zoh=False, threads=None):
        """Vector-Jacobian products of scan_fwd (Delta*B form, or the exact ZOH
        form with zoh=True) for the loss sum(dy * y) + sum(dhL * hL).  Returns a dict with dx, ddt, dz (None
        without z), dBm, dCm, dA, dDskip, ddt_bias and dh0."""
        x = np.asarray(x)
        batch, dim, L = x.shape
        A = np.asarray(A)
        N = A.shape[1]
        x = _f64(x, (batch, dim, L), "x")
        dt = _f64(dt, (batch, dim, L), "dt")
        A = _f64(A, (dim, N), "A")
        Bm = _f64(Bm, (batch, N, L), "Bm")
        Cm = _f64(Cm, (batch, N, L), "Cm")
        dy = _f64(dy, (batch, dim, L), "dy")
        dt_bias = _f64(dt_bias, (dim,), "dt_bias")
        Dskip = _f64(Dskip, (dim,), "Dskip")
        z = _f64(z, (batch, dim, L), "z")
        h0 = _f64(h0, (batch, dim, N), "h0")
        dhL = _f64(dhL, (batch, dim, N), "dhL")
        g = {k: np.empty(shape, np.float64) for k, shape in (
            ("dx", (batch, dim, L)), ("ddt", (batch, dim, L)), ("ddt_bias", (dim,)),
            ("dA", (dim, N)), ("dBm", (batch, N, L)), ("dCm", (batch, N, L)), ("dDskip", (dim,)),
            ("dh0", (batch, dim, N)))}
        g["dz"] = np.empty((batch, dim, L), np.float64) if z is not None else None
        nt = threads or os.cpu_count() or 1
        rc = self._lib.ssm_oracle_scan_bwd_f64(
            batch, dim, L, N, 1 if zoh else 0, _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(Bm), _ptr(Cm),
            _ptr(Dskip), _ptr(z), _ptr(h0), _ptr(dy), _ptr(dhL), _ptr(g["dx"]), _ptr(g["ddt"]),
            _ptr(g["ddt_bias"]), _ptr(g["dA"]), _ptr(g["dBm"]), _ptr(g["dCm"]), _ptr(g["dDskip"]),
            _ptr(g["dz"]), _ptr(g["dh0"]), int(nt))
        if rc != 0:
            raise RuntimeError("oracle scan backward failed with code %d" % rc)
        return g

    def conv1d(self, x, weight, bias=None, state0=None, silu=True, threads=None):
        """Causal depthwise conv: y[batch,dim,L] and the final conv state
        [batch,dim,W-1] (the last W-1 inputs of state0 followed by x)."""
        x = np.asarray(x)
        if x.ndim != 3:
            raise ValueError("x must be [batch, dim, L]")
        batch, dim, L = x.shape
        weight = np.asarray(weight)
        W = weight.shape[1]
        x = _f64(x, (batch, dim, L), "x")
        weight = _f64(weight, (dim, W), "weight")
        bias = _f64(bias, (dim,), "bias")
        state0 = _f64(state0, (batch, dim, W - 1), "state0")
        y = np.empty((batch, dim, L), np.float64)
        stateL = np.empty((batch, dim, W - 1), np.float64)
        nt = threads or os.cpu_count() or 1
        rc = self._lib.ssm_oracle_conv1d_f64(
            batch, dim, L, W, 1 if silu else 0, _ptr(x), _ptr(weight), _ptr(bias), _ptr(state0),
            _ptr(y), _ptr(stateL), int(nt))
        if rc != 0:
            raise RuntimeError("oracle conv1d failed with code %d" % rc)
        return y, stateL

    def conv1d_update(self, state, x, weight, bias=None, silu=True, threads=None):
        """One decode step of the conv; returns (y[batch,dim], new_state)."""
        state = np.array(state, dtype=np.float64, order="C", copy=True)
        batch, dim, H = state.shape
        x = _f64(x, (batch, dim), "x")
        weight = _f64(weight, (dim, H + 1), "weight")
        bias = _f64(bias, (dim,), "bias")
        y = np.empty((batch, dim), np.float64)
        nt = threads or os.cpu_count() or 1
        rc = self._lib.ssm_oracle_conv1d_update_f64(
            batch, dim, H + 1, 1 if silu else 0, _ptr(state), _ptr(x), _ptr(weight), _ptr(bias),
            _ptr(y), int(nt))
        if rc != 0:
            raise RuntimeError("oracle conv1d update failed with code %d" % rc)
        return y, state


_default = None


def default():
    """The oracle built from ``ssm_oracle.c`` without mutants (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _default = Oracle(_build.LIB)
    return _default


def scan_fwd(*args, **kw):
    return default().scan_fwd(*args, **kw)


def state_update(*args, **kw):
    return default().state_update(*args, **kw)


def scan_bwd(*args, **kw):
    return default().scan_bwd(*args, **kw)


def conv1d(*args, **kw):
    return default().conv1d(*args, **kw)


def conv1d_update(*args, **kw):
    return default().conv1d_update(*args, **kw)
