"""Pins for the fp64 CPU oracle: each checks it against something the pages or
the mathematics fix independently of the oracle's own code.

Sources are the pages "Mamba: Linear-Time Sequence Modeling with Selective
State Spaces" (reading guide to arXiv 2312.00752; sections "Method", "The
selection mechanism (S6)", "Hardware-aware state expansion", Q&A) and
"Mamba选择性状态空间机制：效率提升10倍的核心突破" (soft186.com; dynamic
parameterization and chunked-computation sections).

Every pin is a plain function of an oracle handle so that the meta-test at the
bottom can run all of them against deliberately wrong builds of the oracle and
show that each planted mistake is caught by at least one pin.
"""
import itertools
import json
import math
import os

import mpmath
import numpy as np
import pytest
from scipy.special import expit

import oracle
from oracle import _build

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
mpmath.mp.dps = 40


def _mp_eval(expr):
    if isinstance(expr, (int, float)):
        return mpmath.mpf(expr)
    return mpmath.mpf(eval(expr, {"__builtins__": {}}, {"log": mpmath.log, "exp": mpmath.exp}))


def _arr(obj):
    if obj is None:
        return None
    a = np.asarray(obj, dtype=object)
    return np.vectorize(lambda e: float(_mp_eval(e)), otypes=[np.float64])(a)


def _rand_problem(rng, batch, dim, L, N, gate=True, h0=True, skip=True):
    p = dict(
        x=rng.standard_normal((batch, dim, L)),
        dt=rng.standard_normal((batch, dim, L)),
        A=-rng.uniform(0.5, 4.0, (dim, N)),
        Bm=rng.standard_normal((batch, N, L)),
        Cm=rng.standard_normal((batch, N, L)),
        dt_bias=rng.uniform(-4.0, 0.0, dim),
    )
    if skip:
        p["Dskip"] = rng.normal(1.0, 0.3, dim)
    if gate:
        p["z"] = rng.standard_normal((batch, dim, L))
    if h0:
        p["h0"] = rng.standard_normal((batch, dim, N))
    return p


# --------------------------------------------------------------------------
# P1: short sequences worked out by hand ("Method" equations; golden fixture)
# --------------------------------------------------------------------------
def pin_hand_examples(o):
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        spec = json.load(f)
    for case in spec["cases"]:
        kw = {k: _arr(case[k]) for k in ("dt_bias", "Dskip", "z", "h0")}
        y, hL = o.scan_fwd(_arr(case["x"]), _arr(case["dt"]), _arr(case["A"]), _arr(case["Bm"]),
                           _arr(case["Cm"]), zoh=(case["mode"] == "zoh"), **kw)
        np.testing.assert_allclose(y, _arr(case["y"]), rtol=1e-14, atol=1e-14, err_msg=case["name"])
        np.testing.assert_allclose(hL, _arr(case["hL"]), rtol=1e-14, atol=1e-14,
                                   err_msg=case["name"])


# --------------------------------------------------------------------------
# P2: with Delta, B, C constant in time the system is LTI and equals the
# convolution y = K * x + D x with K_k = sum_n C_n Abar_n^k Bbar_n
# ("Method"; Q&A contrasting recurrence and convolution modes).
# --------------------------------------------------------------------------
def pin_lti_convolution(o):
    rng = np.random.default_rng(11)
    batch, dim, L, N = 2, 3, 300, 5
    x = rng.standard_normal((batch, dim, L))
    dt_const = rng.standard_normal((batch, dim))
    dt = np.repeat(dt_const[:, :, None], L, axis=2)
    dt_bias = rng.uniform(-3.0, 0.5, dim)
    A = -rng.uniform(0.2, 3.0, (dim, N))
    Bc = rng.standard_normal((batch, N))
    Cc = rng.standard_normal((batch, N))
    Bm = np.repeat(Bc[:, :, None], L, axis=2)
    Cm = np.repeat(Cc[:, :, None], L, axis=2)
    Dskip = rng.normal(1.0, 0.2, dim)
    for zoh in (False, True):
        y, hL = o.scan_fwd(x, dt, A, Bm, Cm, dt_bias=dt_bias, Dskip=Dskip, zoh=zoh)
        for b in range(batch):
            for d in range(dim):
                u = dt_const[b, d] + dt_bias[d]
                delta = math.log1p(math.exp(u)) if u < 30 else u
                abar = np.exp(delta * A[d])
                if zoh:
                    bbar = np.expm1(delta * A[d]) / A[d] * Bc[b]
                else:
                    bbar = delta * Bc[b]
                k = np.arange(L)
                K = (Cc[b][None, :] * bbar[None, :] * abar[None, :] ** k[:, None]).sum(axis=1)
                ref = np.convolve(K, x[b, d])[:L] + Dskip[d] * x[b, d]
                np.testing.assert_allclose(y[b, d], ref, rtol=1e-10, atol=1e-11)
                # final state: sum_j Abar^(L-1-j) Bbar x_j
                hl = (abar[None, :] ** (L - 1 - k)[:, None] * bbar[None, :] * x[b, d][:, None]).sum(0)
                np.testing.assert_allclose(hL[b, d], hl, rtol=1e-10, atol=1e-11)


# --------------------------------------------------------------------------
# P3: Delta -> 0 keeps the state and ignores the input (Q&A on Delta and
# gating): with dt_bias = -40, y = (C_t . h0 + D x_t) silu(z_t).
# --------------------------------------------------------------------------
def pin_small_delta(o):
    rng = np.random.default_rng(12)
    p = _rand_problem(rng, 2, 3, 50, 4)
    p["dt_bias"] = np.full(3, -40.0)
    p["dt"] = np.clip(p["dt"], -2.0, 2.0)
    y, hL = o.scan_fwd(**p)
    ch0 = np.einsum("bnl,bdn->bdl", p["Cm"], p["h0"])
    ref = (ch0 + p["Dskip"][None, :, None] * p["x"]) * p["z"] * expit(p["z"])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hL, p["h0"], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# P4: large Delta resets the state to the current input (Q&A on Delta and
# gating): with dt_bias = +40, |dt| <= 4 and A <= -2, Abar <= e^-72, so
# h_t = Delta_t B_t x_t and y_t = (Delta_t (C_t . B_t) x_t + D x_t) silu(z_t).
# --------------------------------------------------------------------------
def pin_large_delta(o):
    rng = np.random.default_rng(13)
    p = _rand_problem(rng, 2, 3, 40, 4)
    p["dt_bias"] = np.full(3, 40.0)
    p["dt"] = np.clip(p["dt"], -4.0, 4.0)
    p["A"] = -rng.uniform(2.0, 4.0, (3, 4))
    y, hL = o.scan_fwd(**p)
    u = p["dt"] + 40.0
    delta = u + np.log1p(np.exp(-u))
    cb = np.einsum("bnl,bnl->bl", p["Cm"], p["Bm"])
    ref = (delta * cb[:, None, :] * p["x"] + p["Dskip"][None, :, None] * p["x"]) * p["z"] * expit(p["z"])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    hl_ref = delta[:, :, -1:] * p["Bm"][:, None, :, -1] * p["x"][:, :, -1:]
    np.testing.assert_allclose(hL, hl_ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# P5: the gated-RNN special case (S6 section): N = 1, A = -1, B = C = 1.
# Hand-derived fixture plus random u checked against the logistic function.
# --------------------------------------------------------------------------
def pin_gated_rnn(o):
    with open(os.path.join(GOLDEN, "gated_rnn.json")) as f:
        spec = json.load(f)
    u = _arr(spec["u"])
    x = np.asarray(spec["x"], np.float64)
    L = len(u)
    ones = np.ones((1, 1, L))
    for mode in ("zoh", "delta"):
        y, hL = o.scan_fwd(x[None, None], u[None, None], np.array([[-1.0]]), ones, ones,
                           zoh=(mode == "zoh"))
        ref = _arr(spec[mode]["y"])
        np.testing.assert_allclose(y[0, 0], ref, rtol=1e-14, atol=1e-14, err_msg=mode)
        np.testing.assert_allclose(hL[0, 0, 0], ref[-1], rtol=1e-14, err_msg=mode)
    # random sequence against the logistic form (scipy's expit / log1p)
    rng = np.random.default_rng(14)
    L = 200
    u = rng.normal(0.0, 3.0, L)
    x = rng.standard_normal(L)
    ones = np.ones((1, 1, L))
    for zoh in (True, False):
        y, _ = o.scan_fwd(x[None, None], u[None, None], np.array([[-1.0]]), ones, ones, zoh=zoh)
        h, ref = 0.0, np.empty(L)
        for t in range(L):
            g_in = expit(u[t]) if zoh else np.logaddexp(0.0, u[t])
            h = expit(-u[t]) * h + g_in * x[t]
            ref[t] = h
        np.testing.assert_allclose(y[0, 0], ref, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# P6: the recurrence is an associative scan ("Hardware-aware state
# expansion": computed with a parallel associative scan).  On tiny inputs every
# bracketing of the combine (a1,b1) o (a2,b2) = (a1 a2, a2 b1 + b2) must give
# the oracle's sequential final state and every prefix.
# --------------------------------------------------------------------------
def _bracketings(items):
    if len(items) == 1:
        yield items[0]
        return
    for split in range(1, len(items)):
        for left in _bracketings(items[:split]):
            for right in _bracketings(items[split:]):
                yield (left[0] * right[0], right[0] * left[1] + right[1])


def pin_bracketings(o):
    rng = np.random.default_rng(15)
    for L in (1, 2, 3, 5, 8):
        N = 3
        p = _rand_problem(rng, 1, 1, L, N, gate=False, h0=False, skip=False)
        y, hL = o.scan_fwd(**p)
        u = p["dt"][0, 0] + p["dt_bias"][0]
        delta = np.logaddexp(0.0, u)
        for n in range(N):
            pairs = [(math.exp(delta[t] * p["A"][0, n]), delta[t] * p["Bm"][0, n, t] * p["x"][0, 0, t])
                     for t in range(L)]
            finals = [br[1] for br in _bracketings(pairs)]
            assert len(finals) == math.comb(2 * (L - 1), L - 1) // L
            np.testing.assert_allclose(finals, hL[0, 0, n], rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# P7: split and resume (the cache holds the state after the scan: the
# "everything-about-mamba-paper" page; Q&A on generation).
# --------------------------------------------------------------------------
def pin_split_resume(o):
    rng = np.random.default_rng(16)
    p = _rand_problem(rng, 2, 3, 97, 4)
    y, hL = o.scan_fwd(**p)
    for cut in (1, 40, 96):
        first = {k: (v[..., :cut] if k in ("x", "dt", "z", "Bm", "Cm") else v) for k, v in p.items()}
        rest = {k: (v[..., cut:] if k in ("x", "dt", "z", "Bm", "Cm") else v) for k, v in p.items()}
        y1, h1 = o.scan_fwd(**first)
        rest["h0"] = h1
        y2, h2 = o.scan_fwd(**rest)
        np.testing.assert_allclose(np.concatenate([y1, y2], axis=2), y, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(h2, hL, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# P8: decoding one token at a time with a fixed D x N state equals the scan
# (Q&A on generation: O(1) per step, no KV cache).
# --------------------------------------------------------------------------
def pin_decode_equals_scan(o):
    rng = np.random.default_rng(17)
    p = _rand_problem(rng, 3, 4, 25, 8)
    y, hL = o.scan_fwd(**p)
    state = p["h0"].copy()
    for t in range(25):
        yt, state = o.state_update(state, p["x"][..., t], p["dt"][..., t], p["A"], p["Bm"][..., t],
                                   p["Cm"][..., t], dt_bias=p["dt_bias"], Dskip=p["Dskip"],
                                   z=p["z"][..., t])
        np.testing.assert_allclose(yt, y[..., t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(state, hL, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# P9: linearity in x when h0 = 0 and Delta, B, C, z are fixed (the
# recurrence of "Method" is linear in its input).
# --------------------------------------------------------------------------
def pin_linearity(o):
    rng = np.random.default_rng(18)
    p = _rand_problem(rng, 2, 3, 60, 4, h0=False)
    x1, x2 = p["x"], rng.standard_normal(p["x"].shape)
    al, be = 0.7, -1.3
    ya, ha = o.scan_fwd(**{**p, "x": x1})
    yb, hb = o.scan_fwd(**{**p, "x": x2})
    yc, hc = o.scan_fwd(**{**p, "x": al * x1 + be * x2})
    np.testing.assert_allclose(yc, al * ya + be * yb, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(hc, al * ha + be * hb, rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------
# P10: equivariance.  B and C are per-token N-vectors shared by all channels
# while Delta, A, D are per channel (S6 section): permuting channels together
# with their per-channel parameters permutes the output, and batch rows are
# independent.
# --------------------------------------------------------------------------
def pin_equivariance(o):
    rng = np.random.default_rng(19)
    p = _rand_problem(rng, 3, 5, 33, 4)
    y, hL = o.scan_fwd(**p)
    perm = rng.permutation(5)
    q = dict(p)
    for k in ("x", "dt", "z", "h0"):
        q[k] = p[k][:, perm]
    for k in ("A", "Dskip", "dt_bias"):
        q[k] = p[k][perm]
    yq, hq = o.scan_fwd(**q)
    np.testing.assert_allclose(yq, y[:, perm], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(hq, hL[:, perm], rtol=1e-13, atol=1e-14)
    # batch rows are independent: solving row 1 alone gives the same answer
    r = {k: (v[1:2] if k in ("x", "dt", "z", "h0", "Bm", "Cm") else v) for k, v in p.items()}
    yr, hr = o.scan_fwd(**r)
    np.testing.assert_allclose(yr[0], y[1], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(hr[0], hL[1], rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------
# P11: softplus and silu against high-precision values over the whole range
# the workloads reach (S6 section: Delta = softplus(.)); checked through L = 1,
# N = 1 scans whose outputs isolate each function.
# --------------------------------------------------------------------------
def pin_softplus_silu(o):
    us = np.array([-60.0, -30.0, -12.5, -7.0, -1e-3, 0.0, 1e-3, 0.5, 3.0, 19.0, 45.0])
    # y = Delta * B * x with h0 = 0, A = -1, B = C = x = 1, no skip, no gate
    for u in us:
        y, _ = o.scan_fwd(np.ones((1, 1, 1)), np.array([[[u]]]), np.array([[-1.0]]),
                          np.ones((1, 1, 1)), np.ones((1, 1, 1)))
        ref = mpmath.log1p(mpmath.exp(mpmath.mpf(u)))
        assert abs(y[0, 0, 0] - float(ref)) <= 4e-16 * float(ref), (u, y[0, 0, 0], ref)
    # gate: Delta = ln 2 (u = 0), so y = ln2 * silu(z)
    for zv in (-40.0, -5.0, -0.25, 0.0, 0.3, 2.0, 35.0):
        y, _ = o.scan_fwd(np.ones((1, 1, 1)), np.zeros((1, 1, 1)), np.array([[-1.0]]),
                          np.ones((1, 1, 1)), np.ones((1, 1, 1)), z=np.array([[[zv]]]))
        ref = mpmath.log(2) * zv / (1 + mpmath.exp(-mpmath.mpf(zv)))
        assert abs(y[0, 0, 0] - float(ref)) <= 4e-16 * abs(float(ref)) + 1e-300, (zv, y, ref)


# --------------------------------------------------------------------------
# Causal depthwise conv in front of the scan (glossary entry "Mamba Block";
# conv state in the inference cache, "everything-about-mamba-paper";
# d_conv = 4, the basic-model example of "Mamba选择性状态空间机制：效率提升10倍的核心突破").
# --------------------------------------------------------------------------
def _rand_conv(rng, batch, dim, L, W, state=True):
    return dict(x=rng.standard_normal((batch, dim, L)), weight=rng.standard_normal((dim, W)),
                bias=rng.standard_normal(dim),
                state0=rng.standard_normal((batch, dim, W - 1)) if state else None)


def pin_conv_hand_examples(o):
    with open(os.path.join(GOLDEN, "conv_hand_examples.json")) as f:
        spec = json.load(f)
    for case in spec["cases"]:
        y, sL = o.conv1d(_arr(case["x"]), _arr(case["weight"]), bias=_arr(case["bias"]),
                         state0=_arr(case["state0"]), silu=case["silu"])
        np.testing.assert_allclose(y, _arr(case["y"]), rtol=1e-14, atol=1e-14, err_msg=case["name"])
        np.testing.assert_allclose(sL, _arr(case["stateL"]), rtol=0, atol=0, err_msg=case["name"])


def pin_conv_library(o):
    """Special case of a library routine: torch's grouped conv1d (a
    cross-correlation) over the history-extended input, in fp64 on the CPU."""
    import torch
    rng = np.random.default_rng(31)
    for W in (2, 3, 4):
        for silu in (False, True):
            p = _rand_conv(rng, 2, 5, 37, W)
            y, _ = o.conv1d(p["x"], p["weight"], bias=p["bias"], state0=p["state0"], silu=silu)
            e = torch.from_numpy(np.concatenate([p["state0"], p["x"]], axis=2))
            ref = torch.nn.functional.conv1d(e, torch.from_numpy(p["weight"])[:, None, :],
                                             torch.from_numpy(p["bias"]), groups=5).numpy()
            if silu:
                ref = ref * expit(ref)
            np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-14)


def pin_conv_impulse(o):
    """A unit impulse at t0 with zero history returns the taps newest-last:
    y[t] = bias + w[W-1-(t-t0)] for t0 <= t < t0 + W, and bias elsewhere."""
    W, L, t0 = 4, 12, 5
    w = np.array([[0.5, -1.25, 2.0, 3.5]])
    x = np.zeros((1, 1, L))
    x[0, 0, t0] = 1.0
    y, sL = o.conv1d(x, w, bias=np.array([0.25]), silu=False)
    ref = np.full(L, 0.25)
    for t in range(t0, t0 + W):
        ref[t] += w[0, W - 1 - (t - t0)]
    np.testing.assert_array_equal(y[0, 0], ref)
    np.testing.assert_array_equal(sL[0, 0], x[0, 0, L - (W - 1):])


def pin_conv_split_resume(o):
    """Feeding the final conv state of x[:, :, :L1] as the history of
    x[:, :, L1:] reproduces the whole run, also for pieces shorter than W-1."""
    rng = np.random.default_rng(32)
    for W in (2, 3, 4):
        p = _rand_conv(rng, 2, 3, 29, W)
        y, sL = o.conv1d(**p)
        for cut in (1, 2, 13, 28):
            y1, s1 = o.conv1d(p["x"][:, :, :cut], p["weight"], p["bias"], p["state0"])
            y2, s2 = o.conv1d(p["x"][:, :, cut:], p["weight"], p["bias"], s1)
            np.testing.assert_allclose(np.concatenate([y1, y2], axis=2), y, rtol=1e-14, atol=1e-15)
            np.testing.assert_array_equal(s2, sL)


def pin_conv_decode_equals_prefill(o):
    rng = np.random.default_rng(33)
    p = _rand_conv(rng, 3, 4, 9, 4)
    y, sL = o.conv1d(**p)
    state = p["state0"].copy()
    for t in range(9):
        yt, state = o.conv1d_update(state, p["x"][:, :, t], p["weight"], p["bias"])
        np.testing.assert_allclose(yt, y[:, :, t], rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(state, sL)


# --------------------------------------------------------------------------
# Backward pass ("Hardware-aware state expansion": the backward recomputes the
# states).  The oracle returns the vector-Jacobian products of the forward
# map for l = sum(dy * y) + sum(dhL * hL); these pins tie it to the (pinned)
# forward oracle.
# --------------------------------------------------------------------------
def _bwd_problem(seed, batch=2, dim=3, L=23, N=4):
    rng = np.random.default_rng(seed)
    p = _rand_problem(rng, batch, dim, L, N)
    dy = rng.standard_normal((batch, dim, L))
    dhL = rng.standard_normal((batch, dim, N))
    return rng, p, dy, dhL


def _loss(o, p, dy, dhL, zoh=False):
    y, hL = o.scan_fwd(**p, zoh=zoh)
    return float((dy * y).sum() + (dhL * hL).sum())


def pin_bwd_linear_inputs(o):
    """The loss is affine in each of x, h0, Bm, Cm and Dskip when the other
    inputs are held fixed, so the directional derivative along v is exactly
    l(input = v) - l(input = 0): <grad, v> must match it to rounding (no step
    size involved)."""
    rng, p, dy, dhL = _bwd_problem(41)
    g = o.scan_bwd(dy=dy, dhL=dhL, **p)
    for name, gname in (("x", "dx"), ("h0", "dh0"), ("Bm", "dBm"), ("Cm", "dCm"),
                        ("Dskip", "dDskip")):
        v = rng.standard_normal(p[name].shape)
        lhs = (_loss(o, {**p, name: v}, dy, dhL)
               - _loss(o, {**p, name: np.zeros_like(v)}, dy, dhL))
        rhs = float((g[gname] * v).sum())
        assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs)), (name, lhs, rhs)


def pin_bwd_finite_differences(o):
    """Central differences of the forward oracle along random directions, for
    every input including the non-linear ones (dt, dt_bias, A, z)."""
    rng, p, dy, dhL = _bwd_problem(42)
    g = o.scan_bwd(dy=dy, dhL=dhL, **p)
    names = {"x": "dx", "dt": "ddt", "dt_bias": "ddt_bias", "A": "dA", "Bm": "dBm", "Cm": "dCm",
             "Dskip": "dDskip", "z": "dz", "h0": "dh0"}
    eps = 1e-6
    for name, gname in names.items():
        v = rng.standard_normal(p[name].shape)
        fd = (_loss(o, {**p, name: p[name] + eps * v}, dy, dhL)
              - _loss(o, {**p, name: p[name] - eps * v}, dy, dhL)) / (2 * eps)
        an = float((g[gname] * v).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def pin_bwd_zoh(o):
    """The exact ZOH form ([MAMBA] Method): the same exact directional
    derivatives for the inputs the loss is affine in, and central
    differences for the rest, through the ZOH forward oracle; one channel
    has A = 0 (B-bar = Delta B there, and its A gradient takes the series
    limit Delta^2 / 2)."""
    rng, p, dy, dhL = _bwd_problem(44)
    p["A"][1, 2] = 0.0
    g = o.scan_bwd(dy=dy, dhL=dhL, zoh=True, **p)
    for name, gname in (("x", "dx"), ("h0", "dh0"), ("Bm", "dBm"), ("Cm", "dCm")):
        v = rng.standard_normal(p[name].shape)
        lhs = (_loss(o, {**p, name: v}, dy, dhL, True)
               - _loss(o, {**p, name: np.zeros_like(v)}, dy, dhL, True))
        rhs = float((g[gname] * v).sum())
        assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs)), (name, lhs, rhs)
    eps = 1e-6
    for name, gname in (("dt", "ddt"), ("dt_bias", "ddt_bias"), ("A", "dA"), ("z", "dz")):
        v = rng.standard_normal(p[name].shape)
        fd = (_loss(o, {**p, name: p[name] + eps * v}, dy, dhL, True)
              - _loss(o, {**p, name: p[name] - eps * v}, dy, dhL, True)) / (2 * eps)
        an = float((g[gname] * v).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    # the A = 0 entry alone, where the forward switches to its limit branch
    v = np.zeros_like(p["A"])
    v[1, 2] = 1.0
    fd = (_loss(o, {**p, "A": p["A"] + eps * v}, dy, dhL, True)
          - _loss(o, {**p, "A": p["A"] - eps * v}, dy, dhL, True)) / (2 * eps)
    assert abs(fd - g["dA"][1, 2]) <= 1e-6 * max(1.0, abs(fd)), (fd, g["dA"][1, 2])


def pin_bwd_no_gate_no_state(o):
    """Without gate, skip, bias and h0 the same identities hold, and the
    returned dh0 is the adjoint at t = -1 (finite differences through h0)."""
    rng, p, dy, dhL = _bwd_problem(43, L=9, N=2)
    for k in ("z", "Dskip", "dt_bias", "h0"):
        p[k] = None
    g = o.scan_bwd(dy=dy, dhL=dhL, **p)
    assert g["dz"] is None
    v = rng.standard_normal(dhL.shape)
    eps = 1e-6
    fd = (_loss(o, {**p, "h0": eps * v}, dy, dhL) - _loss(o, {**p, "h0": -eps * v}, dy, dhL)) / (2 * eps)
    assert abs(fd - float((g["dh0"] * v).sum())) <= 1e-7 * max(1.0, abs(fd))
    v = rng.standard_normal(p["dt"].shape)
    fd = (_loss(o, {**p, "dt": p["dt"] + eps * v}, dy, dhL)
          - _loss(o, {**p, "dt": p["dt"] - eps * v}, dy, dhL)) / (2 * eps)
    assert abs(fd - float((g["ddt"] * v).sum())) <= 1e-6 * max(1.0, abs(fd))
    # the bias gradient is the time-and-batch sum of the dt gradient
    np.testing.assert_allclose(g["ddt_bias"], g["ddt"].sum(axis=(0, 2)), rtol=1e-12, atol=1e-13)


PINS = [pin_hand_examples, pin_lti_convolution, pin_small_delta, pin_large_delta, pin_gated_rnn,
        pin_bracketings, pin_split_resume, pin_decode_equals_scan, pin_linearity,
        pin_equivariance, pin_softplus_silu, pin_conv_hand_examples, pin_conv_library,
        pin_conv_impulse, pin_conv_split_resume, pin_conv_decode_equals_prefill,
        pin_bwd_linear_inputs, pin_bwd_finite_differences, pin_bwd_zoh, pin_bwd_no_gate_no_state]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.default())


def test_threads_do_not_change_results():
    rng = np.random.default_rng(20)
    p = _rand_problem(rng, 3, 7, 41, 4)
    y1, h1 = oracle.default().scan_fwd(**p, threads=1)
    y8, h8 = oracle.default().scan_fwd(**p, threads=8)
    assert np.array_equal(y1, y8) and np.array_equal(h1, h8)


def test_bad_arguments_rejected():
    o = oracle.default()
    with pytest.raises(ValueError):
        o.scan_fwd(np.zeros((1, 1, 4)), np.zeros((1, 1, 3)), np.zeros((1, 2)), np.zeros((1, 2, 4)),
                   np.zeros((1, 2, 4)))
    with pytest.raises(RuntimeError):
        o.scan_fwd(np.zeros((1, 1, 0)), np.zeros((1, 1, 0)), np.zeros((1, 2)), np.zeros((1, 2, 0)),
                   np.zeros((1, 2, 0)))


@pytest.mark.parametrize("k", sorted(oracle.MUTANTS), ids=lambda k: "m%d" % k)
def test_planted_mistake_is_caught(k, tmp_path):
    """Each deliberately wrong oracle build fails at least one pin."""
    mutant = oracle.Oracle(_build.build_mutant(k, str(tmp_path)))
    assert mutant.mutant == k
    failed = []
    for pin in PINS:
        try:
            pin(mutant)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "mutant %d (%s) passed every pin" % (k, oracle.MUTANTS[k])
