"""Seeded synthetic inputs shaped like Mamba selective-scan layers.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the scan's arithmetic.  The tests, the benchmark and the
smoke check all take their inputs from here, so the HIP path and the CPU
oracle read exactly the same bits.

Recipe (the pages' layer sizes; no dataset or trained weights involved):
  * x, raw dt, z, Bm, Cm ~ N(0, 1), drawn in fp32 in blocks of 64 rows from
    ``numpy.random.default_rng([seed, tensor_id, b, row // 64])`` so any
    row can be regenerated from its block alone.
  * A[d, n] = -(n + 1), fp32.
  * dt_bias[d] = softplus^-1(Delta0_d) with Delta0_d log-uniform on
    [1e-3, 1e-1] per channel, so softplus(dt_bias) alone spans that range;
    the raw dt ~ N(0, 1) is added on top.
  * Dskip = 1 for the tiny case, else N(1, 0.1).
  * h0 (when asked for) and the decode state ~ N(0, 1), fp32.
  * bf16 tensors are the fp32 draws rounded to nearest-even.
  * Conv taps weight[d, k] and bias[d] (width W = 4 unless stated) follow the
    default initialisation of a depthwise conv layer, U(-1/sqrt(W), 1/sqrt(W)),
    fp32; the conv state (when asked for) ~ N(0, 1), fp32.
"""
from dataclasses import dataclass, field
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TENSOR_IDS = {"x": 0, "dt": 1, "z": 2, "Bm": 3, "Cm": 4, "Dskip": 5, "delta0": 6, "h0": 7,
              "conv_w": 8, "conv_b": 9, "conv_state": 10}


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    dim: int
    dstate: int
    seqlen: int          # L for the scan; number of decode steps for "decode"
    dtype: str           # storage dtype of x, dt, z, Bm, Cm: "f32" or "bf16"
    dskip: str           # "ones" or "normal"
    seed: int
    decode: bool = False
    note: str = field(default="", compare=False)

    @property
    def elements(self):
        return self.batch * self.dim * self.seqlen * self.dstate


# The five workloads: a tiny fp32 case, Mamba-130M- and Mamba-2.8B-shaped
# layers, a 2^20-long fp32 sequence and a 256-step decode loop.
WORKLOADS = [
    Workload("tiny-fp32 b1 d4 N4 L64", 1, 4, 4, 64, "f32", "ones", 1000),
    Workload("mamba-130m-layer b8 d1536 N16 L2048 bf16", 8, 1536, 16, 2048, "bf16", "normal", 1001),
    Workload("mamba-2.8b-layer b4 d5120 N16 L2048 bf16", 4, 5120, 16, 2048, "bf16", "normal", 1002),
    Workload("long-fp32 b1 d1536 N16 L1048576", 1, 1536, 16, 1 << 20, "f32", "normal", 1003),
    Workload("decode b64 d5120 N16 x256 steps bf16", 64, 5120, 16, 256, "bf16", "normal", 1004,
             decode=True),
]


def bf16_bits(f32):
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_values(bits):
    """Exact fp32 values of bf16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


ROWS_PER_BLOCK = 64


def normal_block(seed, name, b, block, rows, length):
    """Rows [64 block, 64 block + rows) of tensor `name`, batch row b."""
    rng = np.random.default_rng([seed, TENSOR_IDS[name], b, block])
    return rng.standard_normal((rows, length), dtype=np.float32)


def normal_row(seed, name, b, row, length, total_rows):
    blk = row // ROWS_PER_BLOCK
    rows = min(ROWS_PER_BLOCK, total_rows - blk * ROWS_PER_BLOCK)
    return normal_block(seed, name, b, blk, rows, length)[row - blk * ROWS_PER_BLOCK]


def _fill_rows(seed, name, batch, rows, length, threads):
    out = np.empty((batch, rows, length), np.float32)

    def work(job):
        b, blk = job
        r0 = blk * ROWS_PER_BLOCK
        n = min(ROWS_PER_BLOCK, rows - r0)
        out[b, r0:r0 + n] = normal_block(seed, name, b, blk, n, length)

    nblk = (rows + ROWS_PER_BLOCK - 1) // ROWS_PER_BLOCK
    jobs = [(b, k) for b in range(batch) for k in range(nblk)]
    if threads > 1 and batch * rows * length > (1 << 22):
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, jobs))
    else:
        for j in jobs:
            work(j)
    return out


def _store(f32, dtype):
    return bf16_bits(f32) if dtype == "bf16" else np.ascontiguousarray(f32, np.float32)


@dataclass
class Inputs:
    """Host-side inputs.  Tensors named in ``stored`` are uint16 bf16 bits for
    bf16 workloads and float32 otherwise; A, Dskip, dt_bias, h0 are float32."""
    wl: Workload
    dtype: str
    x: np.ndarray
    dt: np.ndarray
    z: np.ndarray
    Bm: np.ndarray
    Cm: np.ndarray
    A: np.ndarray
    Dskip: np.ndarray
    dt_bias: np.ndarray
    h0: np.ndarray = None

    stored = ("x", "dt", "z", "Bm", "Cm")

    def values(self, name):
        """Exact float64 values of a tensor as the kernels read them."""
        a = getattr(self, name)
        if a is None:
            return None
        if name in self.stored and self.dtype == "bf16":
            return bf16_values(a).astype(np.float64)
        return np.asarray(a, dtype=np.float64)


def parameters(wl, dim=None, dstate=None):
    """A, Dskip, dt_bias for a workload (fp32)."""
    dim = dim or wl.dim
    dstate = dstate or wl.dstate
    A = -np.tile(np.arange(1, dstate + 1, dtype=np.float32), (dim, 1))
    if wl.dskip == "ones":
        Dskip = np.ones(dim, np.float32)
    else:
        Dskip = np.random.default_rng([wl.seed, TENSOR_IDS["Dskip"]]).normal(
            1.0, 0.1, dim).astype(np.float32)
    u = np.random.default_rng([wl.seed, TENSOR_IDS["delta0"]]).uniform(
        math.log(1e-3), math.log(1e-1), dim)
    delta0 = np.exp(u)
    dt_bias = np.log(np.expm1(delta0)).astype(np.float32)
    return A, Dskip, dt_bias


def conv_parameters(wl, width=4, dim=None):
    """Depthwise conv taps [dim, width] and bias [dim] (fp32)."""
    dim = dim or wl.dim
    bound = 1.0 / math.sqrt(width)
    w = np.random.default_rng([wl.seed, TENSOR_IDS["conv_w"], width]).uniform(
        -bound, bound, (dim, width)).astype(np.float32)
    b = np.random.default_rng([wl.seed, TENSOR_IDS["conv_b"], width]).uniform(
        -bound, bound, dim).astype(np.float32)
    return w, b


def conv_state(wl, width=4, threads=None):
    """A conv state [batch, dim, width - 1] ~ N(0, 1) (fp32)."""
    threads = threads or min(16, os.cpu_count() or 1)
    return _fill_rows(wl.seed, "conv_state", wl.batch, wl.dim, width - 1, threads)


def make_inputs(wl, with_h0=False, threads=None, seqlen=None):
    """All inputs of a workload.  For the decode workload, x/dt/z are
    [batch, dim, steps] and Bm/Cm are [batch, N, steps]: step s reads
    ``[..., s]``."""
    threads = threads or min(16, os.cpu_count() or 1)
    L = seqlen or wl.seqlen
    x = _fill_rows(wl.seed, "x", wl.batch, wl.dim, L, threads)
    dt = _fill_rows(wl.seed, "dt", wl.batch, wl.dim, L, threads)
    z = _fill_rows(wl.seed, "z", wl.batch, wl.dim, L, threads)
    Bm = _fill_rows(wl.seed, "Bm", wl.batch, wl.dstate, L, threads)
    Cm = _fill_rows(wl.seed, "Cm", wl.batch, wl.dstate, L, threads)
    A, Dskip, dt_bias = parameters(wl)
    h0 = None
    if with_h0 or wl.decode:
        h0 = _fill_rows(wl.seed, "h0", wl.batch, wl.dim, wl.dstate, threads)
    return Inputs(wl, wl.dtype, _store(x, wl.dtype), _store(dt, wl.dtype), _store(z, wl.dtype),
                  _store(Bm, wl.dtype), _store(Cm, wl.dtype), A, Dskip, dt_bias, h0)


def row_inputs(wl, b, d, seqlen=None):
    """The inputs of the single row (b, d) as a batch-1, dim-1 problem
    (float64 values exactly as stored), regenerated from the row seeds."""
    L = seqlen or wl.seqlen

    def vals(name, row):
        total = wl.dstate if name in ("Bm", "Cm") else wl.dim
        f = normal_row(wl.seed, name, b, row, L, total)
        return (bf16_values(bf16_bits(f)) if wl.dtype == "bf16" else f).astype(np.float64)

    A, Dskip, dt_bias = parameters(wl)
    out = {
        "x": vals("x", d)[None, None],
        "dt": vals("dt", d)[None, None],
        "z": vals("z", d)[None, None],
        "Bm": np.stack([vals("Bm", n) for n in range(wl.dstate)])[None],
        "Cm": np.stack([vals("Cm", n) for n in range(wl.dstate)])[None],
        "A": A[d:d + 1].astype(np.float64),
        "Dskip": Dskip[d:d + 1].astype(np.float64),
        "dt_bias": dt_bias[d:d + 1].astype(np.float64),
    }
    return out
