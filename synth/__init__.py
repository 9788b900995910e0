"""Seeded synthetic inputs for the fused gate-up SwiGLU workloads.

This module draws inputs and nothing else: it holds none of the method's
arithmetic (no sigmoid, no SiLU, no gradient). The tests, the bench and the
oracle's timing leg all take their inputs from here, so the CPU oracle and the
HIP path always see the same bits.

Workload shapes follow the Liger-Kernel Megatron SwiGLU page (§Summary: the
Megatron training shape S=2048, B=4 in bf16 with ffn_local 4096 and 32768;
§Background: one packed [tokens, 2n] fc1 output with gate in columns [0, n)
and up in [n, 2n); §Megatron feature compatibility: fp32 and bf16, 2D and 3D
inputs, any TP width). The pages measure on that training shape, not on a
dataset; fc1 activations are stood in for by the distributions below.

Recipe (each tensor is drawn in float64 and rounded once, directly, to the
workload dtype with round-to-nearest-even):

* Each tensor is cut into blocks of ``BLOCK_ROWS`` consecutive rows. Block
  ``b`` of tensor ``t`` (0 = gate half, 1 = up half, 2 = dy) is drawn from its
  own PCG64 stream seeded with ``[seed, t, b]``, so any block can be drawn
  alone, blocks can be drawn in parallel, and the values do not depend on how
  many blocks exist.
* "normal": standard normal draws.
* "normal_var2": standard normal draws times sqrt(2) (variance 2).
* "mix_sat": three draws per block in this order: a standard normal block, a
  mask block (uniform [0, 1) < 0.1) and a uniform [-30, 30) block; elements
  where the mask is set take the uniform value. This drives sigmoid into
  saturation on one element in ten.
"""

from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, field

import numpy as np

BLOCK_ROWS = 512

GATE, UP, DY = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: x is [rows, 2n] (viewed as ``shape``), dy is [rows, n]."""

    name: str
    shape: tuple          # logical shape of x, last dim = 2n
    dtype: str            # "fp32" or "bf16"
    seed: int
    gate_dist: str = "normal"
    up_dist: str = "normal"
    dy_dist: str = "normal"
    in_place: bool = False
    note: str = ""

    @property
    def n(self) -> int:
        return self.shape[-1] // 2

    @property
    def rows(self) -> int:
        return int(math.prod(self.shape[:-1]))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2


# The workloads. Names state what each one is and its size.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32_s16_b4_n128", (16, 4, 256), "fp32", 0,
                 note="tiny fp32 check, fwd + out-of-place bwd"),
        Workload("dense_bf16_s2048_b4_n4096", (2048, 4, 8192), "bf16", 2,
                 note="Megatron dense MLP shape, ffn_local 4096"),
        Workload("wide_bf16_s2048_b4_n32768", (2048, 4, 65536), "bf16", 3,
                 note="wide FFN, ffn_local 32768: the headline bandwidth shape"),
        Workload("odd_fp32_s4096_b1_n11008", (4096, 1, 22016), "fp32", 4,
                 gate_dist="mix_sat", up_dist="normal_var2",
                 note="odd width with sigmoid saturation"),
        Workload("inplace_wide_bf16_t8192_n32768", (8192, 65536), "bf16", 5,
                 in_place=True, note="2D input, backward over the input buffer"),
        Workload("inplace_tp_bf16_t8192_n1792", (8192, 3584), "bf16", 6,
                 in_place=True, note="2D input, one TP shard's width, in-place backward"),
    ]
}

HEADLINE = "wide_bf16_s2048_b4_n32768"
SMALL = "tiny_fp32_s16_b4_n128"


def _f64_to_bf16_bits_inputs(v: np.ndarray) -> np.ndarray:
    """Round finite float64 draws to bf16 bit patterns, nearest-even, in one step.

    Works on the float64 bit pattern: keep sign, exponent and the top 7
    mantissa bits, rounding the 45 dropped bits to nearest, ties to even.
    Only for the value ranges drawn here (zero or normal bf16 results);
    anything else is rejected rather than rounded.
    """
    v = np.ascontiguousarray(v, dtype=np.float64)
    a = np.abs(v)
    nz = a != 0.0
    if np.any(nz & ((a < 2.0 ** -126) | (a >= 2.0 ** 127))) or not np.all(np.isfinite(v)):
        raise ValueError("input draw outside the normal bf16 range")
    bits = v.view(np.uint64)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    r = (bits + np.uint64((1 << 44) - 1) + lsb) >> np.uint64(45)   # sign|exp11|mant7
    sign = (r >> np.uint64(18)) & np.uint64(1)
    exp11 = (r >> np.uint64(7)) & np.uint64(0x7FF)
    mant = r & np.uint64(0x7F)
    exp8 = exp11.astype(np.int64) - (1023 - 127)
    out = (sign << np.uint64(15)) | (np.clip(exp8, 0, 255).astype(np.uint64) << np.uint64(7)) | mant
    out = np.where(nz, out, sign << np.uint64(15))
    return out.astype(np.uint16)


def _draw_block(dist: str, seed: int, tensor: int, block: int, shape) -> np.ndarray:
    rng = np.random.default_rng([seed, tensor, block])
    if dist == "normal":
        return rng.standard_normal(shape)
    if dist == "normal_var2":
        return rng.standard_normal(shape) * math.sqrt(2.0)
    if dist == "mix_sat":
        base = rng.standard_normal(shape)
        mask = rng.random(shape) < 0.1
        unif = rng.uniform(-30.0, 30.0, shape)
        return np.where(mask, unif, base)
    raise ValueError(f"unknown distribution {dist!r}")


def _to_dtype(v: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return v.astype(np.float32)          # IEEE nearest-even
    if dtype == "bf16":
        return _f64_to_bf16_bits_inputs(v)   # uint16 bit patterns
    raise ValueError(dtype)


def _fill(out: np.ndarray, col0: int, dist: str, w: Workload, tensor: int,
          row_lo: int, row_hi: int, width: int, threads: int) -> None:
    """Fill out[:, col0:col0+width] with rows [row_lo, row_hi) of one tensor."""
    b_lo, b_hi = row_lo // BLOCK_ROWS, (row_hi - 1) // BLOCK_ROWS + 1

    def job(b):
        r0, r1 = b * BLOCK_ROWS, min((b + 1) * BLOCK_ROWS, w.rows)
        blk = _to_dtype(_draw_block(dist, w.seed, tensor, b, (r1 - r0, width)), w.dtype)
        s0, s1 = max(r0, row_lo), min(r1, row_hi)
        out[s0 - row_lo:s1 - row_lo, col0:col0 + width] = blk[s0 - r0:s1 - r0]

    if threads <= 1 or b_hi - b_lo <= 1:
        for b in range(b_lo, b_hi):
            job(b)
    else:
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(job, range(b_lo, b_hi)))


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def storage_dtype(dtype: str):
    """numpy storage type: float32 for fp32, uint16 bit patterns for bf16."""
    return np.float32 if dtype == "fp32" else np.uint16


def make_x(w: Workload, row_lo: int = 0, row_hi: int | None = None,
           threads: int | None = None) -> np.ndarray:
    """Rows [row_lo, row_hi) of the packed fc1 output x, shape [rows, 2n]."""
    row_hi = w.rows if row_hi is None else row_hi
    threads = default_threads() if threads is None else threads
    out = np.empty((row_hi - row_lo, 2 * w.n), storage_dtype(w.dtype))
    if row_hi > row_lo:
        _fill(out, 0, w.gate_dist, w, GATE, row_lo, row_hi, w.n, threads)
        _fill(out, w.n, w.up_dist, w, UP, row_lo, row_hi, w.n, threads)
    return out


def make_dy(w: Workload, row_lo: int = 0, row_hi: int | None = None,
            threads: int | None = None) -> np.ndarray:
    """Rows [row_lo, row_hi) of the upstream gradient dy, shape [rows, n]."""
    row_hi = w.rows if row_hi is None else row_hi
    threads = default_threads() if threads is None else threads
    out = np.empty((row_hi - row_lo, w.n), storage_dtype(w.dtype))
    if row_hi > row_lo:
        _fill(out, 0, w.dy_dist, w, DY, row_lo, row_hi, w.n, threads)
    return out


def sample_rows(w: Workload, count: int, seed: int = 12345) -> np.ndarray:
    """Sorted row indices for sampled checks at full size: the first and last
    row, both sides of every block boundary that falls in a small window, and
    a seeded uniform draw of the rest."""
    rng = np.random.default_rng([seed, w.seed])
    fixed = {0, w.rows - 1, min(BLOCK_ROWS, w.rows - 1), max(0, w.rows - BLOCK_ROWS)}
    k = max(0, min(count, w.rows) - len(fixed))
    extra = rng.choice(w.rows, size=k, replace=False) if k else []
    return np.array(sorted(fixed | set(int(r) for r in extra)), dtype=np.int64)
