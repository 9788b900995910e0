"""Helpers shared by the GPU tests: host <-> device transfer of the stored
types, and the parity checks against the oracle.

Parity bars (elementwise, over every compared element):
* fp32: |got - ref| <= 1e-5 * |ref|, and got is exactly +-0 where ref is 0;
* bf16: at most 2 bf16 steps (ordinal distance, +0 == -0) from the oracle's
  float64 value rounded once to bf16, nearest-even.
"""

from __future__ import annotations

import concurrent.futures as cf

import numpy as np
import torch

import oracle
import synth

FP32_REL_TOL = 1e-5
BF16_ULP_TOL = 2


def to_dev(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "fp32":
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).to(device).view(
        torch.bfloat16)


def from_dev(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy float32 values or uint16 bf16 bit patterns."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def torch_dtype(dtype: str):
    return torch.float32 if dtype == "fp32" else torch.bfloat16


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


class Stat:
    """Accumulated comparison result of one output."""

    def __init__(self, what: str, dtype: str):
        self.what, self.dtype = what, dtype
        self.count = 0
        self.bad = 0
        self.worst = 0.0            # max relative error (fp32) or max ulp (bf16)
        self.example = None

    def merge(self, other: "Stat"):
        self.count += other.count
        self.bad += other.bad
        if other.worst > self.worst:
            self.worst = other.worst
        if self.example is None:
            self.example = other.example

    def ok(self) -> bool:
        return self.bad == 0

    def __str__(self):
        unit = "ulp" if self.dtype == "bf16" else "rel"
        return (f"{self.what}: {self.count} elements, max {self.worst:.3g} {unit}, "
                f"{self.bad} outside tolerance" + (f", e.g. {self.example}" if self.example else ""))


def compare(got: np.ndarray, ref: np.ndarray, dtype: str, what: str, mask=None) -> Stat:
    """got: stored values (float32 or uint16 bits); ref: float64 oracle values."""
    st = Stat(what, dtype)
    if mask is not None:
        got, ref = got[mask], ref[mask]
    st.count = int(ref.size)
    if ref.size == 0:
        return st
    if dtype == "fp32":
        g = got.astype(np.float64)
        err = np.abs(g - ref)
        with np.errstate(divide="ignore", invalid="ignore"):
            rel = np.where(ref != 0, err / np.abs(ref), np.where(g == 0, 0.0, np.inf))
        bad = ~(rel <= FP32_REL_TOL)
        st.worst = float(np.nanmax(rel)) if rel.size else 0.0
    else:
        d = oracle.bf16_ulp_distance(got, oracle.round_f64_to_bf16_bits(ref))
        bad = d > BF16_ULP_TOL
        st.worst = float(d.max())
    st.bad = int(bad.sum())
    if st.bad:
        i = int(np.flatnonzero(bad.ravel())[0])
        st.example = (i, float(np.asarray(ref).ravel()[i]), got.ravel()[i].item())
    return st


def compare_workload_chunks(w: synth.Workload, x_h, dy_h, outs: dict, rows_per_chunk=None,
                            threads=None):
    """Compare full outputs against the oracle, chunk by chunk over rows.

    outs maps a label to (kind, array) with kind "fwd" ([rows, n]) or
    "bwd" ([rows, 2n]); arrays are host copies of the device results."""
    threads = threads or synth.default_threads()
    rows_per_chunk = rows_per_chunk or max(1, (1 << 23) // max(1, 2 * w.n))
    chunks = [(r, min(r + rows_per_chunk, w.rows)) for r in range(0, w.rows, rows_per_chunk)]

    def job(c):
        r0, r1 = c
        xf = oracle.widen(x_h[r0:r1], w.dtype)
        res = {}
        need_bwd = any(k == "bwd" for k, _ in outs.values())
        yref = oracle.oracle_fwd(xf)
        dref = oracle.oracle_bwd(xf, oracle.widen(dy_h[r0:r1], w.dtype)) if need_bwd else None
        for label, (kind, arr) in outs.items():
            ref = yref if kind == "fwd" else dref
            res[label] = compare(arr[r0:r1], ref, w.dtype, label)
        return res

    total = {label: Stat(label, w.dtype) for label in outs}
    with cf.ThreadPoolExecutor(threads) as ex:
        for res in ex.map(job, chunks):
            for label, st in res.items():
                total[label].merge(st)
    return total
