"""The C-ABI library on the host: it loads, exports what the header declares,
and rejects bad arguments before any HIP call (no GPU needed; no call here
passes validation, so nothing is ever launched)."""

from __future__ import annotations

import ctypes
import glob
import math
import os
import re
import subprocess

import mpmath
import numpy as np
import pytest

import swiglu_activation_amd as sw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gpu_visible() -> bool:
    import torch
    return torch.cuda.is_available()


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sw.library_path()):
        from swiglu_activation_amd import build
        build.build()
    return sw.load_library()


def _declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\([^;{]*\)\s*;", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    assert _declared_functions() == sorted(sw.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", sw.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    for code in range(9):
        s = sw.swiglu_status_string(code)
        assert s.startswith("SWIGLU_")
    assert "UNKNOWN" in sw.swiglu_status_string(99)


# Fake, never-dereferenced addresses: every call below must fail validation.
# They are only passed where no GPU is reachable, so a test mistake that let
# one through could not launch a kernel on them.
A, B, C = 0x100000, 0x900000, 0x1100000

no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="fake device addresses are only "
                                 "passed to the library on hosts without a GPU")
F32, BF16 = sw.SWIGLU_DTYPE_F32, sw.SWIGLU_DTYPE_BF16


def fwd(lib, x, xs, y, ys, rows, n, dt=BF16):
    return lib.swiglu_gateup_fwd(x, xs, y, ys, rows, n, dt, None)


def bwd(lib, dy, dys, x, xs, dx, dxs, rows, n, dt=BF16, ip=0):
    return lib.swiglu_gateup_bwd(dy, dys, x, xs, dx, dxs, rows, n, dt, ip, None)


@no_gpu_only
def test_fwd_validation(lib):
    assert fwd(lib, A, 16, B, 8, 4, 8, dt=7) == sw.SWIGLU_ERR_BAD_DTYPE
    assert fwd(lib, A, 16, B, 8, 4, 8, dt=-1) == sw.SWIGLU_ERR_BAD_DTYPE
    assert fwd(lib, A, 16, B, 8, -1, 8) == sw.SWIGLU_ERR_BAD_SHAPE
    assert fwd(lib, A, 16, B, 8, 4, -8) == sw.SWIGLU_ERR_BAD_SHAPE
    assert fwd(lib, A, 2 ** 33, B, 2 ** 32, 4, 2 ** 31) == sw.SWIGLU_ERR_BAD_SHAPE
    assert fwd(lib, A, 15, B, 8, 4, 8) == sw.SWIGLU_ERR_BAD_STRIDE
    assert fwd(lib, A, 16, B, 7, 4, 8) == sw.SWIGLU_ERR_BAD_STRIDE
    assert fwd(lib, A, 2 ** 40, B, 8, 2 ** 40, 8) == sw.SWIGLU_ERR_BAD_SHAPE   # byte span overflows
    assert fwd(lib, None, 16, B, 8, 4, 8) == sw.SWIGLU_ERR_NULL_POINTER
    assert fwd(lib, A, 16, None, 8, 4, 8) == sw.SWIGLU_ERR_NULL_POINTER
    # y overlaps x: x spans [A, A + (3*16+16)*2) bytes
    assert fwd(lib, A, 16, A + 64, 8, 4, 8) == sw.SWIGLU_ERR_ALIASING
    assert fwd(lib, A + 32, 16, A, 8, 4, 8) == sw.SWIGLU_ERR_ALIASING   # y spans [A, A+64)
    assert fwd(lib, A, 16, A, 8, 4, 8, dt=F32) == sw.SWIGLU_ERR_ALIASING


@no_gpu_only
def test_empty_problems_launch_nothing(lib):
    # No HIP call is made for an empty problem, so these succeed without a GPU.
    assert fwd(lib, None, 16, None, 8, 0, 8) == sw.SWIGLU_OK
    assert fwd(lib, None, 0, None, 0, 5, 0) == sw.SWIGLU_OK
    assert bwd(lib, None, 8, None, 16, None, 16, 0, 8) == sw.SWIGLU_OK
    assert bwd(lib, None, 0, None, 0, None, 0, 3, 0, ip=1) == sw.SWIGLU_OK


@no_gpu_only
def test_bwd_validation(lib):
    assert bwd(lib, A, 8, B, 16, C, 16, 4, 8, dt=3) == sw.SWIGLU_ERR_BAD_DTYPE
    assert bwd(lib, A, 8, B, 16, C, 16, -2, 8) == sw.SWIGLU_ERR_BAD_SHAPE
    assert bwd(lib, A, 7, B, 16, C, 16, 4, 8) == sw.SWIGLU_ERR_BAD_STRIDE
    assert bwd(lib, A, 8, B, 15, C, 16, 4, 8) == sw.SWIGLU_ERR_BAD_STRIDE
    assert bwd(lib, A, 8, B, 16, C, 15, 4, 8) == sw.SWIGLU_ERR_BAD_STRIDE
    assert bwd(lib, None, 8, B, 16, C, 16, 4, 8) == sw.SWIGLU_ERR_NULL_POINTER
    assert bwd(lib, A, 8, None, 16, C, 16, 4, 8) == sw.SWIGLU_ERR_NULL_POINTER
    assert bwd(lib, A, 8, B, 16, None, 16, 4, 8) == sw.SWIGLU_ERR_NULL_POINTER
    # out of place: dx must not overlap x or dy
    assert bwd(lib, A, 8, B, 16, B + 32, 16, 4, 8) == sw.SWIGLU_ERR_ALIASING
    assert bwd(lib, A, 8, B, 16, A, 16, 4, 8) == sw.SWIGLU_ERR_ALIASING
    # in place: dx must be NULL or x, and dy must not overlap x
    assert bwd(lib, A, 8, B, 16, C, 16, 4, 8, ip=1) == sw.SWIGLU_ERR_ALIASING
    assert bwd(lib, B + 16, 8, B, 16, None, 0, 4, 8, ip=1) == sw.SWIGLU_ERR_ALIASING
    assert bwd(lib, A, 8, B, 15, None, 0, 4, 8, ip=1) == sw.SWIGLU_ERR_BAD_STRIDE
    # in place ignores dx_row_stride (x's is used), so a bad one is not an error
    # by itself; this call still fails, on the NULL x.
    assert bwd(lib, A, 8, None, 16, None, 3, 4, 8, ip=1) == sw.SWIGLU_ERR_NULL_POINTER


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 16)
    with pytest.raises(ValueError):
        sw.swiglu_gateup_fwd(x)
    with pytest.raises(ValueError):
        sw.swiglu_gateup_bwd(torch.zeros(4, 8), x)
    with pytest.raises(ValueError):
        sw.swiglu_gateup_bias_scale_fwd(x, torch.zeros(16))
    with pytest.raises(ValueError):
        sw.swiglu_silu_mul_fwd(torch.zeros(4, 8), torch.zeros(4, 8))
    with pytest.raises(ValueError):
        sw.swiglu_fc1_fwd(torch.zeros(4, 64, dtype=torch.bfloat16),
                          torch.zeros(128, 64, dtype=torch.bfloat16))


def test_row_flattening():
    import torch
    t = torch.zeros(3, 5, 16)
    assert sw._rows_and_stride(t, "t") == (15, 16)
    wide = torch.zeros(6, 40)[:, :16]
    assert sw._rows_and_stride(wide, "t") == (6, 40)
    assert sw._rows_and_stride(torch.zeros(1, 1, 16), "t") == (1, 16)
    with pytest.raises(ValueError):
        sw._rows_and_stride(torch.zeros(4, 6, 16).transpose(0, 1), "t")
    with pytest.raises(ValueError):
        sw._rows_and_stride(torch.zeros(16, 4).t(), "t")


def _hex_const(src: str, name: str) -> float:
    m = re.search(rf"constexpr float {name} = (-?0x[0-9a-fA-Fp.+-]+)f;", src)
    assert m, name
    return float.fromhex(m.group(1))


def test_kernel_constants_match_their_definitions():
    """The fp32 constants in the kernel source equal the splits of log2(e),
    ln 2, g0 = -1 - W(1/e) and e^{g0}, derived here at 50 digits."""
    src = open(os.path.join(ROOT, "swiglu_activation_amd", "csrc", "swiglu_device.h")).read()
    with mpmath.workdps(50):
        l2e = 1 / mpmath.log(2)
        g0 = -1 - mpmath.lambertw(1 / mpmath.e).real

        def split(v):
            hi = float(np.float32(float(v)))
            lo = float(np.float32(float(v - mpmath.mpf(hi))))
            return hi, lo

        assert (_hex_const(src, "kLog2eHi"), _hex_const(src, "kLog2eLo")) == split(l2e)
        assert _hex_const(src, "kLn2") == float(np.float32(float(mpmath.log(2))))
        assert (_hex_const(src, "kG0Hi"), _hex_const(src, "kG0Lo")) == split(g0)
        assert _hex_const(src, "kC") == float(np.float32(float(mpmath.exp(g0))))
        assert abs(float(mpmath.exp(g0) + 1 + g0)) < 1e-40


def bsf(lib, x, xs, bias, scale, ss, y, ys, rows, n, dt=BF16):
    return lib.swiglu_gateup_bias_scale_fwd(x, xs, bias, scale, ss, y, ys, rows, n, dt, None)


def bsb(lib, dy, dys, x, xs, bias, scale, ss, dx, dxs, db, ds, dss, ws, wsb, rows, n, dt=BF16, ip=0):
    return lib.swiglu_gateup_bias_scale_bwd(dy, dys, x, xs, bias, scale, ss, dx, dxs, db, ds, dss,
                                            ws, wsb, rows, n, dt, ip, None)


def test_bias_scale_workspace_size(lib):
    ws = lambda r, n, b, s: lib.swiglu_gateup_bias_scale_workspace_size(r, n, b, s)  # noqa: E731
    r256 = lambda v: (v + 255) // 256 * 256  # noqa: E731
    assert ws(8192, 32768, 0, 0) == 0
    assert ws(0, 32768, 1, 1) == 0 and ws(8, 0, 1, 1) == 0 and ws(-1, 8, 1, 1) == 0
    # dbias: one fp32 partial row of 2n per group of 64 rows (the smaller of
    # the tile kernel's 64-row and the row loop's 128-row groups); dscale: one
    # fp32 partial per row and 64-element chunk of the widest plan (1-element
    # accesses: ceil(n / 256) tiles of 4 chunks)
    groups = (8192 + 63) // 64
    assert ws(8192, 32768, 1, 0) == r256(groups * 2 * 32768 * 4)
    assert ws(8192, 32768, 0, 1) == r256(8192 * 128 * 4 * 4)
    assert ws(8192, 32768, 1, 1) == r256(groups * 2 * 32768 * 4) + r256(8192 * 128 * 4 * 4)
    assert ws(300, 1001, 1, 1) == r256(5 * 2002 * 4) + r256(300 * 4 * 4 * 4)


@no_gpu_only
def test_bias_scale_validation(lib):
    D = 0x2100000   # dbias / dscale / workspace fake addresses far from A, B, C
    assert bsf(lib, A, 16, B, None, 1, C, 8, 4, 8, dt=9) == sw.SWIGLU_ERR_BAD_DTYPE
    assert bsf(lib, A, 16, B, C + 4096, 0, C, 8, 4, 8) == sw.SWIGLU_ERR_BAD_STRIDE   # scale stride
    assert bsf(lib, A, 16, None, None, 1, A + 8, 8, 4, 8) == sw.SWIGLU_ERR_ALIASING   # y over x
    assert bsf(lib, A, 16, C + 8, None, 1, C, 8, 4, 8) == sw.SWIGLU_ERR_ALIASING     # y over bias
    # dbias without bias, dscale without scale
    assert bsb(lib, A, 8, B, 16, None, None, 1, C, 16, D, None, 1, D + 4096, 1 << 20, 4, 8) == \
        sw.SWIGLU_ERR_NULL_POINTER
    assert bsb(lib, A, 8, B, 16, None, None, 1, C, 16, None, D, 1, D + 4096, 1 << 20, 4, 8) == \
        sw.SWIGLU_ERR_NULL_POINTER
    # workspace missing / too small / misaligned
    bias = D + (1 << 16)
    assert bsb(lib, A, 8, B, 16, bias, None, 1, C, 16, D, None, 1, None, 0, 4, 8) == \
        sw.SWIGLU_ERR_WORKSPACE
    assert bsb(lib, A, 8, B, 16, bias, None, 1, C, 16, D, None, 1, D + 8192, 16, 4, 8) == \
        sw.SWIGLU_ERR_WORKSPACE
    assert bsb(lib, A, 8, B, 16, bias, None, 1, C, 16, D, None, 1, D + 8200, 1 << 20, 4, 8) == \
        sw.SWIGLU_ERR_WORKSPACE
    # dbias overlapping the workspace, dx overlapping bias
    assert bsb(lib, A, 8, B, 16, bias, None, 1, C, 16, D, None, 1, D, 1 << 20, 4, 8) == \
        sw.SWIGLU_ERR_ALIASING
    assert bsb(lib, A, 8, B, 16, C + 32, None, 1, C, 16, D, None, 1, D + 8192, 1 << 20, 4, 8) == \
        sw.SWIGLU_ERR_ALIASING
    # dscale stride below 1
    assert bsb(lib, A, 8, B, 16, None, bias, 1, C, 16, None, D, 0, D + 8192, 1 << 20, 4, 8) == \
        sw.SWIGLU_ERR_BAD_STRIDE


def bsn(lib, dy, dys, x, xs, bias, scale, ss, dx, dxs, db, ds, dss, rows, n, dt=BF16, ip=0):
    return lib.swiglu_gateup_bias_scale_bwd_noalloc(dy, dys, x, xs, bias, scale, ss, dx, dxs, db,
                                                    ds, dss, rows, n, dt, ip, None)


def test_noalloc_limit_in_header_and_binding():
    text = open(os.path.join(ROOT, "include", "swiglu_gateup.h")).read()
    m = re.search(r"#define SWIGLU_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == sw.NOALLOC_SCRATCH_BYTES


@no_gpu_only
def test_noalloc_validation(lib):
    """The allocation-free backward checks what the workspace one checks, and
    refuses a problem whose partials exceed the static scratch before any HIP
    call (so these fake addresses are never used)."""
    D = 0x2100000
    bias = D + (1 << 16)
    lim = sw.NOALLOC_SCRATCH_BYTES
    assert bsn(lib, A, 8, B, 16, bias, None, 1, C, 16, D, None, 1, 4, 8, dt=5) == \
        sw.SWIGLU_ERR_BAD_DTYPE
    assert bsn(lib, A, 7, B, 16, bias, None, 1, C, 16, D, None, 1, 4, 8) == sw.SWIGLU_ERR_BAD_STRIDE
    assert bsn(lib, A, 8, B, 16, None, None, 1, C, 16, D, None, 1, 4, 8) == \
        sw.SWIGLU_ERR_NULL_POINTER                                   # dbias without bias
    assert bsn(lib, A, 8, B, 16, C + 32, None, 1, C, 16, D, None, 1, 4, 8) == \
        sw.SWIGLU_ERR_ALIASING                                       # dx over bias
    assert bsn(lib, A, 8, B, 16, bias, None, 1, C, 16, bias + 8, None, 1, 4, 8) == \
        sw.SWIGLU_ERR_ALIASING                                       # dbias over bias
    # past the limit: 16384 rows of n = 65536 with both sums, fake addresses
    # spaced so that no two views overlap
    rows, n = 16384, 65536
    assert lib.swiglu_gateup_bias_scale_workspace_size(rows, n, 1, 1) > lim
    G = 1 << 40
    assert bsn(lib, 1 * G, n, 2 * G, 2 * n, 3 * G, 4 * G, 1, 5 * G, 2 * n, 6 * G, 7 * G, 1,
               rows, n) == sw.SWIGLU_ERR_SCRATCH_LIMIT
    # the same problem with dbias only stays within the limit (64 MiB of
    # partials exactly is allowed) only if it fits; either way the status is
    # decided by the size the workspace query reports
    need_db = lib.swiglu_gateup_bias_scale_workspace_size(rows, n, 1, 0)
    st = bsn(lib, 1 * G, n, 2 * G, 2 * n, 3 * G, 4 * G, 1, 5 * G, 2 * n, 6 * G, None, 1, rows, n)
    assert st == (sw.SWIGLU_ERR_SCRATCH_LIMIT if need_db > lim else sw.SWIGLU_ERR_HIP)
    # an empty problem launches nothing (dbias would be zero-filled: not asked)
    assert bsn(lib, None, 8, None, 16, None, None, 1, None, 16, None, None, 1, 0, 8) == sw.SWIGLU_OK


def fc1(lib, a, lda, w, ldw, y, ldy, x, ldx, m, n, k, dt=BF16, ws=None):
    return lib.swiglu_fc1_fwd(a, lda, w, ldw, y, ldy, x, ldx, m, n, k, dt, ws, None)


@no_gpu_only
def test_fc1_validation(lib):
    D = 0x2100000
    ok = dict(a=A, lda=64, w=B, ldw=64, y=C, ldy=128, x=None, ldx=0, m=4, n=128, k=64)

    def call(**kw):
        args = {**ok, **kw}
        return fc1(lib, args["a"], args["lda"], args["w"], args["ldw"], args["y"], args["ldy"],
                   args["x"], args["ldx"], args["m"], args["n"], args["k"], kw.get("dt", BF16),
                   kw.get("ws"))

    assert call(dt=F32) == sw.SWIGLU_ERR_BAD_DTYPE
    # shapes: n and k multiples of 64, n <= 2^30, nothing negative
    assert call(n=96) == sw.SWIGLU_ERR_BAD_SHAPE
    assert call(k=32, lda=32, ldw=32) == sw.SWIGLU_ERR_BAD_SHAPE
    assert call(m=-1) == sw.SWIGLU_ERR_BAD_SHAPE
    assert call(n=(1 << 30) + 64, ldy=(1 << 30) + 64) == sw.SWIGLU_ERR_BAD_SHAPE
    assert call(k=0, lda=0, ldw=0) == sw.SWIGLU_ERR_BAD_SHAPE        # an empty sum
    # strides below the widths
    assert call(lda=56) == sw.SWIGLU_ERR_BAD_STRIDE
    assert call(ldw=56) == sw.SWIGLU_ERR_BAD_STRIDE
    assert call(ldy=120) == sw.SWIGLU_ERR_BAD_STRIDE
    assert call(x=D, ldx=248) == sw.SWIGLU_ERR_BAD_STRIDE
    # 16-byte pointers and strides that are multiples of 8 elements
    assert call(lda=68) == sw.SWIGLU_ERR_BAD_STRIDE
    assert call(ldy=132) == sw.SWIGLU_ERR_BAD_STRIDE
    assert call(a=A + 8) == sw.SWIGLU_ERR_BAD_STRIDE
    assert call(y=C + 2) == sw.SWIGLU_ERR_BAD_STRIDE
    assert call(x=D + 4, ldx=256) == sw.SWIGLU_ERR_BAD_STRIDE
    # the copies address 8 weight or token rows by one 32-bit byte offset:
    # lda and ldw are at most 2^28 elements
    assert call(lda=(1 << 28) + 8) == sw.SWIGLU_ERR_BAD_STRIDE
    assert call(ldw=(1 << 28) + 8) == sw.SWIGLU_ERR_BAD_STRIDE
    # NULL inputs or output
    assert call(a=None) == sw.SWIGLU_ERR_NULL_POINTER
    assert call(w=None) == sw.SWIGLU_ERR_NULL_POINTER
    assert call(y=None) == sw.SWIGLU_ERR_NULL_POINTER
    # outputs overlapping inputs or each other (a spans 4 * 64 * 2 = 512 bytes,
    # w 256 * 64 * 2 = 32 KiB, y 4 * 128 * 2 bytes)
    assert call(y=A + 256) == sw.SWIGLU_ERR_ALIASING
    assert call(y=B + 16384) == sw.SWIGLU_ERR_ALIASING
    assert call(x=A, ldx=256) == sw.SWIGLU_ERR_ALIASING
    assert call(x=B + 4096, ldx=256) == sw.SWIGLU_ERR_ALIASING
    assert call(x=C + 512, ldx=256) == sw.SWIGLU_ERR_ALIASING
    # the tile-queue workspace: 16-byte aligned, apart from every operand
    assert lib.swiglu_fc1_workspace_size() == 9 * 128
    assert call(ws=D + 8) == sw.SWIGLU_ERR_BAD_STRIDE
    assert call(ws=A + 256) == sw.SWIGLU_ERR_ALIASING
    assert call(ws=B - 1024) == sw.SWIGLU_ERR_ALIASING               # its 1152 bytes reach w
    assert call(ws=C + 512) == sw.SWIGLU_ERR_ALIASING
    assert call(x=D, ldx=256, ws=D + 1024) == sw.SWIGLU_ERR_ALIASING


@no_gpu_only
def test_fc1_empty_problems_launch_nothing(lib):
    assert fc1(lib, None, 64, None, 64, None, 128, None, 0, 0, 128, 64) == sw.SWIGLU_OK
    assert fc1(lib, None, 64, None, 64, None, 0, None, 0, 5, 0, 64) == sw.SWIGLU_OK
    assert fc1(lib, None, 0, None, 0, None, 128, None, 0, 0, 128, 0) == sw.SWIGLU_OK


@no_gpu_only
def test_launch_failure_is_reported():
    """Arguments that pass every check, on a host with no GPU: the launch
    itself fails and each entry point returns SWIGLU_ERR_HIP (the status a
    caller sees for any HIP launch error)."""
    D = 0x2100000
    H = sw.SWIGLU_ERR_HIP
    assert fwd(lib_(), A, 16, B, 8, 4, 8) == H
    assert bwd(lib_(), A, 8, B, 16, C, 16, 4, 8) == H
    assert bwd(lib_(), A, 8, B, 16, None, 0, 4, 8, ip=1) == H
    L = lib_()
    assert L.swiglu_silu_mul_fwd(A, 8, A + 4096, 8, B, 8, 4, 8, BF16, None) == H
    assert L.swiglu_silu_mul_bwd(A, 8, B, 8, B + 4096, 8, C, 8, C + 4096, 8, 4, 8, BF16, 0,
                                 None) == H
    assert bsf(L, A, 16, B, None, 1, C, 8, 4, 8) == H
    bias = D + (1 << 16)
    assert bsb(L, A, 8, B, 16, bias, None, 1, C, 16, D, None, 1, D + 8192, 1 << 20, 4, 8) == H
    # the allocation-free backward: the scratch address lookup fails first
    assert bsn(L, A, 8, B, 16, bias, None, 1, C, 16, D, None, 1, 4, 8) == H
    assert bsn(L, A, 8, B, 16, bias, None, 1, C, 16, None, None, 1, 4, 8) == H   # no sums
    assert fc1(L, A, 64, B, 64, C, 128, None, 0, 4, 128, 64) == H


def lib_():
    return sw.load_library()
