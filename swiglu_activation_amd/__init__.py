"""Fused gate-up SwiGLU for AMD MI355X: Python binding of libswiglu_gateup.so.

The binding only marshals arguments: it flattens leading dimensions into rows,
reads row strides, allocates outputs with torch, and passes device pointers
and torch's current HIP stream to the C ABI (include/swiglu_gateup.h). Every
step of the computation runs in the HIP kernels. There is no fallback: if the
library is missing or cannot be loaded, every call raises.

Layout (Liger-Kernel Megatron SwiGLU page, §Background): x is the packed fc1
output [..., 2n] with the gate in [..., :n] and up in [..., n:]; 2D and 3D
inputs are accepted (§Megatron feature compatibility).
"""

from __future__ import annotations

import ctypes
import os

__all__ = ["swiglu_gateup_fwd", "swiglu_gateup_bwd", "swiglu_silu_mul_fwd", "swiglu_silu_mul_bwd",
           "swiglu_gateup_bias_scale_fwd", "swiglu_gateup_bias_scale_bwd",
           "swiglu_gateup_bias_scale_workspace_size", "swiglu_gateup_bias_scale_bwd_noalloc",
           "swiglu_fc1_fwd", "swiglu_fc1_workspace_size", "swiglu_status_string", "SwiGLUError",
           "library_path",
           "load_library", "EXPORTS", "NOALLOC_SCRATCH_BYTES"]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG_DIR, "libswiglu_gateup.so")

# Status codes and dtype codes of include/swiglu_gateup.h.
SWIGLU_OK = 0
SWIGLU_ERR_NULL_POINTER = 1
SWIGLU_ERR_BAD_SHAPE = 2
SWIGLU_ERR_BAD_STRIDE = 3
SWIGLU_ERR_BAD_DTYPE = 4
SWIGLU_ERR_ALIASING = 5
SWIGLU_ERR_HIP = 6
SWIGLU_ERR_WORKSPACE = 7
SWIGLU_ERR_SCRATCH_LIMIT = 8
NOALLOC_SCRATCH_BYTES = 64 << 20     # SWIGLU_NOALLOC_SCRATCH_BYTES of the header
SWIGLU_DTYPE_F32 = 0
SWIGLU_DTYPE_BF16 = 1
_BAD_DTYPE_CODE = -1    # passed for any other torch dtype; the library rejects it

EXPORTS = ("swiglu_gateup_fwd", "swiglu_gateup_bwd", "swiglu_silu_mul_fwd", "swiglu_silu_mul_bwd",
           "swiglu_gateup_bias_scale_fwd", "swiglu_gateup_bias_scale_bwd",
           "swiglu_gateup_bias_scale_workspace_size", "swiglu_gateup_bias_scale_bwd_noalloc",
           "swiglu_fc1_fwd", "swiglu_fc1_workspace_size", "swiglu_status_string")

_lib = None


class SwiGLUError(RuntimeError):
    """A nonzero swiglu_status from the library."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {swiglu_status_string(status)}")


class SwiGLUArgumentError(SwiGLUError, ValueError):
    """The library rejected the arguments (nothing was launched)."""


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libswiglu_gateup.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built; run `python -m swiglu_activation_amd.build` "
            "(or __graft_entry__.build()) first. There is no non-HIP fallback.")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, vp, cint = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.swiglu_gateup_fwd.argtypes = [vp, i64, vp, i64, i64, i64, cint, vp]
    lib.swiglu_gateup_fwd.restype = cint
    lib.swiglu_gateup_bwd.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64, cint, cint, vp]
    lib.swiglu_gateup_bwd.restype = cint
    lib.swiglu_silu_mul_fwd.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64, cint, vp]
    lib.swiglu_silu_mul_fwd.restype = cint
    lib.swiglu_silu_mul_bwd.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, i64, i64,
                                        cint, cint, vp]
    lib.swiglu_silu_mul_bwd.restype = cint
    lib.swiglu_gateup_bias_scale_fwd.argtypes = [vp, i64, vp, vp, i64, vp, i64, i64, i64, cint, vp]
    lib.swiglu_gateup_bias_scale_fwd.restype = cint
    lib.swiglu_gateup_bias_scale_workspace_size.argtypes = [i64, i64, cint, cint]
    lib.swiglu_gateup_bias_scale_workspace_size.restype = ctypes.c_size_t
    lib.swiglu_gateup_bias_scale_bwd.argtypes = [vp, i64, vp, i64, vp, vp, i64, vp, i64, vp, vp,
                                                 i64, vp, ctypes.c_size_t, i64, i64, cint, cint, vp]
    lib.swiglu_gateup_bias_scale_bwd.restype = cint
    lib.swiglu_gateup_bias_scale_bwd_noalloc.argtypes = [vp, i64, vp, i64, vp, vp, i64, vp, i64,
                                                         vp, vp, i64, i64, i64, cint, cint, vp]
    lib.swiglu_gateup_bias_scale_bwd_noalloc.restype = cint
    lib.swiglu_fc1_fwd.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, i64, i64, i64, cint, vp, vp]
    lib.swiglu_fc1_fwd.restype = cint
    lib.swiglu_fc1_workspace_size.argtypes = []
    lib.swiglu_fc1_workspace_size.restype = ctypes.c_size_t
    lib.swiglu_status_string.argtypes = [cint]
    lib.swiglu_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def swiglu_status_string(status: int) -> str:
    return load_library().swiglu_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status == SWIGLU_OK:
        return
    if status == SWIGLU_ERR_HIP:
        raise SwiGLUError(status, what)
    raise SwiGLUArgumentError(status, what)


# ---------------------------------------------------------------------------
# Tensor marshalling
# ---------------------------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return SWIGLU_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return SWIGLU_DTYPE_BF16
    return _BAD_DTYPE_CODE


def _rows_and_stride(t, name: str):
    """View t as [rows, width] with unit column stride: (rows, row_stride)."""
    if t.dim() < 1:
        raise ValueError(f"{name} must have at least one dimension")
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride in its last dimension")
    rows = 1
    for s in t.shape[:-1]:
        rows *= int(s)
    if t.dim() == 1:
        return rows, int(t.shape[-1])
    # leading dims must collapse into one row index with a single stride
    row_stride = None
    expect = None
    for d in range(t.dim() - 2, -1, -1):
        if t.shape[d] == 1:
            continue
        if row_stride is None:
            row_stride = int(t.stride(d))
            expect = row_stride * int(t.shape[d])
        else:
            if int(t.stride(d)) != expect:
                raise ValueError(f"leading dimensions of {name} do not collapse into rows")
            expect = int(t.stride(d)) * int(t.shape[d])
    if row_stride is None:          # a single row
        row_stride = int(t.shape[-1])
    return rows, row_stride


def _require_device(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on a HIP device (device pointers only)")
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError("all tensors must be on the same device")


def _stream_handle(device, stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def swiglu_gateup_fwd(x, y=None, *, stream=None):
    """y = silu(x[..., :n]) * x[..., n:] for x of shape [..., 2n] (fp32 or bf16).

    ``y`` (optional) is the [..., n] output; allocated when omitted. The
    kernel is enqueued on ``stream`` (default: torch's current stream)."""
    import torch
    lib = load_library()
    _require_device(x, y)
    if x.dim() < 1 or x.shape[-1] % 2:
        raise ValueError("last dimension of x must be even (2n)")
    n = x.shape[-1] // 2
    if y is None:
        y = torch.empty(tuple(x.shape[:-1]) + (n,), dtype=x.dtype, device=x.device)
    if y.dtype != x.dtype:
        raise ValueError("x and y must have the same dtype")
    rows, xs = _rows_and_stride(x, "x")
    yrows, ys = _rows_and_stride(y, "y")
    if yrows != rows or y.shape[-1] != n:
        raise ValueError(f"y must hold {rows} rows of {n} elements")
    with torch.cuda.device(x.device):
        st = lib.swiglu_gateup_fwd(x.data_ptr(), xs, y.data_ptr(), ys, rows, n,
                                   _dtype_code(x), _stream_handle(x.device, stream))
    _check(st, "swiglu_gateup_fwd")
    return y


def swiglu_gateup_bwd(dy, x, dx=None, *, in_place: bool = False, stream=None):
    """Gradient of swiglu_gateup_fwd with respect to x: [dgate | dup], [..., 2n].

    silu is recomputed from the saved input ``x``. Out of place (default) the
    result goes to ``dx`` (allocated when omitted). With ``in_place=True`` it
    overwrites ``x``, which is returned."""
    import torch
    lib = load_library()
    _require_device(dy, x, dx)
    if x.dim() < 1 or x.shape[-1] % 2:
        raise ValueError("last dimension of x must be even (2n)")
    n = x.shape[-1] // 2
    if dy.dtype != x.dtype:
        raise ValueError("dy and x must have the same dtype")
    rows, xs = _rows_and_stride(x, "x")
    dyrows, dys = _rows_and_stride(dy, "dy")
    if dyrows != rows or dy.shape[-1] != n:
        raise ValueError(f"dy must hold {rows} rows of {n} elements")
    if in_place:
        if dx is not None and dx.data_ptr() != x.data_ptr():
            raise ValueError("in_place backward writes into x; pass dx=None or dx=x")
        dx_ptr, dxs = None, 0
        out = x
    else:
        if dx is None:
            dx = torch.empty(tuple(x.shape), dtype=x.dtype, device=x.device)
        if dx.dtype != x.dtype:
            raise ValueError("dx and x must have the same dtype")
        dxrows, dxs = _rows_and_stride(dx, "dx")
        if dxrows != rows or dx.shape[-1] != 2 * n:
            raise ValueError(f"dx must hold {rows} rows of {2 * n} elements")
        dx_ptr = dx.data_ptr()
        out = dx
    with torch.cuda.device(x.device):
        st = lib.swiglu_gateup_bwd(dy.data_ptr(), dys, x.data_ptr(), xs, dx_ptr, dxs, rows, n,
                                   _dtype_code(x), 1 if in_place else 0,
                                   _stream_handle(x.device, stream))
    _check(st, "swiglu_gateup_bwd")
    return out


def _same_rows(t, rows, n, name):
    r, s = _rows_and_stride(t, name)
    if r != rows or t.shape[-1] != n:
        raise ValueError(f"{name} must hold {rows} rows of {n} elements")
    return s


def swiglu_silu_mul_fwd(gate, up, y=None, *, stream=None):
    """y = silu(gate) * up for two tensors of the same shape [..., n]."""
    import torch
    lib = load_library()
    _require_device(gate, up, y)
    if gate.shape != up.shape:
        raise ValueError("gate and up must have the same shape")
    if gate.dtype != up.dtype:
        raise ValueError("gate and up must have the same dtype")
    n = gate.shape[-1] if gate.dim() else 1
    rows, gs = _rows_and_stride(gate, "gate")
    us = _same_rows(up, rows, n, "up")
    if y is None:
        y = torch.empty(tuple(gate.shape), dtype=gate.dtype, device=gate.device)
    if y.dtype != gate.dtype:
        raise ValueError("y must have the dtype of gate")
    ys = _same_rows(y, rows, n, "y")
    with torch.cuda.device(gate.device):
        st = lib.swiglu_silu_mul_fwd(gate.data_ptr(), gs, up.data_ptr(), us, y.data_ptr(), ys,
                                     rows, n, _dtype_code(gate), _stream_handle(gate.device, stream))
    _check(st, "swiglu_silu_mul_fwd")
    return y


def swiglu_silu_mul_bwd(dy, gate, up, dgate=None, dup=None, *, in_place: bool = False, stream=None):
    """(dgate, dup) for y = silu(gate) * up. With in_place=True they overwrite
    gate and up, which are returned."""
    import torch
    lib = load_library()
    _require_device(dy, gate, up, dgate, dup)
    if gate.shape != up.shape or dy.shape != gate.shape:
        raise ValueError("dy, gate and up must have the same shape")
    if not (dy.dtype == gate.dtype == up.dtype):
        raise ValueError("dy, gate and up must have the same dtype")
    n = gate.shape[-1] if gate.dim() else 1
    rows, gs = _rows_and_stride(gate, "gate")
    us = _same_rows(up, rows, n, "up")
    dys = _same_rows(dy, rows, n, "dy")
    if in_place:
        for t, src, name in ((dgate, gate, "dgate"), (dup, up, "dup")):
            if t is not None and t.data_ptr() != src.data_ptr():
                raise ValueError(f"in_place backward writes into the inputs; pass {name}=None")
        dgate, dup = gate, up
        dg_ptr = du_ptr = None
        dgs = dus = 0
    else:
        if dgate is None:
            dgate = torch.empty(tuple(gate.shape), dtype=gate.dtype, device=gate.device)
        if dup is None:
            dup = torch.empty(tuple(gate.shape), dtype=gate.dtype, device=gate.device)
        if dgate.dtype != gate.dtype or dup.dtype != gate.dtype:
            raise ValueError("dgate and dup must have the dtype of gate")
        dgs = _same_rows(dgate, rows, n, "dgate")
        dus = _same_rows(dup, rows, n, "dup")
        dg_ptr, du_ptr = dgate.data_ptr(), dup.data_ptr()
    with torch.cuda.device(gate.device):
        st = lib.swiglu_silu_mul_bwd(dy.data_ptr(), dys, gate.data_ptr(), gs, up.data_ptr(), us,
                                     dg_ptr, dgs, du_ptr, dus, rows, n, _dtype_code(gate),
                                     1 if in_place else 0, _stream_handle(gate.device, stream))
    _check(st, "swiglu_silu_mul_bwd")
    return dgate, dup


# ---------------------------------------------------------------------------
# Bias and per-token scale variants
# ---------------------------------------------------------------------------

def _bias_arg(bias, x, n):
    if bias is None:
        return None
    _require_device(bias, x)
    if bias.dim() != 1 or bias.shape[0] != 2 * n or (n and bias.stride(0) != 1):
        raise ValueError(f"bias must be a contiguous [{2 * n}] tensor")
    if bias.dtype != x.dtype:
        raise ValueError("bias must have the dtype of x")
    return bias.data_ptr()


def _per_row_arg(t, x, rows, name):
    """A per-row fp32 tensor shaped like x's leading dims, optionally with a
    trailing 1: (pointer, stride)."""
    import torch
    if t is None:
        return None, 1
    _require_device(t, x)
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32")
    lead = tuple(x.shape[:-1])
    if tuple(t.shape) == lead:
        t2 = t.unsqueeze(-1)
    elif tuple(t.shape) == lead + (1,):
        t2 = t
    else:
        raise ValueError(f"{name} must have shape {lead} or {lead + (1,)}")
    r, s_ = _rows_and_stride(t2, name)
    assert r == rows
    return t.data_ptr(), max(1, s_)


def swiglu_gateup_bias_scale_workspace_size(rows: int, n: int, want_dbias: bool,
                                            want_dscale: bool) -> int:
    return int(load_library().swiglu_gateup_bias_scale_workspace_size(
        int(rows), int(n), int(bool(want_dbias)), int(bool(want_dscale))))


def swiglu_gateup_bias_scale_fwd(x, bias=None, scale=None, y=None, *, stream=None):
    """y = scale * silu(z[..., :n]) * z[..., n:] with z = x + bias.

    bias: [2n] of x's dtype or None; scale: float32 per row (shape
    x.shape[:-1], optionally with a trailing 1) or None."""
    import torch
    lib = load_library()
    _require_device(x, y)
    if x.dim() < 1 or x.shape[-1] % 2:
        raise ValueError("last dimension of x must be even (2n)")
    n = x.shape[-1] // 2
    rows, xs = _rows_and_stride(x, "x")
    bp = _bias_arg(bias, x, n)
    sp, ss = _per_row_arg(scale, x, rows, "scale")
    if y is None:
        y = torch.empty(tuple(x.shape[:-1]) + (n,), dtype=x.dtype, device=x.device)
    if y.dtype != x.dtype:
        raise ValueError("x and y must have the same dtype")
    ys = _same_rows(y, rows, n, "y")
    with torch.cuda.device(x.device):
        st = lib.swiglu_gateup_bias_scale_fwd(x.data_ptr(), xs, bp, sp, ss, y.data_ptr(), ys, rows,
                                              n, _dtype_code(x), _stream_handle(x.device, stream))
    _check(st, "swiglu_gateup_bias_scale_fwd")
    return y


def swiglu_gateup_bias_scale_bwd(dy, x, bias=None, scale=None, dx=None, *, want_dbias=None,
                                 want_dscale=None, in_place: bool = False, workspace=None,
                                 stream=None):
    """Backward of swiglu_gateup_bias_scale_fwd: returns (dx, dbias, dscale).

    dbias ([2n] float32) is computed when want_dbias (default: bias given),
    dscale (float32, shaped like scale) when want_dscale (default: scale
    given). workspace: a device tensor of at least
    swiglu_gateup_bias_scale_workspace_size(...) bytes, allocated if None."""
    import torch
    lib = load_library()
    _require_device(dy, x, dx)
    if x.dim() < 1 or x.shape[-1] % 2:
        raise ValueError("last dimension of x must be even (2n)")
    n = x.shape[-1] // 2
    if dy.dtype != x.dtype:
        raise ValueError("dy and x must have the same dtype")
    rows, xs = _rows_and_stride(x, "x")
    dys = _same_rows(dy, rows, n, "dy")
    bp = _bias_arg(bias, x, n)
    sp, ss = _per_row_arg(scale, x, rows, "scale")
    want_dbias = bias is not None if want_dbias is None else bool(want_dbias)
    want_dscale = scale is not None if want_dscale is None else bool(want_dscale)
    dbias = torch.empty(2 * n, dtype=torch.float32, device=x.device) if want_dbias else None
    dscale = (torch.empty(tuple(scale.shape), dtype=torch.float32, device=x.device)
              if want_dscale and scale is not None else None)
    if want_dscale and scale is None:
        dscale = torch.empty(tuple(x.shape[:-1]), dtype=torch.float32, device=x.device)
    dsp, dss = _per_row_arg(dscale, x, rows, "dscale") if dscale is not None else (None, 1)
    if in_place:
        if dx is not None and dx.data_ptr() != x.data_ptr():
            raise ValueError("in_place backward writes into x; pass dx=None or dx=x")
        dx_ptr, dxs, out = None, 0, x
    else:
        if dx is None:
            dx = torch.empty(tuple(x.shape), dtype=x.dtype, device=x.device)
        if dx.dtype != x.dtype:
            raise ValueError("dx and x must have the same dtype")
        dxs = _same_rows(dx, rows, 2 * n, "dx")
        dx_ptr, out = dx.data_ptr(), dx
    need = swiglu_gateup_bias_scale_workspace_size(rows, n, want_dbias, want_dscale)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if workspace is not None:
        _require_device(workspace, x)
        wp, wb = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    else:
        wp, wb = None, 0
    with torch.cuda.device(x.device):
        st = lib.swiglu_gateup_bias_scale_bwd(
            dy.data_ptr(), dys, x.data_ptr(), xs, bp, sp, ss, dx_ptr, dxs,
            dbias.data_ptr() if dbias is not None else None, dsp, dss, wp, wb, rows, n,
            _dtype_code(x), 1 if in_place else 0, _stream_handle(x.device, stream))
    _check(st, "swiglu_gateup_bias_scale_bwd")
    return out, dbias, dscale


def swiglu_gateup_bias_scale_bwd_noalloc(dy, x, dx=None, dbias=None, dscale=None, *, bias=None,
                                         scale=None, in_place: bool = False, stream=None):
    """swiglu_gateup_bias_scale_bwd without any allocation: the caller passes
    every output (dx, unless in_place; dbias [2n] float32 to get dbias;
    dscale float32 shaped like scale to get dscale) and the partial sums go to
    the library's static per-GPU scratch. Calls that may overlap in time on
    one GPU race on that scratch. Problems needing more than
    NOALLOC_SCRATCH_BYTES of partials raise (SWIGLU_ERR_SCRATCH_LIMIT).
    Returns (dx or x, dbias, dscale)."""
    lib = load_library()
    _require_device(dy, x, dx, dbias, dscale)
    if x.dim() < 1 or x.shape[-1] % 2:
        raise ValueError("last dimension of x must be even (2n)")
    n = x.shape[-1] // 2
    if dy.dtype != x.dtype:
        raise ValueError("dy and x must have the same dtype")
    rows, xs = _rows_and_stride(x, "x")
    dys = _same_rows(dy, rows, n, "dy")
    bp = _bias_arg(bias, x, n)
    sp, ss = _per_row_arg(scale, x, rows, "scale")
    if dbias is not None:
        import torch
        if dbias.dtype != torch.float32 or dbias.dim() != 1 or dbias.shape[0] != 2 * n or \
                (n and dbias.stride(0) != 1):
            raise ValueError(f"dbias must be a contiguous float32 [{2 * n}] tensor")
    dsp, dss = _per_row_arg(dscale, x, rows, "dscale") if dscale is not None else (None, 1)
    if in_place:
        if dx is not None and dx.data_ptr() != x.data_ptr():
            raise ValueError("in_place backward writes into x; pass dx=None or dx=x")
        dx_ptr, dxs, out = None, 0, x
    else:
        if dx is None:
            raise ValueError("the allocation-free backward needs dx (or in_place=True)")
        if dx.dtype != x.dtype:
            raise ValueError("dx and x must have the same dtype")
        dxs = _same_rows(dx, rows, 2 * n, "dx")
        dx_ptr, out = dx.data_ptr(), dx
    import torch
    with torch.cuda.device(x.device):
        st = lib.swiglu_gateup_bias_scale_bwd_noalloc(
            dy.data_ptr(), dys, x.data_ptr(), xs, bp, sp, ss, dx_ptr, dxs,
            dbias.data_ptr() if dbias is not None else None, dsp, dss, rows, n,
            _dtype_code(x), 1 if in_place else 0, _stream_handle(x.device, stream))
    _check(st, "swiglu_gateup_bias_scale_bwd_noalloc")
    return out, dbias, dscale


# ---------------------------------------------------------------------------
# fc1 projection with the SwiGLU epilogue
# ---------------------------------------------------------------------------

def swiglu_fc1_workspace_size() -> int:
    return int(load_library().swiglu_fc1_workspace_size())


# One zeroed fc1 workspace per (device, stream): the kernel leaves it zeroed,
# and launches on one stream never overlap.
_fc1_workspaces: dict = {}


def _fc1_workspace(device, stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    if torch.cuda.is_current_stream_capturing():
        # memory allocated under capture belongs to the graph's pool: the
        # captured launch uses one workgroup per tile instead
        return None
    key = (torch.device(device).index, s.cuda_stream)
    ws = _fc1_workspaces.get(key)
    if ws is None:
        with torch.cuda.stream(s):
            ws = torch.zeros(swiglu_fc1_workspace_size(), dtype=torch.uint8, device=device)
        _fc1_workspaces[key] = ws
    return ws


def swiglu_fc1_fwd(a, w, y=None, *, x_out=None, stream=None, workspace=None):
    """y = silu(a @ w[:n].T) * (a @ w[n:].T) for bf16 a [..., k] and w [2n, k].

    x_out: None, True (allocate) or a [..., 2n] tensor that receives a @ w.T.
    Returns y, or (y, x_out) when x_out is requested. n and k must be
    multiples of 64, rows 16-byte aligned, and the row strides of a and w at
    most 2^28 elements; anything else raises ValueError (the C entry point's
    status).

    workspace: None (a zeroed buffer kept per device and stream; none while
    the stream is being captured into a graph), False (none: one workgroup
    per tile), or a device tensor of swiglu_fc1_workspace_size() bytes that
    is all zero and not in use by another launch. The outputs are the same
    bits either way."""
    import torch
    lib = load_library()
    _require_device(a, w, y, x_out if isinstance(x_out, torch.Tensor) else None)
    if w.dim() != 2 or w.shape[0] % 2:
        raise ValueError("w must be [2n, k]")
    n, k = w.shape[0] // 2, w.shape[1]
    if a.shape[-1] != k:
        raise ValueError(f"a must have {k} columns")
    if a.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise ValueError("swiglu_fc1_fwd needs bfloat16 a and w")
    m, lda = _rows_and_stride(a, "a")
    _, ldw = _rows_and_stride(w, "w")
    if y is None:
        y = torch.empty(tuple(a.shape[:-1]) + (n,), dtype=a.dtype, device=a.device)
    if y.dtype != torch.bfloat16:
        raise ValueError("y must be bfloat16")
    ldy = _same_rows(y, m, n, "y")
    want_x = x_out is not None and x_out is not False
    if x_out is True:
        x_out = torch.empty(tuple(a.shape[:-1]) + (2 * n,), dtype=a.dtype, device=a.device)
    xp, ldx = None, 0
    if want_x:
        if x_out.dtype != torch.bfloat16:
            raise ValueError("x_out must be bfloat16")
        ldx = _same_rows(x_out, m, 2 * n, "x_out")
        xp = x_out.data_ptr()
    if workspace is None:
        workspace = _fc1_workspace(a.device, stream)
    elif workspace is False:
        workspace = None
    wsp = None
    if workspace is not None:
        _require_device(workspace, a)
        if workspace.numel() * workspace.element_size() < swiglu_fc1_workspace_size():
            raise ValueError("fc1 workspace smaller than swiglu_fc1_workspace_size()")
        wsp = workspace.data_ptr()
    with torch.cuda.device(a.device):
        st = lib.swiglu_fc1_fwd(a.data_ptr(), lda, w.data_ptr(), ldw, y.data_ptr(), ldy, xp, ldx,
                                m, n, k, _dtype_code(a), wsp, _stream_handle(a.device, stream))
    _check(st, "swiglu_fc1_fwd")
    return (y, x_out) if want_x else y
