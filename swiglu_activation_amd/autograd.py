"""Autograd ops and a Megatron-style module over the HIP kernels.

Behaviour follows the Liger-Kernel Megatron SwiGLU page:
* §Background / §What's added: a differentiable op on the packed fc1 output
  [..., 2n] (gate first, up second) whose backward recomputes silu from the
  saved input; only that input is saved.
* §How to use: the module is called with the positional arguments of
  Megatron's bias_swiglu_impl -- (intermediate, bias, fp8_input_store,
  cpu_offload_input) -- so it can stand in for it.
* §Optional in_place: with in_place=True the backward writes [dgate | dup]
  over the saved fc1 output instead of a new buffer (opt-in, off by default).
* §Known issues: writes through a raw pointer do not bump torch's version
  counter, so a second backward through the same graph (retain_graph=True)
  would read gradients as if they were activations; the op remembers that
  its in-place backward ran and raises on a second one.
* §Scope: FP8 input retention and CPU offload are served by Megatron's own
  path. There is no Megatron here, so they are errors (the behaviour the
  page gives for fallback_impl=None). A bias on the fc1 output, which the
  page also leaves to Megatron, is served here by the bias kernels, and so is
  the per-token-scale (router-weighted) form the page lists as a follow-up.
* §Background: the two-tensor op for models whose gate and up projections
  are separate tensors.

The fc1 projection followed by the SwiGLU (Liger-Kernel test/cute page,
§MLP1 numerical reference: fused MLP1-with-activation variants) is wired in
as Fc1SwiGLU. Its forward either runs the projection as a library GEMM
(torch.matmul) and then the fused gate-up SwiGLU kernel on the [tokens, 2n]
product (the default), or, with fused_epilogue=True, the one kernel that
computes the projection with the SwiGLU as its epilogue and also writes the
product. The default is the faster of the two on MI355X: with the product
written (as the backward needs it), the GEMM then the SwiGLU took 5.92 ms
against 6.11 ms for the fused kernel at 8192 tokens, hidden 8192 and
n = 32768, and the two were level at hidden 4096, n = 4096. The backward is
the SwiGLU backward kernel followed by the two weight and input GEMMs of
the projection (plain library GEMMs through torch.matmul).

Every SwiGLU computation runs in libswiglu_gateup.so; this module only wires
it into autograd.
"""

from __future__ import annotations

import torch

from . import (swiglu_fc1_fwd, swiglu_gateup_bias_scale_bwd, swiglu_gateup_bias_scale_fwd,
               swiglu_gateup_bwd, swiglu_gateup_fwd, swiglu_silu_mul_bwd, swiglu_silu_mul_fwd,
               _rows_and_stride)

__all__ = ["FusedGateUpSiLUMul", "FusedGateUpSiLUMulBiasScale", "SiLUMul", "MegatronSwiGLU",
           "Fc1SwiGLU", "FusedFc1SwiGLU", "fc1_swiglu", "fused_gate_up_swiglu", "silu_mul",
           "weighted_swiglu"]


def _as_row_view(t: torch.Tensor) -> torch.Tensor:
    """t itself if the kernels can address it as [rows, width] with a single
    row stride, else a contiguous copy (autograd may hand in expanded or
    transposed gradients)."""
    try:
        _rows_and_stride(t, "t")
        return t
    except ValueError:
        return t.contiguous()


class FusedGateUpSiLUMul(torch.autograd.Function):
    """y = silu(x[..., :n]) * x[..., n:]; dx = [dgate | dup]."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, in_place: bool = False):
        x = _as_row_view(x)
        y = swiglu_gateup_fwd(x)
        ctx.save_for_backward(x)
        ctx.in_place = bool(in_place)
        ctx.already_backward = False
        return y

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        (x,) = ctx.saved_tensors
        dy = _as_row_view(dy)
        if ctx.in_place:
            if ctx.already_backward:
                raise RuntimeError(
                    "FusedGateUpSiLUMul: backward called a second time with in_place=True; the "
                    "first backward overwrote the saved fc1 output with its gradient. Use "
                    "in_place=False to backpropagate through this graph more than once.")
            ctx.already_backward = True
            dx = swiglu_gateup_bwd(dy, x, in_place=True)
        else:
            dx = swiglu_gateup_bwd(dy, x)
        return dx, None


class SiLUMul(torch.autograd.Function):
    """y = silu(gate) * up on two tensors; returns (dgate, dup) in backward."""

    @staticmethod
    def forward(ctx, gate: torch.Tensor, up: torch.Tensor, in_place: bool = False):
        gate, up = _as_row_view(gate), _as_row_view(up)
        y = swiglu_silu_mul_fwd(gate, up)
        ctx.save_for_backward(gate, up)
        ctx.in_place = bool(in_place)
        ctx.already_backward = False
        return y

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        gate, up = ctx.saved_tensors
        dy = _as_row_view(dy)
        if ctx.in_place:
            if ctx.already_backward:
                raise RuntimeError(
                    "SiLUMul: backward called a second time with in_place=True; the first "
                    "backward overwrote the saved gate and up with their gradients.")
            ctx.already_backward = True
        dgate, dup = swiglu_silu_mul_bwd(dy, gate, up, in_place=ctx.in_place)
        return dgate, dup, None


class FusedGateUpSiLUMulBiasScale(torch.autograd.Function):
    """y = s * silu(z[..., :n]) * z[..., n:] with z = x + bias; bias ([2n])
    and the per-token scale s (shape x.shape[:-1], or with a trailing 1) are
    optional. Gradients for x, bias and s."""

    @staticmethod
    def forward(ctx, x, bias, scale, in_place: bool = False):
        x = _as_row_view(x)
        s32 = None
        if scale is not None:
            s32 = scale if scale.dtype == torch.float32 else scale.float()
        y = swiglu_gateup_bias_scale_fwd(x, bias, s32)
        ctx.save_for_backward(x, bias, s32)
        ctx.scale_dtype = None if scale is None else scale.dtype
        ctx.in_place = bool(in_place)
        ctx.already_backward = False
        return y

    @staticmethod
    def backward(ctx, dy):
        x, bias, s32 = ctx.saved_tensors
        dy = _as_row_view(dy)
        if ctx.in_place:
            if ctx.already_backward:
                raise RuntimeError(
                    "FusedGateUpSiLUMulBiasScale: backward called a second time with "
                    "in_place=True; the first backward overwrote the saved fc1 output.")
            ctx.already_backward = True
        want_db = bias is not None and ctx.needs_input_grad[1]
        want_ds = s32 is not None and ctx.needs_input_grad[2]
        dx, dbias, dscale = swiglu_gateup_bias_scale_bwd(
            dy, x, bias, s32, want_dbias=want_db, want_dscale=want_ds, in_place=ctx.in_place)
        if dbias is not None:
            dbias = dbias.to(bias.dtype)
        if dscale is not None:
            dscale = dscale.to(ctx.scale_dtype)
        return dx, dbias, dscale, None


def fused_gate_up_swiglu(x: torch.Tensor, in_place: bool = False) -> torch.Tensor:
    return FusedGateUpSiLUMul.apply(x, in_place)


def silu_mul(gate: torch.Tensor, up: torch.Tensor, in_place: bool = False) -> torch.Tensor:
    return SiLUMul.apply(gate, up, in_place)


def weighted_swiglu(x: torch.Tensor, weights: torch.Tensor, bias=None,
                    in_place: bool = False) -> torch.Tensor:
    """Per-token-scaled fused SwiGLU for MoE routed experts:
    weights * silu(z[..., :n]) * z[..., n:], z = x + bias (bias optional)."""
    return FusedGateUpSiLUMulBiasScale.apply(x, bias, weights, in_place)


class MegatronSwiGLU(torch.nn.Module):
    """Drop-in for Megatron's bias_swiglu_impl on the packed [s, b, 2n] or
    [tokens, 2n] fc1 output.

    Called as module(intermediate, bias, fp8_input_store, cpu_offload_input)
    with the same positional order. bias ([2n]) may be None or a tensor;
    fp8_input_store=True and cpu_offload_input=True raise NotImplementedError.
    """

    def __init__(self, in_place: bool = False):
        super().__init__()
        self.in_place = bool(in_place)

    def extra_repr(self) -> str:
        return f"in_place={self.in_place}"

    def forward(self, intermediate: torch.Tensor, bias=None, fp8_input_store: bool = False,
                cpu_offload_input: bool = False) -> torch.Tensor:
        if fp8_input_store:
            raise NotImplementedError("MegatronSwiGLU: fp8_input_store=True is not supported")
        if cpu_offload_input:
            raise NotImplementedError("MegatronSwiGLU: cpu_offload_input=True is not supported")
        if intermediate.dim() not in (2, 3):
            raise ValueError(f"MegatronSwiGLU: expected a 2D or 3D input, got {intermediate.dim()}D")
        if intermediate.shape[-1] % 2:
            raise ValueError("MegatronSwiGLU: the last dimension must be 2 * ffn_hidden (even)")
        if bias is not None:
            return FusedGateUpSiLUMulBiasScale.apply(intermediate, bias, None, self.in_place)
        return FusedGateUpSiLUMul.apply(intermediate, self.in_place)


class Fc1SwiGLU(torch.autograd.Function):
    """y = silu(a W_g^T) * (a W_u^T) for bf16 a [..., k] and W = [W_g; W_u]
    [2n, k]. Saves a, W and the product a W^T. fused_epilogue: compute it
    with the fc1 kernel that has the SwiGLU as its epilogue (one launch) rather
    than a library GEMM followed by the SwiGLU kernel (the default, faster on
    MI355X at the shapes measured)."""

    @staticmethod
    def forward(ctx, a: torch.Tensor, w: torch.Tensor, fused_epilogue: bool = False):
        k = w.shape[1]
        a2 = _as_row_view(a.reshape(-1, k))
        if fused_epilogue:
            y, x = swiglu_fc1_fwd(a2, w, x_out=True)
        else:
            x = torch.matmul(a2, w.t())                # [m, 2n] = [gate | up]
            y = swiglu_gateup_fwd(x)
        ctx.save_for_backward(a2, w, x)
        ctx.a_shape = tuple(a.shape)
        return y.reshape(tuple(a.shape[:-1]) + (w.shape[0] // 2,))

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        a2, w, x = ctx.saved_tensors
        n = w.shape[0] // 2
        dy2 = _as_row_view(dy.reshape(-1, n))
        dx = swiglu_gateup_bwd(dy2, x)                 # [m, 2n] = [dgate | dup]
        da = dx @ w if ctx.needs_input_grad[0] else None
        dw = dx.t() @ a2 if ctx.needs_input_grad[1] else None
        return (da.reshape(ctx.a_shape) if da is not None else None), dw, None


def fc1_swiglu(a: torch.Tensor, w: torch.Tensor, fused_epilogue: bool = False) -> torch.Tensor:
    return Fc1SwiGLU.apply(a, w, fused_epilogue)


class FusedFc1SwiGLU(torch.nn.Module):
    """The first half of a SwiGLU MLP: a bias-free fc1 projection to [gate | up]
    (weight [2 * ffn_hidden, hidden], the Linear layout) followed by the
    SwiGLU, with no chunk or copy between them. bf16 only. fused_epilogue
    selects the single fc1 kernel with the SwiGLU in its epilogue; by default
    the projection is a library GEMM and the SwiGLU the fused gate-up kernel,
    which measured faster (see Fc1SwiGLU)."""

    def __init__(self, hidden: int, ffn_hidden: int, device=None, dtype=torch.bfloat16,
                 fused_epilogue: bool = False):
        super().__init__()
        if dtype != torch.bfloat16:
            raise ValueError("FusedFc1SwiGLU is bf16 only")
        self.fused_epilogue = fused_epilogue
        self.weight = torch.nn.Parameter(torch.empty(2 * ffn_hidden, hidden, device=device,
                                                     dtype=dtype))
        torch.nn.init.normal_(self.weight, std=hidden ** -0.5)

    def forward(self, a: torch.Tensor) -> torch.Tensor:
        return Fc1SwiGLU.apply(a, self.weight, self.fused_epilogue)
