"""PyTorch autograd wrapper: a linear layer y = x . w^T whose backward is the
HLQ/HOT backward of libhlq.so.

"HOT: Hadamard-based Optimized Training" (scime.ai summary, "Approach"): the
stored activation is compressed at forward time (activation buffer
compression), and the backward runs Hadamard quantization on g_x and Hadamard
low-rank approximation plus INT8 on g_w.  The forward product itself is
unchanged by the method; what this wrapper keeps for the backward is the ACBP
form of x (INT4 codes + one fp32 scale per token) instead of x, and its
backward is one ``hlq_linear_backward`` call.  For bf16 x and w with I a
multiple of 32 the forward is one ``hlq_linear_forward`` launch (the bf16
MFMA product with the codes of x emitted by the same launch); otherwise
torch's matmul and ``hlq_compress_act``.  Leading dimensions of x are
flattened into tokens.  No bias (its gradient is not part of the method).
"""
from __future__ import annotations

import torch

from . import hlq


class HLQLinearFunction(torch.autograd.Function):
    """y = x . w^T; backward by ``hlq_linear_backward`` on the ACBP codes of x."""

    @staticmethod
    def forward(ctx, x, w, block, rank, gx_mode, gw_mode, reduction):
        if x.shape[-1] != w.shape[1]:
            raise ValueError("x [..., I] and w [O, I] disagree on I")
        x2 = x.reshape(-1, x.shape[-1]).contiguous()
        if x2.dtype == torch.bfloat16 and w.dtype == torch.bfloat16 and x2.shape[1] % 32 == 0:
            y, codes, scales = hlq.hlq_linear_forward(x2, w.contiguous())
        else:
            y = x2 @ w.t()
            codes, scales = hlq.hlq_compress_act(x2)
        ctx.save_for_backward(codes, scales, w)
        ctx.cfg = (block, rank, gx_mode, gw_mode, reduction)
        ctx.x_shape, ctx.x_dtype = x.shape, x.dtype
        return y.reshape(*x.shape[:-1], w.shape[0])

    @staticmethod
    def backward(ctx, g_y):
        codes, scales, w = ctx.saved_tensors
        block, rank, gx_mode, gw_mode, reduction = ctx.cfg
        gy2 = g_y.reshape(-1, g_y.shape[-1])
        if gy2.dtype != w.dtype:
            gy2 = gy2.to(w.dtype)
        gy2 = gy2.contiguous()
        g_x, g_w = hlq.hlq_linear_backward(gy2, codes, scales, w.contiguous(), block, rank,
                                           gx_mode, gw_mode, reduction)
        g_x = g_x.reshape(ctx.x_shape).to(ctx.x_dtype) if ctx.needs_input_grad[0] else None
        g_w = g_w.to(w.dtype) if ctx.needs_input_grad[1] else None
        return g_x, g_w, None, None, None, None, None


def hlq_linear(x, w, block, rank, gx_mode=hlq.HLQ_PER_TOKEN, gw_mode=hlq.HLQ_PER_TOKEN,
               reduction=hlq.HLQ_SUM):
    """Functional form of :class:`HLQLinear`."""
    return HLQLinearFunction.apply(x, w, block, rank, gx_mode, gw_mode, reduction)


class HLQLinear(torch.nn.Module):
    """Bias-free linear layer (weight [out_features, in_features]) trained with
    the HLQ/HOT backward.  ``block`` and ``rank`` are the Hadamard block and the
    low-rank r of the g_w path; the token count of every batch must be a
    multiple of ``block``, and out_features too."""

    def __init__(self, in_features, out_features, block=16, rank=8,
                 gx_mode=hlq.HLQ_PER_TOKEN, gw_mode=hlq.HLQ_PER_TOKEN, reduction=hlq.HLQ_SUM,
                 device=None, dtype=None):
        super().__init__()
        self.weight = torch.nn.Parameter(
            torch.empty((out_features, in_features), device=device, dtype=dtype))
        torch.nn.init.kaiming_uniform_(self.weight, a=5 ** 0.5)
        self.block, self.rank = block, rank
        self.gx_mode, self.gw_mode, self.reduction = gx_mode, gw_mode, reduction

    def forward(self, x):
        return hlq_linear(x, self.weight, self.block, self.rank, self.gx_mode, self.gw_mode,
                          self.reduction)

    def extra_repr(self):
        return (f"in_features={self.weight.shape[1]}, out_features={self.weight.shape[0]}, "
                f"block={self.block}, rank={self.rank}, gx_mode={self.gx_mode}, "
                f"gw_mode={self.gw_mode}")
