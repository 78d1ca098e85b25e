"""The dual-weight GLU as an autograd Function over the library's two entry points.

Mirrors the segKI "Plan B" design (DeepSpeed PR #8602, comment "Plan B:
Dual-Weight GEMV", section "Plan B Design"): the Function keeps hidden, gate_w and up_w, reads the weight
Parameters in place in both directions, and returns gradients for all three,
so training and generation share one forward and one set of weights.
Forward: glu_dual_gemv; backward: glu_dual_gemv_backward (up to 65536 rows
of hidden per call).  Only argument marshalling happens here.
"""
import torch

from . import api


class DualWeightGlu(torch.autograd.Function):
    @staticmethod
    def forward(ctx, hidden, gate_w, up_w):
        ctx.save_for_backward(hidden, gate_w, up_w)
        return api.dual_gemv(hidden, gate_w, up_w)

    @staticmethod
    def backward(ctx, dout):
        hidden, gate_w, up_w = ctx.saved_tensors
        dh, dwg, dwu = api.dual_gemv_backward(hidden.contiguous(), gate_w.contiguous(), up_w.contiguous(),
                                              dout.contiguous())
        return dh, dwg, dwu


def dual_weight_glu(hidden: torch.Tensor, gate_w: torch.Tensor, up_w: torch.Tensor) -> torch.Tensor:
    """out = silu(hidden @ gate_w.T) * (hidden @ up_w.T) with bf16 rounding per tensor, differentiable."""
    return DualWeightGlu.apply(hidden, gate_w, up_w)
