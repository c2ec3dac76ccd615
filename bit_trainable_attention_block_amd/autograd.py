"""A training-step wrapper over the four C-ABI calls: SageBwd attention as a
torch.autograd.Function (SageBwd paper summary, "method step details":
forward steps (1)-(5), backward steps (1)-(7)).

    O = sage_attention(Q, K, V, causal=True)     # Q, K, V: [B, H, N, D] bf16/fp16 on the GPU
    O.backward(dO)                               # Q.grad, K.grad, V.grad in the input dtype

Forward: sage_quantize then sage_fwd; the INT8 codes, scales and means, V,
O and the logsumexp L are kept for the backward (3 bytes of codes per element
beside the 16-bit V: the backward recomputes S and P from the codes, it does
not keep them, and forms dP from V's 16-bit values).  Backward: sage_bwd_pre on the incoming dO, then
sage_bwd.  The library computes every step; this module only allocates the
buffers and passes pointers and the current stream; sage_cast_grads rounds
the float32 gradients to the input dtype.  Without libsage.so the calls
raise.
"""
from __future__ import annotations

import torch

from . import binding as bd


class SageAttentionFunction(torch.autograd.Function):
    """autograd.Function over sage_quantize / sage_fwd / sage_bwd_pre / sage_bwd."""

    @staticmethod
    def forward(ctx, Q, K, V, causal: bool, k_smooth: bool, q_smooth: bool, sm_scale: float, bq: int,
                qk_norm: bool, fp8: bool):
        if not (Q.is_cuda and K.is_cuda and V.is_cuda):
            raise ValueError("sage_attention: Q, K, V must be GPU tensors")
        if Q.dtype not in (torch.bfloat16, torch.float16) or K.dtype != Q.dtype or V.dtype != Q.dtype:
            raise ValueError("sage_attention: Q, K, V must share one dtype, bf16 or fp16")
        if Q.dim() != 4 or K.shape != Q.shape or V.shape != Q.shape:
            raise ValueError("sage_attention: Q, K, V must be [B, H, N, D] of one shape")
        B, H, N, D = Q.shape
        sh = bd.Shape(B=B, H=H, N=N, D=D, bq=bq, bkv=64,
                      dtype=bd.SAGE_BF16 if Q.dtype == torch.bfloat16 else bd.SAGE_FP16,
                      causal=bool(causal), k_smooth=bool(k_smooth), q_smooth=bool(q_smooth),
                      sm_scale=float(sm_scale), qk_norm=bool(qk_norm), fp8=bool(fp8))
        Q, K, V = Q.contiguous(), K.contiguous(), V.contiguous()
        qt = bd.quantize(sh, Q, K, V)
        O, L = bd.fwd(sh, qt)
        ctx.sh = sh
        ctx.qt = qt          # codes, scales and means
        if qk_norm:
            ctx.save_for_backward(O, L, V, Q, K)   # the norm's gradient needs the input rows
        else:
            ctx.save_for_backward(O, L, V)
        return O

    @staticmethod
    def backward(ctx, dO):
        O, L, V = ctx.saved_tensors[:3]
        sh = ctx.sh
        dO = dO.to(O.dtype).contiguous()
        dot = bd.bwd_pre(sh, O, dO)
        dQ, dK, dV = bd.bwd(sh, ctx.qt, dot, V, dO, L)
        if sh.qk_norm:
            Q, K = ctx.saved_tensors[3:]
            bd.qk_norm_bwd(sh, Q, K, ctx.qt, dQ, dK)
        ctx.qt = None
        dQ, dK, dV = bd.cast_grads(sh, dQ, dK, dV)   # float32 -> the input dtype, in the library
        return dQ, dK, dV, None, None, None, None, None, None, None


def sage_attention(Q, K, V, causal: bool = False, k_smooth: bool = True, q_smooth: bool = False,
                   sm_scale: float = 0.0, bq: int = 128, qk_norm: bool = False, fp8: bool = False):
    """SageBwd INT8 attention with gradients (sm_scale 0 selects 1/sqrt(D)).
    qk_norm=True applies QK-norm (unit gain) to Q and K inside sage_quantize
    and returns gradients w.r.t. the un-normalised inputs.  fp8=True runs the
    E4M3 variant (E4M3 codes in place of INT8; see include/sage.h)."""
    return SageAttentionFunction.apply(Q, K, V, causal, k_smooth, q_smooth, sm_scale, bq, qk_norm, fp8)
