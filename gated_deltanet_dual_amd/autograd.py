"""torch.autograd wrapper of the dual-stream Gated DeltaNet layer.

``gdn_dual(varlen, q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n,
block_size, h0=None, scale=0.0, flags=0, ckpt_stride=1, window=0)`` returns
``(o, on, h_final)`` and records the reverse mode: the forward runs
flare_gdn_dual_fwd with the chunk-start states saved, the backward runs
flare_gdn_dual_bwd with the incoming output gradients.  By default every
chunk-start state is kept and so is the forward's workspace, whose chunk
matrices the backward then reads.  With ckpt_stride > 1 only every
ckpt_stride-th state is kept (the backward rebuilds the others) and nothing
else survives the forward; window > 0 runs both passes in windows of that
many chunks of every document, so their workspaces no longer grow with the
sequence.  Marshalling only, like the binding it calls: every step of the
computation runs in the library's HIP kernels.

Method: "FLARE: Diffusion for Hybrid Language Model" (papernotes.org notes),
Key designs items 2-3 (the dual-stream forward and the block-level gradient
injection into the causal chain).
"""
from __future__ import annotations

import torch

from . import Varlen, gdn_dual_bwd, gdn_dual_fwd, workspace_bytes, _io_of

_GRADS = ("dq", "dk", "dv", "dalpha", "dbeta", "dqn", "dkn", "dvn", "dalpha_n", "dbeta_n")


class GDNDualFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, varlen, block_size, scale, flags, stride, window, q, k, v, alpha, beta, qn, kn, vn, alpha_n,
                beta_n, h0):
        T, H, d = q.shape
        fws = None
        nbytes = workspace_bytes(varlen, H, d, block_size, _io_of(q), flags, window=window)
        if nbytes > 0:
            fws = torch.empty((nbytes,), dtype=torch.uint8, device=q.device)
        o, on, hf, ckpt = gdn_dual_fwd(varlen, q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n, block_size,
                                       h0=h0, scale=scale, flags=flags, want_ckpt=True, workspace=fws,
                                       ckpt_stride=stride, window=window)
        ctx.varlen, ctx.block_size, ctx.scale, ctx.flags = varlen, block_size, scale, flags
        ctx.stride, ctx.window = stride, window
        ctx.has_h0 = h0 is not None
        # the one-pass forward's chunk matrices serve the backward; the memory
        # modes keep nothing but the strided checkpoints
        ctx.fws = fws if stride == 1 and window == 0 else None
        ctx.save_for_backward(q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n, h0, ckpt)
        return o, on, hf

    @staticmethod
    def backward(ctx, d_o, d_on, dh_final):
        q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n, h0, ckpt = ctx.saved_tensors
        d_o = torch.zeros_like(q) if d_o is None else d_o.contiguous()
        d_on = torch.zeros_like(q) if d_on is None else d_on.contiguous()
        if dh_final is not None:
            dh_final = dh_final.contiguous()
        g = gdn_dual_bwd(ctx.varlen, q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n, ctx.block_size, ckpt,
                         d_o, d_on, h0=h0, dh_final=dh_final, scale=ctx.scale, flags=ctx.flags,
                         want_dh0=ctx.has_h0, fwd_workspace=ctx.fws, ckpt_stride=ctx.stride, window=ctx.window)
        ctx.fws = None
        return (None,) * 6 + tuple(g[n] for n in _GRADS) + (g["dh0"] if ctx.has_h0 else None,)


def gdn_dual(varlen: Varlen, q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n, block_size, h0=None, scale=0.0,
             flags=0, ckpt_stride=1, window=0):
    """Differentiable dual-stream forward: (o, on, h_final).  Gradients flow
    to q, k, v, alpha, beta of both streams and to h0 (when given).
    ckpt_stride / window: the memory modes described above (window a multiple
    of ckpt_stride)."""
    return GDNDualFunction.apply(varlen, int(block_size), float(scale), int(flags), int(ckpt_stride), int(window),
                                 q, k, v, alpha, beta, qn, kn, vn, alpha_n, beta_n, h0)
