"""Attention as a torch.autograd.Function over the library's forward and
backward entry points.

``attention(q, k, v, ...)`` returns O and, when the inputs require gradients,
records the library's backward: dQ, dK, dV come from fa_bwd (or its grouped,
masked and dropout variants), which rebuilds P from O and the saved
logsumexp.  Only the arguments are marshalled here; every step runs in the
library's kernels.
"""

from __future__ import annotations

import torch

from . import binding


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal, scale, dropout_p, seed, offset, tiles):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        if dropout_p > 0.0:
            o, lse = binding.fwd_dropout(q, k, v, dropout_p, seed, offset, causal=causal, scale=scale, tiles=tiles)
        elif tiles is not None:
            o, lse = binding.fwd_masked(q, k, v, tiles, causal=causal, scale=scale)
        else:
            o, lse = binding.fwd(q, k, v, causal=causal, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.tiles = tiles
        ctx.params = (causal, scale, dropout_p, seed, offset)
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, do, _dlse):
        q, k, v, o, lse = ctx.saved_tensors
        causal, scale, dropout_p, seed, offset = ctx.params
        do = do.contiguous()
        if dropout_p > 0.0:
            dq, dk, dv = binding.bwd_dropout(q, k, v, o, lse, do, dropout_p, seed, offset, causal=causal, scale=scale,
                                             tiles=ctx.tiles)
        elif ctx.tiles is not None:
            dq, dk, dv = binding.bwd_masked(q, k, v, o, lse, do, ctx.tiles, causal=causal, scale=scale)
        else:
            dq, dk, dv = binding.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
        return dq, dk, dv, None, None, None, None, None, None


def attention(q, k, v, causal=False, scale=None, dropout_p=0.0, key_mask=None, seed=None, offset=0,
              return_lse=False):
    """Exact attention O = softmax(scale * Q K^T + M) V, differentiable.

    q: [B, H, N, D]; k, v: [B, H_kv, N, D] (H_kv divides H); fp16 or bf16 on
    the GPU.  key_mask: optional [B, N] (nonzero = visible).  dropout_p > 0
    drops probabilities with the library's regenerated Philox mask; seed
    (drawn from torch's generator when None) and offset identify it, and the
    backward uses the same pair.  Returns O, or (O, LSE) with return_lse.
    """
    if scale is None:
        scale = q.shape[-1] ** -0.5
    if dropout_p > 0.0 and seed is None:
        seed = int(torch.randint(0, 2 ** 62, (1,)).item())
    tiles = binding.mask_tiles(key_mask) if key_mask is not None else None
    o, lse = _Attention.apply(q, k, v, bool(causal), float(scale), float(dropout_p), int(seed or 0), int(offset),
                              tiles)
    return (o, lse) if return_lse else o
