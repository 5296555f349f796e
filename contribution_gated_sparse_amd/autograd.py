"""``torch.autograd`` entry to the MALA operator: the forward is ``mala_fwd``
(online allocation, Sec. 2.2 Eq. 3) and the backward is ``mala_bwd`` on the
saved log-normalizer (offline allocation, Sec. 2.2 Eq. 4), exactly as a
training step pairs them (Alg. 1 and 2). This module only routes tensors
between autograd and the two C-ABI calls; all arithmetic runs in libmala.

Queries may be the last N_q of N_k positions (chunked prefill): the causal
mask is bottom-right aligned, key k being visible to query row q iff
k <= q + (N_k - N_q).
"""
from __future__ import annotations

from typing import Optional

import torch

from .mala import mala_bwd, mala_fwd


class MalaAttentionFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, tau: float, causal: bool, softmax_scale: Optional[float],
                fast_grad: bool, gate_pass: bool):
        # the gate pass scores only the tiles the forward kept (nested
        # support, Sec. 2.2), which needs the forward's tile mask
        out = mala_fwd(q, k, v, tau, causal=causal, softmax_scale=softmax_scale, want_kept=False,
                       want_mask=gate_pass)
        ctx.save_for_backward(q, k, v, out["o"], out["lse"], out["mask"])
        ctx.cfg = (tau, causal, softmax_scale, fast_grad, gate_pass)
        return out["o"]

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, o, lse, fmask = ctx.saved_tensors
        tau, causal, scale, fast_grad, gate_pass = ctx.cfg
        g = mala_bwd(q, k, v, o, lse, d_o.contiguous(), tau, causal=causal, softmax_scale=scale,
                     want_kept=False, fast_grad=fast_grad, gate_pass=gate_pass,
                     fwd_mask=fmask if gate_pass else None)
        return g["dq"], g["dk"], g["dv"], None, None, None, None, None


def mala_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tau: float,
                   causal: bool = True, softmax_scale: Optional[float] = None,
                   fast_grad: bool = False, gate_pass: bool = False) -> torch.Tensor:
    """MALA attention with autograd. q [B,Hq,Nq,d], k, v [B,Hkv,Nk,d] (bf16 or
    fp32, contiguous, on the GPU); returns O [B,Hq,Nq,d]. ``gate_pass``: the
    backward takes its decisions in a separate score pass over the tiles the
    forward kept (the forward then also stores its tile mask, int8
    [B,Hq,ceil(Nq/32),ceil(Nk/64)], until the backward) and skips the steps
    without a kept tile (for inputs where few tiles are kept)."""
    return MalaAttentionFunction.apply(q, k, v, tau, causal, softmax_scale, fast_grad, gate_pass)
