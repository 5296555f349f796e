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
                fast_grad: bool, gate_pass, nested: bool):
        # the nested backward scores only the tiles the forward kept, which
        # needs the forward's tile mask; the automatic walk choice reads the
        # forward's kept-tile counters
        auto = gate_pass == "auto"
        out = mala_fwd(q, k, v, tau, causal=causal, softmax_scale=softmax_scale, want_kept=auto,
                       want_mask=nested)
        ctx.save_for_backward(q, k, v, out["o"], out["lse"], out["mask"], out["kept"])
        ctx.cfg = (tau, causal, softmax_scale, fast_grad, gate_pass, nested)
        return out["o"]

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, o, lse, fmask, fkept = ctx.saved_tensors
        tau, causal, scale, fast_grad, gate_pass, nested = ctx.cfg
        auto = gate_pass == "auto"
        g = mala_bwd(q, k, v, o, lse, d_o.contiguous(), tau, causal=causal, softmax_scale=scale,
                     want_kept=False, fast_grad=fast_grad, gate_pass=False if auto else gate_pass,
                     fwd_mask=fmask if nested else None, fwd_kept=fkept if auto else None)
        return g["dq"], g["dk"], g["dv"], None, None, None, None, None, None


def mala_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tau: float,
                   causal: bool = True, softmax_scale: Optional[float] = None,
                   fast_grad: bool = False, gate_pass=False,
                   nested: bool = False) -> torch.Tensor:
    """MALA attention with autograd. q [B,Hq,Nq,d], k, v [B,Hkv,Nk,d] (bf16 or
    fp32, contiguous, on the GPU); returns O [B,Hq,Nq,d].

    ``gate_pass``: True: the backward takes every decision in a separate
    score pass over all legal tiles (MALA_FLAG_GATE_PASS), then skips the
    steps without a kept tile (for inputs where few tiles are kept). "auto":
    the forward also returns its kept-tile counters, and the backward
    chooses between that mode and the default walk on the device, from its
    own decisions on a sample of the key tiles (mala_bwd_auto).
    ``nested``: the backward scores only the tiles the forward kept
    (mala_bwd_nested, which runs in the gate-pass mode): the forward also
    stores its tile mask, int8 [B,Hq,ceil(Nq/32),ceil(Nk/64)], until the
    backward. This relies on the nesting of the supports (Sec. 2.2) instead
    of recomputing the scores of forward-skipped tiles, which the paper's
    backward does before every skip decision (App. A.1)."""
    if gate_pass not in (False, True, "auto"):
        raise ValueError('gate_pass must be False, True or "auto"')
    if gate_pass == "auto" and nested:
        raise ValueError('nested runs the gate-pass walks: gate_pass="auto" does not apply')
    return MalaAttentionFunction.apply(q, k, v, tau, causal, softmax_scale, fast_grad, gate_pass,
                                       nested)
