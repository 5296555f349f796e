"""Fidelity and matched-work measurements of the MALA operator (App. C.2,
C.3; Sec. 3, Table 1), computed with torch from the operator's outputs.

Measurement only: nothing here is a step of the operator, which runs in
libmala's kernels. These functions turn the library's outputs (O, the
log-normalizer z, the forward tile mask) into the quantities the paper
reports:

* omitted normalized mass per row, 1 - Z_R / Z = 1 - exp(z_R - z) (App. C.2),
  bounded by tau / (1 + tau) (Prop. 1);
* head-level relative L2 errors of outputs and gradients against the tau = 0
  operator (App. C.3);
* a per-instance reference-mass control at matched work (App. C.2): for every
  forward decision (query head x query block) it keeps exactly as many key
  tiles as MALA kept there, chosen by their mass under the unscreened
  softmax; both supports are scored the same way, so the comparison isolates
  the allocation.
"""
from __future__ import annotations

import torch


def omitted_mass(lse: torch.Tensor, lse_dense: torch.Tensor) -> torch.Tensor:
    """1 - exp(z_R - z) per row, in fp64 (App. C.2)."""
    return 1.0 - torch.exp(lse.double() - lse_dense.double())


def head_rel_l2(x: torch.Tensor, x0: torch.Tensor) -> torch.Tensor:
    """||x - x0|| / ||x0|| per (batch, head) over that head's [N, d] block
    (App. C.3), flattened over batch and heads."""
    num = (x.double() - x0.double()).pow(2).sum((-1, -2)).sqrt()
    den = x0.double().pow(2).sum((-1, -2)).sqrt().clamp_min(1e-300)
    return (num / den).flatten()


def mean_p95(t: torch.Tensor) -> dict:
    """Mean and 95th percentile (nearest rank from below) of a tensor."""
    t = t.flatten().double()
    return {"mean": float(t.mean()), "p95": float(t.sort().values[int(0.95 * (t.numel() - 1))])}


def reference_mass_control(q, k, v, scale: float, lse_dense, mask, bq: int, bk: int):
    """MALA's forward support against the matched-work reference-mass control.

    q [B,Hq,N,d], k, v [B,Hkv,N,d] (causal, N_q = N_k); lse_dense [B,Hq,N]: z
    of the tau = 0 operator; mask [B,Hq,Tr,Tc] int8: the forward tile mask
    (1 kept) on the bq x bk partition. For every (batch, head) the unscreened
    probabilities P = exp(s - z) are formed in fp32, summed per row and key
    tile, and per decision block; the control keeps, in each decision block,
    the same number of key tiles as MALA, those of largest block mass (ties
    broken toward the lower tile index).

    Returns dict with ``control_support`` (bool [B,Hq,Tr,Tc]) and, per
    support (``mala``, ``control``), ``omitted_mass`` (fp64 [B,Hq,N]: the
    unscreened mass outside the support's kept tiles) and ``o_rel_l2`` (fp64
    [B,Hq,N]: relative L2 error of softmax attention restricted to the
    support against unscreened attention)."""
    B, HQ, N, _ = q.shape
    G = HQ // k.shape[1]
    Tr, Tc = mask.shape[2], mask.shape[3]
    dev = q.device
    causal = torch.ones(N, N, dtype=torch.bool, device=dev).tril()
    control = torch.zeros(mask.shape, dtype=torch.bool, device=dev)
    om = {n: torch.zeros((B, HQ, N), dtype=torch.float64, device=dev) for n in ("mala", "control")}
    rl2 = {n: torch.zeros((B, HQ, N), dtype=torch.float64, device=dev) for n in ("mala", "control")}
    pad_k = Tc * bk - N
    pad_q = Tr * bq - N
    for b in range(B):
        for h in range(HQ):
            kh, vh = k[b, h // G].float(), v[b, h // G].float()
            p = torch.exp((q[b, h].float() @ kh.T) * scale - lse_dense[b, h, :, None].float())
            p = p.masked_fill(~causal, 0.0)                            # unscreened P
            o_ref = p @ vh
            o_ref = o_ref / p.sum(-1, keepdim=True)
            pt = torch.nn.functional.pad(p, (0, pad_k)).view(N, Tc, bk).sum(-1)   # [N, Tc]
            blk = torch.nn.functional.pad(pt, (0, 0, 0, pad_q)).view(Tr, bq, Tc).sum(1)
            keep = mask[b, h] == 1
            cnt = keep.sum(-1)
            order = torch.argsort(blk, dim=-1, descending=True, stable=True)
            rank = torch.empty_like(order)
            rank.scatter_(1, order, torch.arange(Tc, device=dev).expand(Tr, Tc).contiguous())
            ctrl = rank < cnt[:, None]
            control[b, h] = ctrl
            for name, sup in (("mala", keep), ("control", ctrl)):
                rows = sup.repeat_interleave(bq, 0)[:N]                     # [N, Tc]
                om[name][b, h] = 1.0 - (pt.double() * rows).sum(-1) / p.double().sum(-1)
                pk = p * rows.repeat_interleave(bk, 1)[:, :N]
                o = (pk @ vh) / pk.sum(-1, keepdim=True)
                rl2[name][b, h] = ((o - o_ref).norm(dim=-1)
                                   / o_ref.norm(dim=-1).clamp_min(1e-30)).double()
    return {"control_support": control,
            "mala": {"omitted_mass": om["mala"], "o_rel_l2": rl2["mala"]},
            "control": {"omitted_mass": om["control"], "o_rel_l2": rl2["control"]}}
