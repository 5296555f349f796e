"""CPU pins of the derived rounding bound that the GPU parity tests apply to
large gradient entries (parity_util.grad_rounding_bounds).

A backward that takes the oracle's decisions and fp64 values but rounds what
a bf16-operand kernel rounds (P to bf16 in dV^T = dO^T P; dS to bf16 in
dK^T = Q^T dS; dS as a bf16 hi + lo pair in dQ = dS K, or as one bf16 value
with the fast-gradient flag; D from a perturbed stored O; each output to
bf16) must stay inside the bound on every element, and come close to it
somewhere: a bound far above every error would pass a wrong kernel.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import mala_oracle as O
from parity_util import (add_output_rounding, grad_rounding_bounds, o_rounding_dk_term,
                         o_rounding_dq_term, tiling)


def _bf(a):
    """Round to bf16 (round to nearest even), back to fp64."""
    return torch.from_numpy(np.ascontiguousarray(a)).float().to(torch.bfloat16).double().numpy()


def _emulated_backward(q, k, v, do, scale, fwd, bmask, o_lib, split_dq):
    b_, hq, n, d = q.shape
    g = hq // k.shape[1]
    _, (bbq, bbk, _), _ = tiling()
    keys = np.arange(n)
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(b_):
        for h in range(hq):
            kh = h // g
            s = scale * q[b, h] @ k[b, kh].T
            legal = keys[None, :] <= keys[:, None]
            z32 = fwd["lse"][b, h].astype(np.float32).astype(np.float64)
            kept = bmask[b, h][keys // bbq][:, keys // bbk] == O.KEPT
            p = np.where(legal & kept, np.exp(s - z32[:, None]), 0.0)
            dd = (o_lib[b, h] * do[b, h]).sum(-1)
            ds = p * (do[b, h] @ v[b, kh].T - dd[:, None])
            dv[b, kh] += _bf(p).T @ do[b, h]
            dk[b, kh] += scale * _bf(ds).T @ q[b, h]
            hi = _bf(ds)
            dsq = hi + _bf(ds - hi) if split_dq else hi
            dq[b, h] = scale * dsq @ k[b, kh]
    return {"dq": _bf(dq), "dk": _bf(dk), "dv": _bf(dv)}


@pytest.mark.parametrize("tau", [1e-4, 1.0])
@pytest.mark.parametrize("split_dq", [True, False])
def test_bound_holds_and_is_tight_for_an_emulated_bf16_backward(tau, split_dq):
    x = W.make_structured(400, hq=2, hkv=1, d=128)
    q, k, v, do = (x[n].float().numpy().astype(np.float64) for n in ("q", "k", "v", "do"))
    sc = x["scale"]
    (fbq, fbk, _), (bbq, bbk, _), _ = tiling()
    fwd = O.mala_fwd(q, k, v, tau, sc, True, fbq, fbk)
    ref = O.mala_bwd(q, k, v, fwd["o"], fwd["lse"], do, tau, sc, True, bbq, bbk,
                     o_storage="bf16", lse_storage="f32")
    # the library's stored O: the oracle's, moved by up to u of itself (the
    # P V product's bf16 P), then rounded to bf16
    rng = np.random.default_rng(20260101)
    o_lib = _bf(fwd["o"] * (1 + 2 ** -8 * (2 * rng.random(fwd["o"].shape) - 1)))
    got = _emulated_backward(q, k, v, do, sc, fwd, ref["mask"], o_lib, split_dq)
    bound = add_output_rounding(
        grad_rounding_bounds(q, k, v, do, sc, True, fwd, ref["mask"], "bf16", split_dq=split_dq,
                             lse_gpu=fwd["lse"].astype(np.float32), o_gpu=o_lib), ref, "bf16")
    for n in ("dq", "dk", "dv"):
        err = np.abs(got[n] - ref[n])
        ratio = err / np.maximum(bound[n], 1e-300)
        assert (err <= bound[n] * (1 + 1e-9) + 1e-300).all(), (n, float(ratio.max()))
        # tight where the rounding terms dominate: some element comes within
        # a factor of two of its bound
        assert ratio.max() >= 0.5, (n, float(ratio.max()))


@pytest.mark.parametrize("case", ["structured", "sinks", "one_row"])
def test_o_rounding_terms_bound_dq_and_dk(case):
    """The bf16-O rounding terms (o_rounding_dq_term, o_rounding_dk_term)
    bound how far dQ and dK move when the stored O moves by up to its bf16
    rounding: the oracle's backward on the same decisions and z, with O moved
    by one bf16 unit in the direction that moves D = rowsum(O o dO) most, moves
    dQ and dK within the terms on every element, and reaches a fifth of them
    somewhere (the terms allow 4u, two units per side)."""
    (fbq, fbk, _), (bbq, bbk, _), _ = tiling()
    if case == "one_row":
        # one query row, non-causal, tau = 100: dQ and dK near zero
        x = W.make_prefill(W.CONFIGS[2], n=411, hq=2, hkv=2, d=128, planted=4, seed=192)
        x["q"], x["do"] = x["q"][:, :, -1:], x["do"][:, :, -1:]
        causal, tau = False, 100.0
    else:
        kw = {"sink_logit": 30.0} if case == "sinks" else {}
        x = W.make_structured(300, hq=2, hkv=1, d=128, **kw)
        causal, tau = True, 1.0
    q, k, v, do = (x[n].float().numpy().astype(np.float64) for n in ("q", "k", "v", "do"))
    sc = x["scale"]
    fwd = O.mala_fwd(q, k, v, tau, sc, causal, fbq, fbk)
    ref = O.mala_bwd(q, k, v, fwd["o"], fwd["lse"], do, tau, sc, causal, bbq, bbk,
                     o_storage="bf16", lse_storage="f32")
    o_ref = _bf(fwd["o"])
    o_moved = o_ref + 2.0 ** -8 * np.abs(o_ref) * np.sign(do)
    got = O.mala_bwd(q, k, v, o_moved, fwd["lse"], do, tau, sc, causal, bbq, bbk,
                     lse_storage="f32", replay=ref["mask"], band=np.inf)
    assert np.array_equal(got["mask"], ref["mask"])
    terms = {"dq": o_rounding_dq_term(q, k, v, do, sc, causal, fwd, ref),
             "dk": o_rounding_dk_term(q, k, v, do, sc, causal, fwd, ref)}
    for n, t in terms.items():
        err = np.abs(got[n] - ref[n])
        assert (err <= t * (1 + 1e-9) + 1e-300).all(), n
        assert float((err / np.maximum(t, 1e-300)).max()) >= 0.2, n

