"""Shared helpers of the GPU parity tests: run the library, run the oracle on
the exact same (rounded) inputs, and compare decisions and values."""
from __future__ import annotations

import numpy as np
import torch

from oracle import mala_oracle as O

# Near-tie band of a decision margin (nats): decisions this close to the
# threshold may go either way between an fp64 and an fp32 evaluation.
BAND = {"f32": 1e-4, "bf16": 1e-3}
# Value tolerances, stated for unit-scale tensors: fp32 inputs max error 1e-5
# against the oracle; bf16 inputs max error 2e-2 and relative Frobenius error
# 1e-2. The max error is taken relative to the tensor's scale,
# max|got - ref| <= tol * max(1, max|ref|): a gradient entry is a sum of
# terms of the tensor's magnitude, and bf16 (fp32) operands round each term by
# up to 2^-9 (2^-24) of it, so an entry of size 1 inside a tensor of size 14
# cannot be within 2e-2 absolute in any bf16-operand implementation. The
# strict element-wise absolute error is reported next to it.
TOL_F32 = 1e-5
TOL_BF16_ABS = 2e-2
TOL_BF16_FRO = 1e-2


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def dtype_name(t: torch.Tensor) -> str:
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def tiling():
    from contribution_gated_sparse_amd import mala_get_tiling
    return mala_get_tiling(0), mala_get_tiling(1), mala_get_tiling(2)


STATS = []


def compare_values(name, got, ref, kind, rows=None):
    """Return (max_abs, rel_fro) and assert the tolerance of ``kind``."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    diff = np.abs(got - ref)
    mx = float(diff.max()) if diff.size else 0.0
    rmax = float(np.abs(ref).max()) if ref.size else 0.0
    den = float(np.linalg.norm(ref.ravel()))
    fro = float(np.linalg.norm((got - ref).ravel()) / den) if den > 0 else mx
    scaled = mx / max(1.0, rmax)
    msg = (f"{name}: max abs {mx:.3e}, max|ref| {rmax:.3e}, max abs / max(1, max|ref|) "
           f"{scaled:.3e}, rel fro {fro:.3e}")
    STATS.append(msg)
    print(msg)
    if kind == "f32":
        assert scaled <= TOL_F32, msg
    else:
        assert scaled <= TOL_BF16_ABS, msg
        assert fro <= TOL_BF16_FRO, msg
    return mx, fro


def check_forward(x, tau, causal=True, blocks=None, max_ties=None):
    """Run mala_fwd on x = dict(q, k, v, scale) and the oracle on the same
    values. Returns (gpu, oracle, stats). ``blocks`` samples (b, h, i) query
    blocks of B_q rows for the oracle (all blocks if None)."""
    from contribution_gated_sparse_amd import mala_fwd
    q, k, v = x["q"], x["k"], x["v"]
    kind = dtype_name(q)
    (bq, bk, _), _, _ = tiling()
    g = mala_fwd(q, k, v, tau, causal=causal, softmax_scale=x["scale"], want_mask=True)
    torch.cuda.synchronize()
    gmask = g["mask"].cpu().numpy()
    gkept = g["kept"].cpu().numpy()
    qn, kn, vn = np64(q), np64(k), np64(v)
    r = O.mala_fwd(qn, kn, vn, tau, x["scale"], causal, bq, bk, blocks=blocks,
                   replay=gmask, band=BAND[kind])
    done = r["done"]                                   # [B, H, Tr]
    # every decision of every checked block matches, near ties replayed
    om = r["mask"][done]
    gm = gmask[done]
    assert np.array_equal(om, gm), (
        f"forward decisions differ outside the near-tie band: "
        f"{int((om != gm).sum())} of {om.size}")
    kept_o = (r["mask"] == O.KEPT).sum(-1)[done]
    assert np.array_equal(kept_o, gkept[done]), "kept-tile counters differ"
    rows = np.repeat(done, bq, axis=-1)[..., : q.shape[2]]
    go, gl = np64(g["o"]), np64(g["lse"])
    e_o = compare_values("O", go, r["o"], kind, rows)
    d_l = float(np.abs(gl[rows] - r["lse"][rows]).max()) if rows.any() else 0.0
    assert d_l <= (1e-5 if kind == "f32" else 2e-3), f"LSE error {d_l:.3e}"
    if max_ties is not None:
        assert r["near_ties"] <= max_ties, f"{r['near_ties']} near-tie decisions"
    visited = om != O.NOT_VISITED
    stats = dict(o_max_abs=e_o[0], o_rel_fro=e_o[1], lse_max_abs=d_l, near_ties=r["near_ties"],
                 kept_frac=float((om == O.KEPT).sum() / max(1, visited.sum())))
    return g, r, stats


def check_nesting(fmask, bmask):
    """Backward-kept tiles lie inside forward-kept tiles (Sec. 2.2): the
    backward partition refines the forward one."""
    (fbq, fbk, _), (bbq, bbk, _), _ = tiling()
    assert fbq % bbq == 0 and fbk % bbk == 0
    rq, rk = fbq // bbq, fbk // bbk
    tr, tc = bmask.shape[2], bmask.shape[3]
    up = np.repeat(np.repeat(fmask, rq, axis=2), rk, axis=3)[:, :, :tr, :tc]
    bad = (bmask == O.KEPT) & (up != O.KEPT)
    assert not bad.any(), f"{int(bad.sum())} backward-kept tiles outside the forward support"
