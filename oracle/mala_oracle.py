"""CPU fp64 oracle of MassAlloc Attention (MALA): test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module. It shares no code with the GPU library: it is a plain,
slow, obviously correct restatement of the operator defined in
"MassAlloc Attention: Let Attention Allocate Its Own Compute" (arXiv
2609.32712), written with numpy in float64.

Notation follows the paper. One query head and its key/value head are
processed at a time; the softmax scale is folded into the scores
(s_qk = scale * <q_q, k_k>); logarithms are natural (Sec. 2.1).

Readings where the paper leaves a step open (each is listed with the
tolerance rules in the design notes of this repository):

* the tile partition (B_q, B_k) is a parameter; queries and keys are both
  tiled from position 0; forward and backward use the same partition;
* causal legality is bottom-right aligned: key k is visible to query row q
  iff k <= q + (N_k - N_q), so L_q = q + (N_k - N_q) + 1 (L_q = N_k when not
  causal); this gives L_q = q + 1 for equal lengths and L_0 = N_k for a
  single decode row (Sec. 2.1);
* tau = 0 makes log(tau / L_q) = -inf, so nothing is skipped (Sec. 2.3);
* a decision whose margin lies within a near-tie band (a decision that sits
  on the threshold within rounding) may be replayed from another
  implementation's choice, in the forward (whose rule is path dependent, so
  later decisions stay comparable) and in the backward; every other decision
  is the oracle's own;
* split-KV decode: chunks aligned to absolute position 0, tiles aligned to
  the chunk start, newest tile first inside each chunk, one decision per
  query head (Sec. 2.4 and App. A.1, "Fused decoding execution").

Every function is pinned by tests against something other than itself: the
tau = 0 limit against torch's fp64 scaled-dot-product attention and autograd,
per-key brute force of Eq. 2/3 in ratio form (for the forward and for the
split decode, whose splits gate against their own partial normalizers with
L = N_k), Proposition 1, the per-key bound of its proof and Eqs. 9-10,
support nesting, and a closed form for constant scores.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

NEG_INF = -np.inf

# Decisions recorded in masks.
SKIPPED = 0
KEPT = 1
NOT_VISITED = -1


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def visible_counts(nq: int, nk: int, causal: bool) -> np.ndarray:
    """L_q for every query row (Sec. 2.1, definition of C_q and L_q)."""
    if not causal:
        return np.full(nq, float(nk))
    return np.arange(nq, dtype=np.float64) + (nk - nq) + 1.0


def row_threshold(tau: float, counts: np.ndarray) -> np.ndarray:
    """log(tau / L_q), the right-hand side of Eq. 3 and Eq. 4; -inf at tau=0."""
    if tau == 0.0:
        return np.full(counts.shape, NEG_INF)
    return math.log(tau) - np.log(counts)


def legal(rows: np.ndarray, nk: int, nq: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), nk]: is key k causally visible to query row q."""
    keys = np.arange(nk)
    if not causal:
        return np.ones((rows.size, nk), dtype=bool)
    return keys[None, :] <= (rows[:, None] + (nk - nq))


def scores(qrows: np.ndarray, k: np.ndarray, scale: float, ok: np.ndarray) -> np.ndarray:
    """S = scale * Q K^T with illegal entries set to -inf (Sec. 2.2)."""
    s = scale * (qrows @ k.T)
    return np.where(ok, s, NEG_INF)


def _logsumexp_rows(x: np.ndarray) -> np.ndarray:
    """log sum exp along the last axis; -inf for an all -inf row."""
    m = np.max(x, axis=-1)
    mf = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        out = np.log(np.sum(np.exp(x - mf[..., None]), axis=-1)) + mf
    return np.where(np.isfinite(m), out, NEG_INF)


def _tile_stats(s: np.ndarray, bk: int):
    """Per-row max and log-sum-exp of every key tile of a score strip."""
    nr, nk = s.shape
    tc = -(-nk // bk)
    pad = tc * bk - nk
    if pad:
        s = np.concatenate([s, np.full((nr, pad), NEG_INF)], axis=1)
    st = s.reshape(nr, tc, bk)
    return np.max(st, axis=2), _logsumexp_rows(st)


# --------------------------------------------------------------------------
# Dense reference (the tau -> 0 limit, Sec. 2.3)
# --------------------------------------------------------------------------

def dense_fwd(q, k, v, scale: float, causal: bool = True):
    """Plain causal softmax attention. q: [B,Hq,Nq,d], k,v: [B,Hkv,Nk,d].
    Returns O [B,Hq,Nq,d] and z = log sum_k exp(s_qk) [B,Hq,Nq]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    b_, hq, nq, _ = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    g = hq // hkv
    o = np.zeros(q.shape[:3] + (v.shape[3],))
    z = np.zeros((b_, hq, nq))
    ok = legal(np.arange(nq), nk, nq, causal)
    for b in range(b_):
        for h in range(hq):
            s = scores(q[b, h], k[b, h // g], scale, ok)
            zz = _logsumexp_rows(s)
            p = np.exp(s - zz[:, None])
            o[b, h] = p @ v[b, h // g]
            z[b, h] = zz
    return o, z


# --------------------------------------------------------------------------
# Forward: online allocation (Sec. 2.2 "Online Sparse Softmax", Eq. 1-3,
# Algorithm 1, App. A.1 "Fused forward execution")
# --------------------------------------------------------------------------

def fwd_block(s: np.ndarray, c: np.ndarray, bk: int, valid_rows: np.ndarray,
              replay: Optional[np.ndarray] = None, band: float = 0.0):
    """Decisions for one query block.

    s: [B_q, N_k] scores of the block (illegal entries -inf), c: [B_q] row
    thresholds log(tau/L_q), valid_rows: [B_q] bool (rows < N_q).
    Returns (decision[T_c], margin[T_c], Lambda[B_q], kept_cols bool[N_k],
    near_ties). margin = min over constraining rows of c_r - (t_r - Lambda_r):
    the tile is skipped iff margin > 0 (Eq. 3 with m + log l = log Z, Eq. 1).
    """
    nr, nk = s.shape
    tc = -(-nk // bk)
    tmax, tlse = _tile_stats(s, bk)
    dec = np.full(tc, NOT_VISITED, dtype=np.int8)
    marg = np.full(tc, np.nan)
    lam = np.full(nr, NEG_INF)        # log Z_q^(t) of the running retained set
    kept_cols = np.zeros(nk, dtype=bool)
    ties = 0
    has = np.isfinite(tmax) & valid_rows[:, None]
    tiles_with_legal = np.nonzero(has.any(axis=0))[0]
    if tiles_with_legal.size == 0:
        return dec, marg, lam, kept_cols, ties
    top = int(tiles_with_legal.max())
    for j in range(top, -1, -1):          # diagonal first, then earlier keys
        rows = has[:, j]
        if not rows.any():
            continue                      # no row is constrained: not a legal tile
        with np.errstate(invalid="ignore"):
            ratio_log = tmax[rows, j] - lam[rows]      # log r_qj (Eq. 2); +inf if Z=0
        terms = c[rows] - ratio_log
        mu = float(np.min(terms))
        skip = mu > 0.0
        if replay is not None and abs(mu) < band:
            ties += 1
            skip = replay[j] == SKIPPED
        marg[j] = mu
        if skip:
            dec[j] = SKIPPED              # m, l and O unchanged
            continue
        dec[j] = KEPT
        lam[rows] = np.logaddexp(lam[rows], tlse[rows, j])
        kept_cols[j * bk:(j + 1) * bk] = True
    return dec, marg, lam, kept_cols, ties


def mala_fwd(q, k, v, tau: float, scale: float, causal: bool = True,
             bq: int = 64, bk: int = 64, blocks: Optional[Iterable] = None,
             replay: Optional[np.ndarray] = None, band: float = 0.0):
    """MALA forward. q: [B,Hq,Nq,d]; k, v: [B,Hkv,Nk,d] (GQA: head h reads KV
    head h // (Hq/Hkv)).

    Returns dict with o [B,Hq,Nq,d], lse [B,Hq,Nq] (z_q = log Z_{R,q}),
    mask [B,Hq,T_r,T_c] (KEPT/SKIPPED/NOT_VISITED), margin [B,Hq,T_r,T_c],
    near_ties (count of replayed near-tie decisions), done (bool [B,Hq,T_r]).
    ``blocks`` restricts the work to an iterable of (b, h, i) query blocks;
    other rows are left as NaN. ``replay`` is a mask of the same shape whose
    choice is adopted where |margin| < band.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    b_, hq, nq, _ = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    g = hq // hkv
    tr, tc = -(-nq // bq), -(-nk // bk)
    o = np.full(q.shape[:3] + (v.shape[3],), np.nan)
    lse = np.full((b_, hq, nq), np.nan)
    mask = np.full((b_, hq, tr, tc), NOT_VISITED, dtype=np.int8)
    margin = np.full((b_, hq, tr, tc), np.nan)
    done = np.zeros((b_, hq, tr), dtype=bool)
    counts = visible_counts(nq, nk, causal)
    cthr = row_threshold(tau, counts)
    if blocks is None:
        blocks = [(b, h, i) for b in range(b_) for h in range(hq) for i in range(tr)]
    ties = 0
    for (b, h, i) in blocks:
        r0, r1 = i * bq, min((i + 1) * bq, nq)
        rows = np.arange(r0, r1)
        ok = legal(rows, nk, nq, causal)
        s = scores(q[b, h, r0:r1], k[b, h // g], scale, ok)
        # pad the block to B_q rows; padding rows are invalid
        nr = r1 - r0
        sp = np.full((bq, nk), NEG_INF)
        sp[:nr] = s
        cp = np.zeros(bq)
        cp[:nr] = cthr[r0:r1]
        valid = np.arange(bq) < nr
        rp = replay[b, h, i] if replay is not None else None
        dec, marg, lam, kept_cols, t = fwd_block(sp, cp, bk, valid, rp, band)
        ties += t
        mask[b, h, i] = dec
        margin[b, h, i] = marg
        z = lam[:nr]
        keep = ok & kept_cols[None, :]
        p = np.where(keep, np.exp(s - z[:, None]), 0.0)   # softmax over R_q (Sec. 2.2)
        o[b, h, r0:r1] = p @ v[b, h // g]
        lse[b, h, r0:r1] = z
        done[b, h, i] = True
    return dict(o=o, lse=lse, mask=mask, margin=margin, near_ties=ties, done=done)


# --------------------------------------------------------------------------
# Backward: offline allocation on the final normalizer (Sec. 2.2 "Offline
# Sparse Probability", Eq. 4, Algorithm 2, App. A.1 "Fused backward")
# --------------------------------------------------------------------------

def round_storage(x, dtype: Optional[str]) -> np.ndarray:
    """Value of x once stored in a tensor of ``dtype`` ("f32", "bf16", or
    None for no rounding): round to nearest even at each narrowing."""
    x = _f64(x)
    if dtype is None:
        return x
    f = x.astype(np.float32)
    if dtype == "f32":
        return f.astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def mala_bwd(q, k, v, o, lse, do, tau: float, scale: float, causal: bool = True,
             bq: int = 64, bk: int = 64, qblocks: Optional[Iterable] = None,
             replay: Optional[np.ndarray] = None, band: float = 0.0,
             o_storage: Optional[str] = None, lse_storage: Optional[str] = None):
    """MALA backward on the saved z = lse.

    Returns dict with dq [B,Hq,Nq,d], dk, dv [B,Hkv,Nk,d] (summed over the
    query heads of each KV head), mask [B,Hq,T_r,T_c] and margin (skip iff
    margin > 0, margin = -max over legal entries of s - z_q - log(tau/L_q)).
    ``qblocks`` restricts the query blocks processed (an iterable of i); then
    dq is exact on those rows, dk/dv hold only their contributions.
    ``replay`` (a mask of the same shape) is adopted where |margin| < band:
    such a decision sits on the threshold within rounding (App. B, last
    paragraph), and the gradients then follow the replayed support.
    ``o_storage``: Algorithm 2 forms rowsum(O o dO) from the output the forward
    stored; when that output is kept in a narrower dtype ("bf16", "f32"),
    D is computed from o rounded to it.
    ``lse_storage``: likewise, Algorithm 2 reads the log-normalizer the forward
    saved; when it is stored in a narrower dtype ("f32"), the gate and P use
    lse rounded to it.
    """
    q, k, v, o, lse, do = map(_f64, (q, k, v, o, lse, do))
    lse = round_storage(lse, lse_storage)
    b_, hq, nq, _ = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    g = hq // hkv
    tr, tc = -(-nq // bq), -(-nk // bk)
    dq = np.zeros_like(q)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    mask = np.full((b_, hq, tr, tc), NOT_VISITED, dtype=np.int8)
    margin = np.full((b_, hq, tr, tc), np.nan)
    counts = visible_counts(nq, nk, causal)
    cthr = row_threshold(tau, counts)
    dvec = np.sum(round_storage(o, o_storage) * do, axis=-1)   # rowsum(O o dO), Algorithm 2
    ilist = list(range(tr)) if qblocks is None else list(qblocks)
    for b in range(b_):
        for h in range(hq):
            kh = h // g
            for i in ilist:
                r0, r1 = i * bq, min((i + 1) * bq, nq)
                rows = np.arange(r0, r1)
                ok = legal(rows, nk, nq, causal)
                s = scores(q[b, h, r0:r1], k[b, kh], scale, ok)
                z = lse[b, h, r0:r1]
                with np.errstate(invalid="ignore"):
                    x = s - z[:, None] - cthr[r0:r1, None]   # Eq. 4, left minus right
                x = np.where(ok, x, NEG_INF)
                tmx, _ = _tile_stats(x, bk)
                tmax = np.max(tmx, axis=0)                    # per key tile
                keep_cols = np.zeros(nk, dtype=bool)
                for j in range(tc):
                    if not np.isfinite(tmax[j]) and tmax[j] < 0:
                        continue                              # no legal entry
                    margin[b, h, i, j] = -tmax[j]
                    skip = tmax[j] < 0.0                      # all entries below: skip
                    if replay is not None and abs(tmax[j]) < band:
                        skip = replay[b, h, i, j] == SKIPPED
                    if skip:
                        mask[b, h, i, j] = SKIPPED
                    else:
                        mask[b, h, i, j] = KEPT
                        keep_cols[j * bk:(j + 1) * bk] = True
                keep = ok & keep_cols[None, :]
                p = np.where(keep, np.exp(s - z[:, None]), 0.0)
                dp = do[b, h, r0:r1] @ v[b, kh].T
                ds = p * (dp - dvec[b, h, r0:r1, None])
                dq[b, h, r0:r1] = scale * (ds @ k[b, kh])
                dk[b, kh] += scale * (ds.T @ q[b, h, r0:r1])
                dv[b, kh] += p.T @ do[b, h, r0:r1]
    return dict(dq=dq, dk=dk, dv=dv, mask=mask, margin=margin)


def dense_bwd(q, k, v, do, scale: float, causal: bool = True):
    """Gradients of dense causal attention (the tau = 0 limit)."""
    o, z = dense_fwd(q, k, v, scale, causal)
    r = mala_bwd(q, k, v, o, z, do, 0.0, scale, causal, bq=q.shape[2] or 1,
                 bk=k.shape[2] or 1)
    return r["dq"], r["dk"], r["dv"]


# --------------------------------------------------------------------------
# Split-KV decode (Sec. 2.4, App. A.1 "Fused decoding execution")
# --------------------------------------------------------------------------

def mala_decode(q, k_cache, v_cache, seqlens, tau: float, scale: float,
                chunk: int = 256, bk: int = 64, replay: Optional[np.ndarray] = None,
                band: float = 0.0):
    """One decode step. q: [B,Hq,d] is the query at position N_k - 1 of each
    sequence; k_cache, v_cache: [B,Hkv,cap,d]; seqlens: [B] = N_k (the current
    token included). Each chunk of ``chunk`` keys starts with an empty state
    and applies the forward rule with L = N_k; chunks merge by the standard
    normalizer-aware reduction.

    Returns dict with o [B,Hq,d], lse [B,Hq], mask [B,Hq,n_chunks,chunk//bk],
    margin (same shape), v_tiles (bool [B,Hkv,n_chunks,chunk//bk]: some head
    of the group kept the tile, so its V is read), near_ties.
    """
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    b_, hq, _ = q.shape
    hkv, cap = kc.shape[1], kc.shape[2]
    g = hq // hkv
    seqlens = [int(x) for x in seqlens]
    nch = -(-max(seqlens + [1]) // chunk)
    tpc = chunk // bk
    o = np.zeros((b_, hq, vc.shape[3]))
    lse = np.zeros((b_, hq))
    mask = np.full((b_, hq, nch, tpc), NOT_VISITED, dtype=np.int8)
    margin = np.full((b_, hq, nch, tpc), np.nan)
    vt = np.zeros((b_, hkv, nch, tpc), dtype=bool)
    ties = 0
    for b in range(b_):
        n = seqlens[b]
        c = row_threshold(tau, np.array([float(n)]))
        for h in range(hq):
            kh = h // g
            s = scale * (kc[b, kh, :n] @ q[b, h])       # all N_k keys are visible
            kept = np.zeros(n, dtype=bool)
            lam_chunks = []
            for ci in range(-(-n // chunk)):
                c0, c1 = ci * chunk, min((ci + 1) * chunk, n)
                sp = np.full((1, c1 - c0), NEG_INF)
                sp[0] = s[c0:c1]
                rp = replay[b, h, ci] if replay is not None else None
                dec, marg, lam, kc_cols, t = fwd_block(sp, c, bk, np.array([True]), rp, band)
                ties += t
                ntile = dec.size
                mask[b, h, ci, :ntile] = dec
                margin[b, h, ci, :ntile] = marg
                vt[b, kh, ci, :ntile] |= dec == KEPT
                kept[c0:c1] = kc_cols
                lam_chunks.append(lam[0])
            z = _logsumexp_rows(np.array(lam_chunks)[None, :])[0]
            p = np.where(kept, np.exp(s - z), 0.0)
            o[b, h] = p @ vc[b, kh, :n]
            lse[b, h] = z
    return dict(o=o, lse=lse, mask=mask, margin=margin, v_tiles=vt, near_ties=ties)


# --------------------------------------------------------------------------
# Fidelity measure (App. C.2)
# --------------------------------------------------------------------------

def omitted_mass(lse_screened, lse_reference):
    """1 - exp(z_screened - z_reference) (App. C.2)."""
    return 1.0 - np.exp(_f64(lse_screened) - _f64(lse_reference))
