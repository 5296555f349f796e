"""Pins of the CPU oracle against what the paper and mathematics fix.

Nothing here touches the GPU library. Each pin is an independent check:
a library routine (torch fp64 SDPA + autograd) at tau = 0, brute force of the
per-key definitions (Eq. 2-4 in ratio form, scalar Python loops), the
forward guarantees of Appendix B (Prop. 1, Eq. 9, Eq. 10), support nesting
(Sec. 2.2), first-tile retention (Sec. 2.2, App. A.1), and a closed form for
constant scores derived from Eq. 3.
"""
import math

import numpy as np
import pytest
import torch

from oracle import mala_oracle as O


def rand_problem(seed, b=1, hq=2, hkv=1, nq=16, nk=None, d=4, qstd=1.5):
    rng = np.random.default_rng(seed)
    nk = nq if nk is None else nk
    q = rng.standard_normal((b, hq, nq, d)) * qstd
    k = rng.standard_normal((b, hkv, nk, d))
    v = rng.standard_normal((b, hkv, nk, d))
    do = rng.standard_normal((b, hq, nq, d))
    return q, k, v, do


# ---------------------------------------------------------------- tau = 0

@pytest.mark.parametrize("shape", [(2, 4, 2, 37, 16), (1, 3, 3, 64, 8), (1, 2, 1, 5, 4)])
@pytest.mark.parametrize("blk", [(8, 8), (4, 16), (64, 64)])
def test_tau0_forward_matches_torch_sdpa(shape, blk):
    b, hq, hkv, n, d = shape
    q, k, v, _ = rand_problem(1, b, hq, hkv, n, d=d)
    scale = 1.0 / math.sqrt(d)
    r = O.mala_fwd(q, k, v, 0.0, scale, True, *blk)
    g = hq // hkv
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(k).repeat_interleave(g, dim=1)
    tv = torch.from_numpy(v).repeat_interleave(g, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    np.testing.assert_allclose(r["o"], ref.numpy(), atol=1e-12, rtol=0)
    s = (tq @ tk.transpose(-1, -2)) * scale
    s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(r["lse"], torch.logsumexp(s, -1).numpy(), atol=1e-12, rtol=0)
    assert (r["mask"] != O.SKIPPED).all()


@pytest.mark.parametrize("shape", [(1, 4, 2, 37, 16), (2, 2, 2, 20, 8)])
def test_tau0_backward_matches_torch_autograd(shape):
    b, hq, hkv, n, d = shape
    q, k, v, do = rand_problem(2, b, hq, hkv, n, d=d)
    scale = 1.0 / math.sqrt(d)
    f = O.mala_fwd(q, k, v, 0.0, scale, True, 8, 8)
    r = O.mala_bwd(q, k, v, f["o"], f["lse"], do, 0.0, scale, True, 8, 8)
    g = hq // hkv
    tq = torch.from_numpy(q).requires_grad_()
    tk = torch.from_numpy(k).requires_grad_()
    tv = torch.from_numpy(v).requires_grad_()
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(g, 1), tv.repeat_interleave(g, 1), is_causal=True, scale=scale)
    out.backward(torch.from_numpy(do))
    np.testing.assert_allclose(r["dq"], tq.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(r["dk"], tk.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(r["dv"], tv.grad.numpy(), atol=1e-11, rtol=0)


def test_dense_reference_matches_torch():
    q, k, v, do = rand_problem(3, 1, 2, 2, 24, d=8)
    o, z = O.dense_fwd(q, k, v, 0.3, True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True, scale=0.3)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)


def test_noncausal_tau0_matches_torch():
    q, k, v, _ = rand_problem(4, 1, 2, 2, 12, nk=30, d=8)
    r = O.mala_fwd(q, k, v, 0.0, 0.35, False, 4, 8)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=False, scale=0.35)
    np.testing.assert_allclose(r["o"], ref.numpy(), atol=1e-12)


# ---------------------------------------------------------------- brute force

def brute_forward(q, k, v, tau, scale, bq, bk, causal=True):
    """Scalar loops over Eq. 2 and Eq. 3 in ratio form: skip a tile iff every
    valid row with a legal key has exp(max s) / Z_t < tau / L_q."""
    b_, hq, nq, d = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    g = hq // hkv
    tr, tc = -(-nq // bq), -(-nk // bk)
    mask = np.full((b_, hq, tr, tc), -1, dtype=np.int8)
    o = np.zeros((b_, hq, nq, v.shape[3]))
    lse = np.zeros((b_, hq, nq))
    for b in range(b_):
        for h in range(hq):
            kh = h // g
            for i in range(tr):
                rows = list(range(i * bq, min(i * bq + bq, nq)))
                sc = {}
                for qq in rows:
                    for kk in range(nk):
                        if (not causal) or kk <= qq + nk - nq:
                            sc[(qq, kk)] = scale * sum(q[b, h, qq, e] * k[b, kh, kk, e] for e in range(d))
                Z = {qq: 0.0 for qq in rows}
                kept = {qq: [] for qq in rows}
                tiles = [j for j in range(tc) if any((qq, kk) in sc for qq in rows
                                                     for kk in range(j * bk, min(j * bk + bk, nk)))]
                for j in sorted(tiles, reverse=True):
                    skip = True
                    for qq in rows:
                        keys = [kk for kk in range(j * bk, min(j * bk + bk, nk)) if (qq, kk) in sc]
                        if not keys:
                            continue
                        L = (qq + nk - nq + 1) if causal else nk
                        if Z[qq] == 0.0:
                            skip = False
                            continue
                        ratio = math.exp(max(sc[(qq, kk)] for kk in keys)) / Z[qq]
                        if not ratio < tau / L:
                            skip = False
                    mask[b, h, i, j] = 0 if skip else 1
                    if not skip:
                        for qq in rows:
                            for kk in range(j * bk, min(j * bk + bk, nk)):
                                if (qq, kk) in sc:
                                    Z[qq] += math.exp(sc[(qq, kk)])
                                    kept[qq].append(kk)
                for qq in rows:
                    for kk in kept[qq]:
                        o[b, h, qq] += math.exp(sc[(qq, kk)]) / Z[qq] * v[b, kh, kk]
                    lse[b, h, qq] = math.log(Z[qq])
    return mask, o, lse


def brute_backward_mask(q, k, lse, tau, scale, bq, bk):
    """Eq. 4 in ratio form: skip iff exp(s) / Z_R < tau / L_q for every legal entry."""
    b_, hq, nq, d = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    g = hq // hkv
    tr, tc = -(-nq // bq), -(-nk // bk)
    mask = np.full((b_, hq, tr, tc), -1, dtype=np.int8)
    for b in range(b_):
        for h in range(hq):
            for i in range(tr):
                for j in range(tc):
                    any_legal, skip = False, True
                    for qq in range(i * bq, min(i * bq + bq, nq)):
                        for kk in range(j * bk, min(j * bk + bk, nk)):
                            if kk > qq + nk - nq:
                                continue
                            any_legal = True
                            s = scale * sum(q[b, h, qq, e] * k[b, h // g, kk, e] for e in range(d))
                            if not math.exp(s) / math.exp(lse[b, h, qq]) < tau / (qq + nk - nq + 1):
                                skip = False
                    if any_legal:
                        mask[b, h, i, j] = 0 if skip else 1
    return mask


TAUS = [0.0, 1e-3, 0.05, 0.3, 1.0, 3.0, 20.0, 1e3]


@pytest.mark.parametrize("blk", [1, 2, 4])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_forward_matches_bruteforce(blk, seed):
    q, k, v, _ = rand_problem(10 + seed, 1, 2, 1, 16, d=4, qstd=2.5)
    skipped = 0
    for tau in TAUS:
        r = O.mala_fwd(q, k, v, tau, 0.7, True, blk, blk)
        m, o, lse = brute_forward(q, k, v, tau, 0.7, blk, blk)
        np.testing.assert_array_equal(r["mask"], m)
        np.testing.assert_allclose(r["o"], o, atol=1e-12)
        np.testing.assert_allclose(r["lse"], lse, atol=1e-12)
        skipped += int((m == 0).sum())
    assert skipped > 0   # the sweep exercises the skip branch


@pytest.mark.parametrize("bq,bk,nq,nk", [(2, 4, 13, 13), (4, 2, 9, 15), (3, 3, 7, 7)])
def test_forward_bruteforce_rectangular_tiles(bq, bk, nq, nk):
    q, k, v, _ = rand_problem(20, 1, 2, 2, nq, nk=nk, d=4, qstd=2.5)
    for tau in [0.5, 4.0, 50.0]:
        r = O.mala_fwd(q, k, v, tau, 0.7, True, bq, bk)
        m, o, lse = brute_forward(q, k, v, tau, 0.7, bq, bk)
        np.testing.assert_array_equal(r["mask"], m)
        np.testing.assert_allclose(r["o"], o, atol=1e-12)
    r = O.mala_fwd(q, k, v, 4.0, 0.7, False, bq, bk)
    m, o, _ = brute_forward(q, k, v, 4.0, 0.7, bq, bk, causal=False)
    np.testing.assert_array_equal(r["mask"], m)
    np.testing.assert_allclose(r["o"], o, atol=1e-12)


@pytest.mark.parametrize("blk", [1, 2, 4])
def test_backward_mask_matches_bruteforce(blk):
    q, k, v, do = rand_problem(30, 1, 2, 1, 16, d=4, qstd=2.5)
    skipped = 0
    for tau in TAUS:
        f = O.mala_fwd(q, k, v, tau, 0.7, True, blk, blk)
        r = O.mala_bwd(q, k, v, f["o"], f["lse"], do, tau, 0.7, True, blk, blk)
        m = brute_backward_mask(q, k, f["lse"], tau, 0.7, blk, blk)
        # exact ties (tau = 1 on a row's only key) are decided by rounding:
        # compare every decision whose margin is clear of them
        clear = ~(np.abs(r["margin"]) < 1e-9)
        np.testing.assert_array_equal(r["mask"][clear], m[clear])
        skipped += int((m == 0).sum())
    assert skipped > 0


def test_backward_grads_bruteforce():
    """Gradients from the per-entry backward equations of Algorithm 2,
    written as scalar loops over kept entries."""
    q, k, v, do = rand_problem(31, 1, 2, 1, 10, d=3, qstd=2.5)
    tau, sc, blk = 2.0, 0.7, 2
    f = O.mala_fwd(q, k, v, tau, sc, True, blk, blk)
    r = O.mala_bwd(q, k, v, f["o"], f["lse"], do, tau, sc, True, blk, blk)
    _, hq, n, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(hq):
        for qq in range(n):
            D = sum(f["o"][0, h, qq, e] * do[0, h, qq, e] for e in range(d))
            for kk in range(qq + 1):
                if r["mask"][0, h, qq // blk, kk // blk] != 1:
                    continue
                s = sc * sum(q[0, h, qq, e] * k[0, 0, kk, e] for e in range(d))
                p = math.exp(s - f["lse"][0, h, qq])
                dp = sum(do[0, h, qq, e] * v[0, 0, kk, e] for e in range(d))
                ds = p * (dp - D)
                for e in range(d):
                    dv[0, 0, kk, e] += p * do[0, h, qq, e]
                    dk[0, 0, kk, e] += sc * ds * q[0, h, qq, e]
                    dq[0, h, qq, e] += sc * ds * k[0, 0, kk, e]
    assert (r["mask"] == 0).any() and (r["mask"] == 1).any()
    np.testing.assert_allclose(r["dq"], dq, atol=1e-12)
    np.testing.assert_allclose(r["dk"], dk, atol=1e-12)
    np.testing.assert_allclose(r["dv"], dv, atol=1e-12)


# ------------------------------------------------ Appendix B guarantees

@pytest.mark.parametrize("tau", [1e-3, 0.1, 1.0, 5.0, 100.0])
@pytest.mark.parametrize("blk", [1, 4, 8])
def test_prop1_and_eq9_eq10(tau, blk):
    q, k, v, _ = rand_problem(40, 2, 2, 2, 64, d=8, qstd=3.0)
    sc = 0.5
    r = O.mala_fwd(q, k, v, tau, sc, True, blk, blk)
    od, zd = O.dense_fwd(q, k, v, sc, True)
    eps = O.omitted_mass(r["lse"], zd)
    assert (eps <= tau / (1 + tau) + 1e-12).all()                    # Eq. 6
    n = q.shape[2]
    vmax = np.linalg.norm(v, axis=-1).max()
    for b in range(2):
        for h in range(2):
            s = sc * q[b, h] @ k[b, h].T
            ok = np.tril(np.ones((n, n), bool))
            s = np.where(ok, s, -np.inf)
            p = np.exp(s - zd[b, h][:, None])
            kept = np.zeros((n, n), bool)
            m = r["mask"][b, h]
            for i in range(m.shape[0]):
                for j in range(m.shape[1]):
                    if m[i, j] == 1:
                        kept[i * blk:(i + 1) * blk, j * blk:(j + 1) * blk] = True
            kept &= ok
            pt = np.where(kept, np.exp(s - r["lse"][b, h][:, None]), 0.0)
            L = np.arange(n) + 1.0
            omitted = ok & ~kept
            ratio = np.exp(s - r["lse"][b, h][:, None])
            assert (ratio[omitted] < np.broadcast_to(tau / L[:, None], (n, n))[omitted]).all()   # Eq. 7
            l1 = np.abs(p - pt).sum(-1)
            np.testing.assert_allclose(l1, 2 * eps[b, h], atol=1e-12)                        # Eq. 9
            dnorm = np.linalg.norm(od[b, h] - r["o"][b, h], axis=-1)
            assert (dnorm <= 2 * tau / (1 + tau) * vmax + 1e-12).all()                       # Eq. 10


@pytest.mark.parametrize("tau", [0.01, 0.5, 2.0, 30.0])
@pytest.mark.parametrize("blk", [2, 4, 16])
def test_nesting_and_first_tile(tau, blk):
    q, k, v, do = rand_problem(50, 1, 4, 2, 48, d=8, qstd=3.0)
    f = O.mala_fwd(q, k, v, tau, 0.5, True, blk, blk)
    r = O.mala_bwd(q, k, v, f["o"], f["lse"], do, tau, 0.5, True, blk, blk)
    # forward-skipped => backward-skipped (Sec. 2.2)
    assert not ((f["mask"] == O.SKIPPED) & (r["mask"] == O.KEPT)).any()
    # same visited set
    np.testing.assert_array_equal(f["mask"] != O.NOT_VISITED, r["mask"] != O.NOT_VISITED)
    # the diagonal tile is the first tested and always kept in forward
    tr = f["mask"].shape[2]
    for i in range(tr):
        assert (f["mask"][..., i, i] == O.KEPT).all()


# ------------------------------------------------ constant scores closed form

def closed_form_kept(tau, i, B):
    """Number of kept off-diagonal tiles of query block i when all scores are
    equal (derived from Eq. 3: with r tiles kept the binding row is the block's
    first when tau > 1, and the next tile is skipped iff tau(1 + rB) > iB + 1)."""
    if tau <= 1.0:
        return i
    r = 0
    while r < i and not tau * (1 + r * B) > i * B + 1:
        r += 1
    return r


@pytest.mark.parametrize("tau", [0.5, 2.0, 3.5, 7.25])
@pytest.mark.parametrize("B", [2, 4, 8])
def test_constant_scores_closed_form(tau, B):
    n, d = 8 * B, 4
    rng = np.random.default_rng(60)
    q = rng.standard_normal((1, 1, n, d))
    k = np.zeros((1, 1, n, d))
    v = rng.standard_normal((1, 1, n, d))
    do = rng.standard_normal((1, 1, n, d))
    for i in range(n // B):
        for r in range(i + 1):
            assert tau * (1 + r * B) != i * B + 1      # no exact ties
    f = O.mala_fwd(q, k, v, tau, 1.0, True, B, B)
    for i in range(n // B):
        rs = closed_form_kept(tau, i, B)
        expect = np.full(n // B, -1)
        expect[: i + 1] = 0
        expect[i - rs: i + 1] = 1
        np.testing.assert_array_equal(f["mask"][0, 0, i], expect)
        for a in range(B):
            row = i * B + a
            keys = np.arange((i - rs) * B, row + 1)
            np.testing.assert_allclose(f["o"][0, 0, row], v[0, 0, keys].mean(0), atol=1e-12)
            np.testing.assert_allclose(f["lse"][0, 0, row], math.log(keys.size), atol=1e-12)
    b = O.mala_bwd(q, k, v, f["o"], f["lse"], do, tau, 1.0, True, B, B)
    if tau > 1.0:      # every tile is skipped in backward: the diagonal is not forced
        assert not (b["mask"] == O.KEPT).any()
        assert np.abs(b["dq"]).max() == 0 and np.abs(b["dk"]).max() == 0 and np.abs(b["dv"]).max() == 0
    else:
        assert ((b["mask"] == O.KEPT) == (f["mask"] == O.KEPT)).all()


# ------------------------------------------------ decode

def test_decode_tau0_is_dense_last_row():
    rng = np.random.default_rng(70)
    b, hq, hkv, cap, d = 3, 4, 2, 700, 8
    q = rng.standard_normal((b, hq, d)) * 2
    kc = rng.standard_normal((b, hkv, cap, d))
    vc = rng.standard_normal((b, hkv, cap, d))
    lens = [700, 513, 64]
    r = O.mala_decode(q, kc, vc, lens, 0.0, 0.4, 256, 64)
    for bb in range(b):
        n = lens[bb]
        for h in range(hq):
            s = 0.4 * kc[bb, h // 2, :n] @ q[bb, h]
            p = np.exp(s - s.max())
            np.testing.assert_allclose(r["o"][bb, h], (p / p.sum()) @ vc[bb, h // 2, :n], atol=1e-12)
            np.testing.assert_allclose(r["lse"][bb, h], np.log(np.exp(s - s.max()).sum()) + s.max(), atol=1e-12)


@pytest.mark.parametrize("tau", [1e-3, 0.5, 4.0, 100.0])
def test_decode_single_chunk_equals_forward_rule(tau):
    """With one chunk covering the context, the split rule is the forward
    rule of a one-row query block at position N_k - 1 (L_0 = N_k)."""
    rng = np.random.default_rng(71)
    n, d, bk = 200, 8, 16
    q = rng.standard_normal((1, 1, n, d)) * 3
    k = rng.standard_normal((1, 1, n, d))
    v = rng.standard_normal((1, 1, n, d))
    f = O.mala_fwd(q[:, :, -1:], k, v, tau, 0.5, True, 1, bk)
    r = O.mala_decode(q[:, :, -1], k, v, [n], tau, 0.5, 256, bk)
    np.testing.assert_allclose(r["o"][0, 0], f["o"][0, 0, 0], atol=1e-12)
    np.testing.assert_allclose(r["lse"][0, 0], f["lse"][0, 0, 0], atol=1e-12)
    nt = -(-n // bk)
    np.testing.assert_array_equal(r["mask"][0, 0, 0, :nt], f["mask"][0, 0, 0, :nt])


@pytest.mark.parametrize("tau", [1e-4, 1.0, 50.0])
def test_decode_split_bound_and_first_tiles(tau):
    rng = np.random.default_rng(72)
    b, hq, cap, d = 2, 4, 1100, 8
    q = rng.standard_normal((b, hq, d)) * 3
    kc = rng.standard_normal((b, 1, cap, d))
    vc = rng.standard_normal((b, 1, cap, d))
    lens = [1100, 1025]
    r = O.mala_decode(q, kc, vc, lens, tau, 0.5, 256, 64)
    for bb in range(b):
        n = lens[bb]
        nch = -(-n // 256)
        # the newest tile of every chunk is tested first and kept (empty state)
        for ci in range(nch):
            tiles = -(-(min(n, 256 * ci + 256) - 256 * ci) // 64)
            assert (r["mask"][bb, :, ci, tiles - 1] == O.KEPT).all()
        # each chunk tests against its own partial normalizer, which is no
        # larger than the merged one, so every omitted key's ratio to the
        # merged normalizer is below tau / N_k (the step of Prop. 1's proof,
        # with L = N_k for the decode row), and the omitted mass obeys the
        # forward bound of Prop. 1
        for h in range(hq):
            s = 0.5 * kc[bb, 0, :n] @ q[bb, h]
            zd = np.log(np.exp(s - s.max()).sum()) + s.max()
            eps = 1 - np.exp(r["lse"][bb, h] - zd)
            assert eps <= tau / (1 + tau) + 1e-12
            omitted = ~decode_kept_keys(r["mask"][bb, h], n, 256, 64)
            assert omitted.any() or tau < 10.0
            assert (np.exp(s[omitted] - r["lse"][bb, h]) < tau / n).all()


def decode_kept_keys(mask_bh, n, chunk, bk):
    """Boolean [n]: key lies in a tile that its split kept."""
    kept = np.zeros(n, bool)
    for ci in range(mask_bh.shape[0]):
        for t in range(mask_bh.shape[1]):
            if mask_bh[ci, t] == O.KEPT:
                kept[ci * chunk + t * bk: min(n, ci * chunk + (t + 1) * bk)] = True
    return kept


def brute_decode(q, kc, vc, lens, tau, scale, chunk, bk):
    """Scalar loops over the split rule (Sec. 2.4, App. A.1 "Fused decoding
    execution") in ratio form. Every split of ``chunk`` keys starts with an
    empty normalizer Z = 0 and tests its tiles newest first; a tile is skipped
    iff Z > 0 and exp(max s) / Z < tau / N_k, where N_k counts the query's
    whole causal context (the decode row's L_0), not the split's keys; a kept
    tile adds exp(s) of its keys to the split's Z. The output is the softmax
    over the union of the splits' kept keys."""
    b_, hq, d = q.shape
    g = hq // kc.shape[1]
    nch = -(-max(lens) // chunk)
    mask = np.full((b_, hq, nch, chunk // bk), -1, dtype=np.int8)
    o = np.zeros((b_, hq, vc.shape[3]))
    lse = np.zeros((b_, hq))
    for b in range(b_):
        n = lens[b]
        for h in range(hq):
            kh = h // g
            s = [scale * sum(q[b, h, e] * kc[b, kh, kk, e] for e in range(d)) for kk in range(n)]
            kept = []
            for ci in range(-(-n // chunk)):
                c0, c1 = ci * chunk, min(ci * chunk + chunk, n)
                Z = 0.0
                for t in reversed(range(-(-(c1 - c0) // bk))):
                    keys = list(range(c0 + t * bk, min(c0 + (t + 1) * bk, c1)))
                    skip = Z > 0.0 and math.exp(max(s[kk] for kk in keys)) / Z < tau / n
                    mask[b, h, ci, t] = 0 if skip else 1
                    if not skip:
                        for kk in keys:
                            Z += math.exp(s[kk])
                            kept.append(kk)
            tot = sum(math.exp(s[kk]) for kk in kept)
            for kk in kept:
                o[b, h] += math.exp(s[kk]) / tot * vc[b, kh, kk]
            lse[b, h] = math.log(tot)
    return mask, o, lse


DECODE_TAUS = [0.0, 1e-3, 0.05, 0.5, 2.0, 20.0, 1e3]


def _decode_pin_problem():
    rng = np.random.default_rng(73)
    b, hq, hkv, cap, d = 2, 4, 2, 300, 6
    q = rng.standard_normal((b, hq, d)) * 2.5
    kc = rng.standard_normal((b, hkv, cap, d))
    vc = rng.standard_normal((b, hkv, cap, d))
    return q, kc, vc, [300, 161]


@pytest.mark.parametrize("tau", DECODE_TAUS)
def test_decode_multi_split_matches_bruteforce(tau):
    """Several splits per sequence (64-key splits, 16-key tiles): the
    oracle's decisions, output and log-normalizer equal the per-key scalar
    loops of the split rule with L = N_k."""
    q, kc, vc, lens = _decode_pin_problem()
    r = O.mala_decode(q, kc, vc, lens, tau, 0.6, 64, 16)
    m, o, lse = brute_decode(q, kc, vc, lens, tau, 0.6, 64, 16)
    np.testing.assert_array_equal(r["mask"], m)
    np.testing.assert_allclose(r["o"], o, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse, atol=1e-12)
    if tau >= 0.5:
        assert (m == O.SKIPPED).any()      # the sweep exercises the skip branch


# ------------------------------------------------ mutation checks of the pins

def _mutant_fwd_block(kind):
    orig = O.fwd_block

    def mutant(s, c, bk, valid_rows, replay=None, band=0.0):
        if kind == "ascending":
            # visit tiles in ascending order instead of from the diagonal
            nr, nk = s.shape
            tc = -(-nk // bk)
            dec = np.full(tc, -1, dtype=np.int8)
            lam = np.full(nr, -np.inf)
            kept = np.zeros(nk, bool)
            tmax, tlse = O._tile_stats(s, bk)
            has = np.isfinite(tmax) & valid_rows[:, None]
            for j in range(tc):
                rows = has[:, j]
                if not rows.any():
                    continue
                mu = np.min(c[rows] - (tmax[rows, j] - lam[rows]))
                if mu > 0:
                    dec[j] = 0
                    continue
                dec[j] = 1
                lam[rows] = np.logaddexp(lam[rows], tlse[rows, j])
                kept[j * bk:(j + 1) * bk] = True
            return dec, np.zeros(tc), lam, kept, 0
        if kind == "no_length_norm":
            return orig(s, c + np.log(np.arange(1, c.size + 1)), bk, valid_rows, replay, band)
        if kind == "non_strict":
            return orig(s, c + 1e-9, bk, valid_rows, replay, band)
        raise ValueError(kind)
    return mutant


@pytest.mark.parametrize("kind", ["ascending", "no_length_norm"])
def test_pins_catch_planted_forward_mistakes(kind, monkeypatch):
    q, k, v, _ = rand_problem(12, 1, 2, 1, 16, d=4, qstd=2.5)
    monkeypatch.setattr(O, "fwd_block", _mutant_fwd_block(kind))
    caught = False
    for tau in TAUS:
        r = O.mala_fwd(q, k, v, tau, 0.7, True, 2, 2)
        m, _, _ = brute_forward(q, k, v, tau, 0.7, 2, 2)
        if not np.array_equal(r["mask"], m):
            caught = True
    assert caught


def _split_local_length_mutant(tau):
    """fwd_block as the decode would call it if L counted only the keys of
    the split being gated instead of the query's whole context."""
    orig = O.fwd_block

    def mutant(s, c, bk, valid_rows, replay=None, band=0.0):
        c_local = np.full(c.shape, math.log(tau) - math.log(s.shape[1]))
        return orig(s, c_local, bk, valid_rows, replay, band)
    return mutant


def test_pins_catch_split_local_length(monkeypatch):
    """A decode that uses the split's own length in tau / L fails both the
    brute-force pin of the split rule and the per-key bound exp(s_k) / Z_R <
    tau / N_k on omitted keys."""
    q, kc, vc, lens = _decode_pin_problem()
    refs = {tau: brute_decode(q, kc, vc, lens, tau, 0.6, 64, 16) for tau in DECODE_TAUS[1:]}
    mismatched = 0
    for tau, (m, _, _) in refs.items():
        monkeypatch.setattr(O, "fwd_block", _split_local_length_mutant(tau))
        r = O.mala_decode(q, kc, vc, lens, tau, 0.6, 64, 16)
        mismatched += int((r["mask"] != m).sum())
    # the per-key bound sees the mutant where one split holds most of the
    # mass (its partial normalizer is then close to the merged one): here
    # the newest of four 64-key splits, whose keys are twice as long
    rng = np.random.default_rng(74)
    q = rng.standard_normal((1, 4, 6)) * 2.5
    kc = rng.standard_normal((1, 1, 256, 6))
    vc = rng.standard_normal((1, 1, 256, 6))
    kc[:, :, 192:] *= 2.0
    bound_broken = 0
    for tau in (0.05, 0.2, 0.5, 5.0):
        monkeypatch.setattr(O, "fwd_block", _split_local_length_mutant(tau))
        r = O.mala_decode(q, kc, vc, [256], tau, 0.6, 64, 16)
        monkeypatch.undo()
        ok = O.mala_decode(q, kc, vc, [256], tau, 0.6, 64, 16)
        for h in range(4):
            s = 0.6 * kc[0, 0] @ q[0, h]
            for res, tally in ((r, True), (ok, False)):
                omitted = ~decode_kept_keys(res["mask"][0, h], 256, 64, 16)
                broken = int((np.exp(s[omitted] - res["lse"][0, h]) >= tau / 256).sum())
                if tally:
                    bound_broken += broken
                else:
                    assert broken == 0       # the oracle itself keeps the bound
    monkeypatch.undo()
    assert mismatched > 0 and bound_broken > 0


def test_pins_catch_forced_backward_diagonal(monkeypatch):
    """A backward that always keeps the diagonal tile fails the closed form."""
    orig = O.mala_bwd

    def mutant(*a, **kw):
        r = orig(*a, **kw)
        m = r["mask"]
        for i in range(min(m.shape[2], m.shape[3])):
            m[..., i, i] = np.where(m[..., i, i] == O.SKIPPED, O.KEPT, m[..., i, i])
        return r
    monkeypatch.setattr(O, "mala_bwd", mutant)
    with pytest.raises(AssertionError):
        test_constant_scores_closed_form(2.0, 4)


def test_round_storage_matches_torch_casts():
    """The oracle's model of a stored bf16/fp32 tensor is torch's round-to-
    nearest-even cast."""
    rng = np.random.default_rng(80)
    x = rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))
    t = torch.from_numpy(x)
    np.testing.assert_array_equal(O.round_storage(x, "bf16"),
                                  t.float().to(torch.bfloat16).double().numpy())
    np.testing.assert_array_equal(O.round_storage(x, "f32"), t.float().double().numpy())
    np.testing.assert_array_equal(O.round_storage(x, None), x)
