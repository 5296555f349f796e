"""GPU parity at the full sizes of the benchmark workloads (8K, 32K and 128K
causal prefill + backward; 128K split-KV decode), run through the same entry
points and flags as bench.py, against the CPU fp64 oracle on sampled outputs.

The oracle cannot redo a whole 32K or 128K problem in seconds, so each test
checks outputs it can compute one by one:
  - forward: O, LSE and every tile decision of sampled 32-row query blocks of
    one query head (first, early, middle, late and last blocks);
  - backward dQ and the backward decisions of the same blocks;
  - backward dK and dV of the last 64 keys of one KV head: causally only the
    last 64 query rows of the group's heads reach them, so the oracle runs on
    those rows alone (bottom-right alignment keeps their positions);
  - decode: whole steps (every head, every split) of the 128K decode batch,
    with the default 256-key splits and with the automatic split length;
  - the backward with the gate pass on the structured 32K workload: sampled
    blocks against the oracle, and every decision, dK and dV against the
    default backward.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import mala_oracle as O
from parity_util import (BAND, assert_bitwise_where_agree, check_dq_o_rounding, check_lse,
                         check_ties, compare_values, np64, o_rounding_dq_term, tiling)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # collected on CPU only to be deselected
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = "cuda"
TAU = 1e-4


def lib():
    import contribution_gated_sparse_amd as m
    return m


def _agree(gm, om, margin, what, max_ties=8):
    """Decisions agree wherever the oracle visited and the margin is clear of
    the near-tie band; the near ties themselves are counted and bounded."""
    seen = om != O.NOT_VISITED
    clear = seen & ~(np.abs(np.nan_to_num(margin, nan=np.inf)) < BAND["bf16"])
    bad = int((gm[clear] != om[clear]).sum())
    assert bad == 0, f"{what}: {bad} decisions differ outside the near-tie band"
    ties = int((seen & ~clear).sum())
    check_ties(f"{what} near ties (of {int(seen.sum())})", ties, max_ties)
    return ties


# C3 runs at every tolerance of its sweep (tau = 0 is dense attention)
@pytest.mark.parametrize("cid,tau", [(2, 1e-4), (3, 0.0), (3, 1e-5), (3, 1e-4), (3, 1e-3),
                                     (4, 1e-4)])
def test_prefill_full_size_sampled(cid, tau):
    m = lib()
    cfg = W.CONFIGS[cid]
    x = W.make_prefill(cfg, device=DEV)
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    scale = x["scale"]
    B, HQ, N, D = q.shape
    HKV = k.shape[1]
    G = HQ // HKV
    (fbq, fbk, _), (bbq, bbk, _), _ = tiling()
    assert N % 64 == 0 and fbq == bbq
    print(f"[full-size] config {cid} tau={tau}: B={B} Hq={HQ} Hkv={HKV} N={N} d={D}", flush=True)

    g = m.mala_fwd(q, k, v, tau, softmax_scale=scale, want_mask=True)
    gb = m.mala_bwd(q, k, v, g["o"], g["lse"], do, tau, softmax_scale=scale, want_mask=True)
    torch.cuda.synchronize()

    kh = HKV - 1
    heads = list(range(kh * G, (kh + 1) * G))
    h = heads[-1]
    tr = N // fbq
    blocks = sorted({0, 1, tr // 3, tr // 2 + 1, tr - 3, tr - 1})

    # ---- forward and dQ on sampled blocks of head h
    kn, vn = np64(k[:, kh:kh + 1]), np64(v[:, kh:kh + 1])
    qh, doh = np64(q[:, h:h + 1]), np64(do[:, h:h + 1])
    fmask = g["mask"][:, h:h + 1].cpu().numpy()
    r = O.mala_fwd(qh, kn, vn, tau, scale, True, fbq, fbk,
                   blocks=[(0, 0, i) for i in blocks], replay=fmask, band=BAND["bf16"])
    _agree(fmask, r["mask"], r["margin"], "forward")
    kept = g["kept"][:, h:h + 1].cpu().numpy()
    for i in blocks:
        assert kept[0, 0, i] == int((r["mask"][0, 0, i] == O.KEPT).sum())
    rows = np.zeros((1, 1, N), bool)
    for i in blocks:
        rows[..., i * fbq:(i + 1) * fbq] = True
    compare_values("O", np64(g["o"][:, h:h + 1]), r["o"], "bf16", rows)
    check_lse("LSE", np64(g["lse"][:, h:h + 1])[rows], r["lse"][rows], "bf16")

    bmask = gb["mask"][:, h:h + 1].cpu().numpy()
    rb = O.mala_bwd(qh, kn, vn, r["o"], r["lse"], doh, tau, scale, True, bbq, bbk,
                    qblocks=blocks, replay=bmask, band=BAND["bf16"], o_storage="bf16",
                    lse_storage="f32")
    _agree(bmask, rb["mask"], rb["margin"], "backward")
    compare_values("dQ", np64(gb["dq"][:, h:h + 1]), rb["dq"], "bf16", rows)

    # ---- dK, dV of the last 64 keys of KV head kh: only the group's last 64
    # query rows see them
    t = 64
    qt, dot = np64(q[:, heads, N - t:]), np64(do[:, heads, N - t:])
    ft = g["mask"][:, heads, -(t // fbq):].cpu().numpy()
    rt = O.mala_fwd(qt, kn, vn, tau, scale, True, fbq, fbk, replay=ft, band=BAND["bf16"])
    _agree(ft, rt["mask"], rt["margin"], "forward (tail)")
    compare_values("O tail", np64(g["o"][:, heads, N - t:]), rt["o"], "bf16")
    bt = gb["mask"][:, heads, -(t // bbq):].cpu().numpy()
    rbt = O.mala_bwd(qt, kn, vn, rt["o"], rt["lse"], dot, tau, scale, True, bbq, bbk,
                     replay=bt, band=BAND["bf16"], o_storage="bf16",
                    lse_storage="f32")
    _agree(bt, rbt["mask"], rbt["margin"], "backward (tail)")
    compare_values("dQ tail", np64(gb["dq"][:, heads, N - t:]), rbt["dq"], "bf16")
    compare_values("dK tail", np64(gb["dk"][:, kh:kh + 1, N - t:]), rbt["dk"][:, :, N - t:], "bf16")
    compare_values("dV tail", np64(gb["dv"][:, kh:kh + 1, N - t:]), rbt["dv"][:, :, N - t:], "bf16")


def test_gate_pass_full_size_structured():
    """MALA_FLAG_GATE_PASS at the bench's structured 32K workload (sink keys,
    local band, retrieval keys; most tiles skipped): decisions and dQ of
    sampled blocks against the oracle, the decision masks against the default
    backward's, and the whole dK and dV against the default backward's; the
    nested call (the forward's kept tiles only) against the gate pass."""
    m = lib()
    x = W.make_structured(32768, hq=32, hkv=8, d=128, device=DEV, dtype="bf16", with_do=False)
    q, k, v, scale = x["q"], x["k"], x["v"], x["scale"]
    do = W.rademacher(q.shape, seed=20269002, device=DEV, dtype="bf16")
    B, HQ, N, D = q.shape
    HKV = k.shape[1]
    G = HQ // HKV
    (fbq, fbk, _), (bbq, bbk, _), _ = tiling()
    print(f"[full-size] gate pass, structured: Hq={HQ} Hkv={HKV} N={N}", flush=True)
    g = m.mala_fwd(q, k, v, TAU, softmax_scale=scale, want_mask=True)
    ga = m.mala_bwd(q, k, v, g["o"], g["lse"], do, TAU, softmax_scale=scale, want_mask=True)
    gb = m.mala_bwd(q, k, v, g["o"], g["lse"], do, TAU, softmax_scale=scale, want_mask=True,
                    gate_pass=True)
    torch.cuda.synchronize()

    ma, mb = ga["mask"].cpu().numpy(), gb["mask"].cpu().numpy()
    assert np.array_equal(ma == O.NOT_VISITED, mb == O.NOT_VISITED)
    assert int((mb == O.KEPT).sum()) < 0.1 * int((mb != O.NOT_VISITED).sum())
    # the two score products round differently: decisions may differ only at
    # near ties, which are rare
    assert int((ma != mb).sum()) <= 16, f"{int((ma != mb).sum())} decisions differ"
    kept_a, kept_b = ga["kept"].cpu().numpy(), gb["kept"].cpu().numpy()
    assert np.array_equal(kept_b, (mb == O.KEPT).sum(-1))
    assert int(np.abs(kept_a - kept_b).sum()) <= int((ma != mb).sum())

    kh = 0                                   # the KV head whose key block 0 holds the sinks
    h = kh * G
    tr = N // fbq
    blocks = sorted({0, 1, tr // 3, tr // 2 + 1, tr - 3, tr - 1})
    kn, vn = np64(k[:, kh:kh + 1]), np64(v[:, kh:kh + 1])
    qh, doh = np64(q[:, h:h + 1]), np64(do[:, h:h + 1])
    r = O.mala_fwd(qh, kn, vn, TAU, scale, True, fbq, fbk, blocks=[(0, 0, i) for i in blocks],
                   replay=g["mask"][:, h:h + 1].cpu().numpy(), band=BAND["bf16"])
    rows = np.zeros((1, 1, N), bool)
    for i in blocks:
        rows[..., i * fbq:(i + 1) * fbq] = True
    bmask = mb[:, h:h + 1]
    rb = O.mala_bwd(qh, kn, vn, r["o"], r["lse"], doh, TAU, scale, True, bbq, bbk,
                    qblocks=blocks, replay=bmask, band=BAND["bf16"], o_storage="bf16",
                    lse_storage="f32")
    _agree(bmask, rb["mask"], rb["margin"], "backward (gate pass)")
    # dQ on these inputs is at the conditioning limit of a bf16-stored O (in
    # sink-led rows dP - D nearly cancels): the stated bar plus the bf16-O
    # rounding term of o_rounding_dq_term, element by element and in norm
    term = o_rounding_dq_term(qh, kn, vn, doh, scale, True, r, rb, rows)
    check_dq_o_rounding("dQ (gate pass, structured)", np64(gb["dq"][:, h:h + 1])[rows],
                        rb["dq"][rows], term)
    # the dQ kernel is the default path's: the same decisions give the same dQ
    assert_bitwise_where_agree(ma, mb, ga, gb, G, dkdv=False)

    for n_ in ("dk", "dv"):
        a, b_ = np64(gb[n_]), np64(ga[n_])
        scaled = float(np.abs(a - b_).max() / max(1.0, np.abs(b_).max()))
        fro = float(np.linalg.norm(a - b_) / max(np.linalg.norm(b_), 1e-30))
        assert scaled <= 2e-2 and fro <= 1e-2, f"{n_}: {scaled:.3e} {fro:.3e}"

    # on the forward's kept tiles only (mala_bwd_nested): the gate pass's
    # decisions restricted to those tiles, which exact arithmetic makes the
    # same decisions, and then the same gradients bit for bit
    gc = m.mala_bwd(q, k, v, g["o"], g["lse"], do, TAU, softmax_scale=scale, want_mask=True,
                    fwd_mask=g["mask"])
    torch.cuda.synchronize()
    mc = gc["mask"].cpu().numpy()
    up = np.repeat(np.repeat(g["mask"].cpu().numpy(), fbq // bbq, axis=2), fbk // bbk,
                   axis=3)[:, :, :mb.shape[2], :mb.shape[3]]
    assert np.array_equal(mc, np.where((mb == O.KEPT) & (up != O.KEPT), O.SKIPPED, mb))
    assert int((mc != mb).sum()) <= 16, f"{int((mc != mb).sum())} decisions differ"
    assert np.array_equal(gc["kept"].cpu().numpy(), (mc == O.KEPT).sum(-1))
    assert_bitwise_where_agree(mb, mc, gb, gc, G)


@pytest.mark.parametrize("step,split_keys", [(0, 0), (63, 0), (0, -1)])
def test_decode_full_size(step, split_keys):
    m = lib()
    x = W.make_decode(W.CONFIGS[5], device=DEV)
    kc, vc, qs = x["k_cache"], x["v_cache"], x["q_steps"]
    cache0 = x["cache"]
    B, HQ = qs.shape[1], qs.shape[2]
    n = cache0 + step + 1
    print(f"[full-size] decode step {step}: B={B} Hq={HQ} N_k={n} split_keys={split_keys}",
          flush=True)
    _, _, (_, dbk, chunk) = tiling()
    q = qs[step].contiguous()
    lens = [n] * B
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    g = m.mala_decode(q, kc, vc, seq, TAU, max_n_k=n, softmax_scale=x["scale"], want_mask=True,
                      split_keys=split_keys)
    torch.cuda.synchronize()
    chunk = g["split"]
    gmask = g["mask"].cpu().numpy()
    r = O.mala_decode(np64(q), np64(kc[:, :, :n]), np64(vc[:, :, :n]), lens, TAU, x["scale"],
                      chunk, dbk, replay=gmask, band=BAND["bf16"])
    assert np.array_equal(gmask, r["mask"]), "decode decisions differ outside the near-tie band"
    kept = g["kept"].cpu().numpy()
    assert np.array_equal(kept[:, :HQ], (r["mask"] == O.KEPT).sum((-1, -2)))
    assert np.array_equal(kept[:, HQ:], r["v_tiles"].sum((-1, -2)))
    compare_values("decode O", np64(g["o"]), r["o"], "bf16")
    check_lse("decode LSE", np64(g["lse"]), r["lse"], "bf16")
