#!/usr/bin/env python3
"""Benchmark of the MALA operator on one MI355X.

One step = one pass of the whole hot path over synthetic inputs resident in
HBM: MALA forward + backward on the 32K causal GQA problem (B=1, 32 query /
8 KV heads, d=128, bf16, tau=1e-4) followed by one split-KV decode step on the
128K decode batch (8 sequences, 8 query / 1 KV head, 256-key splits), whose
new K/V rows are appended to the caches inside the step.

Prints one JSON line. ``value`` is the step's dense-equivalent throughput:
the FLOPs dense causal attention would spend on the same work (forward 4d and
backward 10d per legal query/key pair, decode 4d per key), divided by the
measured step time. Per-stage times come from HIP events on the stream the
library launches on. The CPU fp64 oracle is timed on a bounded sample of the
same 32K problem as a baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--tau", type=float, default=1e-4)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the CPU oracle baseline sample (0 = skip)")
    ap.add_argument("--no-128k", action="store_true", help="skip the 128K prefill extra")
    ap.add_argument("--no-structured", action="store_true",
                    help="skip the structured-logit extra (skip speedups against tau = 0)")
    ap.add_argument("--fast-grad", action="store_true", help="single-bf16 dS in the backward")
    ap.add_argument("--only", default="", help="profiling: 'fwd', 'bwd' or 'decode' alone")
    ap.add_argument("--profile-structured", type=float, default=None, metavar="TAU",
                    help="for rocprofv3: two passes of the structured 32K forward + backward, "
                         "of the backward with the gate pass, and of the structured 128K decode "
                         "(256-key splits, then one split per sequence) at TAU; prints no JSON")
    ap.add_argument("--profile", action="store_true",
                    help="for rocprofv3: one warm-up step, one step, then a 1 GiB device copy "
                         "that calibrates the byte counters; prints no JSON")
    return ap.parse_args()


def causal_pairs(n: int) -> int:
    return n * (n + 1) // 2


def fwd_tiles(nq, nk, bq, bk):
    """Score tiles visited by the causal forward (per head)."""
    off = nk - nq
    tot = 0
    for i in range(-(-nq // bq)):
        last = min(i * bq + bq - 1, nq - 1)
        tot += min(last + off, nk - 1) // bk + 1
    return tot


def bwd_tiles(nq, nk, bq, bk):
    """Legal backward tiles (per head)."""
    off = nk - nq
    tot = 0
    for i in range(-(-nq // bq)):
        last = min(i * bq + bq - 1, nq - 1)
        tot += min(last + off, nk - 1) // bk + 1
    return tot


def matched_work(m, F, W, torch, dev, fbq, fbk, preset, n=8192):
    """Allocation at matched work (Sec. 3, Table 1; App. C.2) on structured
    inputs: MALA's forward support against a per-instance reference-mass
    control that keeps, for every decision (head x query block), exactly as
    many key tiles as MALA kept there, chosen by their mass under the
    unscreened softmax (fidelity.reference_mass_control). Both supports are
    scored the same way in fp32 from the unscreened scores: omitted mass per
    row and the relative L2 error of the output they imply."""
    z = W.make_structured_preset(preset, n, hq=32, hkv=8, d=128, device=dev, dtype="bf16",
                                 with_do=False)
    q, k, v, scale = z["q"], z["k"], z["v"], z["scale"]
    _, HQ, N, _ = q.shape
    lse0 = m.mala_fwd(q, k, v, 0.0, softmax_scale=scale)["lse"]
    res = {"n": n, "heads": HQ, "decision": f"{fbq} query rows x {fbk} keys"}
    for tau_ in (1e-4, 1.0):
        mask = m.mala_fwd(q, k, v, tau_, softmax_scale=scale, want_mask=True)["mask"]
        r = F.reference_mass_control(q, k, v, scale, lse0, mask, fbq, fbk)
        row = {"slots_per_query": round(int((mask == 1).sum()) * fbk * fbq / (HQ * N), 1)}
        for name in ("mala", "control"):
            row[name] = {"omitted_mass": F.mean_p95(r[name]["omitted_mass"]),
                         "o_rel_l2": F.mean_p95(r[name]["o_rel_l2"])}
        res[f"tau={tau_:g}"] = row
    return res


def profile_structured(tau, m, W, torch, dev):
    """Kernel launches for a profiler on the structured inputs: two passes
    (the first warms up) of the 32K forward + backward, two of the backward
    with the separate gate pass, two with the walk chosen on the device
    (mala_bwd_auto), two of the forward writing its tile mask and
    the nested backward on it, then of the 128K decode with 256-key splits
    and with one split per sequence."""
    x = W.make_structured(32768, hq=32, hkv=8, d=128, device=dev, dtype="bf16", with_do=False)
    q, k, v = x["q"], x["k"], x["v"]
    do = W.rademacher(q.shape, seed=20269002, device=dev, dtype="bf16")
    for _ in range(2):
        f = m.mala_fwd(q, k, v, tau, softmax_scale=x["scale"])
        m.mala_bwd(q, k, v, f["o"], f["lse"], do, tau, softmax_scale=x["scale"])
        torch.cuda.synchronize()
    for _ in range(2):   # the backward with the separate gate pass
        m.mala_bwd(q, k, v, f["o"], f["lse"], do, tau, softmax_scale=x["scale"], gate_pass=True)
        torch.cuda.synchronize()
    for _ in range(2):   # the walk chosen on the device from the forward's kept counters
        m.mala_bwd(q, k, v, f["o"], f["lse"], do, tau, softmax_scale=x["scale"], fwd_kept=f["kept"])
        torch.cuda.synchronize()
    for _ in range(2):   # the forward's tile mask and the backward on its kept tiles
        f = m.mala_fwd(q, k, v, tau, softmax_scale=x["scale"], want_mask=True)
        m.mala_bwd(q, k, v, f["o"], f["lse"], do, tau, softmax_scale=x["scale"],
                   fwd_mask=f["mask"])
        torch.cuda.synchronize()
    del x, q, k, v, do, f
    torch.cuda.empty_cache()
    n = 131072
    y = W.make_structured(n, hq=8, hkv=1, d=128, batch=8, device=dev, dtype="bf16", with_do=False)
    kc, vc = y["k"], y["v"]
    qd = y["q"][:, :, n - 1].contiguous()
    del y
    seq = torch.full((qd.shape[0],), n, dtype=torch.int32, device=dev)
    for sk in (0, n):
        for _ in range(2):
            m.mala_decode(qd, kc, vc, seq, tau, max_n_k=n, softmax_scale=x_scale(128),
                          split_keys=sk)
            torch.cuda.synchronize()
    print(f"structured profile run done (tau={tau:g})", flush=True)


NESTED_NOTE = ("outside the method: mala_bwd_nested skips the backward score recomputation of "
               "the tiles the forward skipped, while the paper's backward recomputes Q K^T "
               "before every skip decision (App. A.1); its speedups are not the method's")


def prefill_128k_structured(args, m, W, torch, dev, fb, bb, preset):
    """One GPU's share of the 128K layer (B=1, 8 query / 1 KV head, d=128)
    on the structured preset at tau = 0 and tau = 1: the forward, the default
    backward and the backward with the walk chosen on the device
    (mala_bwd_auto). The pages quote their 128K operator ratios at tau = 1 on
    other hardware (context only)."""
    (fbq, fbk), (bbq, bbk) = fb, bb
    x = W.make_structured_preset(preset, 131072, hq=8, hkv=1, d=128, device=dev, dtype="bf16",
                                 with_do=False)
    q, k, v = x["q"], x["k"], x["v"]
    do = W.rademacher(q.shape, seed=20269002, device=dev, dtype="bf16")
    B, HQ, N, _ = q.shape
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn):
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        t = 0.0
        for _ in range(args.steps):
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            t += ev[0].elapsed_time(ev[1])
        return round(t / args.steps, 3)

    out = {}
    for tau_ in (0.0, 1.0):
        fo, bo = {}, {}
        tf = timed(lambda: fo.update(m.mala_fwd(q, k, v, tau_, softmax_scale=x["scale"])))
        tb = timed(lambda: bo.update(m.mala_bwd(q, k, v, fo["o"], fo["lse"], do, tau_,
                                                softmax_scale=x["scale"])))
        ta = timed(lambda: m.mala_bwd(q, k, v, fo["o"], fo["lse"], do, tau_,
                                      softmax_scale=x["scale"], fwd_kept=fo["kept"]))
        out[tau_] = dict(fwd_ms=tf, bwd_ms=tb, bwd_auto_ms=ta, slots_per_query={
            "fwd": round(float(fo["kept"].double().sum()) * fbk * fbq / (B * HQ * N), 1),
            "bwd": round(float(bo["kept"].double().sum()) * bbk * bbq / (B * HQ * N), 1)})
        del fo, bo
    z, r = out[0.0], out[1.0]
    r["fwd_speedup"] = round(z["fwd_ms"] / r["fwd_ms"], 4)
    r["bwd_speedup"] = round(z["bwd_ms"] / r["bwd_ms"], 4)
    r["bwd_speedup_auto"] = round(z["bwd_ms"] / r["bwd_auto_ms"], 4)
    r["speedup_vs_tau0"] = round((z["fwd_ms"] + z["bwd_ms"]) / (r["fwd_ms"] + r["bwd_ms"]), 4)
    r["speedup_vs_tau0_auto"] = round((z["fwd_ms"] + z["bwd_ms"]) / (r["fwd_ms"] + r["bwd_auto_ms"]),
                                      4)
    del x, q, k, v, do
    return {"shape": "B=1, 8 query / 1 KV head, d=128, L=131072", **{f"tau={t:g}": out[t] for t in out}}


def structured_section(args, m, F, W, torch, dev, tiling, preset):
    """Extra, not part of ``value``: the same kernels on structured-logit inputs
    (sink keys, a local band, sparse retrieval keys; the named preset of
    workloads.make_structured_preset), where the tolerance does skip tiles,
    timed against tau = 0. Prefill: 32K, 32/8 heads; decode: 8 sequences of
    131072 keys, 8/1 heads, the query of each sequence being the sequence's
    last row."""
    (fbq, fbk), (bbq, bbk), (dbk, dchunk) = tiling
    taus = (0.0, 1e-4, 1e-2, 1.0)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    res = {"inputs": f"workloads.make_structured_preset({preset!r}) (bf16)",
           "nested": NESTED_NOTE}

    x = W.make_structured_preset(preset, 32768, hq=32, hkv=8, d=128, device=dev, dtype="bf16",
                                 with_do=False)
    q, k, v = x["q"], x["k"], x["v"]
    # dO: a deterministic Rademacher probe (App. C.3)
    do = W.rademacher(q.shape, seed=20269002, device=dev, dtype="bf16")
    B, HQ, N, D = q.shape
    fo = dict(o=torch.empty_like(q), lse=torch.empty(q.shape[:3], device=dev),
              kept=torch.empty((B, HQ, -(-N // fbq)), dtype=torch.int32, device=dev))
    bo = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
              kept=torch.empty((B, HQ, -(-N // bbq)), dtype=torch.int32, device=dev))
    bg = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v))
    ba = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v))
    fn = dict(o=torch.empty_like(q), lse=torch.empty(q.shape[:3], device=dev),
              mask=torch.empty((B, HQ, -(-N // fbq), -(-N // fbk)), dtype=torch.int8, device=dev))
    bn = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v))
    vis_f = fwd_tiles(N, N, fbq, fbk) * B * HQ
    vis_b = bwd_tiles(N, N, bbq, bbk) * B * HQ
    pre = {}
    for tau_ in taus:
        def run():
            m.mala_fwd(q, k, v, tau_, softmax_scale=x["scale"], out=fo)
            ev[1].record()
            m.mala_bwd(q, k, v, fo["o"], fo["lse"], do, tau_, softmax_scale=x["scale"], out=bo,
                       fast_grad=args.fast_grad)
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        tf = tb = 0.0
        for _ in range(args.steps):
            ev[0].record()
            run()
            ev[2].record()
            torch.cuda.synchronize()
            tf += ev[0].elapsed_time(ev[1])
            tb += ev[1].elapsed_time(ev[2])
        pre[tau_] = dict(fwd_ms=round(tf / args.steps, 3), bwd_ms=round(tb / args.steps, 3),
                         fwd_kept_frac=round(int(fo["kept"].sum()) / vis_f, 4),
                         bwd_kept_frac=round(int(bo["kept"].sum()) / vis_b, 4))
        # the same backward with the separate gate pass (MALA_FLAG_GATE_PASS):
        # dK/dV then walks only the steps with a kept tile
        def run_gate():
            m.mala_bwd(q, k, v, fo["o"], fo["lse"], do, tau_, softmax_scale=x["scale"], out=bg,
                       fast_grad=args.fast_grad, gate_pass=True)
        for _ in range(args.warmup):
            run_gate()
        torch.cuda.synchronize()
        tg = 0.0
        for _ in range(args.steps):
            ev[0].record()
            run_gate()
            ev[2].record()
            torch.cuda.synchronize()
            tg += ev[0].elapsed_time(ev[2])
        pre[tau_]["bwd_gate_pass_ms"] = round(tg / args.steps, 3)
        pre[tau_]["gate_pass_vs_default"] = {   # max |difference| / max(1, max |default|)
            n_: float((bg[n_].float() - bo[n_].float()).abs().max()
                      / bo[n_].float().abs().max().clamp_min(1.0)) for n_ in ("dq", "dk", "dv")}
        # the walk chosen on the device from the forward's kept counters
        # (mala_bwd_auto): the gate-pass walks below half of the legal tiles
        def run_auto():
            m.mala_bwd(q, k, v, fo["o"], fo["lse"], do, tau_, softmax_scale=x["scale"], out=ba,
                       fast_grad=args.fast_grad, fwd_kept=fo["kept"])
        for _ in range(args.warmup):
            run_auto()
        torch.cuda.synchronize()
        ta = 0.0
        for _ in range(args.steps):
            ev[0].record()
            run_auto()
            ev[2].record()
            torch.cuda.synchronize()
            ta += ev[0].elapsed_time(ev[2])
        pre[tau_]["bwd_auto_ms"] = round(ta / args.steps, 3)
        # which walk ran: its result equals that walk's own call bit for bit
        same = lambda r: all(torch.equal(ba[n_], r[n_]) for n_ in ("dq", "dk", "dv"))
        pre[tau_]["bwd_auto_walk"] = ("gate_pass" if same(bg) else
                                      "default" if same(bo) else "neither")
        # the gate pass as a training step pairs it: the forward also writes its
        # tile mask, and the backward scores only the tiles the forward kept
        # (mala_bwd_nested; nested support, Sec. 2.2)
        def run_nested():
            m.mala_fwd(q, k, v, tau_, softmax_scale=x["scale"], out=fn, want_mask=True,
                       want_kept=False)
            ev[1].record()
            m.mala_bwd(q, k, v, fn["o"], fn["lse"], do, tau_, softmax_scale=x["scale"], out=bn,
                       fast_grad=args.fast_grad, fwd_mask=fn["mask"])
        for _ in range(args.warmup):
            run_nested()
        torch.cuda.synchronize()
        tf = tb = 0.0
        for _ in range(args.steps):
            ev[0].record()
            run_nested()
            ev[2].record()
            torch.cuda.synchronize()
            tf += ev[0].elapsed_time(ev[1])
            tb += ev[1].elapsed_time(ev[2])
        pre[tau_]["fwd_with_mask_ms"] = round(tf / args.steps, 3)
        pre[tau_]["bwd_nested_ms"] = round(tb / args.steps, 3)
        pre[tau_]["nested_equals_gate_pass"] = all(
            torch.equal(bn[n_], bg[n_]) for n_ in ("dq", "dk", "dv"))
        # fidelity against tau = 0 (App. C.1/C.3 quantities): omitted normalized
        # mass per row, 1 - Z_R / Z = 1 - exp(z_tau - z_0), bounded by
        # tau / (1 + tau) (Prop. 1), and the relative L2 error of each output row
        if tau_ == 0.0:
            lse0, o0 = fo["lse"].clone(), fo["o"].float()
            g0 = {n_: bo[n_].clone() for n_ in ("dq", "dk", "dv")}
        eps = (1.0 - torch.exp(fo["lse"] - lse0)).flatten().double()
        rl2 = ((fo["o"].float() - o0).norm(dim=-1) / o0.norm(dim=-1).clamp_min(1e-30)).flatten()
        bound = tau_ / (1.0 + tau_)
        pre[tau_]["omitted_mass"] = {
            "mean": float(eps.mean()), "p95": float(eps.sort().values[int(0.95 * (eps.numel() - 1))]),
            "max": float(eps.max()), "bound": bound,
            # fp32 LSEs resolve the mass to ~1e-5
            "rows_over_bound": int((eps > bound + 1e-5).sum())}
        pre[tau_]["o_rel_l2"] = {"mean": float(rl2.mean()),
                                 "p95": float(rl2.sort().values[int(0.95 * (rl2.numel() - 1))]),
                                 "max": float(rl2.max())}
        # head-level relative L2 errors (App. C.3): output and dQ per query
        # head, dK and dV per KV head
        pre[tau_]["head_rel_l2"] = {"o": F.mean_p95(F.head_rel_l2(fo["o"], o0))}
        for n_ in ("dq", "dk", "dv"):
            pre[tau_]["head_rel_l2"][n_] = F.mean_p95(F.head_rel_l2(bo[n_], g0[n_]))
        # mean post-score key slots per query (Eq. 11): kept tiles x B_k over
        # the block's rows
        pre[tau_]["slots_per_query"] = {
            "fwd": round(float(fo["kept"].double().sum()) * fbk * fbq / (B * HQ * N), 1),
            "bwd": round(float(bo["kept"].double().sum()) * bbk * bbq / (B * HQ * N), 1)}
    for tau_ in taus:
        pre[tau_]["speedup_vs_tau0"] = round(
            (pre[0.0]["fwd_ms"] + pre[0.0]["bwd_ms"]) / (pre[tau_]["fwd_ms"] + pre[tau_]["bwd_ms"]), 4)
        pre[tau_]["fwd_speedup"] = round(pre[0.0]["fwd_ms"] / pre[tau_]["fwd_ms"], 4)
        pre[tau_]["bwd_speedup"] = round(pre[0.0]["bwd_ms"] / pre[tau_]["bwd_ms"], 4)
        pre[tau_]["speedup_vs_tau0_gate_pass"] = round(
            (pre[0.0]["fwd_ms"] + pre[0.0]["bwd_ms"])
            / (pre[tau_]["fwd_ms"] + pre[tau_]["bwd_gate_pass_ms"]), 4)
        pre[tau_]["bwd_speedup_gate_pass"] = round(pre[0.0]["bwd_ms"] / pre[tau_]["bwd_gate_pass_ms"], 4)
        pre[tau_]["speedup_vs_tau0_auto"] = round(
            (pre[0.0]["fwd_ms"] + pre[0.0]["bwd_ms"])
            / (pre[tau_]["fwd_ms"] + pre[tau_]["bwd_auto_ms"]), 4)
        pre[tau_]["bwd_speedup_auto"] = round(pre[0.0]["bwd_ms"] / pre[tau_]["bwd_auto_ms"], 4)
        pre[tau_]["speedup_vs_tau0_nested"] = round(
            (pre[0.0]["fwd_ms"] + pre[0.0]["bwd_ms"])
            / (pre[tau_]["fwd_with_mask_ms"] + pre[tau_]["bwd_nested_ms"]), 4)
        pre[tau_]["bwd_speedup_nested"] = round(pre[0.0]["bwd_ms"] / pre[tau_]["bwd_nested_ms"], 4)
    res["prefill_32k"] = {f"tau={t:g}": pre[t] for t in taus}
    del x, q, k, v, do, fo, bo, bg, fn, bn, g0
    torch.cuda.empty_cache()
    res["matched_work_8k"] = matched_work(m, F, W, torch, dev, fbq, fbk, preset)
    torch.cuda.empty_cache()
    res["prefill_128k"] = prefill_128k_structured(args, m, W, torch, dev, (fbq, fbk), (bbq, bbk),
                                                  preset)
    torch.cuda.empty_cache()

    n = 131072
    y = W.make_structured_preset(preset, n, hq=8, hkv=1, d=128, batch=8, device=dev,
                                 dtype="bf16", with_do=False)
    kc, vc = y["k"], y["v"]
    qd = y["q"][:, :, n - 1].contiguous()
    del y
    torch.cuda.empty_cache()
    DB, DHQ, DHKV = kc.shape[0], qd.shape[1], kc.shape[1]
    seq = torch.full((DB,), n, dtype=torch.int32, device=dev)
    out = dict(o=torch.empty_like(qd), lse=torch.empty(qd.shape[:2], device=dev),
               kept=torch.empty((DB, DHQ + DHKV), dtype=torch.int32, device=dev))
    tiles = DB * DHKV * (-(-n // dbk))
    dec = {}
    for tau_ in taus:
        for _ in range(args.warmup + 2):
            m.mala_decode(qd, kc, vc, seq, tau_, max_n_k=n, softmax_scale=x_scale(128), out=out)
        torch.cuda.synchronize()
        reps = 20
        ev[0].record()
        for _ in range(reps):
            m.mala_decode(qd, kc, vc, seq, tau_, max_n_k=n, softmax_scale=x_scale(128), out=out)
        ev[1].record()
        torch.cuda.synchronize()
        kept = out["kept"].cpu()
        vt = int(kept[:, DHQ:].sum())
        dec[tau_] = dict(us_per_step=round(ev[0].elapsed_time(ev[1]) / reps * 1e3, 2),
                         head_kept_frac=round(int(kept[:, :DHQ].sum()) / (tiles * DHQ // DHKV), 4),
                         v_tiles_kept_frac=round(vt / tiles, 4),
                         bytes_per_step=DB * DHKV * n * 128 * 2 + vt * dbk * 128 * 2)
    for tau_ in taus:
        dec[tau_]["speedup_vs_tau0"] = round(dec[0.0]["us_per_step"] / dec[tau_]["us_per_step"], 4)
    res["decode_128k"] = {f"tau={t:g}": dec[t] for t in taus}

    # split length: each split tests its tiles against its own partial
    # normalizer, so longer splits skip more tiles but leave fewer splits to
    # run in parallel (App. A.1 "Fused decoding execution")
    sweep = {}
    for label, sk in (("256", 0), ("auto", m.DECODE_SPLIT_AUTO), ("4096", 4096),
                      ("unsplit", n)):
        row = {}
        for tau_ in (0.0, 1e-4, 1.0):
            reps = 3 if label == "unsplit" else 20
            for _ in range(2):
                r = m.mala_decode(qd, kc, vc, seq, tau_, max_n_k=n, softmax_scale=x_scale(128),
                                  out=out, split_keys=sk)
                out["ws"] = r["ws"]         # reused by the timed calls
            torch.cuda.synchronize()
            ev[0].record()
            for _ in range(reps):
                m.mala_decode(qd, kc, vc, seq, tau_, max_n_k=n, softmax_scale=x_scale(128),
                              out=out, split_keys=sk)
            ev[1].record()
            torch.cuda.synchronize()
            vt = int(out["kept"][:, DHQ:].sum())
            row[f"tau={tau_:g}"] = dict(us_per_step=round(ev[0].elapsed_time(ev[1]) / reps * 1e3, 2),
                                        v_tiles_kept_frac=round(vt / tiles, 4))
        row["split_keys"] = r["split"]
        sweep[label] = row
    res["decode_128k_split_length"] = sweep
    return res


TRAFFIC_MD = os.path.join(ROOT, "profiles", "mala_kernels_prefill32k_decode128k_hbm_traffic.md")
KERNEL_ROWS = {"fwd": ("fwd_bf16_d128_kernel", "fwd_bf16.hip"),
               "bwd_dkdv": ("bwd_dkdv_kernel<128, false>", "bwd_bf16.hip"),
               "bwd_dq": ("bwd_dq_d128_kernel<true>", "bwd_bf16.hip")}


def measured_traffic(kernel: str):
    """HBM bytes per launch of ``kernel`` from the committed FETCH_SIZE /
    WRITE_SIZE summary (copy-calibrated), or None when the kernel's sources
    have changed since those counters were taken."""
    import hashlib
    import re
    if kernel not in KERNEL_ROWS or not os.path.exists(TRAFFIC_MD):
        return None
    row, src = KERNEL_ROWS[kernel]
    csrc = os.path.join(ROOT, "contribution_gated_sparse_amd", "csrc")
    h = hashlib.sha256()
    for f in (src, "mala_device.h", "mala_internal.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    for line in open(TRAFFIC_MD):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 7 and cells[0] == row and re.fullmatch(r"[0-9a-f]{16}", cells[6]):
            return float(cells[5]) * 1e9 if cells[6] == h.hexdigest()[:16] else None
    return None


def x_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the MALA operator "
              "runs on a single MI355X here (heads are independent, so a multi-GPU run would "
              "shard heads across GPUs with no exchange inside the operator).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import contribution_gated_sparse_amd as m
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = m.load_library()
    (fbq, fbk, _), (bbq, bbk, _) = m.mala_get_tiling(0), m.mala_get_tiling(1)
    _, dbk, dchunk = m.mala_get_tiling(2)
    tau = args.tau
    if args.profile_structured is not None:
        profile_structured(args.profile_structured, m, W, torch, dev)
        return

    # ------------------------------------------------------------ inputs
    cfg = W.CONFIGS[3]
    x = W.make_prefill(cfg, device=dev)
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    B, HQ, N, D = q.shape
    HKV = k.shape[1]
    scale = x["scale"]
    fo = dict(o=torch.empty_like(q), lse=torch.empty(q.shape[:3], device=dev),
              kept=torch.empty((B, HQ, -(-N // fbq)), dtype=torch.int32, device=dev))
    bo = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
              kept=torch.empty((B, HQ, -(-N // bbq)), dtype=torch.int32, device=dev))
    dcfg = W.CONFIGS[5]
    y = W.make_decode(dcfg, device=dev)
    kc, vc, qs = y["k_cache"], y["v_cache"], y["q_steps"]
    DB, DHQ, DHKV = kc.shape[0], qs.shape[2], kc.shape[1]
    cache0, nsteps = y["cache"], y["steps"]
    cap = kc.shape[2]
    # the rows each step appends, staged outside the caches
    k_new = kc[:, :, cache0:cache0 + nsteps].clone()
    v_new = vc[:, :, cache0:cache0 + nsteps].clone()
    seqlens = [torch.full((DB,), cache0 + t + 1, dtype=torch.int32, device=dev)
               for t in range(nsteps)]
    do_ = dict(o=torch.empty_like(qs[0]), lse=torch.empty(qs.shape[1:3], device=dev),
               kept=torch.empty((DB, DHQ + DHKV), dtype=torch.int32, device=dev))
    torch.cuda.synchronize()

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]

    def prefill(tau_, events=True):
        if events:
            ev[0].record()
        m.mala_fwd(q, k, v, tau_, softmax_scale=scale, out=fo)
        if events:
            ev[1].record()
        m.mala_bwd(q, k, v, fo["o"], fo["lse"], do, tau_, softmax_scale=scale, out=bo,
                   fast_grad=args.fast_grad, events=ev[2:5] if events else None,
                   stages=(m.mala.BWD_PREP, m.mala.BWD_DKDV, m.mala.BWD_DQ) if events else None)

    def decode(t, events=True):
        n = cache0 + t + 1
        kc[:, :, n - 1].copy_(k_new[:, :, t])          # append the current token (caller-owned)
        vc[:, :, n - 1].copy_(v_new[:, :, t])
        if events:
            ev[5].record()
        m.mala_decode(qs[t], kc, vc, seqlens[t], tau, max_n_k=n, softmax_scale=y["scale"],
                      out=do_, events=ev[6:8] if events else None)

    names = ["fwd", "bwd_prep", "bwd_dkdv", "bwd_dq", "append", "dec_split", "dec_combine"]

    def phase_ms():
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(7)]

    if args.profile:
        prefill(tau, events=False)
        decode(0, events=False)
        torch.cuda.synchronize()
        prefill(tau, events=False)
        decode(1, events=False)
        torch.cuda.synchronize()
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)                         # 1 GiB read + 1 GiB written
        torch.cuda.synchronize()
        print("profile run done: 2 steps + 1 GiB copy", flush=True)
        return

    only = args.only
    # ------------------------------------------------------------ warmup + timed steps
    for i in range(args.warmup):
        if only in ("", "fwd", "bwd"):
            prefill(tau)
        if only in ("", "decode"):
            decode(i % nsteps)
    torch.cuda.synchronize()
    acc = np.zeros(7)
    t0 = time.perf_counter()
    for i in range(args.steps):
        if only in ("", "fwd", "bwd"):
            prefill(tau)
        if only in ("", "decode"):
            decode(i % nsteps)
        if only == "":
            torch.cuda.synchronize()
            acc += phase_ms()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / max(1, args.steps)
    if only:
        print(json.dumps({"only": only, "ms_per_step": wall}))
        return
    ph = acc / args.steps
    fwd_ms, bwd_ms = ph[0], ph[1] + ph[2] + ph[3]
    dec_us = (ph[5] + ph[6]) * 1e3
    step_ms = float(ph.sum())

    # counters of the last step
    fk = fo["kept"].cpu().numpy()
    bk_ = bo["kept"].cpu().numpy()
    vis_f = fwd_tiles(N, N, fbq, fbk) * B * HQ
    vis_b = bwd_tiles(N, N, bbq, bbk) * B * HQ
    kept_f, kept_b = int(fk.sum()), int(bk_.sum())

    # ------------------------------------------------------------ tau = 0, same kernels
    for _ in range(args.warmup):
        prefill(0.0)
    torch.cuda.synchronize()
    acc0 = np.zeros(7)
    for _ in range(args.steps):
        prefill(0.0)
        torch.cuda.synchronize()
        acc0 += phase_ms()
    ph0 = acc0 / args.steps
    fwd0_ms, bwd0_ms = ph0[0], ph0[1] + ph0[2] + ph0[3]

    # ------------------------------------------------------------ decode: all steps
    # the 64 steps run back to back as a serving loop would issue them; events
    # recorded in the stream bracket each step's append and its decode call
    # (split and merge launched back to back), and are read after one
    # synchronization at the end. A second pass records an event between the
    # split and the merge as well, for the breakdown: that event itself costs
    # a few microseconds, so the step time is the first pass's.
    for t in range(nsteps):
        decode(t, events=False)
    torch.cuda.synchronize()
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nsteps)]
    for t in range(nsteps):
        e = sev[t]
        e[0].record()
        n = cache0 + t + 1
        kc[:, :, n - 1].copy_(k_new[:, :, t])
        vc[:, :, n - 1].copy_(v_new[:, :, t])
        e[1].record()
        m.mala_decode(qs[t], kc, vc, seqlens[t], tau, max_n_k=n, softmax_scale=y["scale"],
                      out=do_)
        e[2].record()
    torch.cuda.synchronize()
    dec_all_us = sum(e[1].elapsed_time(e[2]) for e in sev) / nsteps * 1e3
    dappend_us = sum(e[0].elapsed_time(e[1]) for e in sev) / nsteps * 1e3
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nsteps)]
    for t in range(nsteps):
        e = bev[t]
        e[0].record()
        m.mala_decode(qs[t], kc, vc, seqlens[t], tau, max_n_k=cache0 + t + 1,
                      softmax_scale=y["scale"], out=do_, events=e[1:3])
    torch.cuda.synchronize()
    dsplit_us = sum(e[0].elapsed_time(e[1]) for e in bev) / nsteps * 1e3
    dmerge_us = sum(e[1].elapsed_time(e[2]) for e in bev) / nsteps * 1e3
    dkept = do_["kept"].cpu().numpy()
    n_last = cache0 + nsteps
    dec_vtiles = int(dkept[:, DHQ:].sum())
    dec_tiles_total = DB * DHKV * sum(min(4, -(-(min(n_last, c * dchunk + dchunk) - c * dchunk)
                                                // dbk)) for c in range(-(-n_last // dchunk)))

    # ------------------------------------------------------------ work accounting
    pairs = B * HQ * causal_pairs(N)
    dense_fwd = 4 * D * pairs
    dense_bwd = 10 * D * pairs
    dec_keys = DB * DHQ * (cache0 + 1)          # approx. per step (N_k of step 0)
    dense_dec = 4 * D * DB * DHQ * (cache0 + nsteps // 2)
    step_flops = dense_fwd + dense_bwd + dense_dec
    value = step_flops / (step_ms * 1e-3) / 1e12
    E_f = vis_f * fbq * fbk
    S_f = kept_f * fbq * fbk
    E_b = vis_b * bbq * bbk
    S_b = kept_b * bbq * bbk
    alg = {
        "fwd": 2 * D * E_f + 2 * D * S_f,                         # QK on visited, PV on kept
        "bwd_dkdv": 2 * D * E_b + 6 * D * S_b,                    # S on legal; dP, dV, dK on kept
        "bwd_dq": 2 * D * S_b,                                    # dQ on kept
    }
    tms = {"fwd": ph[0], "bwd_dkdv": ph[2], "bwd_dq": ph[3]}
    dec_bytes = (DB * DHKV * n_last * D * 2                      # every K row
                 + dec_vtiles * dbk * D * 2                      # V of kept tiles
                 + 2 * DB * DHQ * D * 2)                         # q in, o out
    dominant = max(tms, key=lambda n: tms[n])
    roof = {"kernel": dominant, "bound": "mfma",
            "achieved": alg[dominant] / (tms[dominant] * 1e-3) / 1e12,
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dominant)      # HBM bytes per launch (rocprofv3)
    roof["algorithmic_per_launch"] = alg[dominant]
    # the same ratio over each whole operator: the forward kernel alone, and
    # the backward's prep + dK/dV + dQ (algorithmic FLOPs 2d E + 8d S_b, Eq. 16)
    alg_bwd = alg["bwd_dkdv"] + alg["bwd_dq"]
    roof["whole_fwd_frac"] = alg["fwd"] / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
    roof["whole_bwd_frac"] = alg_bwd / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
    roof["kernel_fracs"] = {n: round(alg[n] / (tms[n] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
                            for n in alg}

    out = {
        "metric": "MALA fwd+bwd ms & effective TFLOP/s vs tau=0 dense at 32K/128K; decode us/step",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "wall_ms_per_step": round(wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_32k_bf16_gqa32x8 fwd+bwd (B=1, Hq=32, Hkv=8, L=32768, "
                               "d=128, tau=%g) + decode_128k_bf16_b8_gqa8x1 one step" % tau,
                   "tau": tau, "grad_mode": "fast" if args.fast_grad else "split"},
        "roofline": roof,
        "prefill_32k": {
            "fwd_ms": round(fwd_ms, 3), "bwd_ms": round(bwd_ms, 3),
            "bwd_stage_ms": {"prep": round(ph[1], 3), "dkdv": round(ph[2], 3),
                             "dq": round(ph[3], 3)},
            "fwd_eff_tflops": round(dense_fwd / (fwd_ms * 1e-3) / 1e12, 1),
            "bwd_eff_tflops": round(dense_bwd / (bwd_ms * 1e-3) / 1e12, 1),
            "fwd_kept_frac": kept_f / vis_f, "bwd_kept_frac": kept_b / vis_b,
            "slots_f": S_f / (B * HQ * N), "slots_b": S_b / (B * HQ * N),
            "tau0_fwd_ms": round(fwd0_ms, 3), "tau0_bwd_ms": round(bwd0_ms, 3),
            "speedup_vs_tau0": round((fwd0_ms + bwd0_ms) / (fwd_ms + bwd_ms), 4),
            "alg_tflops": {n: round(alg[n] / (tms[n] * 1e-3) / 1e12, 1) for n in alg},
        },
        "decode_128k": {
            "us_per_step": round(dec_all_us, 2),
            "split_us_with_mid_event": round(dsplit_us, 2),
            "merge_us_with_mid_event": round(dmerge_us, 2), "append_us": round(dappend_us, 2),
            "in_step_us": round((ph[4] + ph[5] + ph[6]) * 1e3, 2),
            "v_tiles_kept_frac": dec_vtiles / dec_tiles_total,
            # the whole step (split + merge): algorithmic bytes / step time
            "hbm_gbs": round(dec_bytes / (dec_all_us * 1e-6) / 1e9, 1),
            "hbm_frac": round(dec_bytes / (dec_all_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "split_hbm_frac": round(dec_bytes / (dsplit_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "bytes_per_step": dec_bytes,
        },
    }
    out["peak_memory"] = peak_memory(m, torch, q, k, v, do, scale, tau, args.fast_grad,
                                     qs[0], kc, vc, seqlens[0], cache0 + 1, y["scale"])

    # ------------------------------------------------------------ 128K prefill extra
    if not args.no_128k:
        del x, q, k, v, do, fo, bo
        torch.cuda.empty_cache()
        x4 = W.make_prefill(W.CONFIGS[4], device=dev)
        q4, k4, v4, do4 = x4["q"], x4["k"], x4["v"], x4["do"]
        n4 = q4.shape[2]
        f4 = dict(o=torch.empty_like(q4), lse=torch.empty(q4.shape[:3], device=dev))
        b4 = dict(dq=torch.empty_like(q4), dk=torch.empty_like(k4), dv=torch.empty_like(v4))
        res = {}
        for tau_ in (tau, 0.0):
            for _ in range(max(1, args.warmup // 2)):
                m.mala_fwd(q4, k4, v4, tau_, softmax_scale=x4["scale"], out=f4)
                m.mala_bwd(q4, k4, v4, f4["o"], f4["lse"], do4, tau_, softmax_scale=x4["scale"],
                           out=b4, fast_grad=args.fast_grad)
            torch.cuda.synchronize()
            tf = tb = 0.0
            reps = max(1, args.steps // 2)
            for _ in range(reps):
                ev[0].record()
                m.mala_fwd(q4, k4, v4, tau_, softmax_scale=x4["scale"], out=f4)
                ev[1].record()
                m.mala_bwd(q4, k4, v4, f4["o"], f4["lse"], do4, tau_, softmax_scale=x4["scale"],
                           out=b4, fast_grad=args.fast_grad)
                ev[2].record()
                torch.cuda.synchronize()
                tf += ev[0].elapsed_time(ev[1])
                tb += ev[1].elapsed_time(ev[2])
            res[tau_] = (tf / reps, tb / reps)
        p4 = q4.shape[0] * q4.shape[1] * causal_pairs(n4)
        out["prefill_128k"] = {
            "fwd_ms": round(res[tau][0], 3), "bwd_ms": round(res[tau][1], 3),
            "fwd_eff_tflops": round(4 * 128 * p4 / (res[tau][0] * 1e-3) / 1e12, 1),
            "bwd_eff_tflops": round(10 * 128 * p4 / (res[tau][1] * 1e-3) / 1e12, 1),
            "tau0_fwd_ms": round(res[0.0][0], 3), "tau0_bwd_ms": round(res[0.0][1], 3),
            "speedup_vs_tau0": round(sum(res[0.0]) / sum(res[tau]), 4),
        }
        del x4, q4, k4, v4, do4, f4, b4
        torch.cuda.empty_cache()
        x = W.make_prefill(cfg, device=dev)   # for the CPU sample below
        q, k, v, do = x["q"], x["k"], x["v"], x["do"]

    # ------------------------------------------------------------ structured-logit extra
    if not args.no_structured:
        keep_cpu = (q.cpu(), k.cpu(), v.cpu(), do.cpu()) if args.cpu_seconds > 0 else None
        del x, q, k, v, do
        torch.cuda.empty_cache()
        from contribution_gated_sparse_amd import fidelity as F
        out["structured"] = {
            preset: structured_section(args, m, F, W, torch, dev,
                                       ((fbq, fbk), (bbq, bbk), (dbk, dchunk)), preset)
            for preset in ("sparse", "calibrated")}
        if keep_cpu is not None:
            q, k, v, do = (t.to(dev) for t in keep_cpu)

    # ------------------------------------------------------------ CPU oracle baseline
    if args.cpu_seconds > 0:
        gf = m.mala_fwd(q, k, v, tau, softmax_scale=scale, want_mask=True)
        gb = m.mala_bwd(q, k, v, gf["o"], gf["lse"], do, tau, softmax_scale=scale,
                        want_mask=True, fast_grad=args.fast_grad)
        torch.cuda.synchronize()
        gpu = dict(fmask=gf["mask"], o=gf["o"], lse=gf["lse"], bmask=gb["mask"], dq=gb["dq"])
        out["cpu_baseline"], out["parity"] = cpu_baseline(
            q, k, v, do, scale, tau, (fbq, fbk), (bbq, bbk), args.cpu_seconds, gpu)
    print(json.dumps(out), flush=True)


def peak_memory(m, torch, q, k, v, do, scale, tau, fast_grad, qd, kc, vc, seq, n_k, dscale):
    """Peak device memory each operator call allocates (outputs and
    workspace, inputs resident beforehand), at tau and at tau = 0, from
    torch's allocator statistics (Sec. 3 "Operator Latency and Memory"
    compares MALA's peak operator memory with dense attention's). The bytes
    are those requested: the allocator's block sizes can exceed them by an
    unsplit remainder of a reused cached block, which depends on what was
    freed before, not on the call."""
    def cur():
        return torch.cuda.memory_stats().get("requested_bytes.all.current",
                                             torch.cuda.memory_allocated())

    def peak():
        return torch.cuda.memory_stats().get("requested_bytes.all.peak",
                                             torch.cuda.max_memory_allocated())
    res = {}
    # a first pass over both tolerances takes any one-time allocation (the
    # binding's cached buffers, the allocator's first blocks of a size) out
    # of the measured one
    for tau_ in (tau, 0.0, tau, 0.0):
        row = {}
        for name in ("fwd", "bwd", "decode"):
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            base = cur()
            torch.cuda.reset_peak_memory_stats()
            if name == "fwd":
                r = m.mala_fwd(q, k, v, tau_, softmax_scale=scale)
            elif name == "bwd":
                f = m.mala_fwd(q, k, v, tau_, softmax_scale=scale)
                torch.cuda.synchronize()
                base = cur()
                torch.cuda.reset_peak_memory_stats()
                r = m.mala_bwd(q, k, v, f["o"], f["lse"], do, tau_, softmax_scale=scale,
                               fast_grad=fast_grad)
            else:
                r = m.mala_decode(qd, kc, vc, seq, tau_, max_n_k=n_k, softmax_scale=dscale)
            torch.cuda.synchronize()
            row[name + "_bytes"] = int(peak() - base)
            del r
        res[f"tau={tau_:g}"] = row
    res["equal_to_tau0"] = res[f"tau={tau:g}"] == res["tau=0"]
    return res


def cpu_baseline(q, k, v, do, scale, tau, ftile, btile, budget, gpu=None):
    """Times the fp64 oracle on a bounded, seeded sample of 32-row query
    blocks of the 32K problem (forward + backward of those rows), and reports
    the dense-equivalent TFLOP/s of the sample. With ``gpu`` (the library's
    forward and backward outputs on the same inputs: masks, O, LSE, dQ) the
    sampled rows are also compared with the oracle's: the strict max-abs
    errors of O, LSE and dQ and the count of differing decisions outside the
    near-tie band (replayed inside it). Returns (baseline, parity)."""
    import numpy as np

    from oracle import mala_oracle as O
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    B, HQ, N, D = q.shape
    g = HQ // k.shape[1]
    rng = np.random.default_rng(7)
    bq = ftile[0]
    nblk = -(-N // bq)
    done_rows, flops, elapsed, nb = 0, 0.0, 0.0, 0
    kv_cache = {}
    err = {"O": 0.0, "LSE": 0.0, "dQ": 0.0}
    bad_decisions = 0
    n64 = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    while elapsed < budget and nb < 256:
        h = int(rng.integers(HQ))
        i = int(rng.integers(nblk))
        kh = h // g
        if kh not in kv_cache:
            kv_cache[kh] = (n64(k[0, kh])[None, None], n64(v[0, kh])[None, None])
        kn, vn = kv_cache[kh]
        r0, r1 = i * bq, min(N, i * bq + bq)
        qn = n64(q[0, h])[None, None]
        dn = n64(do[0, h])[None, None]
        qb = range(i * (bq // btile[0]), min(-(-N // btile[0]), (i + 1) * (bq // btile[0])))
        fmask = gpu["fmask"][:, h:h + 1].cpu().numpy() if gpu else None
        bmask = gpu["bmask"][:, h:h + 1].cpu().numpy() if gpu else None
        t0 = time.perf_counter()
        f = O.mala_fwd(qn, kn, vn, tau, scale, True, ftile[0], ftile[1], blocks=[(0, 0, i)],
                       replay=fmask, band=1e-3 if gpu else 0.0)
        o = np.nan_to_num(f["o"])
        lse = np.nan_to_num(f["lse"])
        rb = O.mala_bwd(qn, kn, vn, o, lse, dn, tau, scale, True, btile[0], btile[1], qblocks=qb,
                        replay=bmask, band=1e-3 if gpu else 0.0, o_storage="bf16",
                        lse_storage="f32")
        elapsed += time.perf_counter() - t0
        nb += 1
        rows = np.arange(r0, r1)
        flops += 14 * D * float((rows + 1).sum())
        done_rows += r1 - r0
        if gpu:
            seen = f["mask"][0, 0, i] != O.NOT_VISITED
            clear = seen & ~(np.abs(np.nan_to_num(f["margin"][0, 0, i], nan=np.inf)) < 1e-3)
            bad_decisions += int((f["mask"][0, 0, i][clear] != fmask[0, 0, i][clear]).sum())
            for j in qb:
                bseen = rb["mask"][0, 0, j] != O.NOT_VISITED
                bclear = bseen & ~(np.abs(np.nan_to_num(rb["margin"][0, 0, j], nan=np.inf)) < 1e-3)
                bad_decisions += int((rb["mask"][0, 0, j][bclear] != bmask[0, 0, j][bclear]).sum())
            err["O"] = max(err["O"], float(np.abs(n64(gpu["o"][0, h, r0:r1]) - f["o"][0, 0, r0:r1]).max()))
            err["LSE"] = max(err["LSE"], float(np.abs(n64(gpu["lse"][0, h, r0:r1])
                                                      - f["lse"][0, 0, r0:r1]).max()))
            err["dQ"] = max(err["dQ"], float(np.abs(n64(gpu["dq"][0, h, r0:r1])
                                                    - rb["dq"][0, 0, r0:r1]).max()))
    base = {"value": round(flops / elapsed / 1e12, 6) if elapsed else None, "unit": "TFLOP/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{nb} random 32-row query blocks (random heads) of the 32K problem, "
                      f"forward + backward of their rows against all causal keys, numpy fp64; "
                      f"{elapsed:.1f} s; dense-equivalent FLOPs / time",
            "cpu": platform.processor() or platform.machine()}
    parity = None
    if gpu:
        bars = {"O": 2e-2, "LSE": 1e-4, "dQ": 2e-2}
        parity = {"workload": "the same 32K problem, the blocks of the CPU sample",
                  "blocks": nb, "max_abs": {n_: float(f"{e:.3e}") for n_, e in err.items()},
                  "bars": bars, "decisions_differing_outside_band": bad_decisions,
                  "within_bars": bad_decisions == 0 and all(err[n_] <= bars[n_] for n_ in bars)}
    return base, parity


if __name__ == "__main__":
    main()
