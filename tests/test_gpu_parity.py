"""GPU parity: libmala (through its C ABI) against the CPU fp64 oracle on the
same seeded inputs. Decisions must match outside the near-tie band (forward
near ties are replayed so that later decisions stay comparable), kept-tile
counters exactly, and values within the stated tolerances."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import mala_oracle as O
from parity_util import (BAND, check_forward, check_nesting, compare_values, dtype_name, np64,
                         tiling)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # collected on CPU only to be deselected
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = "cuda"


def lib():
    import contribution_gated_sparse_amd as m
    return m


def to_dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def check_backward(x, tau, g_fwd, r_fwd, causal=True, qblocks=None, key_rows=None,
                   gate_pass=False, fwd_mask=None):
    m = lib()
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    kind = dtype_name(q)
    _, (bq, bk, _), _ = tiling()
    g = m.mala_bwd(q, k, v, g_fwd["o"], g_fwd["lse"], do, tau, causal=causal,
                   softmax_scale=x["scale"], want_mask=True, gate_pass=gate_pass,
                   fwd_mask=fwd_mask)
    torch.cuda.synchronize()
    gmask = g["mask"].cpu().numpy()
    r = O.mala_bwd(np64(q), np64(k), np64(v), r_fwd["o"], r_fwd["lse"], np64(do), tau,
                   x["scale"], causal, bq, bk, qblocks=qblocks, replay=gmask, band=BAND[kind],
                   o_storage=kind)
    checked = r["mask"] != O.NOT_VISITED
    clear = checked & ~(np.abs(r["margin"]) < BAND[kind])
    assert np.array_equal(gmask[clear], r["mask"][clear]), (
        f"backward decisions differ: {int((gmask[clear] != r['mask'][clear]).sum())}")
    if qblocks is None:
        assert np.array_equal(gmask != O.NOT_VISITED, checked)
        kept_o = (gmask == O.KEPT).sum(-1)
        assert np.array_equal(kept_o, g["kept"].cpu().numpy())
    nq = q.shape[2]
    if qblocks is None:
        rows = np.ones(q.shape[:3], bool)
    else:
        rows = np.zeros(q.shape[:3], bool)
        for i in qblocks:
            rows[:, :, i * bq:min(nq, (i + 1) * bq)] = True
    st = {}
    st["dq"] = compare_values("dQ", np64(g["dq"]), r["dq"], kind, rows)
    if key_rows is not None or qblocks is None:
        kr = slice(None) if key_rows is None else key_rows
        st["dk"] = compare_values("dK", np64(g["dk"])[:, :, kr], r["dk"][:, :, kr], kind)
        st["dv"] = compare_values("dV", np64(g["dv"])[:, :, kr], r["dv"][:, :, kr], kind)
    st["ties"] = int((checked & ~clear).sum())
    return g, r, st


# ------------------------------------------------------------- tiny fp32 config

@pytest.mark.parametrize("tau", [1e-4, 0.0, 1.0, 2.0, 10.0, 1e3])
def test_config1_fp32_fwd_bwd(tau):
    x = to_dev(W.make_prefill(W.CONFIGS[1]))
    g, r, st = check_forward(x, tau, max_ties=2)
    gb, rb, stb = check_backward(x, tau, g, r)
    check_nesting(g["mask"].cpu().numpy(), gb["mask"].cpu().numpy())


# ------------------------------------------------------------- bf16 shapes

SHAPES = [
    # (batch, hq, hkv, nq, nk, d)
    (1, 2, 2, 1, 1, 128),
    (1, 2, 1, 63, 63, 128),
    (1, 4, 1, 65, 65, 128),
    (2, 4, 2, 200, 200, 128),
    (1, 8, 2, 777, 777, 128),
    (1, 2, 2, 300, 300, 64),
    (1, 4, 4, 100, 356, 128),     # chunked prefill: bottom-right causal alignment
    (1, 2, 2, 1, 700, 128),       # one query row against a long prefix
    (1, 16, 1, 130, 130, 128),    # a 16-head GQA group on one KV head
    (3, 4, 2, 33, 97, 64),        # d = 64, batch 3, ragged tiles, chunked
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("tau", [0.0, 1e-4, 1.0, 100.0])
def test_bf16_shapes_fwd_bwd(shape, tau):
    b, hq, hkv, nq, nk, d = shape
    cfg = W.CONFIGS[2]
    x = W.make_prefill(cfg, n=nk, hq=hq, hkv=hkv, d=d, batch=b, planted=4, seed=7 + nq)
    if nq < nk:   # queries are the last nq rows
        x["q"] = x["q"][:, :, nk - nq:].contiguous()
        x["do"] = x["do"][:, :, nk - nq:].contiguous()
    x = to_dev(x)
    g, r, st = check_forward(x, tau, max_ties=4)
    gb, rb, stb = check_backward(x, tau, g, r)
    check_nesting(g["mask"].cpu().numpy(), gb["mask"].cpu().numpy())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noncausal(dtype):
    cfg = W.CONFIGS[2] if dtype == torch.bfloat16 else W.CONFIGS[1]
    d = 128 if dtype == torch.bfloat16 else 64
    x = W.make_prefill(cfg, n=160, hq=2, hkv=1, d=d, planted=3)
    x = to_dev(x)
    for tau in (0.0, 0.5, 50.0):
        g, r, _ = check_forward(x, tau, causal=False, max_ties=4)
        check_backward(x, tau, g, r, causal=False)


def test_fp32_d128_and_gqa():
    x = W.make_prefill(W.CONFIGS[1], n=150, hq=4, hkv=2, d=128, planted=4)
    x["scale"] = 1 / math.sqrt(128)
    x = to_dev(x)
    for tau in (0.0, 1e-4, 3.0):
        g, r, _ = check_forward(x, tau, max_ties=2)
        check_backward(x, tau, g, r)


# ------------------------------------------------------------- skipping inputs

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("tau", [1e-4, 1e-2, 1.0])
def test_structured_skipping_fwd_bwd(dtype, tau):
    """Structured logits (sinks, local band, retrieval keys) make the gate
    skip most far tiles; decisions, counters and values still match."""
    d = 128 if dtype == "bf16" else 64
    x = to_dev(W.make_structured(1000, hq=4, hkv=2, d=d, dtype=dtype,
                                 freqs=48 if d == 128 else 24))
    g, r, st = check_forward(x, tau, max_ties=4)
    assert st["kept_frac"] < 0.8
    gb, rb, stb = check_backward(x, tau, g, r)
    bm = gb["mask"].cpu().numpy()
    assert (bm == O.SKIPPED).sum() > 0
    check_nesting(g["mask"].cpu().numpy(), bm)


# ------------------------------------------------------------- gate pass

@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("tau", [0.0, 1e-4, 1.0, 100.0])
def test_gate_pass_shapes(shape, tau):
    """MALA_FLAG_GATE_PASS: decisions from the separate score pass, dK/dV over
    the steps with a kept tile only; same bar against the oracle."""
    b, hq, hkv, nq, nk, d = shape
    x = W.make_prefill(W.CONFIGS[2], n=nk, hq=hq, hkv=hkv, d=d, batch=b, planted=4, seed=7 + nq)
    if nq < nk:
        x["q"] = x["q"][:, :, nk - nq:].contiguous()
        x["do"] = x["do"][:, :, nk - nq:].contiguous()
    x = to_dev(x)
    print(f"[gate pass] shape={shape} tau={tau}", flush=True)
    g, r, _ = check_forward(x, tau, max_ties=4)
    gb, _, _ = check_backward(x, tau, g, r, gate_pass=True)
    check_nesting(g["mask"].cpu().numpy(), gb["mask"].cpu().numpy())


@pytest.mark.parametrize("tau", [1e-4, 1.0])
def test_gate_pass_structured(tau):
    """On skipping inputs the gate pass takes the default path's decisions
    (outside the near-tie band) and reproduces its gradients."""
    m = lib()
    x = to_dev(W.make_structured(1500, hq=8, hkv=2, d=128))
    g, r, st = check_forward(x, tau, max_ties=4)
    assert st["kept_frac"] < 0.8
    gb, rb, _ = check_backward(x, tau, g, r, gate_pass=True)
    ref = m.mala_bwd(x["q"], x["k"], x["v"], g["o"], g["lse"], x["do"], tau,
                     softmax_scale=x["scale"], want_mask=True)
    torch.cuda.synchronize()
    a, b_ = gb["mask"].cpu().numpy(), ref["mask"].cpu().numpy()
    clear = (a != O.NOT_VISITED) & ~(np.abs(rb["margin"]) < BAND["bf16"])
    assert np.array_equal(a[clear], b_[clear])
    assert (a == O.SKIPPED).sum() > 0
    for n in ("dq", "dk", "dv"):
        u, w = np64(gb[n]), np64(ref[n])
        assert np.abs(u - w).max() <= 2e-2 * max(1.0, np.abs(w).max()), n
    # on the forward's kept tiles only: the same decisions and gradients
    _, a2, b2, want = nested_vs_gate_pass(x, tau, g["mask"])
    if np.array_equal(a2["mask"].cpu().numpy(), want):
        for n in ("dq", "dk", "dv"):
            assert torch.equal(a2[n], b2[n]), n
    assert int((a2["mask"].cpu().numpy() != want).sum()) <= 2


def test_gate_pass_with_fast_grad():
    """Both flags: the gate pass's decisions and dK/dV with the single-bf16 dS
    of MALA_FLAG_FAST_GRAD in dQ; same decisions as the fast default path."""
    m = lib()
    x = to_dev(W.make_structured(900, hq=4, hkv=1, d=128))
    f = m.mala_fwd(x["q"], x["k"], x["v"], 1e-2, softmax_scale=x["scale"])
    a = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], 1e-2,
                   softmax_scale=x["scale"], want_mask=True, fast_grad=True)
    b = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], 1e-2,
                   softmax_scale=x["scale"], want_mask=True, fast_grad=True, gate_pass=True)
    torch.cuda.synchronize()
    ma, mb = a["mask"].cpu().numpy(), b["mask"].cpu().numpy()
    assert int((ma != mb).sum()) <= 2 and (mb == O.SKIPPED).sum() > 0
    if np.array_equal(ma, mb):
        assert torch.equal(a["dq"], b["dq"])
    for n in ("dq", "dk", "dv"):
        u, w = np64(b[n]), np64(a[n])
        assert np.abs(u - w).max() <= 1e-2 * max(1.0, np.abs(w).max()), n


def test_gate_pass_noncausal_and_f32():
    """Non-causal walks through the gate pass; the flag is ignored for fp32."""
    x = to_dev(W.make_prefill(W.CONFIGS[2], n=160, hq=2, hkv=1, d=128, planted=3))
    for tau in (0.0, 0.5, 50.0):
        g, r, _ = check_forward(x, tau, causal=False, max_ties=4)
        check_backward(x, tau, g, r, causal=False, gate_pass=True)
    x = to_dev(W.make_prefill(W.CONFIGS[1], n=150, hq=4, hkv=2, d=64, planted=4))
    g, r, _ = check_forward(x, 1.0, max_ties=2)
    check_backward(x, 1.0, g, r, gate_pass=True)


def expand_fwd(fmask, shape):
    """The forward tile mask on the backward partition (each backward tile
    lies in one forward tile)."""
    (fbq, fbk, _), (bbq, bbk, _), _ = tiling()
    up = np.repeat(np.repeat(fmask, fbq // bbq, axis=2), fbk // bbk, axis=3)
    return up[:, :, :shape[2], :shape[3]]


def nested_vs_gate_pass(x, tau, fwd_mask, causal=True):
    """mala_bwd_nested with ``fwd_mask`` against the gate pass on the same
    inputs: its decisions are the gate pass's restricted to the forward's
    kept tiles, bit for bit; returns both results and the expected mask."""
    m = lib()
    f = m.mala_fwd(x["q"], x["k"], x["v"], tau, causal=causal, softmax_scale=x["scale"])
    a = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], tau, causal=causal,
                   softmax_scale=x["scale"], want_mask=True, gate_pass=True)
    b = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], tau, causal=causal,
                   softmax_scale=x["scale"], want_mask=True, fwd_mask=fwd_mask)
    torch.cuda.synchronize()
    ma, mb = a["mask"].cpu().numpy(), b["mask"].cpu().numpy()
    up = expand_fwd(fwd_mask.cpu().numpy(), ma.shape)
    want = np.where((ma == O.KEPT) & (up != O.KEPT), O.SKIPPED, ma)
    assert np.array_equal(mb, want), f"{int((mb != want).sum())} decisions differ"
    assert np.array_equal(b["kept"].cpu().numpy(), (mb == O.KEPT).sum(-1))
    return f, a, b, want


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("tau", [0.0, 1e-4, 1.0, 100.0])
def test_nested_shapes(shape, tau):
    """mala_bwd_nested on the forward's own mask: the oracle's bar, support
    nested in the forward's, and the gate pass's decisions and gradients
    wherever the two agree (exact arithmetic makes them agree everywhere)."""
    b, hq, hkv, nq, nk, d = shape
    x = W.make_prefill(W.CONFIGS[2], n=nk, hq=hq, hkv=hkv, d=d, batch=b, planted=4, seed=7 + nq)
    if nq < nk:
        x["q"] = x["q"][:, :, nk - nq:].contiguous()
        x["do"] = x["do"][:, :, nk - nq:].contiguous()
    x = to_dev(x)
    print(f"[nested] shape={shape} tau={tau}", flush=True)
    g, r, _ = check_forward(x, tau, max_ties=4)
    gb, _, _ = check_backward(x, tau, g, r, fwd_mask=g["mask"])
    check_nesting(g["mask"].cpu().numpy(), gb["mask"].cpu().numpy())
    _, a, b_, want = nested_vs_gate_pass(x, tau, g["mask"])
    if np.array_equal(a["mask"].cpu().numpy(), want):
        for n in ("dq", "dk", "dv"):
            assert torch.equal(a[n], b_[n]), n


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("density", [0.0, 0.03, 0.5, 1.0])
def test_nested_arbitrary_forward_masks(causal, density):
    """The walk over the forward's kept tiles with masks the forward would not
    write (sparse, dense, empty; more than 64 key tiles, so the look-ahead
    window moves): decisions are exactly the gate pass's on the given tiles,
    and the gradients are the oracle's on that support."""
    nq, nk = 300, 4700
    x = W.make_prefill(W.CONFIGS[2], n=nk, hq=2, hkv=1, d=128, planted=4, seed=11)
    x["q"] = x["q"][:, :, nk - nq:].contiguous()
    x["do"] = x["do"][:, :, nk - nq:].contiguous()
    x = to_dev(x)
    tau = 1e-4
    print(f"[nested mask] causal={causal} density={density}", flush=True)
    fm = lib().mala_fwd(x["q"], x["k"], x["v"], tau, causal=causal, softmax_scale=x["scale"],
                        want_mask=True)["mask"].cpu().numpy()
    rng = np.random.default_rng(int(1000 * density) + causal)
    rand = np.where(rng.random(fm.shape) < density, O.KEPT, O.SKIPPED).astype(np.int8)
    fm = np.where(fm == O.NOT_VISITED, fm, rand)
    f, a, b, want = nested_vs_gate_pass(x, tau, torch.from_numpy(fm).to(DEV), causal=causal)
    if density == 0.0:
        assert not (want == O.KEPT).any()
        for n in ("dq", "dk", "dv"):
            assert not b[n].any(), n
    _, (bq, bk, _), _ = tiling()
    r = O.mala_bwd(np64(x["q"]), np64(x["k"]), np64(x["v"]), np64(f["o"]), np64(f["lse"]),
                   np64(x["do"]), tau, x["scale"], causal, bq, bk, replay=want, band=np.inf,
                   o_storage="bf16")
    assert np.array_equal(r["mask"], want)
    for n in ("dq", "dk", "dv"):
        compare_values(n, np64(b[n]), r[n], "bf16")


def test_backward_modes_are_deterministic():
    """Every backward mode gives the same bits on a second run: the default
    path, the gate pass (whose heavy key blocks sum per-head partials in head
    order) and the nested call."""
    m = lib()
    x = to_dev(W.make_structured(2000, hq=8, hkv=2, d=128))
    f = m.mala_fwd(x["q"], x["k"], x["v"], 1e-4, softmax_scale=x["scale"], want_mask=True)
    for kw in (dict(), dict(gate_pass=True), dict(fwd_mask=f["mask"])):
        runs = [m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], 1e-4,
                           softmax_scale=x["scale"], **kw) for _ in range(2)]
        torch.cuda.synchronize()
        for n in ("dq", "dk", "dv", "kept"):
            assert torch.equal(runs[0][n], runs[1][n]), (n, list(kw))


def test_nested_noncausal_fast_grad_and_f32():
    """The nested call with MALA_FLAG_FAST_GRAD, non-causal, and for fp32
    (where the forward mask is not read and the call is the backward)."""
    m = lib()
    x = to_dev(W.make_structured(900, hq=4, hkv=1, d=128))
    f = m.mala_fwd(x["q"], x["k"], x["v"], 1e-2, softmax_scale=x["scale"], want_mask=True)
    a = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], 1e-2,
                   softmax_scale=x["scale"], want_mask=True, fast_grad=True, gate_pass=True)
    b = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], 1e-2,
                   softmax_scale=x["scale"], want_mask=True, fast_grad=True, fwd_mask=f["mask"])
    torch.cuda.synchronize()
    if torch.equal(a["mask"], b["mask"]):
        for n in ("dq", "dk", "dv"):
            assert torch.equal(a[n], b[n]), n
    assert int((a["mask"] != b["mask"]).sum()) <= 2
    x = to_dev(W.make_prefill(W.CONFIGS[2], n=160, hq=2, hkv=1, d=128, planted=3))
    for tau in (0.0, 0.5, 50.0):
        g, r, _ = check_forward(x, tau, causal=False, max_ties=4)
        check_backward(x, tau, g, r, causal=False, fwd_mask=g["mask"])
    x = to_dev(W.make_prefill(W.CONFIGS[1], n=150, hq=4, hkv=2, d=64, planted=4))
    g, r, _ = check_forward(x, 1.0, max_ties=2)
    check_backward(x, 1.0, g, r, fwd_mask=g["mask"])


# ------------------------------------------------------------- decode

def check_decode(x, lens, tau, steps_q, max_ties=4, split_keys=0):
    m = lib()
    kc, vc = x["k_cache"], x["v_cache"]
    kind = dtype_name(kc)
    _, _, (_, dbk, chunk) = tiling()
    q = steps_q
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    print(f"[decode] {kind} lens={lens} tau={tau} split_keys={split_keys}", flush=True)
    g = m.mala_decode(q, kc, vc, seq, tau, max_n_k=max(lens), softmax_scale=x["scale"],
                      want_mask=True, split_keys=split_keys)
    torch.cuda.synchronize()
    if split_keys == 0:
        assert g["split"] == chunk
    chunk = g["split"]
    gmask = g["mask"].cpu().numpy()
    r = O.mala_decode(np64(q), np64(kc), np64(vc), lens, tau, x["scale"], chunk, dbk,
                      replay=gmask, band=BAND[kind])
    assert np.array_equal(gmask, r["mask"]), "decode decisions differ outside the near-tie band"
    assert r["near_ties"] <= max_ties
    kept = g["kept"].cpu().numpy()
    hq = q.shape[1]
    assert np.array_equal(kept[:, :hq], (r["mask"] == O.KEPT).sum((-1, -2)))
    assert np.array_equal(kept[:, hq:], r["v_tiles"].sum((-1, -2)))
    compare_values("decode O", np64(g["o"]), r["o"], kind)
    dl = float(np.abs(np64(g["lse"]) - r["lse"]).max())
    assert dl <= (1e-5 if kind == "f32" else 2e-3)
    return g, r


@pytest.mark.parametrize("tau", [0.0, 1e-4, 1.0, 50.0])
def test_decode_bf16_small(tau):
    x = W.make_decode(W.CONFIGS[5], cache=1100, steps=3, batch=3, planted=16)
    x = to_dev(x)
    lens = [1103, 1101, 257]
    q = x["q_steps"][2]
    check_decode(x, lens, tau, q.contiguous())


@pytest.mark.parametrize("tau", [0.0, 1e-4, 1.0, 50.0])
def test_decode_f32_small(tau):
    x = W.make_decode(W.CONFIGS[5], cache=600, steps=2, batch=2, hq=4, hkv=2, planted=8)
    x = {k: (v.float() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    x = to_dev(x)
    check_decode(x, [602, 65], tau, x["q_steps"][1].contiguous())


# split lengths other than the default: one tile per split, splits that are
# not whole groups of four tiles, several 32-tile decision words per split,
# the automatic rule, and one split per sequence (App. A.1 "Fused decoding
# execution": each split tests its tiles against its own partial normalizer)
@pytest.mark.parametrize("split_keys", [64, 192, 512, 2560, -1, 8192])
@pytest.mark.parametrize("tau", [0.0, 1e-4, 1.0])
def test_decode_bf16_split_lengths(split_keys, tau):
    x = W.make_decode(W.CONFIGS[5], cache=4100, steps=1, batch=3, planted=24)
    x = to_dev(x)
    g, r = check_decode(x, [4101, 3001, 257], tau, x["q_steps"][0].contiguous(),
                        split_keys=split_keys)
    if split_keys == 8192:
        assert g["split"] == 4160 and g["mask"].shape[2] == 1


# one split per sequence runs as three passes (tile statistics, per-head gate
# replay, P V over kept tiles); other group shapes: 16 query heads per KV head
# (a 1024-thread gate workgroup) and 4 per KV head with two KV heads
@pytest.mark.parametrize("hq,hkv", [(16, 1), (8, 2)])
@pytest.mark.parametrize("tau", [0.0, 1.0])
def test_decode_bf16_unsplit_groups(hq, hkv, tau):
    x = W.make_decode(W.CONFIGS[5], cache=3000, steps=1, batch=2, hq=hq, hkv=hkv, planted=12)
    x = to_dev(x)
    g, r = check_decode(x, [3001, 1500], tau, x["q_steps"][0].contiguous(), split_keys=8192)
    assert g["split"] == 3008 and g["mask"].shape[2] == 1


@pytest.mark.parametrize("split_keys", [64, 320, 2560])
def test_decode_f32_split_lengths(split_keys):
    x = W.make_decode(W.CONFIGS[5], cache=2200, steps=1, batch=2, hq=4, hkv=2, planted=8)
    x = {k: (v.float() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    x = to_dev(x)
    check_decode(x, [2201, 130], 1e-4, x["q_steps"][0].contiguous(), split_keys=split_keys)


def test_decode_clamps_out_of_range_lengths():
    """seqlens_k outside [1, max_n_k] is clamped on the device (the header's
    contract): lengths 0 and 5000 with max_n_k = 701 give exactly the results
    of lengths 1 and 701."""
    m = lib()
    x = to_dev(W.make_decode(W.CONFIGS[5], cache=700, steps=1, batch=2, planted=4))
    q = x["q_steps"][0].contiguous()
    outs = []
    for lens in ([0, 5000], [1, 701]):
        seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
        g = m.mala_decode(q, x["k_cache"], x["v_cache"], seq, 1e-4, max_n_k=701,
                          softmax_scale=x["scale"], want_mask=True)
        torch.cuda.synchronize()
        outs.append({k_: g[k_].cpu() for k_ in ("o", "lse", "mask", "kept")})
    for k_ in outs[0]:
        assert torch.equal(outs[0][k_], outs[1][k_]), k_


def test_decode_group16_and_single_key():
    x = W.make_decode(W.CONFIGS[5], cache=300, steps=1, batch=2, hq=16, hkv=1, planted=4)
    x = to_dev(x)
    check_decode(x, [1, 301], 1e-4, x["q_steps"][0].contiguous())


# ------------------------------------------------------------- empty / errors on device

def test_empty_query_rows():
    m = lib()
    q = torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV)
    k = torch.randn((1, 2, 5, 128), device=DEV).to(torch.bfloat16)
    out = m.mala_fwd(q, k, k, 1e-4)
    assert out["o"].shape == (1, 2, 0, 128)
    b = m.mala_bwd(q, k, k, out["o"], out["lse"], q, 1e-4)
    torch.cuda.synchronize()
    assert torch.count_nonzero(b["dk"]) == 0 and torch.count_nonzero(b["dv"]) == 0
    # the gate-pass walks and the nested call write the zero dK, dV themselves
    f = m.mala_fwd(q, k, k, 1e-4, want_mask=True)
    for kw in (dict(gate_pass=True), dict(fwd_mask=f["mask"])):
        dk = torch.full_like(k, 7.0)
        g = m.mala_bwd(q, k, k, f["o"], f["lse"], q, 1e-4, out=dict(dk=dk), **kw)
        torch.cuda.synchronize()
        assert torch.count_nonzero(g["dk"]) == 0 and torch.count_nonzero(g["dv"]) == 0, kw


def test_fast_grad_flag_same_support():
    """MALA_FLAG_FAST_GRAD changes only the precision of dS in dQ: the
    decisions, dK and dV are identical and dQ stays within tolerance on the
    Gaussian workload."""
    m = lib()
    x = to_dev(W.make_prefill(W.CONFIGS[3], n=600, hq=4, hkv=1, planted=8))
    f = m.mala_fwd(x["q"], x["k"], x["v"], 1e-4, softmax_scale=x["scale"])
    a = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], 1e-4,
                   softmax_scale=x["scale"], want_mask=True)
    b = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], 1e-4,
                   softmax_scale=x["scale"], want_mask=True, fast_grad=True)
    torch.cuda.synchronize()
    assert torch.equal(a["mask"], b["mask"])
    assert torch.equal(a["dv"], b["dv"])
    assert torch.equal(a["dk"], b["dk"])
    r = O.mala_fwd(np64(x["q"]), np64(x["k"]), np64(x["v"]), 1e-4, x["scale"], True,
                   *tiling()[0][:2], replay=m.mala_fwd(x["q"], x["k"], x["v"], 1e-4,
                   softmax_scale=x["scale"], want_mask=True)["mask"].cpu().numpy(), band=1e-3)
    rb = O.mala_bwd(np64(x["q"]), np64(x["k"]), np64(x["v"]), r["o"], r["lse"], np64(x["do"]),
                    1e-4, x["scale"], True, *tiling()[1][:2], o_storage="bf16")
    for name in ("dq", "dk"):
        compare_values(name + " fast", np64(b[name]), rb[name], "bf16")
        compare_values(name + " split", np64(a[name]), rb[name], "bf16")


# ------------------------------------------------------------- autograd entry

@pytest.mark.parametrize("gate_pass", [False, True])
def test_autograd_chunked_prefill_matches_direct_calls(gate_pass):
    """mala_attention (torch.autograd) runs the same two C-ABI calls: its
    output and gradients equal mala_fwd / mala_bwd bit for bit, here on a
    chunked prefill (the last 100 of 356 positions query all 356 keys) whose
    inputs come from an upstream torch op, so the gradient flows through it.
    With ``gate_pass`` the forward also writes its tile mask and the backward
    is mala_bwd_nested on it."""
    m = lib()
    x = to_dev(W.make_prefill(W.CONFIGS[2], n=356, hq=4, hkv=2, planted=4, seed=11))
    scale = x["scale"]
    base = x["q"][:, :, -100:].float().clone().requires_grad_()
    k = x["k"].clone().requires_grad_()
    v = x["v"].clone().requires_grad_()
    do = x["do"][:, :, -100:].contiguous()
    q = (base * 1.0).to(torch.bfloat16).contiguous()        # upstream op
    o = m.mala_attention(q, k, v, 1e-4, softmax_scale=scale, gate_pass=gate_pass)
    o.backward(do)
    qd = q.detach()
    f = m.mala_fwd(qd, k.detach(), v.detach(), 1e-4, softmax_scale=scale, want_mask=gate_pass)
    b = m.mala_bwd(qd, k.detach(), v.detach(), f["o"], f["lse"], do, 1e-4, softmax_scale=scale,
                   fwd_mask=f["mask"])
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), f["o"])
    assert torch.equal(base.grad, b["dq"].float())
    assert torch.equal(k.grad, b["dk"]) and torch.equal(v.grad, b["dv"])


# ------------------------------------------------------------- staged entry points

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_staged_entry_points_match_single_calls(dtype):
    """mala_bwd_stage (PREP, DKDV, DQ) and mala_decode_stage (SPLIT, COMBINE),
    the calls bench.py times one by one, give bit-identical results to
    mala_bwd and mala_decode, including the decisions and the counters."""
    m = lib()
    cfg = W.CONFIGS[2] if dtype == torch.bfloat16 else W.CONFIGS[1]
    x = W.make_prefill(cfg, n=300, hq=4, hkv=2, d=128 if dtype == torch.bfloat16 else 64,
                       planted=4, seed=21)
    x = to_dev({k: (v.to(dtype) if isinstance(v, torch.Tensor) else v) for k, v in x.items()})
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    f = m.mala_fwd(q, k, v, 1e-2, softmax_scale=x["scale"])
    a = m.mala_bwd(q, k, v, f["o"], f["lse"], do, 1e-2, softmax_scale=x["scale"], want_mask=True)
    b = m.mala_bwd(q, k, v, f["o"], f["lse"], do, 1e-2, softmax_scale=x["scale"], want_mask=True,
                   stages=(m.mala.BWD_PREP, m.mala.BWD_DKDV, m.mala.BWD_DQ))
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "mask", "kept"):
        assert torch.equal(a[name], b[name]), name

    y = W.make_decode(W.CONFIGS[5], cache=700, steps=1, batch=2, planted=4)
    y = to_dev({k: (v.to(dtype) if isinstance(v, torch.Tensor) and v.is_floating_point() else v)
                for k, v in y.items()})
    if dtype == torch.float32:
        y["k_cache"], y["v_cache"] = y["k_cache"][..., :64].contiguous(), y["v_cache"][..., :64].contiguous()
        y["q_steps"] = y["q_steps"][..., :64].contiguous()
    qd = y["q_steps"][0].contiguous()
    seq = torch.tensor([701, 300], dtype=torch.int32, device=DEV)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    c = m.mala_decode(qd, y["k_cache"], y["v_cache"], seq, 1e-2, max_n_k=701, want_mask=True)
    e = m.mala_decode(qd, y["k_cache"], y["v_cache"], seq, 1e-2, max_n_k=701, want_mask=True,
                      events=ev)
    torch.cuda.synchronize()
    for name in ("o", "lse", "mask", "kept"):
        assert torch.equal(c[name], e[name]), name
